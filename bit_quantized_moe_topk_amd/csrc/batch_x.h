// fp16 activation copies (header-only): the small-batch gate/up kernel's lane
// layout, and the row-major copy of the prefill tiles; batch.hip and
// mfma.hip read them, and the grouping launches can write them beside their
// own work.
#pragma once

#include "common.h"
#include "gemv.h"

namespace moe {

// Activation operand layout (x16 in fast mode below 256 tokens). The lane
// (token, lane group c) of wave w takes, for each of its NBL blocks b and K
// step kk, eight fp16 values in the weight operand's K order: Q2, weights
// 8 kk .. 8 kk + 7 with each group of four as 0, 2, 1, 3; Q3 (the FP8 form's
// order), weights 16 w' + 4 (i & 3) + 2 h + (i >> 2) at position i for
// kk = 2 w' + h. Each token row stores these operands as 16-byte chunks, the
// chunk of (w, c, q = 4 b + kk) at w H / 64 + 4 q + c: the four lane groups'
// chunks of one step sit side by side, so each load instruction of a wave
// reads 64 contiguous bytes per token rather than 16 bytes from each of 64
// places.
template <int Q, bool XBF16>
__device__ inline uint4 xs_chunk(const void* x, int H, int t, int j, int e) {
  const int NBL = H / 1024, per_w = H / 64;
  const int w = j / per_w, r = j % per_w, q = r >> 2, c = r & 3;
  const int kb = w * (H / 256) + NBL * c + (q >> 2), kk = q & 3;
  const size_t e0 = (size_t)t * H + 32 * kb;
  float f[8];
  if constexpr (Q == 3) {
    // word kk / 2 of the block, half h: pairs (s, s + 4), (s + 8, s + 12) for s = 2 h, 2 h + 1
    const size_t wb = e0 + 16 * (kk >> 1);
    const int h = kk & 1;
    float v[16];
    if constexpr (XBF16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + wb);
      const uint4 a0 = p[0], a1 = p[1];
      const uint32_t u[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(u[i]);
        v[2 * i + 1] = bf16_hi(u[i]);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + wb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 g = p[i];
        v[4 * i] = g.x;
        v[4 * i + 1] = g.y;
        v[4 * i + 2] = g.z;
        v[4 * i + 3] = g.w;
      }
    }
    if (h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = v[4 * (i & 3) + (i >> 2) + 2];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = v[4 * (i & 3) + (i >> 2)];
    }
  } else {
    const size_t cb = e0 + 8 * kk;
    float v[8];
    if constexpr (XBF16) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + cb);
      const uint32_t u[4] = {a0.x, a0.y, a0.z, a0.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(u[i]);
        v[2 * i + 1] = bf16_hi(u[i]);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + cb);
      const float4 g0 = p[0], g1 = p[1];
      v[0] = g0.x; v[1] = g0.y; v[2] = g0.z; v[3] = g0.w;
      v[4] = g1.x; v[5] = g1.y; v[6] = g1.z; v[7] = g1.w;
    }
    f[0] = v[0]; f[1] = v[2]; f[2] = v[1]; f[3] = v[3];
    f[4] = v[4]; f[5] = v[6]; f[6] = v[5]; f[7] = v[7];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = __builtin_ldexpf(f[i], -e);
  return make_uint4(pack_half2(f[0], f[1]), pack_half2(f[2], f[3]), pack_half2(f[4], f[5]),
                    pack_half2(f[6], f[7]));
}

// Row-major fp16 copy of the prefill tiles: 16-byte chunk i holds elements
// 8 i .. 8 i + 7 of the flat [T][H] activations, each group of four as
// 0, 2, 1, 3 (their K order), scaled by 2^-e.
template <bool XBF16>
__device__ inline uint4 x16_chunk(const void* x, long i, int e) {
  float f[8];
  if constexpr (XBF16) {
    const uint4 v = static_cast<const uint4*>(x)[i];
    f[0] = bf16_lo(v.x); f[1] = bf16_lo(v.y); f[2] = bf16_hi(v.x); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_lo(v.w); f[6] = bf16_hi(v.z); f[7] = bf16_hi(v.w);
  } else {
    const float4* src = static_cast<const float4*>(x) + 2 * i;
    const float4 f0 = src[0], f1 = src[1];
    f[0] = f0.x; f[1] = f0.z; f[2] = f0.y; f[3] = f0.w;
    f[4] = f1.x; f[5] = f1.z; f[6] = f1.y; f[7] = f1.w;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) f[u] = __builtin_ldexpf(f[u], -e);
  return make_uint4(pack_half2(f[0], f[1]), pack_half2(f[2], f[3]), pack_half2(f[4], f[5]),
                    pack_half2(f[6], f[7]));
}

// Largest |x| of token row t (every lane of the wave gets it): an integer max
// over the magnitude bits, which order finite values like the values (NaN
// sorts above infinity).
__device__ inline float row_absmax(const void* x, int xbf16, int H, int t) {
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;
  if (xbf16) {
    const uint4* row = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * H);
    for (int j = lane; j < H / 8; j += 64) {
      const uint4 v = row[j];
      const uint32_t a = max(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu);
      const uint32_t b = max(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu);
      m = max(m, max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16)) << 16);
    }
  } else {
    const uint4* row = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + (size_t)t * H);
    for (int j = lane; j < H / 4; j += 64) {
      const uint4 v = row[j];
      m = max(m, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
    }
  }
  return __uint_as_float(wave_max_u32(m));
}

// A request to write one of the copies (xs == nullptr: none), with the
// per-token exponents (row_exp) into xe [T].
struct XsJob {
  const void* x;
  int xbf16, q, H, T;
  uint4* xs;
  int32_t* xe;
};

// The copy named by xj.q (2, 3: the small-batch layout for that code width;
// 0: the prefill copy), one wave per token row: rows w0, w0 + ws, ... Each row
// is scaled by 2^-e (e = row_exp of its largest |x|; the row is read twice,
// the second time from cache) and e goes to xj.xe.
__device__ inline void xs_write_rows(const XsJob& xj, int w0, int ws) {
  const int lane = threadIdx.x & 63;
  const int H = xj.H, per_row = H / 8;
  for (int t = w0; t < xj.T; t += ws) {
    const int e = row_exp(row_absmax(xj.x, xj.xbf16, H, t));
    if (lane == 0) xj.xe[t] = e;
    for (int j = lane; j < per_row; j += 64) {
      uint4 v;
      if (xj.q == 3) v = xj.xbf16 ? xs_chunk<3, true>(xj.x, H, t, j, e) : xs_chunk<3, false>(xj.x, H, t, j, e);
      else if (xj.q == 2) v = xj.xbf16 ? xs_chunk<2, true>(xj.x, H, t, j, e) : xs_chunk<2, false>(xj.x, H, t, j, e);
      else {
        const long i = (long)t * per_row + j;
        v = xj.xbf16 ? x16_chunk<true>(xj.x, i, e) : x16_chunk<false>(xj.x, i, e);
      }
      xj.xs[(size_t)t * per_row + j] = v;
    }
  }
}

}  // namespace moe

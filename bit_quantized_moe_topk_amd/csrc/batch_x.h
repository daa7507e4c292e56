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
__device__ inline uint4 xs_chunk(const void* x, int H, int t, int j) {
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
  return make_uint4(pack_half2(f[0], f[1]), pack_half2(f[2], f[3]), pack_half2(f[4], f[5]),
                    pack_half2(f[6], f[7]));
}

// Row-major fp16 copy of the prefill tiles: 16-byte chunk i holds elements
// 8 i .. 8 i + 7 of the flat [T][H] activations, each group of four as
// 0, 2, 1, 3 (their K order).
template <bool XBF16>
__device__ inline uint4 x16_chunk(const void* x, long i) {
  if constexpr (XBF16) {
    const uint4 v = static_cast<const uint4*>(x)[i];
    return make_uint4(pack_half2(bf16_lo(v.x), bf16_lo(v.y)), pack_half2(bf16_hi(v.x), bf16_hi(v.y)),
                      pack_half2(bf16_lo(v.z), bf16_lo(v.w)), pack_half2(bf16_hi(v.z), bf16_hi(v.w)));
  } else {
    const float4* src = static_cast<const float4*>(x) + 2 * i;
    const float4 f0 = src[0], f1 = src[1];
    return make_uint4(pack_half2(f0.x, f0.z), pack_half2(f0.y, f0.w), pack_half2(f1.x, f1.z),
                      pack_half2(f1.y, f1.w));
  }
}

// Chunks [j0, n) step js (n = T H / 8) of the copy named by Q, written to xs:
// Q = 2, 3 the small-batch layout for that code width, Q = 0 the prefill copy.
__device__ inline void xs_write(const void* x, int xbf16, int Q, int H, long j0, long n, long js,
                                uint4* xs) {
  const int per_row = H / 8;
  for (long i = j0; i < n; i += js) {
    const int t = (int)(i / per_row), j = (int)(i % per_row);
    uint4 v;
    if (Q == 3) v = xbf16 ? xs_chunk<3, true>(x, H, t, j) : xs_chunk<3, false>(x, H, t, j);
    else if (Q == 2) v = xbf16 ? xs_chunk<2, true>(x, H, t, j) : xs_chunk<2, false>(x, H, t, j);
    else v = xbf16 ? x16_chunk<true>(x, i) : x16_chunk<false>(x, i);
    xs[i] = v;
  }
}

// A request to write one of the copies (xs == nullptr: none).
struct XsJob {
  const void* x;
  int xbf16, q, H, T;
  uint4* xs;
};

}  // namespace moe

// Gate-weighted combine of the expert outputs.
//
// y[t] = sum_{j<k} o[slot_of[t*k+j]] + o[slot_of[T*k+t]] (shared expert), in
// that order, where o already carries the gate (the down kernels multiply by
// it); fp32 sums, one rounding to y. Every call form except the decode-window
// kernels (which sum in LDS and write y themselves) ends with this gather:
// check mode, the small-batch kernels and the prefill tiles all store one o
// row per assignment slot (fp32 below 256 tokens, bf16 above).
#include "common.h"

namespace moe {
namespace {

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16 bytes of o: 4 fp32 or 8 bf16 values, as fp32.
template <typename OT>
struct Piece {
  static constexpr int N = 16 / sizeof(OT);
  float v[N];
};
__device__ inline Piece<float> unpack(uint4 u, const float*) {
  Piece<float> p;
  p.v[0] = __uint_as_float(u.x);
  p.v[1] = __uint_as_float(u.y);
  p.v[2] = __uint_as_float(u.z);
  p.v[3] = __uint_as_float(u.w);
  return p;
}
__device__ inline Piece<uint16_t> unpack(uint4 u, const uint16_t*) {
  Piece<uint16_t> p;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p.v[2 * i] = __uint_as_float(w[i] << 16);
    p.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return p;
}

constexpr int kCombineBatch = 8;  // slot rows of one token in flight at once

// One thread per 16 bytes of o (4 fp32 or 8 bf16 outputs) of a token row. The
// token's slot indices are read first (one scalar load each), then up to
// kCombineBatch slot rows are requested before any is added; the sum runs in
// slot order j = 0 .. n-1, so the result does not depend on the batching.
template <typename OT, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const OT* __restrict__ o,
                                                      const int32_t* __restrict__ slot_of, int T,
                                                      int k, int has_shared, int H, void* y) {
  constexpr int V = Piece<OT>::N;
  const int c = (blockIdx.x * 256 + threadIdx.x) * V;
  if (c >= H) return;
  const int n = k + has_shared;
  const int A = T * n;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < n; j0 += kCombineBatch) {
      uint4 u[kCombineBatch];
      bool ok[kCombineBatch];
#pragma unroll
      for (int b = 0; b < kCombineBatch; ++b) {
        const int j = j0 + b;
        int sl = -1;
        if (j < n) sl = slot_of[j < k ? t * k + j : T * k + t];
        ok[b] = (unsigned)sl < (unsigned)A;  // false past n, or for an invalid grouping
        u[b] = ok[b] ? *reinterpret_cast<const uint4*>(o + (size_t)sl * H + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < kCombineBatch; ++b) {
        if (!ok[b]) continue;
        const Piece<OT> p = unpack(u[b], o);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += p.v[i];
      }
    }
    if (OUT_F32) {
      float* dst = static_cast<float*>(y) + (size_t)t * H + c;
#pragma unroll
      for (int i = 0; i < V; i += 4)
        *reinterpret_cast<float4*>(dst + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    } else {
      uint32_t w[V / 2];
#pragma unroll
      for (int i = 0; i < V / 2; ++i)
        w[i] = (uint32_t)f32_to_bf16_rne(acc[2 * i]) | ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
      uint16_t* dst = static_cast<uint16_t*>(y) + (size_t)t * H + c;
      if constexpr (V == 8)
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
  }
}

template <typename OT>
hipError_t launch_t(const Experts& ex, const FfnArgs& a, const OT* o, hipStream_t s) {
  constexpr int V = Piece<OT>::N;
  dim3 grid((ex.H / V + 255) / 256, a.T < 65535 ? a.T : 65535);
  if (a.out_f32)
    MOE_LAUNCH("combine", s, (combine_kernel<OT, true>), grid, dim3(256), 0, s, o, a.slot_of, a.T,
               a.k, ex.has_shared, ex.H, a.y);
  else
    MOE_LAUNCH("combine", s, (combine_kernel<OT, false>), grid, dim3(256), 0, s, o, a.slot_of, a.T,
               a.k, ex.has_shared, ex.H, a.y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  if (a.o) return launch_t<float>(ex, a, a.o, s);
  return launch_t<uint16_t>(ex, a, a.ob, s);
}

}  // namespace moe

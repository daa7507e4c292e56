// Gate-weighted combine of the expert outputs.
//
// y[t] = sum_{j<k} o[slot_of[t*k+j]] + o[slot_of[T*k+t]] (shared expert), in
// that order, where o already carries the gate (the down kernels multiply by
// it); fp32 sums, one rounding to y. This is the path for fp32 check mode and
// for fast mode with many tokens; with few tokens the down kernels add straight
// into an fp32 accumulator instead.
#include "common.h"

namespace moe {
namespace {

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float4 load4(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}

// One thread per 4 consecutive output elements of a token row.
template <typename OT, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const OT* __restrict__ o,
                                                      const int32_t* __restrict__ slot_of, int T,
                                                      int k, int has_shared, int H, void* y) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  const int n = k + has_shared;
  const int A = T * n;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < n; ++j) {
      const int a = j < k ? t * k + j : T * k + t;
      const int sl = slot_of[a];
      if ((unsigned)sl >= (unsigned)A) continue;  // only for an invalid grouping
      const float4 v = load4(o + (size_t)sl * H + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    if (OUT_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * H + c) = acc;
    } else {
      uint2 p;
      p.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
      p.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (size_t)t * H + c) = p;
    }
  }
}

template <typename OT>
hipError_t launch_t(const Experts& ex, const FfnArgs& a, const OT* o, hipStream_t s) {
  dim3 grid((ex.H / 4 + 255) / 256, a.T < 65535 ? a.T : 65535);
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

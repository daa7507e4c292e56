// Device-side scheduling of the expert FFN and the gate-weighted combine.
//
// Scheduling never returns to the host: one workgroup reads the per-expert
// assignment counts of the grouping and writes two work lists,
//   GEMV experts : 1 .. gemv_max tokens (weights streamed once, decode shape);
//   MFMA tiles   : kTileM-token tiles of every larger expert,
// which the FFN kernels walk with a fixed-size grid (surplus workgroups exit).
// Only routed experts a token picked are computed (empty experts get no work),
// as in the pages' prefill, which copies and multiplies only routed experts.
//
// Combine: y[t] = sum_{j<k} o[slot_of[t*k+j]] + o[slot_of[T*k+t]] (shared), in
// that order, where o already carries the gate; fp32 sums, one rounding to y.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void sched_kernel(const int32_t* __restrict__ counts, int E_tot,
                                                     int gemv_max, int* hdr, int* gemv,
                                                     int* tiles) {
  __shared__ int n_g[1024], n_t[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (E_tot + nt - 1) / nt;
  const int lo = min(E_tot, tid * per), hi = min(E_tot, lo + per);
  int cg = 0, ct = 0;
  for (int e = lo; e < hi; ++e) {
    const int M = counts[e];
    if (M > 0 && M <= gemv_max) cg += 1;
    else if (M > gemv_max) ct += (M + kTileM - 1) / kTileM;
  }
  n_g[tid] = cg;
  n_t[tid] = ct;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int vg = tid >= off ? n_g[tid - off] : 0;
    const int vt = tid >= off ? n_t[tid - off] : 0;
    __syncthreads();
    n_g[tid] += vg;
    n_t[tid] += vt;
    __syncthreads();
  }
  int pg = n_g[tid] - cg, pt = n_t[tid] - ct;
  for (int e = lo; e < hi; ++e) {
    const int M = counts[e];
    if (M > 0 && M <= gemv_max) {
      gemv[pg++] = e;
    } else if (M > gemv_max) {
      const int n = (M + kTileM - 1) / kTileM;
      for (int i = 0; i < n; ++i) tiles[pt++] = (e << 16) | i;
    }
  }
  if (tid == nt - 1) {
    hdr[0] = n_g[nt - 1];
    hdr[1] = n_t[nt - 1];
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One thread per 4 consecutive output elements.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
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
    const float4 v = *reinterpret_cast<const float4*>(o + (size_t)sl * H + c);
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

}  // namespace

hipError_t launch_sched(const Experts& ex, const FfnArgs& a, int gemv_max_tokens, hipStream_t s) {
  SchedView v = sched_view(a.sched, ex.E_tot);
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, s, a.counts, ex.E_tot, gemv_max_tokens,
                     v.hdr, v.gemv, v.tiles);
  return hipGetLastError();
}

hipError_t launch_combine(const Experts& ex, const FfnArgs& a, int out_f32, hipStream_t s) {
  dim3 grid((ex.H / 4 + 255) / 256, a.T < 65535 ? a.T : 65535);
  if (out_f32)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, a.o, a.slot_of, a.T, a.k,
                       ex.has_shared, ex.H, a.y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, a.o, a.slot_of, a.T, a.k,
                       ex.has_shared, ex.H, a.y);
  return hipGetLastError();
}

}  // namespace moe

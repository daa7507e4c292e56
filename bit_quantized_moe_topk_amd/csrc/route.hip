// Top-k expert selection and softmax gates: one 64-wide wavefront per token
// (the per-token work is topk_token in topk.h).
#include "common.h"
#include "topk.h"

namespace moe {
namespace {

template <int PER_LANE>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gates) {
  __shared__ TopkScratch sc[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<PER_LANE>(logits + (size_t)t * E, E, k, idx + (size_t)t * k, gates + (size_t)t * k,
                       &sc[threadIdx.x >> 6]);
}

template <int P>
hipError_t launch_p(const float* logits, int T, int E, int k, int32_t* idx, float* gates,
                    hipStream_t s) {
  MOE_LAUNCH("topk", s, topk_kernel<P>, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx,
             gates);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* gates,
                       hipStream_t s) {
  const int per = (E + 63) / 64;
  if (per <= 1) return launch_p<1>(logits, T, E, k, idx, gates, s);
  if (per <= 2) return launch_p<2>(logits, T, E, k, idx, gates, s);
  if (per <= 4) return launch_p<4>(logits, T, E, k, idx, gates, s);
  if (per <= 8) return launch_p<8>(logits, T, E, k, idx, gates, s);
  if (per <= 16) return launch_p<16>(logits, T, E, k, idx, gates, s);
  return launch_p<32>(logits, T, E, k, idx, gates, s);
}

}  // namespace moe

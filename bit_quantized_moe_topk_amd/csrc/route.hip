// Top-k expert selection and softmax gates: one 64-wide wavefront per token.
//
// The router scores every expert of the layer for each token and keeps the 10
// best of 512 ("Strata - the details", "How it works"; the Strata README,
// "How does it work?"). Each lane holds ceil(E/64) logits as 64-bit keys
//   key = (orderable(logit) << 32) | (0xFFFFFFFF - expert)
// so one unsigned maximum picks the largest logit and, among equal logits, the
// lower expert index. k rounds of lane-local max + a butterfly max over the
// wave select the experts in rank order; the owning lane retires its key.
#include "common.h"

namespace moe {
namespace {

// Monotone map float -> uint32 (larger float -> larger code). -0 is folded to +0
// so the two compare equal; every NaN maps to 0, below -inf.
__device__ inline uint32_t orderable(float v) {
  if (v != v) return 0u;
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float from_orderable(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;

  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ((uint64_t)orderable(l[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)
                   : 0ull;  // padding never wins while k <= E
  }

  float top = 0.0f, sum = 0.0f;
  int32_t* idx_t = idx + (size_t)t * k;
  float* g_t = gates + (size_t)t * k;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t other = __shfl_xor(best, off, 64);
      best = other > best ? other : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    // retire the winner in the lane that holds it
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (key[i] == best) key[i] = 0ull;
    const float v = from_orderable((uint32_t)(best >> 32));
    if (j == 0) top = v;
    const float ej = expf(v - top);
    sum += ej;
    if (lane == (j & 63)) {
      idx_t[j] = e;
      g_t[j] = ej;  // unnormalised; divided below by the same lane
    }
  }
  for (int j = lane; j < k; j += 64) g_t[j] = g_t[j] / sum;
}

template <int P>
hipError_t launch_p(const float* logits, int T, int E, int k, int32_t* idx, float* gates,
                    hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel<P>, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx,
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

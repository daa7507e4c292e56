// Measured ceilings of the GPU, reported beside its published peaks: a loop
// that does nothing but issue 32x32x16 matrix-core products on register
// operands. It is a measuring stick for the benchmark, not part of the MoE
// layer, and lives in a library of its own (libmoe_peaks.so).
#include <hip/hip_runtime.h>

#include <type_traits>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;  // independent accumulators per wave: the matrix pipe never waits

// Every wave runs `iters` rounds of kChains products; each product is
// 2 * 32 * 32 * 16 = 32,768 flops. The sum of the accumulators is written only
// under a condition the values never meet, which keeps the loop alive.
template <bool BF>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out) {
  typedef typename std::conditional<BF, bf16x8_t, half8_t>::type op_t;
  typedef typename std::conditional<BF, __bf16, _Float16>::type el_t;
  const int lane = threadIdx.x & 63;
  op_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (el_t)(1e-3f * (float)(lane + i));
    b[i] = (el_t)(1e-3f * (float)(lane - i));
  }
  floatx16_t acc[kChains] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (BF)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (s == -1.0f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same loop on the FP8 matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4
// with E4M3 operands and unit scales, 2 * 32 * 32 * 64 = 131,072 flops each.
__global__ __launch_bounds__(256) void mfma_loop_fp8(int iters, float* out) {
  typedef int int8v_t __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63;
  int8v_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + lane;  // E4M3 values near 1
    b[i] = 0x30303030 + i;
  }
  floatx16_t acc[kChains] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (s == -1.0f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Flops one launch of peaks_mfma_loop performs.
double peaks_mfma_loop_flops(int blocks, int iters) {
  return (double)blocks * 4 /* waves */ * iters * kChains * 32768.0;
}

// Flops one launch of the FP8 loop performs.
double peaks_mfma_loop_fp8_flops(int blocks, int iters) {
  return (double)blocks * 4 /* waves */ * iters * kChains * 131072.0;
}

// Launch the loop: `blocks` workgroups of 256 threads, bf16 (1), fp16 (0) or
// FP8 (2) operands, on `stream`. `out` (device, blocks * 256 floats) is never
// written for the operands used here. Returns the hipError_t of the launch.
int peaks_mfma_loop(int bf16, int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  if (bf16 == 2)
    hipLaunchKernelGGL(mfma_loop_fp8, dim3(blocks), dim3(256), 0, stream, iters, out);
  else if (bf16)
    hipLaunchKernelGGL(mfma_loop<true>, dim3(blocks), dim3(256), 0, stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_loop<false>, dim3(blocks), dim3(256), 0, stream, iters, out);
  return (int)hipGetLastError();
}

}  // extern "C"

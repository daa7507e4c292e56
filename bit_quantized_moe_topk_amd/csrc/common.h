// Internal declarations shared by the HIP translation units of libmoe.
// Not part of the public ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Description of one layer's packed experts (device pointers, shapes).
struct Experts {
  int qtype;      // 2 or 3
  int E;          // routed experts
  int has_shared; // 0 or 1
  int E_tot;      // E + has_shared
  int H, I;
  size_t nb;      // blocks per expert = 3*H*I/32
  const uint8_t* codes;  // [E_tot][nb][8]
  const uint8_t* hi;     // [E_tot][nb][4] (Q3) or nullptr
  const uint16_t* dm;    // [E_tot][nb][2] fp16 bits (d, m)
};

// First block of each matrix inside an expert.
__host__ __device__ inline size_t blk_gate(const Experts& x, int e) { return (size_t)e * x.nb; }
__host__ __device__ inline size_t blk_up(const Experts& x, int e) {
  return (size_t)e * x.nb + (size_t)x.I * (x.H / 32);
}
__host__ __device__ inline size_t blk_down(const Experts& x, int e) {
  return (size_t)e * x.nb + 2 * (size_t)x.I * (x.H / 32);
}

// Scheduling thresholds (tokens per expert).
// Experts with 1..kGemvMaxTokens assignments take the GEMV kernels (weights
// streamed once, codes kept exact); the rest take the MFMA tile kernels.
constexpr int kGemvMaxTokens = 4;
constexpr int kTileM = 64;  // tokens per MFMA tile

// Layout of the scheduling area inside the FFN workspace (int32 words).
//   [0] number of GEMV experts   [1] number of MFMA token tiles
//   [8 .. 8+E_tot)               GEMV expert list
//   [8+E_tot .. )                MFMA tile list: (expert << 16 | tile index)
struct SchedView {
  int* hdr;
  int* gemv;
  int* tiles;
};
inline size_t sched_words(int E_tot, int A) { return 8 + (size_t)E_tot + (size_t)A / kTileM + E_tot + 1; }
__host__ __device__ inline SchedView sched_view(int* base, int E_tot) {
  return SchedView{base, base + 8, base + 8 + E_tot};
}

// fp16 bit pattern -> float (exact; v_cvt_f32_f16).
__device__ inline float half_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// ---- launchers (each returns hipGetLastError() after enqueueing) ----------
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* gates,
                       hipStream_t s);

size_t group_scratch_bytes(int T, int k, int E);
hipError_t launch_group(const int32_t* idx, int T, int k, int E, int has_shared, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* slot_of, void* scratch,
                        hipStream_t s);

// FFN: check mode (fp32) and fast mode; both read a grouping and write y.
struct FfnArgs {
  const void* x;
  int xdtype;  // 0 f32, 1 bf16
  int T, k;
  const int32_t* idx;
  const float* gates;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* slot_of;
  void* y;
  int* sched;  // scheduling area
  void* h;     // [A][I] intermediate
  float* o;    // [A][H] gate-scaled expert outputs
};
hipError_t launch_sched(const Experts& ex, const FfnArgs& a, int gemv_max_tokens, hipStream_t s);
hipError_t launch_ffn_check(const Experts& ex, const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_fast(const Experts& ex, const FfnArgs& a, hipStream_t s);
hipError_t launch_combine(const Experts& ex, const FfnArgs& a, int out_f32, hipStream_t s);

}  // namespace moe

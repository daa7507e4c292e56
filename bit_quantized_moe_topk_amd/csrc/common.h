// Internal declarations shared by the HIP translation units of libmoe.
// Not part of the public ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int MOE_MAX_E_DEV = 2048;  // routed experts per layer (MOE_MAX_E)

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
  // Optional tiled copy for the matrix-core tiles (null when not attached):
  // per (expert, matrix, 32-row group, block quad) a record of 64 lanes.
  const uint8_t* t_codes;  // [E_tot][3][R][64][16]
  const uint16_t* t_dm;    // [E_tot][3][R][64][4]
  const uint8_t* t_hi;     // [E_tot][3][R][64][8] (Q3)
};

// Records per matrix of the tiled copy (32 rows x 4 blocks each).
__host__ __device__ inline size_t tiled_records(const Experts& x) {
  return (size_t)x.H * x.I / 4096;
}

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
constexpr int kGemvBatchLimit = 256;  // batches of at least this many tokens take no GEMV pass
constexpr int kTileM = 64;  // assignments per tile of the fp32 check kernels
// Up to this many tokens the per-assignment expert outputs are kept in fp32;
// above it in bf16 (half the traffic of the combine).
constexpr int kF32SlotMaxTokens = 256;

// fp16 bit pattern -> float (exact; v_cvt_f32_f16).
// Bit mask of the lanes below this one in its 64-wide wavefront.
__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ inline float half_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Launch profiling hooks (inactive unless a caller enabled moe_profile_begin).
// While active, prof_open hands out an event pair that the launch attaches to
// the kernel's own dispatch (hipExtLaunchKernelGGL), so the pair brackets the
// kernel's execution on the device, not the queueing around it.
bool prof_open(const char* name, hipEvent_t* start, hipEvent_t* stop);
void prof_close();
#define MOE_LAUNCH(NAME, STREAM, KERNEL, GRID, BLOCK, LDS, S, ...)                           \
  do {                                                                                     \
    hipEvent_t moe_ev_a_ = nullptr, moe_ev_b_ = nullptr;                                   \
    if (::moe::prof_open(NAME, &moe_ev_a_, &moe_ev_b_)) {                                  \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, S, moe_ev_a_, moe_ev_b_, 0, __VA_ARGS__); \
      ::moe::prof_close();                                                                 \
    } else {                                                                               \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, S, __VA_ARGS__);                        \
    }                                                                                      \
  } while (0)

// Compute units of the current device (read once per device).
int device_cus();

// ---- launchers (each returns hipGetLastError() after enqueueing) ----------
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* gates,
                       hipStream_t s);

size_t group_scratch_bytes(int T, int k, int E);
// xj (optional): the small-batch activation layout to write in the same
// launch when the grouping runs in one workgroup; *xs_done tells whether it did.
struct XsJob;
hipError_t launch_group(const int32_t* idx, int T, int k, int E, int has_shared, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* slot_of, void* scratch,
                        hipStream_t s, const XsJob* xj = nullptr, bool* xs_done = nullptr);
hipError_t launch_route_group(const float* logits, int T, int E, int k, int has_shared, int32_t* idx,
                              float* gates, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* slot_of, void* scratch, hipStream_t s,
                              const XsJob* xj = nullptr, bool* xs_done = nullptr);

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
  int out_f32;     // y is float32
  int gmax;        // GEMV token limit (0: every expert takes the MFMA tiles)
  void* h;         // [A][I] intermediate (fp32 check; bf16 fast)
  uint16_t* x16;   // [T][H] fp16 copy of x (fast mode: MFMA tiles; small-batch layout below 256 tokens)
  int32_t* xe;     // [T] exponent e of each token row of x16 (the row holds x * 2^-e)
  int xs_ready;    // x16 already holds the copy the FFN's matrix-core kernels read
  float* o;        // [A][H] fp32 gate-scaled expert outputs (check mode; fast, few tokens)
  uint16_t* ob;    // [A][H] bf16 gate-scaled expert outputs (fast, many tokens)
};
hipError_t launch_ffn_check(const Experts& ex, const FfnArgs& a, hipStream_t s);
bool gemv_supported(int H, int I);
// The two-kernel whole-layer path for a decode verify window (T <= 4).
// Bytes at the head of every moe_layer workspace kept for the one-launch
// decode window's counters (zero between calls; no other call form writes them).
constexpr size_t kWinSyncBytes = 8192;
// Router product (router.hip): the matrix-core kernel from this many bf16 tokens.
constexpr int kRouterMfmaMinT = 256;
bool router_supported(int H, int E);
// Router product and top-k in one launch for bf16 x (E 256 or 512, k <= 64):
// idx, gates [T][k] as launch_topk of the product; logits [T][E] written when
// not null.
bool router_topk_supported(int xdtype, int H, int E, int k);
hipError_t launch_router_topk(const void* x, int T, int H, const uint16_t* w, const float* bias, int E,
                              int k, float* logits, int32_t* idx, float* gates, hipStream_t s);
hipError_t launch_router(const void* x, int xdtype, int T, int H, const uint16_t* w,
                         const float* bias, int E, float* logits, hipStream_t s);
bool window_supported(const Experts& ex, int T, int k);
size_t window_workspace_bytes(const Experts& ex, int T, int k);
hipError_t launch_window(const float* logits, int T, int k, const Experts& ex, const void* x,
                         int xdtype, int32_t* idx, float* gates, void* y, int out_f32, void* ws,
                         hipStream_t s);
// Gate/up + SwiGLU of one expert on the FP8 matrix cores (a measured
// variant, fp8.hip): workspace bytes, shapes it takes, launch.
size_t fp8_gateup_workspace_bytes(const Experts& ex, int T);
bool fp8_gateup_supported(const Experts& ex);
hipError_t launch_fp8_gateup(const Experts& ex, int expert, const uint16_t* x, int T, float* h,
                             void* ws, hipStream_t s);

// The one-launch window starting from hidden states: router roles store the
// logits [T][E] tagged with the launch into lgp (64-bit entries) and, when lg
// is not null, plain into lg; then the window as launch_window. Only where
// window_hidden_supported holds.
bool window_hidden_supported(const Experts& ex, int T, int k);
hipError_t launch_window_hidden(float* lg, uint64_t* lgp, const uint16_t* rw, const float* rbias,
                                int T, int k, const Experts& ex, const void* x, int xdtype,
                                int32_t* idx, float* gates, void* y, int out_f32, void* ws,
                                hipStream_t s);
hipError_t launch_ffn_fast(const Experts& ex, const FfnArgs& a, hipStream_t s);
// MFMA tiles of fast mode (experts with more than gmax assignments); writes x16.
bool mfma_supported(int H, int I);
hipError_t launch_mfma(const Experts& ex, const FfnArgs& a, hipStream_t s);
// fp16 copy of x in the MFMA K order (a.x16), the activation operand of the
// matrix-core FFN kernels.
hipError_t launch_x16(const Experts& ex, const FfnArgs& a, hipStream_t s);
// Small batches (fewer than kGemvBatchLimit tokens): every touched expert on
// the small-batch matrix-core kernels (batch.hip); writes x16, h and the
// per-slot outputs.
bool batch_supported(int H, int I);
hipError_t launch_batch(const Experts& ex, const FfnArgs& a, hipStream_t s);
// A request for the fp16 activation copy into x16: q = 2, 3 the small-batch
// layout for that code width, 0 the prefill tiles' copy, -1 none.
XsJob xs_job(int q, int H, const void* x, int xdtype, int T, uint16_t* x16, int32_t* xe);
// Writes the tiled copy of ex's planes (t_codes, t_dm, t_hi must be set).
hipError_t launch_tile_weights(const Experts& ex, hipStream_t s);
hipError_t launch_combine(const Experts& ex, const FfnArgs& a, hipStream_t s);

}  // namespace moe

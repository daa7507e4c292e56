// Fast mode of the expert FFN on gfx950.
//
// Decode shape (an expert holding 1..4 of the step's assignments): the layer is
// bound by streaming the packed weights ("Strata - the details", "Other GPUs":
// speed scales with memory bandwidth). The GEMV kernels read every touched
// weight once and never expand it. A 2-bit code c becomes the exact bf16 value
// 128 + c*4^s by OR-ing it into the mantissa of 128 (s = the code's offset
// inside its source field, 0..2), v_dot2 multiplies code pairs by bf16
// activation pairs pre-scaled by 4^-s, and the block affine map is applied once
// per block and token:
//     sum_k (d q_k + m) x_k = d * (D - 128 X) + m * S,
// D = sum of the dot2 terms, X = sum of the scaled activations, S = sum x.
// (3-bit codes use s = 0 and OR in the third bit.) Every lane owns one 32-weight
// block of a row; a wave issues all its block loads before computing, then
// reduces its partial sums across the row's lanes in one batched transpose.
//
// Used for experts with 1..4 assignments in batches under 256 tokens whose
// shapes the small-batch matrix-core kernels (batch.hip) do not cover; the
// other experts of such a batch run on the matrix-core tiles (mfma.hip).
//
// Combine: the down kernels store gate * o per assignment slot (fp32 for few
// tokens, bf16 for many) and the combine kernel sums each token's slots in a
// fixed order. (A device-wide atomic sum was slower: same-address atomics from
// all workgroups serialise, and the result would depend on their order.)
#include "common.h"
#include "gemv.h"
#include "sched.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Activation block of token slot m of an expert (zero past M).
template <int Q, bool XF32>
__device__ inline void load_token_xb(const Experts& ex, const FfnArgs& a, int slot0, int m, int M,
                                     int b, XB& xb) {
  if (m < M) {
    int t = token_of(a.perm[slot0 + m], a.T, a.k);
    t = (unsigned)t < (unsigned)a.T ? t : 0;
    const size_t off = (size_t)t * ex.H + 32 * b;
    if (XF32) load_xb_f32<Q>(static_cast<const float*>(a.x) + off, xb);
    else load_xb_bf16<Q>(static_cast<const uint16_t*>(a.x) + off, xb);
  } else {
    zero_xb(xb);
  }
}

// Decode GEMV, gate + up + SwiGLU, one wave: PRW pair-rows of expert e from
// pair-row prw0, for its MP >= M token slots. Lane l owns block (l % BPR) of
// row (l / BPR) of each group of RPI = 64/BPR rows.
template <int BPR, int MP, int Q, bool XF32>
__device__ inline void gemv_gateup_wave(const Experts& ex, const FfnArgs& a, int e, int prw0, int M,
                                        int slot0) {
  constexpr int RPI = 64 / BPR;
  constexpr int PRW = RPI > 4 ? RPI : 4;
  constexpr int P = PRW / RPI;
  constexpr int NV = 2 * P * MP;
  const int lane = threadIdx.x & 63;
  const int b = lane % BPR, rg = lane / BPR;
  QBlock qg[P], qu[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const size_t row = (size_t)prw0 + p * RPI + rg;
    qg[p] = load_qblock<Q>(ex, blk_gate(ex, e) + row * BPR + b);
    qu[p] = load_qblock<Q>(ex, blk_up(ex, e) + row * BPR + b);
  }
  XB xb[MP];
#pragma unroll
  for (int i = 0; i < MP; ++i) load_token_xb<Q, XF32>(ex, a, slot0, i, M, b, xb[i]);
  float v[NV];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float g[MP], u[MP];
    block_values<Q, MP>(qg[p], xb, g);
    block_values<Q, MP>(qu[p], xb, u);
#pragma unroll
    for (int i = 0; i < MP; ++i) {
      v[2 * (p * MP + i)] = g[i];
      v[2 * (p * MP + i) + 1] = u[i];
    }
  }
  int jbase = 0;
  LaneReduce<NV, BPR / 2>::run(v, lane, jbase);
  uint16_t* h = static_cast<uint16_t*>(a.h);
  if constexpr (NV > BPR) {
#pragma unroll
    for (int j = 0; j < NV / BPR; j += 2) {
      const int pi = (jbase + j) >> 1, p = pi / MP, m = pi % MP;
      if (m < M) {
        const int row = prw0 + p * RPI + rg;
        h[(size_t)(slot0 + m) * ex.I + row] = (uint16_t)f32_to_bf16_bits(silu_mul(v[j], v[j + 1]));
      }
    }
  } else {
    constexpr int OFF = BPR / NV;  // lane bit that holds the gate/up index bit
    const float other = __shfl_xor(v[0], OFF, 64);
    const int pi = jbase >> 1, p = pi / MP, m = pi % MP;
    if ((jbase & 1) == 0 && (lane & (OFF - 1)) == 0 && m < M) {
      const int row = prw0 + p * RPI + rg;
      h[(size_t)(slot0 + m) * ex.I + row] = (uint16_t)f32_to_bf16_bits(silu_mul(v[0], other));
    }
  }
}

template <int BPR>
constexpr int gateup_rows() {
  return 4 * (64 / BPR > 4 ? 64 / BPR : 4);
}
template <int BPR>
constexpr int down_rows() {
  return 4 * (64 / BPR > 16 ? 64 / BPR : 16);
}

template <int BPR, int Q, bool XF32>
__global__ __launch_bounds__(kThreads) void gemv_gateup(Experts ex, FfnArgs a) {
  __shared__ WorkMap wm;
  workmap_init(wm, a.counts, ex.E_tot, a.gmax);
  constexpr int WG_ROWS = gateup_rows<BPR>();
  const int per_e = ex.I / WG_ROWS;
  const int wave = threadIdx.x >> 6;
  for (int item = blockIdx.x; item < wm.n_gemv * per_e; item += gridDim.x) {
    const int e = workmap_gemv(wm, ex.E_tot, item / per_e);
    const int M = a.counts[e], slot0 = a.offsets[e];
    const int prw0 = (item % per_e) * WG_ROWS + wave * (WG_ROWS / 4);
    if (M == 1) gemv_gateup_wave<BPR, 1, Q, XF32>(ex, a, e, prw0, M, slot0);
    else if (M == 2) gemv_gateup_wave<BPR, 2, Q, XF32>(ex, a, e, prw0, M, slot0);
    else gemv_gateup_wave<BPR, 4, Q, XF32>(ex, a, e, prw0, M, slot0);
  }
}

// Output of one expert row for one assignment: gate * value, stored per slot
// (fp32 for few tokens, bf16 for many) for the combine kernel.
// Decode GEMV, down projection with the gate folded in, one wave: RW rows of H
// from row r0w for MP >= M token slots.
template <int BPR, int MP, int Q>
__device__ inline void gemv_down_wave(const Experts& ex, const FfnArgs& a, int e, int r0w, int M,
                                      int slot0) {
  constexpr int RPI = 64 / BPR;
  constexpr int RW = RPI > 16 ? RPI : 16;
  constexpr int P = RW / RPI;
  constexpr int NV = P * MP;
  const int lane = threadIdx.x & 63;
  const int b = lane % BPR, rg = lane / BPR;
  QBlock qd[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const size_t row = (size_t)r0w + p * RPI + rg;
    qd[p] = load_qblock<Q>(ex, blk_down(ex, e) + row * BPR + b);
  }
  const uint16_t* h = static_cast<const uint16_t*>(a.h);
  XB xb[MP];
  float gate[MP];
#pragma unroll
  for (int i = 0; i < MP; ++i) {
    if (i < M) {
      load_xb_bf16<Q>(h + (size_t)(slot0 + i) * ex.I + 32 * b, xb[i]);
      gate[i] = gate_of(a, slot0 + i);
    } else {
      zero_xb(xb[i]);
      gate[i] = 0.f;
    }
  }
  float v[NV];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float o[MP];
    block_values<Q, MP>(qd[p], xb, o);
#pragma unroll
    for (int i = 0; i < MP; ++i) v[p * MP + i] = o[i];
  }
  int jbase = 0;
  LaneReduce<NV, BPR / 2>::run(v, lane, jbase);
  constexpr int NF = NV > BPR ? NV / BPR : 1;
  constexpr int REP = NV < BPR ? BPR / NV : 1;  // lanes holding the same sums
  if ((lane & (REP - 1)) != 0) return;
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int idx = jbase + j, p = idx / MP, i = idx % MP;
    if (i < M) emit(ex, a, slot0 + i, r0w + p * RPI + rg, gate[i] * v[j]);
  }
}

template <int BPR, int Q>
__global__ __launch_bounds__(kThreads) void gemv_down(Experts ex, FfnArgs a) {
  __shared__ WorkMap wm;
  workmap_init(wm, a.counts, ex.E_tot, a.gmax);
  constexpr int WG_ROWS = down_rows<BPR>();
  const int per_e = ex.H / WG_ROWS;
  const int wave = threadIdx.x >> 6;
  for (int item = blockIdx.x; item < wm.n_gemv * per_e; item += gridDim.x) {
    const int e = workmap_gemv(wm, ex.E_tot, item / per_e);
    const int M = a.counts[e], slot0 = a.offsets[e];
    const int r0w = (item % per_e) * WG_ROWS + wave * (WG_ROWS / 4);
    if (M == 1) gemv_down_wave<BPR, 1, Q>(ex, a, e, r0w, M, slot0);
    else if (M == 2) gemv_down_wave<BPR, 2, Q>(ex, a, e, r0w, M, slot0);
    else gemv_down_wave<BPR, 4, Q>(ex, a, e, r0w, M, slot0);
  }
}

inline int grid_for(long max_items, int cap) {
  return (int)(max_items < cap ? (max_items > 0 ? max_items : 1) : cap);
}


template <int Q, bool XF32>
hipError_t launch_q(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const int A = a.T * (a.k + ex.has_shared);
  const long max_gemv = A < ex.E_tot ? A : ex.E_tot;
  const int bpr_h = ex.H / 32, bpr_i = ex.I / 32;
  const bool gemv = a.gmax > 0;
  const bool mfma = a.T > a.gmax;  // an expert holds at most T assignments
#define GU(B)                                                                                      \
  case B:                                                                                          \
    MOE_LAUNCH("gemv_gateup", s, (gemv_gateup<B, Q, XF32>),                                        \
               dim3(grid_for(max_gemv * (ex.I / gateup_rows<B>()), 2048)), dim3(kThreads), 0, s, ex, \
               a);                                                                                 \
    break;
#define DN(B)                                                                                    \
  case B:                                                                                        \
    MOE_LAUNCH("gemv_down", s, (gemv_down<B, Q>),                                                \
               dim3(grid_for(max_gemv * (ex.H / down_rows<B>()), 2048)), dim3(kThreads), 0, s, ex, \
               a);                                                                               \
    break;
  if (gemv) {
    switch (bpr_h) { GU(4) GU(8) GU(16) GU(32) GU(64) default: return hipErrorInvalidValue; }
  }
  if (mfma) {
    const hipError_t e = launch_mfma(ex, a, s);
    if (e != hipSuccess) return e;
  }
  if (gemv) {
    switch (bpr_i) { DN(4) DN(8) DN(16) DN(32) DN(64) default: return hipErrorInvalidValue; }
  }
#undef GU
#undef DN
  return hipGetLastError();
}

}  // namespace

// True when the decode GEMV lane layouts cover these shapes.
bool gemv_supported(int H, int I) {
  auto ok = [](int bpr) { return bpr == 4 || bpr == 8 || bpr == 16 || bpr == 32 || bpr == 64; };
  return ok(H / 32) && ok(I / 32);
}

hipError_t launch_ffn_fast(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  if (ex.qtype == 3) return a.xdtype == 0 ? launch_q<3, true>(ex, a, s) : launch_q<3, false>(ex, a, s);
  return a.xdtype == 0 ? launch_q<2, true>(ex, a, s) : launch_q<2, false>(ex, a, s);
}

}  // namespace moe

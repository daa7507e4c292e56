// The whole layer for a decode verify window (T <= 4 tokens) in two kernels.
//
// The pages' decode checks up to 3 drafted tokens plus one in a single pass
// over the layers ("Strata - the details", "How it works": speculation), so a
// layer step sees a handful of tokens and is bound by streaming the touched
// experts' weights. Dependent launches are the cost to avoid here, so:
//   win_gateup: every workgroup routes the window itself (top-k of T logit
//     rows, a few KB), builds the list of active experts with each one's token
//     mask and gates in LDS, and computes gate/up + SwiGLU for its own pair-rows
//     of I across every active expert (row-stationary). Workgroup 0 publishes
//     idx, gates and the active list for the second kernel.
//   win_down: every workgroup owns a few rows of H for all active experts: its
//     waves split the rows and the experts, sum gate * o over their experts in
//     registers, add the expert quarters in LDS in a fixed order and write y.
//     No per-assignment buffer, no atomics and no cross-workgroup wait: y is
//     reproducible run to run.
// Activations enter as bf16 and the codes stay exact (gemv.h).
#include "common.h"
#include "deq16.h"
#include "gemv.h"
#include "sched.h"
#include "topk.h"
#include "batch_x.h"

namespace moe {

constexpr int kWinT = 4;                   // tokens per window, at most
constexpr int kWinMaxK = 64;               // experts per token, at most
constexpr int kWinMaxAct = kWinT * kWinMaxK + 1;
constexpr int kWinThreads = 512;

// Active experts of a window: ascending expert index, shared expert last.
struct WinList {
  int n_act;
  int act_e[kWinMaxAct];
  int act_mask[kWinMaxAct];             // bit t: token t routed to it
  float act_gate[kWinMaxAct][kWinT];    // gate per token (0 when not routed)
};

namespace {

template <int Q, bool XF32>
__device__ inline void load_x_row(const void* x, int H, int t, int b, XB& xb) {
  const size_t off = (size_t)t * H + 32 * b;
  if (XF32) load_xb_f32<Q>(static_cast<const float*>(x) + off, xb);
  else load_xb_bf16<Q>(static_cast<const uint16_t*>(x) + off, xb);
}

// Values of one block for the tokens in `mask` (others 0). `mask` must be
// wave-uniform (a scalar): each code pair is decoded once, then a dot2 chain
// runs for every routed token only, behind scalar branches.
template <int Q>
__device__ inline void block_values_masked(const QBlock& b, const XB (&xb)[kWinT], int mask,
                                           float (&out)[kWinT]) {
  uint32_t pr[16];
  decode_pairs<Q>(b, pr);
  const float d = half_lo(b.dm), m = half_hi(b.dm);
#pragma unroll
  for (int i = 0; i < kWinT; ++i) {
    out[i] = 0.f;
    if (mask & (1 << i)) {
      float D = -128.0f * xb[i].S;
#pragma unroll
      for (int p = 0; p < 16; ++p) D = dot2(pr[p], xb[i].p[p], D);
      out[i] = d * D + m * xb[i].S;
    }
  }
}

// Top-k of one token row with the lane count chosen by E (E <= MOE_MAX_E).
__device__ inline void topk_any(const float* l, int E, int k, int32_t* idx_t, float* g_t,
                                TopkScratch* sc) {
  const int per = (E + 63) / 64;
  if (per <= 1) topk_token<1>(l, E, k, idx_t, g_t, sc);
  else if (per <= 2) topk_token<2>(l, E, k, idx_t, g_t, sc);
  else if (per <= 4) topk_token<4>(l, E, k, idx_t, g_t, sc);
  else if (per <= 8) topk_token<8>(l, E, k, idx_t, g_t, sc);
  else if (per <= 16) topk_token<16>(l, E, k, idx_t, g_t, sc);
  else topk_token<32>(l, E, k, idx_t, g_t, sc);
}

template <int BPR>
constexpr int win_gu_rows() {  // pair-rows of I per workgroup
  return 64 / BPR > 2 ? 64 / BPR : 2;
}
constexpr int kWinWaves = kWinThreads / 64;
template <int BPR>
constexpr int win_dn_rows() {  // rows of H per down workgroup: two row groups
  return 2 * (64 / BPR);
}
constexpr int kWinBatch = 4;   // experts whose weights a wave has in flight at once

// LDS state of the window's routing, built by every workgroup.
struct WinRoute {
  static constexpr bool kSlow = true;  // room for more than 64 assignments
  int lidx[kWinT * kWinMaxK];
  float lgate[kWinT * kWinMaxK];
  int flag[MOE_MAX_E_DEV + 1];
  int tmask[MOE_MAX_E_DEV + 1];
  int wsum[16];
  uint32_t bits[64];  // routed-expert bitmap (experts < 2,048)
  int pref[64];       // set bits before each bitmap word
  WinList wl;
  TopkScratch tks[kWinT];
};

// The same for at most 64 assignments (T k <= 64), without the scan arrays.
struct LayerRoute {
  static constexpr bool kSlow = false;
  int lidx[64];
  float lgate[64];
  uint32_t bits[64];
  int pref[64];
  WinList wl;
  TopkScratch tks[kWinT];
};

// Routing, part 1: wave t selects token t's experts into LDS. Called before
// the activation loads: loads complete in order, so the logits must not queue
// behind them.
// PER > 0: the lane count is fixed (E <= 64 PER), which bounds the registers.
template <int PER = 0, typename RT>
__device__ inline void win_topk(RT& R, const float* __restrict__ logits, int T, int E, int k) {
  const int wave = threadIdx.x >> 6;
  if (wave < T) {
    const float* l = logits + (size_t)wave * E;
    if (PER > 0) topk_token<(PER > 0 ? PER : 1)>(l, E, k, R.lidx + wave * k, R.lgate + wave * k, &R.tks[wave]);
    else topk_any(l, E, k, R.lidx + wave * k, R.lgate + wave * k, &R.tks[wave]);
  }
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// More than 64 assignments: token masks per expert, a block scan over the
// expert flags gives the ranks.
__device__ inline int win_list_scan(WinRoute& R, const Experts& ex, int T, int k, bool publish,
                                    int32_t* idx_out, float* gates_out, WinList* gmeta) {
  const int tid = threadIdx.x, NT = blockDim.x;
  const int E = ex.E, E_tot = ex.E_tot;
  for (int e = tid; e < E_tot; e += NT) R.tmask[e] = 0;
  __syncthreads();
  for (int a = tid; a < T * k; a += NT) atomicOr(&R.tmask[R.lidx[a]], 1 << (a / k));
  if (ex.has_shared && tid == 0) R.tmask[E] = (1 << T) - 1;
  __syncthreads();
  for (int e = tid; e < E_tot; e += NT) R.flag[e] = R.tmask[e] != 0;
  __syncthreads();
  const int n_act = block_exclusive_scan(R.flag, E_tot, R.wsum);
  for (int e = tid; e < E_tot; e += NT) {
    if (R.tmask[e]) {
      const int p = R.flag[e];
      R.wl.act_e[p] = e;
      R.wl.act_mask[p] = R.tmask[e];
#pragma unroll
      for (int t = 0; t < kWinT; ++t) R.wl.act_gate[p][t] = 0.f;
    }
  }
  if (tid == 0) R.wl.n_act = n_act;
  __syncthreads();
  for (int a = tid; a < T * k; a += NT) R.wl.act_gate[R.flag[R.lidx[a]]][a / k] = R.lgate[a];
  if (ex.has_shared && tid < T) R.wl.act_gate[R.flag[E]][tid] = 1.0f;
  __syncthreads();
  if (publish) {
    for (int a = tid; a < T * k; a += NT) {
      idx_out[a] = R.lidx[a];
      gates_out[a] = R.lgate[a];
    }
    if (gmeta && tid == 0) gmeta->n_act = n_act;
    for (int p = tid; gmeta && p < n_act; p += NT) {
      gmeta->act_e[p] = R.wl.act_e[p];
      gmeta->act_mask[p] = R.wl.act_mask[p];
#pragma unroll
      for (int t = 0; t < kWinT; ++t) gmeta->act_gate[p][t] = R.wl.act_gate[p][t];
    }
  }
  return n_act;
}

// Routing, part 2: the active-expert list (ascending expert, shared last) with
// each expert's token mask and gates; workgroup 0 also publishes idx, gates
// and the list. Returns the number of active experts.
//
// Up to 64 assignments (every 4-token window with k <= 16) take one wave: the
// assignments set bits of an expert bitmap, a scan over its 64 words gives
// every expert its rank (the number of routed experts below it), and each
// assignment writes its expert, token bit and gate at that rank.
template <typename RT>
__device__ inline int win_list(RT& R, const Experts& ex, int T, int k, bool publish,
                               int32_t* idx_out, float* gates_out, WinList* gmeta) {
  const int tid = threadIdx.x, NT = blockDim.x;
  const int E = ex.E;
  const int A = T * k;
  if (A <= 64) {
    __syncthreads();  // the top-k waves' lidx, lgate
    if (tid < 64) {
      const int lane = tid;
      R.bits[lane] = 0u;
      wave_sync_lds();
      int e = 0, t = 0;
      float g = 0.f;
      if (lane < A) {
        e = R.lidx[lane];
        g = R.lgate[lane];
        t = lane / k;
        atomicOr(&R.bits[e >> 5], 1u << (e & 31));
      }
      wave_sync_lds();
      const uint32_t w = R.bits[lane];
      const int incl = wave_inclusive_scan(__popc(w));
      R.pref[lane] = incl - __popc(w);
      const int n_routed = __builtin_amdgcn_readlane(incl, 63);
      const int n_act = n_routed + ex.has_shared;
      for (int p = lane; p < n_act; p += 64) {
        R.wl.act_mask[p] = 0;
#pragma unroll
        for (int u = 0; u < kWinT; ++u) R.wl.act_gate[p][u] = 0.f;
      }
      wave_sync_lds();
      if (lane < A) {
        const int rank = R.pref[e >> 5] + __popc(R.bits[e >> 5] & ((1u << (e & 31)) - 1u));
        R.wl.act_e[rank] = e;  // the same value from every assignment of e
        atomicOr(&R.wl.act_mask[rank], 1 << t);
        R.wl.act_gate[rank][t] = g;
      }
      if (ex.has_shared && lane < T) {
        if (lane == 0) {
          R.wl.act_e[n_routed] = E;
          R.wl.act_mask[n_routed] = (1 << T) - 1;
        }
        R.wl.act_gate[n_routed][lane] = 1.0f;
      }
      if (lane == 0) R.wl.n_act = n_act;
    }
    __syncthreads();
    const int n_act = R.wl.n_act;
    if (publish) {
      for (int a = tid; a < A; a += NT) {
        idx_out[a] = R.lidx[a];
        gates_out[a] = R.lgate[a];
      }
      if (gmeta && tid == 0) gmeta->n_act = n_act;
      for (int p = tid; gmeta && p < n_act; p += NT) {
        gmeta->act_e[p] = R.wl.act_e[p];
        gmeta->act_mask[p] = R.wl.act_mask[p];
#pragma unroll
        for (int u = 0; u < kWinT; ++u) gmeta->act_gate[p][u] = R.wl.act_gate[p][u];
      }
    }
    return n_act;
  }
  if constexpr (RT::kSlow) return win_list_scan(R, ex, T, k, publish, idx_out, gates_out, gmeta);
  return 0;  // not reached: callers with this state keep T k <= 64
}

template <int BPR, int Q, bool XF32>
__global__ __launch_bounds__(kWinThreads) void win_gateup(const float* __restrict__ logits, int T,
                                                          int k, Experts ex, const void* x,
                                                          int32_t* idx_out, float* gates_out,
                                                          WinList* gmeta, uint16_t* hwin) {
  __shared__ WinRoute R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = lane % BPR, rg = lane / BPR;
  WinList& wl = R.wl;

  win_topk(R, logits, T, ex.E, k);
  XB xb[kWinT];
#pragma unroll
  for (int t = 0; t < kWinT; ++t) {
    if (t < T) load_x_row<Q, XF32>(x, ex.H, t, b, xb[t]);
    else zero_xb(xb[t]);
  }
  const int n_act = win_list(R, ex, T, k, blockIdx.x == 0, idx_out, gates_out, gmeta);

  // gate/up + SwiGLU for this workgroup's pair-rows; wave w takes the active
  // experts w, w + 8, ..., kWinBatch at a time with all their loads in flight
  constexpr int RPI = 64 / BPR;
  constexpr int PR = win_gu_rows<BPR>();
  constexpr int P = PR / RPI;
  constexpr int NV = 2 * P * kWinT;
  const int r0 = blockIdx.x * PR;
  for (int a0 = wave; a0 < n_act; a0 += kWinWaves * kWinBatch) {
    QBlock qg[kWinBatch][P], qu[kWinBatch][P];
#pragma unroll
    for (int g = 0; g < kWinBatch; ++g) {
      const int ai = a0 + g * kWinWaves;
      if (ai < n_act) {
        const int e = wl.act_e[ai];
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const size_t row = (size_t)r0 + p * RPI + rg;
          qg[g][p] = load_qblock<Q>(ex, blk_gate(ex, e) + row * BPR + b);
          qu[g][p] = load_qblock<Q>(ex, blk_up(ex, e) + row * BPR + b);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kWinBatch; ++g) {
      const int ai = a0 + g * kWinWaves;
      if (ai >= n_act) break;
      const int mask = __builtin_amdgcn_readfirstlane(wl.act_mask[ai]);
      float v[NV];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float gv[kWinT], uv[kWinT];
        block_values_masked<Q>(qg[g][p], xb, mask, gv);
        block_values_masked<Q>(qu[g][p], xb, mask, uv);
#pragma unroll
        for (int t = 0; t < kWinT; ++t) {
          v[2 * (p * kWinT + t)] = gv[t];
          v[2 * (p * kWinT + t) + 1] = uv[t];
        }
      }
      int jbase = 0;
      LaneReduce<NV, BPR / 2>::run(v, lane, jbase);
      if constexpr (NV > BPR) {
#pragma unroll
        for (int j = 0; j < NV / BPR; j += 2) {
          const int pi = (jbase + j) >> 1, p = pi / kWinT, t = pi % kWinT;
          if (mask & (1 << t))
            hwin[((size_t)ai * kWinT + t) * ex.I + r0 + p * RPI + rg] =
                (uint16_t)f32_to_bf16_bits(silu_mul(v[j], v[j + 1]));
        }
      } else {
        constexpr int OFF = BPR / NV;  // lane bit holding the gate/up index bit
        const float other = __shfl_xor(v[0], OFF, 64);
        const int pi = jbase >> 1, p = pi / kWinT, t = pi % kWinT;
        if ((jbase & 1) == 0 && (lane & (OFF - 1)) == 0 && (mask & (1 << t)))
          hwin[((size_t)ai * kWinT + t) * ex.I + r0 + p * RPI + rg] =
              (uint16_t)f32_to_bf16_bits(silu_mul(v[0], other));
      }
    }
  }
}

// Gate/up + SwiGLU of the window on the matrix cores (H a multiple of 1,024,
// at most 4,096). Workgroup (g, s) owns rows 16g .. 16g + 15 of I (gate and
// up) for the active experts s, s + 8, ...; its 8 waves split H into 8 slices.
// A wave computes, per expert, a 16-row x 16-token tile of gate and of up with
// v_mfma_f32_16x16x32_f16 (weights as rows, tokens past T zero): lane group c
// (lane / 16) feeds 8 weights of block (slice start + NBL c + b) per step, so
// each lane streams NBL contiguous blocks of its row, and dequantises them in
// registers (deq16.h). The slices' partial tiles are summed in LDS in slice
// order (deterministic), then SwiGLU; h is stored as fp16 in the MFMA K order
// for every token of the window (the down tiles read all of them).
constexpr int kMmaSlices = 8;   // expert slices: workgroups per 16-row group
constexpr int kMmaBatch = 4;    // experts per round
constexpr int kMmaMaxH = 4096;

// Down projection + combine. A workgroup owns R = 2 * RPI rows of H for every
// active expert: wave w takes row group w % 2 and the experts q, q + 4, ...
// with q = w / 2, and sums gate * o over them in registers; the four expert
// quarters are then added in LDS in quarter order and the workgroup writes y.
template <int BPR, int Q>
__global__ __launch_bounds__(kWinThreads) void win_down(int T, Experts ex, const WinList* gmeta,
                                                        const uint16_t* hwin, void* y,
                                                        int out_f32) {
  constexpr int RPI = 64 / BPR;
  constexpr int R = win_dn_rows<BPR>();
  constexpr int NQ = kWinWaves / (R / RPI);  // expert quarters
  __shared__ WinList wl;
  __shared__ float red[NQ][R][kWinT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = lane % BPR, rg = lane / BPR;
  const int rgrp = wave % (R / RPI), q = wave / (R / RPI);
  const int rloc = rgrp * RPI + rg;
  const size_t row = (size_t)blockIdx.x * R + rloc;
  const int n_act = gmeta->n_act;
  for (int p = tid; p < n_act; p += kWinThreads) {
    wl.act_e[p] = gmeta->act_e[p];
    wl.act_mask[p] = gmeta->act_mask[p];
#pragma unroll
    for (int t = 0; t < kWinT; ++t) wl.act_gate[p][t] = gmeta->act_gate[p][t];
  }
  __syncthreads();

  float acc[kWinT] = {0.f, 0.f, 0.f, 0.f};
  for (int a0 = q; a0 < n_act; a0 += NQ * kWinBatch) {
    QBlock qd[kWinBatch];
#pragma unroll
    for (int g = 0; g < kWinBatch; ++g) {
      const int ai = a0 + g * NQ;
      if (ai < n_act) qd[g] = load_qblock<Q>(ex, blk_down(ex, wl.act_e[ai]) + row * BPR + b);
    }
#pragma unroll
    for (int g = 0; g < kWinBatch; ++g) {
      const int ai = a0 + g * NQ;
      if (ai >= n_act) break;
      const int mask = __builtin_amdgcn_readfirstlane(wl.act_mask[ai]);
      XB xh[kWinT];
#pragma unroll
      for (int t = 0; t < kWinT; ++t) {
        if (mask & (1 << t)) load_xb_bf16<Q>(hwin + ((size_t)ai * kWinT + t) * ex.I + 32 * b, xh[t]);
        else zero_xb(xh[t]);
      }
      float o[kWinT];
      block_values_masked<Q>(qd[g], xh, mask, o);
#pragma unroll
      for (int t = 0; t < kWinT; ++t) acc[t] += wl.act_gate[ai][t] * o[t];
    }
  }
  int jbase = 0;
  LaneReduce<kWinT, BPR / 2>::run(acc, lane, jbase);
  constexpr int NF = kWinT > BPR ? kWinT / BPR : 1;
  constexpr int REP = kWinT < BPR ? BPR / kWinT : 1;
  if ((lane & (REP - 1)) == 0) {
#pragma unroll
    for (int j = 0; j < NF; ++j) red[q][rloc][jbase + j] = acc[j];
  }
  __syncthreads();
  for (int i = tid; i < R * T; i += kWinThreads) {
    const int r = i % R, t = i / R;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < NQ; ++g) s += red[g][r][t];
    const size_t o = (size_t)t * ex.H + (size_t)blockIdx.x * R + r;
    if (out_f32) static_cast<float*>(y)[o] = s;
    else static_cast<uint16_t*>(y)[o] = (uint16_t)f32_to_bf16_bits(s);
  }
}


// Gate/up role: rows 16 rgrp .. 16 rgrp + 15 of I for the active experts es,
// es + 8, ... (es = role % 8). xs holds the window's activations (fp16, MFMA K
// order). Ends after the last h store of the role, behind a barrier.
template <int Q, int NBL>
__device__ inline void gateup_role(const WinList& wl, int n_act, int role, int T, const Experts& ex,
                                   const _Float16* xs, const int* xe,
                                   float (&red)[kWinWaves][kMmaBatch][2][16][kWinT],
                                   uint16_t* hwin) {
  // experts per round (at H = 4096 the activation operand alone takes 64
  // registers: one expert at a time)
  constexpr int kB = NBL >= 4 ? 1 : kMmaBatch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = ex.H;
  const int rgrp = role / kMmaSlices, es = role % kMmaSlices;
  const int c = lane >> 4, r16 = lane & 15;
  const int kb0 = wave * (H / 256) + NBL * c;  // this lane's first block of the wave's slice
  half8_t xf[NBL][4];  // B operand: token r16, the same K as the lane's weights
#pragma unroll
  for (int b = 0; b < NBL; ++b)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half8_t v = {};
      if (r16 < T) v = *reinterpret_cast<const half8_t*>(xs + r16 * H + 32 * (kb0 + b) + 8 * t);
      xf[b][t] = v;
    }
  const size_t roff = (size_t)(16 * rgrp + r16) * (H / 32) + kb0;

  for (int p0 = es; p0 < n_act; p0 += kMmaSlices * kB) {
    WRow<NBL> wg[kB], wu[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int p = p0 + j * kMmaSlices;
      if (p < n_act) {
        const int e = wl.act_e[p];
        wg[j] = load_wrow<Q, NBL>(ex, blk_gate(ex, e) + roff);
        wu[j] = load_wrow<Q, NBL>(ex, blk_up(ex, e) + roff);
      }
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int p = p0 + j * kMmaSlices;
      if (p >= n_act) break;
      floatx4_t ag = {}, au = {};
#pragma unroll
      for (int b = 0; b < NBL; ++b) {
        const WStage sg = wstage_block<Q>(wg[j].c[2 * b], wg[j].c[2 * b + 1], wg[j].hi[b], wg[j].dm[b]);
        const WStage su = wstage_block<Q>(wu[j].c[2 * b], wu[j].c[2 * b + 1], wu[j].hi[b], wu[j].dm[b]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag<Q>(sg, t), xf[b][t], ag, 0, 0, 0);
          au = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag<Q>(su, t), xf[b][t], au, 0, 0, 0);
        }
      }
      // ag[v]: row 4 c + v of the group, token r16
      if (r16 < kWinT) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          red[wave][j][0][4 * c + v][r16] = ag[v];
          red[wave][j][1][4 * c + v][r16] = au[v];
        }
      }
    }
    __syncthreads();
    // rows 4 q + s and 4 q + s + 2 (s = 0, 1) sit side by side in the K
    // order (0, 2, 1, 3): one 32-bit store each, coherent across the chip
    // (agent scope) for the down roles that read h in the same launch
    for (int i = tid; i < kB * 8 * kWinT; i += kWinThreads) {
      const int j = i / (8 * kWinT), pr = (i / kWinT) % 8, t = i % kWinT;
      const int p = p0 + j * kMmaSlices;
      if (p < n_act && t < T && ((wl.act_mask[p] >> t) & 1)) {  // the down roles read routed rows only
        const int ra = 4 * (pr >> 1) + (pr & 1), rb = ra + 2;
        float ga = 0.f, ua = 0.f, gb = 0.f, ub = 0.f;
#pragma unroll
        for (int w = 0; w < kWinWaves; ++w) {
          ga += red[w][j][0][ra][t];
          ua += red[w][j][1][ra][t];
          gb += red[w][j][0][rb][t];
          ub += red[w][j][1][rb][t];
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(hwin + ((size_t)p * kWinT + t) * ex.I + 16 * rgrp +
                                                    4 * (pr >> 1) + 2 * (pr & 1));
        __hip_atomic_store(dst, pack_bf16x2(silu_mul_x(ga, ua, xe[t]), silu_mul_x(gb, ub, xe[t])),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
}

// Down role: rows 8 grp .. 8 grp + 7 of H for every active expert, on
// v_mfma_f32_16x16x32_bf16 (bf16 weights, bf16 h in the MFMA K order). Wave w
// takes K half w & 1 and the experts w / 2, w / 2 + 4, ... in pairs (p, p + 4):
// a pair shares one 16 x 16 tile, rows 0-7 expert p's rows and rows 8-15
// expert p + 4's, columns 0-3 the tokens' h of p and columns 4-7 those of
// p + 4, so each expert's products sit in its own quarter of the tile (the
// other quarters are discarded): a 16-row tile carries 8 rows of two experts,
// which halves each role's dequantisation (the phase is VALU-bound) against
// 16-row roles, over twice the roles. The quarters are scaled by the routing
// gates and summed in registers; the eight waves' sums and the two halves are
// added in LDS in a fixed order and the role writes its rows of y. The
// weights of the first kDnW pairs per wave are requested before wait(), which
// returns once h is complete (false: it never was; the rows become NaN). Only
// the rows of h of routed (expert, token) pairs are read, packed in expert
// order into hs by one copy right after the wait (44 rows at a 4-token window
// with k = 10): one round trip of h, not one per round of experts.
constexpr int kHsBytes = 64 * 1024;   // LDS for h: 63 rows of I = 512 or 127 of I = 256, and a zero row
constexpr int kDnW = 8;     // tiles (expert pairs) per wave whose down weights are in registers
constexpr int kDnRows = 8;  // rows of H per down role

template <int Q, int NBL, typename Wait>
__device__ inline void down_role(const WinList& wl, int n_act, int grp, int T, const Experts& ex,
                                 const uint16_t* hwin, void* y, int out_f32, uint16_t* hs,
                                 float (&red)[kWinWaves][16][kWinT], Wait&& wait) {
  constexpr int kMaxAct = 64 + 1;       // T k <= 64 routed experts, the shared one
  constexpr int kMaxRows = 64 + kWinT;  // routed (expert, token) pairs
  constexpr int kChunk = 8 * kDnW;      // experts per chunk of registers (4 waves x kDnW pairs)
  __shared__ int hoff[kMaxAct + 1];     // first compact row of expert p; hoff[n_act] = rows
  __shared__ int16_t hsrc[kMaxRows];    // compact row -> slot p kWinT + t of hwin
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  n_act = __builtin_amdgcn_readfirstlane(n_act);  // uniform: scalar loop bounds
  const int I = ex.I;
  const int c = lane >> 4, r16 = lane & 15;
  const int ks = wave & 1, eq = wave >> 1;
  const int kb0 = ks * (I / 64) + NBL * c;  // this lane's first block of the wave's K half
  // the lane's weight row: row r16 & 7 of the role, of the pair's expert r16 >> 3
  const size_t roff = (size_t)(kDnRows * grp + (r16 & 7)) * (I / 32) + kb0;
  // the lane's h column: token r16 & 3 of the pair's expert (r16 >> 2) & 1
  // (columns 8-15 unused); its output quarter: rows of expert c >> 1
  const int tcol = r16 & 3, hcol = (r16 >> 2) & 1;
  const bool mine = r16 < 8 && hcol == (c >> 1) && tcol < T;
  const int cap = kHsBytes / (2 * I) - 1;  // rows of h that fit hs; the row after them stays zero
  // pair j of the chunk at c0: experts c0 + 8 j + eq and c0 + 8 j + eq + 4
  WRow<NBL> wd[kDnW];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int j = 0; j < kDnW; ++j) {
      const int p = c0 + 8 * j + eq + 4 * (r16 >> 3);
      if (p < n_act) {
        wd[j] = load_wrow<Q, NBL>(ex, blk_down(ex, wl.act_e[p]) + roff);
      } else {  // no such expert: zero weights (d = m = 0)
#pragma unroll
        for (int b = 0; b < NBL; ++b) {
          wd[j].c[2 * b] = wd[j].c[2 * b + 1] = 0u;
          wd[j].hi[b] = wd[j].dm[b] = 0u;
        }
      }
    }
  };
  // The compact list of the rows of h the role reads: the (expert, token)
  // pairs of the routing in expert order (wave 0; before the weight requests,
  // which then stay in flight through the wait).
  if (__builtin_amdgcn_readfirstlane(wave) == 0) {
    const int tm = (1 << T) - 1;
    const int m0 = lane < n_act ? wl.act_mask[lane] & tm : 0;
    const int m1 = lane + 64 < n_act ? wl.act_mask[lane + 64] & tm : 0;
    const int i0 = wave_inclusive_scan(__popc(m0));
    const int tot0 = __builtin_amdgcn_readlane(i0, 63);
    const int i1 = wave_inclusive_scan(__popc(m1)) + tot0;
    int o0 = i0 - __popc(m0), o1 = i1 - __popc(m1);
    if (lane < n_act) hoff[lane] = o0;
    if (lane + 64 < n_act) hoff[lane + 64] = o1;
    if (lane == 0) hoff[n_act] = __builtin_amdgcn_readlane(i1, 63);
#pragma unroll
    for (int t = 0; t < kWinT; ++t) {
      if ((m0 >> t) & 1) hsrc[o0++] = (int16_t)(lane * kWinT + t);
      if ((m1 >> t) & 1) hsrc[o1++] = (int16_t)((lane + 64) * kWinT + t);
    }
  }
  load_chunk(0);
  // the zero row that stands for every other pair (their gate is 0)
  for (int i = tid; i < I / 8; i += kWinThreads) reinterpret_cast<uint4*>(hs + (size_t)cap * I)[i] = make_uint4(0u, 0u, 0u, 0u);
  const bool ok = wait();  // ends with a barrier
  // every routed row of h straight into LDS (each lane's 16 bytes land at the
  // wave's base + 16 lane), all in flight at once, agent-coherent (h was
  // written in this launch on other CUs); chunk q of compact row r lands at
  // position q ^ (r & 3), so the rows a fragment read takes at one chunk sit
  // on different banks. The launch keeps every window's rows within hs
  // (win_mma_ok). A wave's load covers 64 chunks: one row at I = 512, two at
  // I = 256; its rows' sources are wave-uniform (scalar registers).
  {
    constexpr int kCopy = kHsBytes / 16 / kWinThreads;
    constexpr int kCoherent = 16;  // cache policy: agent scope
    const int n16 = __builtin_amdgcn_readfirstlane(hoff[n_act]) * (I / 8);
    const uint4* src = reinterpret_cast<const uint4*>(hwin);
    uint4* dst = reinterpret_cast<uint4*>(hs);
#pragma unroll
    for (int u = 0; u < kCopy; ++u) {
      const int i0 = u * kWinThreads + 64 * wave;
      if (i0 >= n16) break;
      const int rl = i0 / (I / 8);
      const int s0 = __builtin_amdgcn_readfirstlane(hsrc[rl]);
      const int s1 = __builtin_amdgcn_readfirstlane(hsrc[min(rl + 1, kMaxRows - 1)]);
      const int i = i0 + lane;
      if (i < n16) {
        const int r = i / (I / 8), q = i % (I / 8);
        __builtin_amdgcn_global_load_lds(src + (size_t)(r == rl ? s0 : s1) * (I / 8) + (q ^ (r & 3)),
                                         (__attribute__((address_space(3))) void*)(dst + i0), 16, 0,
                                         kCoherent);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the LDS writes have landed
  __syncthreads();
  floatx4_t acc = {};
  for (int c0 = 0; c0 < n_act; c0 += kChunk) {
    if (c0 > 0) {  // more than kChunk experts: the next chunk's weights
      load_chunk(c0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
#pragma unroll
    for (int j = 0; j < kDnW; ++j) {
      const int p = c0 + 8 * j + eq;  // the pair (p, p + 4)
      if (p >= n_act) break;
      // the column's row: compact when its token is routed to its expert,
      // else the zero row (columns 8-15, tokens past T, a missing p + 4)
      const int pc = p + 4 * hcol;
      const int m = r16 < 8 && pc < n_act ? wl.act_mask[pc] : 0;
      const bool cv = (m >> tcol) & 1;
      const int r = cv ? hoff[pc] + __popc(m & ((1 << tcol) - 1)) : cap;
      const uint16_t* hp = hs + (size_t)r * I;
      bf16x8_t hv[NBL][4];
#pragma unroll
      for (int b = 0; b < NBL; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          hv[b][t] = *reinterpret_cast<const bf16x8_t*>(hp + 8 * ((4 * (kb0 + b) + t) ^ (r & 3)));
      floatx4_t o = {};
#pragma unroll
      for (int b = 0; b < NBL; ++b) {
        const WStage sw = wstage_block<Q>(wd[j].c[2 * b], wd[j].c[2 * b + 1], wd[j].hi[b], wd[j].dm[b]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag_bf<Q>(sw, t), hv[b][t], o, 0, 0, 0);
      }
      // o[v]: tile row 4 c + v, column r16; kept where the row's expert is
      // the column's (c >> 1 == hcol)
      const float g = mine && cv ? wl.act_gate[pc][tcol] : 0.f;
#pragma unroll
      for (int v2 = 0; v2 < 4; ++v2) acc[v2] += g * o[v2];
      __builtin_amdgcn_sched_barrier(0);  // one pair's h operands in registers at a time
    }
  }
  if (mine) {  // (half, row, token): rows 4 c + v of the tile are row (4 c + v) & 7 of expert half c >> 1
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * c + v][tcol] = acc[v];
  }
  __syncthreads();
  if (tid < kDnRows * kWinT) {
    const int r = tid / kWinT, t = tid % kWinT;
    if (t < T) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWinWaves; ++w) s += red[w][r][t] + red[w][kDnRows + r][t];
      if (!ok) s = __uint_as_float(0x7FC00000u);
      const size_t o = (size_t)t * ex.H + kDnRows * grp + r;
      if (out_f32) static_cast<float*>(y)[o] = s;
      else static_cast<uint16_t*>(y)[o] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

// Counters of the one-launch window, at the head of the workspace, each on a
// 128-byte line of its own (atomics on one address serialise, so every up
// counter is shared by at most 16 workgroups). up[] counts over all launches
// on the workspace (mod 2^32), kSyncGroup per launch each, whatever the
// layer's shape: the 16 gate/up roles of group g add one each to up[g], and
// the launch's last down role adds kSyncGroup to every up[g] past the
// launch's groups. So after n complete launches every up[g] = 16 n and
// epoch = n, and a launch finds them consistent whatever happened in earlier
// ones, including waits that timed out (late gate/up roles still finish
// before their launch ends). dn[16] count the down roles of the running
// launch (ceil(D / 16) per line) and dn_all the lines that completed; the
// last role of a line zeroes it, the launch's last down role zeroes dn_all
// and raises epoch, so both are zero between launches. `guard`
// is never written: non-zero means the head was not zeroed. `spin`: 0, or a
// bound in wall-clock ticks on the down roles' wait (a testing aid).
// Launches that start from hidden states (RT launches): rt_seq[r] counts
// the RT launches on the workspace for router role r (the role adds one at its
// start; an RT launch without that role has its last down role add it), and
// rt_epoch counts them too (raised by each RT launch's last down role), so the
// role's add returns the launch's number n = rt_epoch, however late the role
// runs; launches that start from logits touch neither. The role tags
// every logit it stores with n + 1 (tag and value in one 64-bit store), then
// adds one to rt_all without waiting for the stores; the role that completes
// rt_all sets it back to zero (router roles never wait, so it is zero between
// launches) and writes n + 1 into the 16 go lines. The other workgroups watch
// one go line each (few waves per line), then read the logits, again until
// every tag shows their launch (the tags, not the order of the stores, make
// the values current). A workgroup whose wait runs out writes epoch + 1 into
// `poison` before it counts; down roles that find it after their own wait
// write NaN, so no launch mixes routings.
constexpr int kSyncGroup = 16;   // workgroups per counter
constexpr int kSyncLine = 32;    // uint32 per 128-byte line
struct WinSync {
  uint32_t guard[kSyncLine];
  uint32_t spin[kSyncLine];
  uint32_t epoch[kSyncLine];     // launches completed
  uint32_t dn_all[kSyncLine];    // down-role lines complete (this launch)
  uint32_t up[16][kSyncLine];    // gate/up roles of group g whose h is released
  uint32_t rt_epoch[kSyncLine];  // RT launches completed
  uint32_t rt_seq[kSyncLine];    // RT launches seen by router role r (r < 32)
  uint32_t rt_all[kSyncLine];    // router roles whose logits are issued (this launch)
  uint32_t go[16][kSyncLine];    // n + 1 once every router role of launch n has issued its logits
  uint32_t poison[kSyncLine];    // epoch + 1: a workgroup of that launch routed without logits
  uint32_t dn[16][kSyncLine];    // down roles finished (this launch), ceil(D / 16) per line
};
static_assert(sizeof(WinSync) <= kWinSyncBytes, "the window counters fit the workspace head");

constexpr int kLayerPer = 8;  // logits per lane in the one-launch window: E <= 512
constexpr long long kWinSpinTicks = 1ll << 24;  // wall-clock ticks a down role waits for h at most
constexpr int kRtExperts = 2 * kWinWaves;       // experts per router role (two per wave)
static_assert(64 * kLayerPer <= kSyncLine * kRtExperts, "a launch counter per router role");

// A logit of the launch numbered n - 1 as stored by a router role: tag n in
// the high word, the value's bits in the low word (one 64-bit store).
__device__ inline void store_tagged(uint64_t* p, uint32_t tag, float v, float* plain) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  if (plain) *plain = v;
}

__device__ inline uint32_t sync_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t sync_add(uint32_t* p, uint32_t v = 1u) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void sync_zero(uint32_t* p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Router role r for bf16 x (matrix cores): the logits of experts 16 r ..
// 16 r + 15 for the window's tokens. Wave w takes K slice w of H / 8 and runs
// kM = H / 256 v_mfma_f32_16x16x32_bf16 on it (router rows as the 16 rows of
// A, tokens as the columns of B, tokens past T zero): lane (i, c) = (lane %
// 16, lane / 16) feeds 8 elements of row i per product from its own
// contiguous quarter of the slice, for the router row and for the token row
// alike (the same K permutation on both operands). Every load is issued at
// entry. Products of bf16 values are exact in f32; the eight slices' partial
// tiles are added in LDS in wave order, so the logits are reproducible.
template <int NBG>
__device__ inline void router_role_mma(int r, const uint16_t* __restrict__ x, int T, int H,
                                       const uint16_t* __restrict__ rw,
                                       const float* __restrict__ rbias, int E, uint32_t tag,
                                       uint64_t* lgp, float* lg, float* red) {
  constexpr int kM = 4 * NBG;  // products per wave (H = 1024 NBG)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, c = lane >> 4;
  const int kq = H / 32;                            // elements of one lane quarter of a slice
  const int k0 = wave * (H / 8) + c * kq;           // this lane's first element
  const int e = min(kRtExperts * r + i, E - 1);
  const uint4* wr = reinterpret_cast<const uint4*>(rw + (size_t)e * H + k0);
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)min(i, T - 1) * H + k0);
  uint4 wv[kM], xv[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    wv[m] = wr[m];
    xv[m] = i < T ? xr[m] : make_uint4(0u, 0u, 0u, 0u);
  }
  const int eo = kRtExperts * r + (tid >> 2);  // expert and token of this thread's sum below
  const float b = (tid < 64 && rbias && eo < E) ? rbias[eo] : 0.f;
  floatx4_t acc = {};
#pragma unroll
  for (int m = 0; m < kM; ++m)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[m]),
                                                  __builtin_bit_cast(bf16x8_t, xv[m]), acc, 0, 0, 0);
  // acc[v]: expert 4 c + v of the role's 16, token i
  if (i < kWinT) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * c + v) * kWinT + i] = acc[v];
  }
  __syncthreads();
  if (tid < 64) {
    const int el = tid >> 2, t = tid & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWinWaves; ++w) v += red[(w * 16 + el) * kWinT + t];
    if (t < T && eo < E)
      store_tagged(lgp + (size_t)t * E + eo, tag, v + b, lg ? lg + (size_t)t * E + eo : nullptr);
  }
}

// Router role r of a launch that starts from hidden states: the router scores
// ("Strata - the details", "How it works": each layer's router runs on the
// GPU in front of its experts) of experts 16 r .. 16 r + 15 for the window's
// tokens, logits[t][e] = x[t] . w[e] (+ bias[e]), stored agent-coherent into
// lg [T][E]. Wave w takes experts 16 r + 2 w and 16 r + 2 w + 1: its router
// rows' 16-byte chunks lane + 64 j (8 elements each) come into registers
// first, the window's rows into LDS as f32 meanwhile; each lane runs an fp32
// fma chain over its chunks and a fixed-order wave sum finishes every dot, so
// the logits are reproducible (the error of an f32 sum of H products).
template <bool XF32>
__device__ inline void router_role(int r, const void* x, int T, int H, const uint16_t* __restrict__ rw,
                                   const float* __restrict__ rbias, int E, uint32_t tag, uint64_t* lgp,
                                   float* lg, float* xsf) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kU = kMmaMaxH / 512;
  const int nu = H / 512;
  uint4 wv[2][kU];
  int e[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    e[i] = kRtExperts * r + 2 * wave + i;
    const uint4* row = reinterpret_cast<const uint4*>(rw + (size_t)min(e[i], E - 1) * H);
#pragma unroll
    for (int j = 0; j < kU; ++j) wv[i][j] = j < nu ? row[lane + 64 * j] : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int i = tid; i < T * (H / 4); i += kWinThreads) {
    const int t = i / (H / 4), q = i - t * (H / 4);
    float4 f;
    if (XF32) {
      f = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * H)[q];
    } else {
      const uint2 u = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)t * H)[q];
      f = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    reinterpret_cast<float4*>(xsf)[i] = f;
  }
  __syncthreads();
  float acc[2][kWinT] = {};
#pragma unroll
  for (int j = 0; j < kU; ++j) {
    if (j < nu) {
      const int q = lane + 64 * j;  // elements 8 q .. 8 q + 7
#pragma unroll
      for (int t = 0; t < kWinT; ++t) {
        if (t < T) {
          const float4 a = reinterpret_cast<const float4*>(xsf + t * H + 8 * q)[0];
          const float4 b = reinterpret_cast<const float4*>(xsf + t * H + 8 * q)[1];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint4 w = wv[i][j];
            float v = acc[i][t];
            v = fmaf(a.x, bf16_lo(w.x), v);
            v = fmaf(a.y, bf16_hi(w.x), v);
            v = fmaf(a.z, bf16_lo(w.y), v);
            v = fmaf(a.w, bf16_hi(w.y), v);
            v = fmaf(b.x, bf16_lo(w.z), v);
            v = fmaf(b.y, bf16_hi(w.z), v);
            v = fmaf(b.z, bf16_lo(w.w), v);
            v = fmaf(b.w, bf16_hi(w.w), v);
            acc[i][t] = v;
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float b = (rbias && e[i] < E) ? rbias[e[i]] : 0.f;
#pragma unroll
    for (int t = 0; t < kWinT; ++t) {
      if (t < T) {
        const float v = wave_sum(acc[i][t]) + b;
        if (lane == 0 && e[i] < E)
          store_tagged(lgp + (size_t)t * E + e[i], tag, v, lg ? lg + (size_t)t * E + e[i] : nullptr);
      }
    }
  }
}

// The whole window in one launch on the matrix cores (H a multiple of 1,024 up
// to 4,096; I 256 or 512). Every workgroup routes the window itself (top-k of
// T logit rows, a few KB, and the active-expert list in LDS). Workgroups
// 0 .. G-1 (G = 8 I / 16) are gate/up roles, the next D = H / 16 down roles.
// A down role requests its weights (which depend only on the routing), then
// waits until every gate/up role has released h. Workgroups are dispatched in
// index order, so a waiting down role never holds back a gate/up role; the
// wait is also bounded in time, past which the role writes NaN rows.
//
// RT (start from hidden states): NR = E / 16 router roles come first and
// store the logits into lg; every other workgroup waits for them (bounded as
// above) before its top-k. A router wait that runs out routes the window to
// experts 0 .. k-1 with NaN gates, so its rows become NaN while every count
// stays balanced. Without RT, lg holds the caller's logits.
template <int Q, bool XF32, int NBG, int NBD, bool RT>
__global__ __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(4)))
void win_layer(float* lg, uint64_t* lgp, const uint16_t* __restrict__ rw, const float* __restrict__ rbias,
               int T, int k, Experts ex, const void* x, int32_t* idx_out, float* gates_out,
               uint16_t* hwin, void* y, int out_f32, WinSync* sync) {
  __shared__ LayerRoute R;
  // gate/up roles: activations (fp16, 32 KB) and partial tiles (16 KB); down roles: h
  __shared__ __attribute__((aligned(16))) char buf[kHsBytes];
  __shared__ float red_dn[kWinWaves][16][kWinT];
  static_assert(kWinT * kMmaMaxH * 2 + kWinWaves * kMmaBatch * 2 * 16 * kWinT * 4 <= kHsBytes, "");
  _Float16* xs = reinterpret_cast<_Float16*>(buf);
  auto& red = *reinterpret_cast<float(*)[kWinWaves][kMmaBatch][2][16][kWinT]>(buf + kWinT * kMmaMaxH * 2);
  __shared__ uint32_t head_s[3];  // guard, spin, epoch
  __shared__ int bad_s;
  __shared__ int xe_w[kWinT];  // per-token exponents of the fp16 activations
  const int tid = threadIdx.x;
  const int H = ex.H;
  const int G = ex.I / 16 * kMmaSlices, D = H / kDnRows;
  const int NR = RT ? (ex.E + kRtExperts - 1) / kRtExperts : 0;
  if (RT && (int)blockIdx.x < NR) {
    __shared__ uint32_t tag_s;
    if (tid == 0) tag_s = sync_add(&sync->rt_seq[blockIdx.x]) + 1u;
    __syncthreads();
    const uint32_t tag = tag_s;
    if constexpr (XF32)
      router_role<true>(blockIdx.x, x, T, H, rw, rbias, ex.E, tag, lgp, lg, reinterpret_cast<float*>(buf));
    else
      router_role_mma<NBG>(blockIdx.x, static_cast<const uint16_t*>(x), T, H, rw, rbias, ex.E, tag, lgp,
                           lg, reinterpret_cast<float*>(buf));
    __syncthreads();  // every wave's stores are issued
    if (tid == 0 && sync_add(sync->rt_all) == (uint32_t)(NR - 1)) {
      sync_zero(sync->rt_all);
      for (int g = 0; g < 16; ++g)
        __hip_atomic_store(sync->go[g], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  const int role = blockIdx.x - NR;

  // the head's words are requested first (their round trip overlaps the
  // activation and logit loads instead of following them)
  uint32_t head_r[3] = {0u, 0u, 0u};
  if (tid == kWinThreads - 64) {
    head_r[0] = sync_load(sync->guard);
    head_r[1] = sync_load(sync->spin);
    head_r[2] = sync_load(sync->epoch);
  }
  if (!RT) win_topk<kLayerPer>(R, lg, T, ex.E, k);
  // the window's activations -> LDS fp16 in the MFMA K order (tokens >= T
  // zero), by the waves that do not select experts, one token row per wave:
  // the row is scaled by 2^-e (row_exp of its largest |x|), e kept in xe_w
  {
    const int t = (tid >> 6) - kWinT, lane = tid & 63;
    if (!XF32 && t >= 0 && t < kWinT) {
      // bf16 rows: the row's quads come into registers once; their largest
      // magnitude gives e, then they are converted from the registers
      constexpr int kQ = kMmaMaxH / 4 / 64;
      uint2 qv[kQ];
      uint32_t m = 0;
      const uint2* row = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)(t < T ? t : 0) * H);
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int q = lane + 64 * i;
        qv[i] = make_uint2(0u, 0u);
        if (t < T && q < H / 4) qv[i] = row[q];
        const uint32_t a = max(qv[i].x & 0x7FFF7FFFu, qv[i].y & 0x7FFF7FFFu);
        m = max(m, max(a & 0xFFFFu, a >> 16));
      }
      const int e = row_exp(__uint_as_float(wave_max_u32(m) << 16));
      if (lane == 0) xe_w[t] = e;
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int q = lane + 64 * i;
        if (q < H / 4) {
          const float v0 = __builtin_ldexpf(bf16_lo(qv[i].x), -e), v1 = __builtin_ldexpf(bf16_hi(qv[i].x), -e);
          const float v2 = __builtin_ldexpf(bf16_lo(qv[i].y), -e), v3 = __builtin_ldexpf(bf16_hi(qv[i].y), -e);
          *reinterpret_cast<uint2*>(xs + t * H + 4 * q) = make_uint2(pack_half2(v0, v2), pack_half2(v1, v3));
        }
      }
    } else if (t >= 0 && t < kWinT) {
      const int e = t < T ? row_exp(row_absmax(x, !XF32, H, t)) : 0;
      if (lane == 0) xe_w[t] = e;
      for (int q = lane; q < H / 4; q += 64) {
        float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
        if (t < T) {
          if (XF32) {
            const float4 f = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * H)[q];
            v0 = f.x; v1 = f.y; v2 = f.z; v3 = f.w;
          } else {
            const uint2 u = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)t * H)[q];
            v0 = bf16_lo(u.x); v1 = bf16_hi(u.x); v2 = bf16_lo(u.y); v3 = bf16_hi(u.y);
          }
          v0 = __builtin_ldexpf(v0, -e); v1 = __builtin_ldexpf(v1, -e);
          v2 = __builtin_ldexpf(v2, -e); v3 = __builtin_ldexpf(v3, -e);
        }
        *reinterpret_cast<uint2*>(xs + t * H + 4 * q) = make_uint2(pack_half2(v0, v2), pack_half2(v1, v3));
      }
    }
  }
  if (tid == kWinThreads - 64) {
    head_s[0] = head_r[0];
    head_s[1] = head_r[1];
    head_s[2] = head_r[2];
  }
  __shared__ int rt_bad_w[kWinT];
  if (RT) {
    // lane 0 of wave 0 watches go line role % 16 (with pauses) until it shows
    // this launch; then wave t < T reads token t's tagged logits
    // (agent-coherent, all in flight at once) until every tag shows it too,
    // and selects its experts from those values. Both waits are bounded like
    // the down roles' wait; a wave that gives up routes to experts 0 .. k-1
    // with NaN gates.
    const int wave = tid >> 6, lane = tid & 63;
    const uint32_t want = sync_load(sync->rt_epoch) + 1u;
    const uint32_t sp = sync_load(sync->spin);
    const long long spin = sp ? (long long)sp : kWinSpinTicks;
    const long long t0 = wall_clock64();
    if (tid == 0) {
      const uint32_t* go = sync->go[role % 16];
      while (sync_load(go) != want && wall_clock64() - t0 <= spin) __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();
    if (wave < T) {
      const uint64_t* l = lgp + (size_t)wave * ex.E;
      float raw[kLayerPer];
      bool bad = false;
      for (;;) {
        bool mine = true;
#pragma unroll
        for (int i = 0; i < kLayerPer; ++i) {
          const uint64_t v = __hip_atomic_load(l + min(lane + 64 * i, ex.E - 1), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          mine = mine && (uint32_t)(v >> 32) == want;
          raw[i] = __uint_as_float((uint32_t)v);
        }
        if (__ballot(!mine) == 0) break;
        if (wall_clock64() - t0 > spin) {
          bad = true;
          break;
        }
      }
      if (!bad) {
        topk_select<kLayerPer>(raw, ex.E, k, R.lidx + wave * k, R.lgate + wave * k, &R.tks[wave]);
      } else {
        for (int j = lane; j < k; j += 64) {
          R.lidx[wave * k + j] = j;
          R.lgate[wave * k + j] = __uint_as_float(0x7FC00000u);
        }
      }
      if (lane == 0) rt_bad_w[wave] = bad;
    }
  }
  const int n_act = win_list(R, ex, T, k, false, nullptr, nullptr, nullptr);  // ends with a barrier
  if (RT && tid == 0) {
    bool bad = false;
    for (int t = 0; t < T; ++t) bad = bad || rt_bad_w[t];
    // counted below (gate/up roles) behind their vmcnt(0); down roles' rows are NaN anyway
    if (bad)
      __hip_atomic_store(sync->poison, head_s[2] + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (head_s[0] != 0u) {  // the head was not zeroed: y becomes NaN
    for (int i = tid; i < T * H; i += kWinThreads) {
      if (out_f32) static_cast<float*>(y)[i] = __uint_as_float(0x7FC00000u);
      else static_cast<uint16_t*>(y)[i] = 0x7FC0u;
    }
    return;
  }
  if (role == 0)
    for (int a = tid; a < T * k; a += kWinThreads) {
      idx_out[a] = R.lidx[a];
      gates_out[a] = R.lgate[a];
    }
  if (role < G) {
    gateup_role<Q, NBG>(R.wl, n_act, role, T, ex, xs, xe_w, red, hwin);
    // The h stores are agent-coherent; a wave's store count reaching zero means
    // they are performed chip-wide, so once every wave has waited for that,
    // the role's count orders them before the down roles' reads (which are
    // agent-coherent too). No cache write-back is needed.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) sync_add(sync->up[role / kSyncGroup]);
    return;
  }
  // Wave 0 watches the launch's group counters (one load, a lane per group,
  // then a pause, so the counters' lines stay quiet for the gate/up roles'
  // atomics) until all are complete; bounded in time, past which the rows
  // become NaN.
  const uint32_t target = (uint32_t)kSyncGroup * (head_s[2] + 1u);
  const long long spin = head_s[1] ? (long long)head_s[1] : kWinSpinTicks;
  auto wait = [&]() -> bool {
    if (tid < 64) {
      const int lane = tid;
      const long long t0 = wall_clock64();
      bool bad = false;
      for (;;) {
        const bool done = lane >= G / kSyncGroup || sync_load(sync->up[lane]) == target;
        if (__ballot(!done) == 0) break;
        if (wall_clock64() - t0 > spin) {
          bad = true;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      // a workgroup of this launch that routed without the logits wrote the
      // poison word before it counted
      if (RT && !bad && lane == 0) bad = sync_load(sync->poison) == head_s[2] + 1u;
      if (lane == 0) bad_s = bad;
    }
    __syncthreads();
    return bad_s == 0;
  };
  const int grp = role - G;
  down_role<Q, NBD>(R.wl, n_act, grp, T, ex, hwin, y, out_f32, reinterpret_cast<uint16_t*>(buf),
                    red_dn, wait);
  // Completion: each down role counts on one of 16 lines (ceil(D / 16) roles
  // per line; atomics on one address serialise, so no single counter takes
  // all D adds); the last role of a line resets it and counts the line on
  // dn_all, and the role that completes dn_all is the launch's last (timed-out
  // roles count too): it tops up the groups this launch's shape has none of,
  // resets dn_all and closes the launch.
  const int per = (D + 15) / 16, line = grp / per, in_line = min(per, D - line * per);
  if (tid == 0 && sync_add(sync->dn[line]) == (uint32_t)(in_line - 1)) {
    sync_zero(sync->dn[line]);
    if (sync_add(sync->dn_all) == (uint32_t)((D + per - 1) / per - 1)) {
      for (int g = G / kSyncGroup; g < 16; ++g) sync_add(sync->up[g], (uint32_t)kSyncGroup);
      if (RT) {
        for (int r = NR; r < kSyncLine; ++r) sync_add(&sync->rt_seq[r]);
        sync_add(sync->rt_epoch);
      }
      sync_zero(sync->dn_all);
      sync_add(sync->epoch);
    }
  }
}

inline bool win_mma_ok(const Experts& ex, int T, int k) {
  // the down roles hold every routed (expert, token) row of h in LDS at once
  const int rows = T * k + T * ex.has_shared;
  return ex.H % 1024 == 0 && ex.H <= kMmaMaxH && (ex.I == 256 || ex.I == 512) &&
         ex.E <= 64 * kLayerPer && T * k <= 64 && rows <= kHsBytes / (2 * ex.I) - 1;
}

template <int BPR_H, int BPR_I, int Q, bool XF32>
hipError_t launch_w(const float* logits, int T, int k, const Experts& ex, const void* x,
                    int32_t* idx, float* gates, WinList* meta, uint16_t* hwin, void* y, int out_f32,
                    hipStream_t s) {
  MOE_LAUNCH("win_gateup", s, (win_gateup<BPR_H, Q, XF32>), dim3(ex.I / win_gu_rows<BPR_H>()),
             dim3(kWinThreads), 0, s, logits, T, k, ex, x, idx, gates, meta, hwin);
  MOE_LAUNCH("win_down", s, (win_down<BPR_I, Q>), dim3(ex.H / win_dn_rows<BPR_I>()),
             dim3(kWinThreads), 0, s, T, ex, meta, hwin, y, out_f32);
  return hipGetLastError();
}

template <int Q, bool XF32, bool RT>
hipError_t launch_layer(float* lg, uint64_t* lgp, const uint16_t* rw, const float* rbias, int T, int k,
                        const Experts& ex, const void* x, int32_t* idx, float* gates, uint16_t* hwin,
                        void* y, int out_f32, WinSync* sync, hipStream_t s) {
  const int NR = RT ? (ex.E + kRtExperts - 1) / kRtExperts : 0;
  const dim3 grid(NR + ex.I / 16 * kMmaSlices + ex.H / kDnRows);
  const char* name = RT ? "win_layer_rt" : "win_layer";
#define L(NBG, NBD)                                                                               \
  MOE_LAUNCH(name, s, (win_layer<Q, XF32, NBG, NBD, RT>), grid, dim3(kWinThreads), 0, s, lg, lgp, \
             rw, rbias, T, k, ex, x, idx, gates, hwin, y, out_f32, sync)
  const int nbg = ex.H / 1024, nbd = ex.I / 256;
  if (nbg == 1 && nbd == 1) L(1, 1);
  else if (nbg == 1) L(1, 2);
  else if (nbg == 2 && nbd == 1) L(2, 1);
  else if (nbg == 2) L(2, 2);
  else if (nbd == 1) L(4, 1);
  else L(4, 2);
#undef L
  return hipGetLastError();
}

template <int Q, bool XF32>
hipError_t launch_wq(int bh, int bi, const float* logits, int T, int k, const Experts& ex,
                     const void* x, int32_t* idx, float* gates, WinList* meta, uint16_t* hwin,
                     void* y, int out_f32, hipStream_t s) {
#define W(BH, BI)                                                                          \
  if (bh == BH && bi == BI)                                                                \
    return launch_w<BH, BI, Q, XF32>(logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
  W(64, 16) W(64, 32) W(64, 64) W(64, 8) W(64, 4)
  W(32, 16) W(32, 32) W(32, 64) W(32, 8) W(32, 4)
  W(16, 16) W(16, 32) W(16, 64) W(16, 8) W(16, 4)
  W(8, 16) W(8, 32) W(8, 64) W(8, 8) W(8, 4)
  W(4, 16) W(4, 32) W(4, 64) W(4, 8) W(4, 4)
#undef W
  return hipErrorInvalidValue;
}

}  // namespace

bool window_supported(const Experts& ex, int T, int k) {
  auto ok = [](int bpr) { return bpr == 4 || bpr == 8 || bpr == 16 || bpr == 32 || bpr == 64; };
  if (!(T >= 1 && T <= kWinT && k <= kWinMaxK && ok(ex.H / 32) && ok(ex.I / 32))) return false;
  const int rows = 2 * (64 / (ex.I / 32));  // down rows per workgroup
  return ex.H % rows == 0 && ex.I % (64 / (ex.H / 32) > 2 ? 64 / (ex.H / 32) : 2) == 0;
}

// Window workspace: counters (kWinSyncBytes; see WinSync) | active list |
// h [n_act][kWinT][I] (bf16; in the MFMA K order for the one-launch form).
namespace {
struct WinLayout {
  size_t sync, meta, h, total;
};
WinLayout win_layout(const Experts& ex, int T, int k) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  WinLayout L{};
  size_t off = 0;
  L.sync = off; off = al(off + kWinSyncBytes);
  L.meta = off; off = al(off + sizeof(WinList));
  L.h = off;    off = al(off + sizeof(uint16_t) * ((size_t)T * k + ex.has_shared) * kWinT * ex.I);
  L.total = off;
  return L;
}
}  // namespace

size_t window_workspace_bytes(const Experts& ex, int T, int k) { return win_layout(ex, T, k).total; }

hipError_t launch_window(const float* logits, int T, int k, const Experts& ex, const void* x,
                         int xdtype, int32_t* idx, float* gates, void* y, int out_f32, void* ws,
                         hipStream_t s) {
  const WinLayout L = win_layout(ex, T, k);
  char* base = static_cast<char*>(ws);
  WinList* meta = reinterpret_cast<WinList*>(base + L.meta);
  uint16_t* hwin = reinterpret_cast<uint16_t*>(base + L.h);
  if (win_mma_ok(ex, T, k)) {
    WinSync* sync = reinterpret_cast<WinSync*>(base + L.sync);
    float* lg = const_cast<float*>(logits);  // read only without RT
    if (ex.qtype == 3)
      return xdtype == 0
                 ? launch_layer<3, true, false>(lg, nullptr, nullptr, nullptr, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s)
                 : launch_layer<3, false, false>(lg, nullptr, nullptr, nullptr, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s);
    return xdtype == 0
               ? launch_layer<2, true, false>(lg, nullptr, nullptr, nullptr, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s)
               : launch_layer<2, false, false>(lg, nullptr, nullptr, nullptr, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s);
  }
  const int bh = ex.H / 32, bi = ex.I / 32;
  if (ex.qtype == 3)
    return xdtype == 0 ? launch_wq<3, true>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s)
                       : launch_wq<3, false>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
  return xdtype == 0 ? launch_wq<2, true>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s)
                     : launch_wq<2, false>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
}

bool window_hidden_supported(const Experts& ex, int T, int k) {
  return window_supported(ex, T, k) && win_mma_ok(ex, T, k);
}

hipError_t launch_window_hidden(float* lg, uint64_t* lgp, const uint16_t* rw, const float* rbias,
                                int T, int k, const Experts& ex, const void* x, int xdtype,
                                int32_t* idx, float* gates, void* y, int out_f32, void* ws,
                                hipStream_t s) {
  if (!window_hidden_supported(ex, T, k)) return hipErrorInvalidValue;
  const WinLayout L = win_layout(ex, T, k);
  char* base = static_cast<char*>(ws);
  uint16_t* hwin = reinterpret_cast<uint16_t*>(base + L.h);
  WinSync* sync = reinterpret_cast<WinSync*>(base + L.sync);
  if (ex.qtype == 3)
    return xdtype == 0
               ? launch_layer<3, true, true>(lg, lgp, rw, rbias, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s)
               : launch_layer<3, false, true>(lg, lgp, rw, rbias, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s);
  return xdtype == 0
             ? launch_layer<2, true, true>(lg, lgp, rw, rbias, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s)
             : launch_layer<2, false, true>(lg, lgp, rw, rbias, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s);
}

}  // namespace moe

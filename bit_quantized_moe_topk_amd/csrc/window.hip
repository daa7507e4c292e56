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
                                   const _Float16* xs,
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
      if (p < n_act && t < T) {  // every token (finite values) for the down tiles
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
        __hip_atomic_store(dst, pack_half2(silu_mul(ga, ua), silu_mul(gb, ub)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
}

// Down role: rows 16 grp .. 16 grp + 15 of H for every active expert; wave w
// takes K half w & 1 and the experts w / 2, w / 2 + 4, ...: per expert a
// 16-row x 16-token tile (tokens past T zero) with h (fp16, MFMA K order) as
// the token operand, scaled by the routing gates and summed in registers; the
// eight partial tiles are added in LDS in wave order and the role writes its
// rows of y. The first round's weights are requested before wait(), which
// returns once h is complete (false: it never was; the rows become NaN). h
// then comes into LDS (hs, kHsBytes) a phase of experts at a time, every load
// of a phase in flight at once.
// experts per wave whose weights are in registers (Q3 rows carry a third-bit
// plane, so fewer of them fit)
template <int Q>
constexpr int dn_batch() {
  return Q == 3 ? 3 : 4;
}
constexpr int kHsBytes = 64 * 1024;   // LDS for h: 16 experts at I = 512, 32 at I = 256

template <int Q, int NBL, typename Wait>
__device__ inline void down_role(const WinList& wl, int n_act, int grp, int T, const Experts& ex,
                                 const uint16_t* hwin, void* y, int out_f32, _Float16* hs,
                                 float (&red)[kWinWaves][16][kWinT], Wait&& wait) {
  constexpr int kDnBatch = dn_batch<Q>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = ex.I;
  const int c = lane >> 4, r16 = lane & 15;
  const int ks = wave & 1, eq = wave >> 1;
  const int kb0 = ks * (I / 64) + NBL * c;  // this lane's first block of the wave's K half
  const size_t roff = (size_t)(16 * grp + r16) * (I / 32) + kb0;
  const bool tok = r16 < T;
  WRow<NBL> wd[kDnBatch];
#pragma unroll
  for (int j = 0; j < kDnBatch; ++j) {  // the first round's weights, before the wait
    const int p = eq + 4 * j;
    if (p < n_act) wd[j] = load_wrow<Q, NBL>(ex, blk_down(ex, wl.act_e[p]) + roff);
  }
  const bool ok = wait();
  floatx4_t acc = {};
  static_assert(kHsBytes / (kWinT * 512 * 2) >= 4 * kDnBatch, "h of one round fits hs (I <= 512)");
  for (int r0 = 0; r0 < n_act; r0 += 4 * kDnBatch) {  // rounds of 4 kDnBatch experts
    const int n16 = min(4 * kDnBatch, n_act - r0) * kWinT * I / 8;
    const uint4* src = reinterpret_cast<const uint4*>(hwin) + (size_t)r0 * kWinT * I / 8;
    // h of the round straight into LDS (each lane's 16 bytes land at the
    // wave's base + 16 lane), no registers held; every load in flight at once,
    // agent-coherent (h was written in this launch on other CUs)
    constexpr int kCopy = kHsBytes / 16 / kWinThreads;
    constexpr int kCoherent = 16;  // cache policy: agent scope
    __syncthreads();  // the previous round's reads of hs are done
#pragma unroll
    for (int u = 0; u < kCopy; ++u)
      if (tid + u * kWinThreads < n16)
        __builtin_amdgcn_global_load_lds(
            src + tid + u * kWinThreads,
            (__attribute__((address_space(3))) void*)(reinterpret_cast<uint4*>(hs) + u * kWinThreads +
                                                      64 * wave),
            16, 0, kCoherent);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the LDS writes have landed
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kDnBatch; ++j) {
      const int p = r0 + eq + 4 * j;
      if (p >= n_act) continue;
      // columns past T read token 0's row (finite; their gate is 0): no
      // branch, so all eight LDS reads of the expert issue together
      const _Float16* hp = hs + ((size_t)(p - r0) * kWinT + (tok ? r16 : 0)) * I;
      half8_t hv[NBL][4];
#pragma unroll
      for (int b = 0; b < NBL; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t) hv[b][t] = *reinterpret_cast<const half8_t*>(hp + 32 * (kb0 + b) + 8 * t);
      floatx4_t o = {};
#pragma unroll
      for (int b = 0; b < NBL; ++b) {
        const WStage sw = wstage_block<Q>(wd[j].c[2 * b], wd[j].c[2 * b + 1], wd[j].hi[b], wd[j].dm[b]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          o = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag<Q>(sw, t), hv[b][t], o, 0, 0, 0);
      }
      const float ga = wl.act_gate[p][r16 & (kWinT - 1)];
      const float g = tok ? ga : 0.f;  // o[v]: row 4 c + v, token r16
#pragma unroll
      for (int v2 = 0; v2 < 4; ++v2) acc[v2] += g * o[v2];
      // this slot's weights for the next round, in flight during the rest of this one
      const int pn = p + 4 * kDnBatch;
      if (pn < n_act) wd[j] = load_wrow<Q, NBL>(ex, blk_down(ex, wl.act_e[pn]) + roff);
    }
  }
  if (r16 < kWinT) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * c + v][r16] = acc[v];
  }
  __syncthreads();
  if (tid < 16 * kWinT) {
    const int r = tid / kWinT, t = tid % kWinT;
    if (t < T) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWinWaves; ++w) s += red[w][r][t];
      if (!ok) s = __uint_as_float(0x7FC00000u);
      const size_t o = (size_t)t * ex.H + 16 * grp + r;
      if (out_f32) static_cast<float*>(y)[o] = s;
      else static_cast<uint16_t*>(y)[o] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

// Counters of the one-launch window, at the head of the workspace, each on a
// 128-byte line of its own (atomics on one address serialise, so every counter
// is shared by at most 16 workgroups). Zero when a launch starts; the launch's
// last down workgroup zeroes them again. `guard` is never written: non-zero
// means the head was not zeroed.
constexpr int kSyncGroup = 16;   // workgroups per counter
constexpr int kSyncLine = 32;    // uint32 per 128-byte line
struct WinSync {
  uint32_t guard[kSyncLine];
  uint32_t up[16][kSyncLine];    // gate/up roles of group g whose h is released
  uint32_t dn[16][kSyncLine];    // down roles of group g finished
  uint32_t dn_all[kSyncLine];    // down groups finished
};
static_assert(sizeof(WinSync) <= kWinSyncBytes, "the window counters fit the workspace head");

constexpr int kLayerPer = 8;  // logits per lane in the one-launch window: E <= 512
constexpr long long kWinSpinTicks = 1ll << 24;  // wall-clock ticks a down role waits for h at most

__device__ inline uint32_t sync_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t sync_add(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void sync_zero(uint32_t* p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The whole window in one launch on the matrix cores (H a multiple of 1,024 up
// to 4,096; I 256 or 512). Every workgroup routes the window itself (top-k of
// T logit rows, a few KB, and the active-expert list in LDS). Workgroups
// 0 .. G-1 (G = 8 I / 16) are gate/up roles, the next D = H / 16 down roles.
// A down role requests its weights (which depend only on the routing), then
// waits until every gate/up role has released h. Workgroups are dispatched in
// index order, so a waiting down role never holds back a gate/up role; the
// wait is also bounded in time, past which the role writes NaN rows.
template <int Q, bool XF32, int NBG, int NBD>
__global__ __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(4)))
void win_layer(const float* __restrict__ logits, int T, int k, Experts ex, const void* x,
               int32_t* idx_out, float* gates_out, uint16_t* hwin, void* y, int out_f32,
               WinSync* sync) {
  __shared__ LayerRoute R;
  // gate/up roles: activations (fp16, 32 KB) and partial tiles (16 KB); down roles: h
  __shared__ __attribute__((aligned(16))) char buf[kHsBytes];
  __shared__ float red_dn[kWinWaves][16][kWinT];
  static_assert(kWinT * kMmaMaxH * 2 + kWinWaves * kMmaBatch * 2 * 16 * kWinT * 4 <= kHsBytes, "");
  _Float16* xs = reinterpret_cast<_Float16*>(buf);
  auto& red = *reinterpret_cast<float(*)[kWinWaves][kMmaBatch][2][16][kWinT]>(buf + kWinT * kMmaMaxH * 2);
  __shared__ uint32_t guard_s;
  __shared__ int bad_s;
  const int tid = threadIdx.x;
  const int H = ex.H;
  const int G = ex.I / 16 * kMmaSlices, D = H / 16;
  const int role = blockIdx.x;

  win_topk<kLayerPer>(R, logits, T, ex.E, k);
  // the window's activations -> LDS fp16 in the MFMA K order (tokens >= T
  // zero), by the waves that do not select experts
  for (int i = tid - 64 * kWinT; i >= 0 && i < kWinT * H / 4; i += kWinThreads - 64 * kWinT) {
    const int t = i / (H / 4), q = i % (H / 4);
    float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
    if (t < T) {
      if (XF32) {
        const float4 f = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * H)[q];
        v0 = f.x; v1 = f.y; v2 = f.z; v3 = f.w;
      } else {
        const uint2 u = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)t * H)[q];
        v0 = bf16_lo(u.x); v1 = bf16_hi(u.x); v2 = bf16_lo(u.y); v3 = bf16_hi(u.y);
      }
    }
    *reinterpret_cast<uint2*>(xs + t * H + 4 * q) = make_uint2(pack_half2(v0, v2), pack_half2(v1, v3));
  }
  if (tid == kWinThreads - 64) guard_s = sync_load(sync->guard);
  const int n_act = win_list(R, ex, T, k, false, nullptr, nullptr, nullptr);  // ends with a barrier

  if (guard_s != 0u) {  // the head was not zeroed: y becomes NaN
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
    gateup_role<Q, NBG>(R.wl, n_act, role, T, ex, xs, red, hwin);
    // The h stores are agent-coherent; a wave's store count reaching zero means
    // they are performed chip-wide, so once every wave has waited for that,
    // the role's count orders them before the down roles' reads (which are
    // agent-coherent too). No cache write-back is needed.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) sync_add(sync->up[role / kSyncGroup]);
    return;
  }
  auto wait = [&]() -> bool {
    if (tid == 0) bad_s = 0;
    __syncthreads();
    if (tid < G / kSyncGroup) {  // lanes of wave 0, one counter each
      const long long t0 = wall_clock64();
      while (sync_load(sync->up[tid]) != (uint32_t)kSyncGroup) {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > kWinSpinTicks) {
          bad_s = 1;
          break;
        }
      }
    }
    __syncthreads();
    return bad_s == 0;
  };
  const int grp = role - G;
  down_role<Q, NBD>(R.wl, n_act, grp, T, ex, hwin, y, out_f32, reinterpret_cast<_Float16*>(buf),
                    red_dn, wait);
  if (tid == 0 && bad_s == 0 && sync_add(sync->dn[grp / kSyncGroup]) == kSyncGroup - 1 &&
      sync_add(sync->dn_all) == (uint32_t)(D / kSyncGroup - 1)) {
    // every gate/up role has released h and every down role has passed its wait
    for (int g = 0; g < G / kSyncGroup; ++g) sync_zero(sync->up[g]);
    for (int g = 0; g < D / kSyncGroup; ++g) sync_zero(sync->dn[g]);
    sync_zero(sync->dn_all);
  }
}

inline bool win_mma_ok(const Experts& ex, int T, int k) {
  return ex.H % 1024 == 0 && ex.H <= kMmaMaxH && (ex.I == 256 || ex.I == 512) &&
         ex.E <= 64 * kLayerPer && T * k <= 64;
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

template <int Q, bool XF32>
hipError_t launch_layer(const float* logits, int T, int k, const Experts& ex, const void* x,
                        int32_t* idx, float* gates, uint16_t* hwin, void* y, int out_f32,
                        WinSync* sync, hipStream_t s) {
  const dim3 grid(ex.I / 16 * kMmaSlices + ex.H / 16);
#define L(NBG, NBD)                                                                               \
  MOE_LAUNCH("win_layer", s, (win_layer<Q, XF32, NBG, NBD>), grid, dim3(kWinThreads), 0, s, logits, \
             T, k, ex, x, idx, gates, hwin, y, out_f32, sync)
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

// Window workspace: counters (kWinSyncBytes, zero between calls) | active list |
// h [n_act][kWinT][I] (fp16 in the MFMA K order for the one-launch form, bf16
// otherwise).
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
    if (ex.qtype == 3)
      return xdtype == 0 ? launch_layer<3, true>(logits, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s)
                         : launch_layer<3, false>(logits, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s);
    return xdtype == 0 ? launch_layer<2, true>(logits, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s)
                       : launch_layer<2, false>(logits, T, k, ex, x, idx, gates, hwin, y, out_f32, sync, s);
  }
  const int bh = ex.H / 32, bi = ex.I / 32;
  if (ex.qtype == 3)
    return xdtype == 0 ? launch_wq<3, true>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s)
                       : launch_wq<3, false>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
  return xdtype == 0 ? launch_wq<2, true>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s)
                     : launch_wq<2, false>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
}

}  // namespace moe

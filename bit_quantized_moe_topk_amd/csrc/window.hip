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
constexpr int kWinGroups = 4;  // expert groups of the down kernel
template <int BPR>
constexpr int win_dn_rows() {  // rows of H per down workgroup: two row groups
  return 2 * (64 / BPR);
}
constexpr int kWinBatch = 4;   // experts whose weights a wave has in flight at once

template <int BPR, int Q, bool XF32>
__global__ __launch_bounds__(kWinThreads) void win_gateup(const float* __restrict__ logits, int T,
                                                          int k, Experts ex, const void* x,
                                                          int32_t* idx_out, float* gates_out,
                                                          WinList* gmeta, uint16_t* hwin) {
  __shared__ int lidx[kWinT * kWinMaxK];
  __shared__ float lgate[kWinT * kWinMaxK];
  __shared__ int flag[MOE_MAX_E_DEV + 1];
  __shared__ int tmask[MOE_MAX_E_DEV + 1];
  __shared__ int wsum[16];
  __shared__ WinList wl;
  __shared__ TopkScratch tks[kWinT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = ex.E, E_tot = ex.E_tot;
  const int b = lane % BPR, rg = lane / BPR;

  // routing: wave t selects token t's experts (before the activation loads:
  // loads complete in order, so the logits must not queue behind them)
  if (wave < T)
    topk_any(logits + (size_t)wave * E, E, k, lidx + wave * k, lgate + wave * k, &tks[wave]);
  XB xb[kWinT];
#pragma unroll
  for (int t = 0; t < kWinT; ++t) {
    if (t < T) load_x_row<Q, XF32>(x, ex.H, t, b, xb[t]);
    else zero_xb(xb[t]);
  }
  for (int e = tid; e < E_tot; e += kWinThreads) tmask[e] = 0;
  __syncthreads();
  for (int a = tid; a < T * k; a += kWinThreads) atomicOr(&tmask[lidx[a]], 1 << (a / k));
  if (ex.has_shared && tid == 0) tmask[E] = (1 << T) - 1;
  __syncthreads();
  for (int e = tid; e < E_tot; e += kWinThreads) flag[e] = tmask[e] != 0;
  __syncthreads();
  const int n_act = block_exclusive_scan(flag, E_tot, wsum);
  for (int e = tid; e < E_tot; e += kWinThreads) {
    if (tmask[e]) {
      const int p = flag[e];
      wl.act_e[p] = e;
      wl.act_mask[p] = tmask[e];
#pragma unroll
      for (int t = 0; t < kWinT; ++t) wl.act_gate[p][t] = 0.f;
    }
  }
  if (tid == 0) wl.n_act = n_act;
  __syncthreads();
  for (int a = tid; a < T * k; a += kWinThreads) wl.act_gate[flag[lidx[a]]][a / k] = lgate[a];
  if (ex.has_shared && tid < T) wl.act_gate[flag[E]][tid] = 1.0f;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int a = tid; a < T * k; a += kWinThreads) {
      idx_out[a] = lidx[a];
      gates_out[a] = lgate[a];
    }
    if (tid == 0) gmeta->n_act = n_act;
    for (int p = tid; p < n_act; p += kWinThreads) {
      gmeta->act_e[p] = wl.act_e[p];
      gmeta->act_mask[p] = wl.act_mask[p];
#pragma unroll
      for (int t = 0; t < kWinT; ++t) gmeta->act_gate[p][t] = wl.act_gate[p][t];
    }
  }

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

// Window workspace: active list | h [n_act][kWinT][I] bf16.
namespace {
struct WinLayout {
  size_t meta, h, total;
};
WinLayout win_layout(const Experts& ex, int T, int k) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  WinLayout L{};
  size_t off = 0;
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
  const int bh = ex.H / 32, bi = ex.I / 32;
  if (ex.qtype == 3)
    return xdtype == 0 ? launch_wq<3, true>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s)
                       : launch_wq<3, false>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
  return xdtype == 0 ? launch_wq<2, true>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s)
                     : launch_wq<2, false>(bh, bi, logits, T, k, ex, x, idx, gates, meta, hwin, y, out_f32, s);
}

}  // namespace moe

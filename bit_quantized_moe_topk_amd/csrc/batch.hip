// Expert FFN for small batches (up to a few hundred tokens, e.g. 16 decode
// streams of a 4-token verify window) on gfx950 matrix cores.
//
// Each expert holds at most T of the batch's assignments, so the layer is
// bound by reading the touched experts' packed weights once ("Strata - the
// details", "Other GPUs": speed follows memory bandwidth). The work is cut
// into many items of equal cost, one per (touched expert, chunk of output
// rows, group of 16 of the expert's tokens), so that every CU streams weights
// and no expert with many tokens leaves a long tail:
//
//   bat_gateup: chunk = 2 groups of 16 rows of I, for gate and up. The 8
//               waves split K (wave w takes blocks w H/256 ...; lane group
//               c = lane / 16 takes NBL consecutive blocks of its row). The
//               lane's 16 tokens stay in registers as the fp16 operand of
//               v_mfma_f32_16x16x32_f16 while the row groups' weights
//               stream through two register sets, dequantised in registers
//               (deq16.h); the next item's first weights are requested while
//               the last row groups compute (Q3 operands: deq16.h, "Q3
//               through the FP8 conversion"). Each row group's eight partial
//               tiles are summed in LDS in wave order, then SwiGLU (each
//               token's activation copy is scaled by 2^-e, xe, which the
//               epilogue undoes); h is stored as bf16 in the MFMA K order.
//   bat_down  : chunk = 128 rows of H (wave w: one group of 16 rows over all
//               of K = I), on bf16 operands (weights dequantised to bf16,
//               bf16 h). The item's 16 h rows come into LDS (double-buffered
//               across items, the next item's rows requested early); outputs
//               are scaled by the routing gate and stored per assignment slot
//               for the combine.
//
// Both grids are persistent (gate/up: two workgroups per CU, down: three):
// every workgroup builds a map of the grouping in LDS (token groups per
// expert, slot offsets, and the token id or gate of every slot) and takes a
// run of consecutive items in (expert, token group, chunk) order, so a token
// group's activations (h rows for down) are loaded once per run; the items of
// one expert, which read the same weights, go to workgroups of one XCD. Waves
// raise their issue priority by the workgroup's progress, so the workgroups
// sharing a CU move together instead of the youngest finishing alone.
#include "common.h"
#include "deq16.h"
#include "gemv.h"
#include "sched.h"
#include "batch_x.h"

namespace moe {
namespace {

constexpr int kBThreads = 512;
constexpr int kBWaves = kBThreads / 64;
constexpr int kGuRows = 2;     // 16-row groups of I per gate/up item (2 or 4)
constexpr int kDnRows = 1;     // 16-row groups of H per wave in a down item (1 or 2)
constexpr int kBMaxI = 512;
constexpr int kBTab = 4096;    // slots whose token id fits the gate/up LDS table
constexpr int kBTabDn = 2048;  // slots whose gate fits the down LDS table

// Grouping map of one launch in LDS. Its two per-expert arrays live in the
// launch's dynamic LDS (bat_map_bytes), so a layer with few experts leaves
// room for more workgroups per CU:
//   base[E_tot + 1]: exclusive prefix over experts of ceil(M / 16), then the total;
//   off[E_tot + 1] : slot offsets (offsets[0..E_tot]).
struct BatMap {
  int wsum[16];
  int n;  // token groups in all
};
inline size_t bat_map_bytes(int E_tot) { return 2 * sizeof(int) * (size_t)(E_tot + 2); }

// One item: expert e, output-row chunk, token group tg (tokens 16 tg ..).
struct BatItem {
  int e, chunk, tg, M, slot0;
};

// Fills the map, and with kTab calls fill(s, perm[s]) for every slot when the
// table is used (A <= kBTab); all kBThreads threads of the block call it.
// Every global load is issued (at a clamped, in-bounds index) before the
// first one is used: the map costs one memory round trip.
template <bool kTab, typename Fill>
__device__ inline void batmap_init(BatMap& bm, int* base, int* off, const FfnArgs& a, int E_tot,
                                   bool use_tab, int A, Fill&& fill) {
  constexpr int kEPer = (MOE_MAX_E_DEV + 2 + kBThreads - 1) / kBThreads;
  constexpr int kSPer = kBTab / kBThreads;
  const int tid = threadIdx.x;
  int ov[kEPer], cv[kEPer], pv[kSPer];
#pragma unroll
  for (int u = 0; u < kEPer; ++u) {
    const int e = tid + kBThreads * u;
    ov[u] = a.offsets[min(e, E_tot)];
    cv[u] = a.counts[min(e, E_tot - 1)];
  }
#pragma unroll
  for (int u = 0; u < kSPer; ++u) pv[u] = kTab ? a.perm[min(tid + kBThreads * u, A - 1)] : 0;
#pragma unroll
  for (int u = 0; u < kEPer; ++u) {
    const int e = tid + kBThreads * u;
    if (e <= E_tot) off[e] = ov[u];
    if (e < E_tot) base[e] = (cv[u] + 15) >> 4;
  }
  if (kTab && use_tab) {
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      const int sl = tid + kBThreads * u;
      if (sl < A) fill(sl, pv[u]);
    }
  }
  __syncthreads();
  const int n = block_exclusive_scan(base, E_tot, bm.wsum);
  if (threadIdx.x == 0) {
    base[E_tot] = n;
    bm.n = n;
  }
  __syncthreads();
}

// Items in (expert, token group, chunk) order: the chunks of one token group
// follow each other, so a workgroup that takes a run of them keeps the
// group's activations (gate/up: registers; down: h rows in LDS).
__device__ inline BatItem bat_item_seq(const int* base, const int* off, int E_tot, int NC, int item) {
  const int gi = item / NC;
  const int e = workmap_find(base, E_tot, gi);
  BatItem it;
  it.e = __builtin_amdgcn_readfirstlane(e);
  it.chunk = __builtin_amdgcn_readfirstlane(item - NC * gi);
  it.tg = __builtin_amdgcn_readfirstlane(gi - base[e]);
  it.slot0 = __builtin_amdgcn_readfirstlane(off[e]);
  it.M = __builtin_amdgcn_readfirstlane(off[e + 1] - off[e]);
  return it;
}

// Column of this workgroup (its run of items is bat_run's). Neighbouring
// columns go to workgroups of one XCD (workgroup g runs
// on XCD g % 8) when the grid is a multiple of 8, so the token groups of one
// expert, which read the same weights, meet in that XCD's L2.
__device__ inline int bat_first() {
  const int g = blockIdx.x, G = gridDim.x;
  return (G % 8) ? g : (g % 8) * (G / 8) + g / 8;
}

// The run of this workgroup's column: items [c n / G, (c + 1) n / G), so the
// runs differ by at most one item and every column has work when n >= G
// (runs of ceil(n / G) would leave the last columns, i.e. whole XCDs, idle).
__device__ inline void bat_run(int n_items, int& first, int& end) {
  const long long c = bat_first(), G = gridDim.x;
  first = (int)(c * n_items / G);
  end = (int)((c + 1) * n_items / G);
}

// --- gate/up ----------------------------------------------------------------

// Waves issue by priority, then age: the workgroup that has finished fewer
// items goes first, so the workgroups on a CU progress together instead of
// the youngest one running alone at the end.
__device__ inline void set_prio_by_progress(int done) {
  if (done == 0) __builtin_amdgcn_s_setprio(3);
  else if (done == 1) __builtin_amdgcn_s_setprio(2);
  else if (done == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

__global__ __launch_bounds__(256) void bat_xs(XsJob xj) {
  xs_write_rows(xj, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
}

// The lane's token operand for token t (a padding column of the tile takes
// some valid token's row: the matrix product keeps columns apart and padding
// columns are never stored).
template <int NBL>
__device__ inline void load_xop(const uint16_t* xs, int H, int t, int wave, int c, half8_t (&xf)[NBL][4]) {
  const uint4* row = reinterpret_cast<const uint4*>(xs) + (uint32_t)(t * (H / 8) + wave * (H / 64) + c);
#pragma unroll
  for (int b = 0; b < NBL; ++b)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xf[b][kk] = __builtin_bit_cast(half8_t, row[4 * (4 * b + kk)]);
}

// One row group: the wave's partial gate and up tiles into red (gate, then
// up: one row's operand planes live at a time).
template <int Q, int NBL>
__device__ inline void gu_partial(const WRow<NBL>& wg, const WRow<NBL>& wu, const half8_t (&xf)[NBL][4],
                                  float (&red)[kBWaves][2][16][17]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane >> 4, r16 = lane & 15;
  floatx4_t ag = {}, au = {};
#pragma unroll
  for (int b = 0; b < NBL; ++b) {
    if constexpr (Q == 3) {
      // one code word (16 weights) of one row at a time
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const WByteWord sg = wbyte_word(wg.c[2 * b + w], wg.hi[b], wg.dm[b], w);
        ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag_byte(sg, 0), xf[b][2 * w], ag, 0, 0, 0);
        ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag_byte(sg, 1), xf[b][2 * w + 1], ag, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const WByteWord su = wbyte_word(wu.c[2 * b + w], wu.hi[b], wu.dm[b], w);
        au = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag_byte(su, 0), xf[b][2 * w], au, 0, 0, 0);
        au = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag_byte(su, 1), xf[b][2 * w + 1], au, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const WStage sg = wstage_block<Q>(wg.c[2 * b], wg.c[2 * b + 1], wg.hi[b], wg.dm[b]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag<Q>(sg, kk), xf[b][kk], ag, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const WStage su = wstage_block<Q>(wu.c[2 * b], wu.c[2 * b + 1], wu.hi[b], wu.dm[b]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        au = __builtin_amdgcn_mfma_f32_16x16x32_f16(wfrag<Q>(su, kk), xf[b][kk], au, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // ag[v]: row 4 c + v of the group, token r16
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    red[wave][0][4 * c + v][r16] = ag[v];
    red[wave][1][4 * c + v][r16] = au[v];
  }
  // the caller reloads this row group's registers next: keep those loads
  // after the arithmetic that still reads them
  __builtin_amdgcn_sched_barrier(0);
}

// Sum of the eight partial tiles (wave order), SwiGLU, h store in the down
// operand's K order, one 32-bit store per pair of positions (2 p, 2 p + 1) and
// token. Q2: positions 4 q + 2 s, + 1 hold rows 4 q + s, 4 q + s + 2; Q3 (16
// rows, one code word of down): positions 2 p, 2 p + 1 hold rows r, r + 4 with
// r = p / 2 + 8 (p & 1). Taken by the 128 threads of waves 2 j, 2 j + 1 (j =
// row group mod 4), so the extra work rotates over the waves.
template <int Q>
__device__ inline void gu_finish(const float (&red)[kBWaves][2][16][17], int j, const BatItem& it,
                                 int row0, int I, uint16_t* h, const int* tok, bool use_tab,
                                 const FfnArgs& a, const int* xe_s) {
  const int rt = (int)threadIdx.x - 128 * (j & 3);
  if (rt < 0 || rt >= 128) return;
  const int pr = rt >> 4, t = rt & 15;
  const int m = 16 * it.tg + t;
  if (m >= it.M) return;
  int tk;  // the slot's token: its activation row's exponent restores g and u
  if (use_tab) {
    tk = tok[it.slot0 + m];
  } else {
    tk = token_of(a.perm[it.slot0 + m], a.T, a.k);
    tk = (unsigned)tk < (unsigned)a.T ? tk : 0;
  }
  const int e = xe_s[tk];
  const int ra = Q == 3 ? (pr >> 1) + 8 * (pr & 1) : 4 * (pr >> 1) + (pr & 1);
  const int rb = ra + (Q == 3 ? 4 : 2);
  float ga = 0.f, ua = 0.f, gb = 0.f, ub = 0.f;
#pragma unroll
  for (int w = 0; w < kBWaves; ++w) {
    ga += red[w][0][ra][t];
    ua += red[w][1][ra][t];
    gb += red[w][0][rb][t];
    ub += red[w][1][rb][t];
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(h + (size_t)(it.slot0 + m) * I + row0 + 2 * pr);
  *dst = pack_bf16x2(silu_mul_x(ga, ua, e), silu_mul_x(gb, ub, e));
}

template <int Q, int NBL>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(4)))
void bat_gateup(Experts ex, FfnArgs a) {
  constexpr int R = kGuRows;
  static_assert(R == 2 || R == 4, "the row-group pipeline takes 2 or 4 groups per item");
  __shared__ BatMap bm;
  extern __shared__ int bat_dyn[];  // base, off (bat_map_bytes)
  __shared__ int tok[kBTab];
  __shared__ int xe_s[kGemvBatchLimit];  // per-token exponents of the activation copy
  __shared__ float red[2][kBWaves][2][16][17];  // two buffers: wave, gate/up, row, token
  const int H = ex.H, I = ex.I, E_tot = ex.E_tot;
  const int A = a.T * (a.k + ex.has_shared);
  const bool use_tab = A <= kBTab;
  int* base = bat_dyn;
  int* off = bat_dyn + E_tot + 2;
  const int xev = (int)threadIdx.x < a.T ? a.xe[threadIdx.x] : 0;  // T < kBThreads
  batmap_init<true>(bm, base, off, a, E_tot, use_tab, A, [&](int s, int asg) {
    const int t = token_of(asg, a.T, a.k);
    tok[s] = (unsigned)t < (unsigned)a.T ? t : 0;
  });
  if ((int)threadIdx.x < a.T) xe_s[threadIdx.x] = xev;  // published by the loop's first barrier
  const int NC = I / (16 * R);
  const int n_items = __builtin_amdgcn_readfirstlane(bm.n * NC);  // uniform: scalar branches
  // a run of consecutive items per workgroup
  int item, item_end;
  bat_run(n_items, item, item_end);
  if (item >= item_end) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kb0 = wave * (H / 256) + NBL * (lane >> 4);  // the lane's first block of its rows
  uint16_t* h = static_cast<uint16_t*>(a.h);
  const uint32_t lane_blk = (uint32_t)(r16 * (H / 32) + kb0);  // block of the lane's row and K slice
  auto wrow = [&](const BatItem& it, int j, size_t mat0) {
    return load_wrow_at<Q, NBL>(ex, mat0 + (size_t)(16 * (R * it.chunk + j)) * (H / 32), lane_blk);
  };

  // the token operand of the item's token group
  auto load_x = [&](const BatItem& it, half8_t (&xf)[NBL][4]) {
    const int m = min(16 * it.tg + r16, it.M - 1), slot = it.slot0 + m;  // padding: the last token
    int t;
    if (use_tab) {
      t = tok[slot];
    } else {
      t = token_of(a.perm[slot], a.T, a.k);
      t = (unsigned)t < (unsigned)a.T ? t : 0;
    }
    load_xop<NBL>(a.x16, H, t, wave, lane >> 4, xf);
  };

  // first item: activations requested first, so its first row group can start
  // while the second one's weights are still in flight
  BatItem it = bat_item_seq(base, off, E_tot, NC, item);
  half8_t xf[NBL][4];
  load_x(it, xf);
  WRow<NBL> ga = wrow(it, 0, blk_gate(ex, it.e)), ua = wrow(it, 0, blk_up(ex, it.e));
  WRow<NBL> gb = wrow(it, 1, blk_gate(ex, it.e)), ub = wrow(it, 1, blk_up(ex, it.e));
  bool new_group = false;
  int done = 0;
  for (;;) {
    set_prio_by_progress(done++);
    if (new_group) load_x(it, xf);
    const int next = item + 1;
    const bool more = next < item_end;
    BatItem nx = it;
    if (more) nx = bat_item_seq(base, off, E_tot, NC, next);
    const int row0 = 16 * R * it.chunk;
    if constexpr (R == 4) {
      // row group 0 (set a), then its weights make way for row group 2
      gu_partial<Q, NBL>(ga, ua, xf, red[0]);
      ga = wrow(it, 2, blk_gate(ex, it.e));
      ua = wrow(it, 2, blk_up(ex, it.e));
      __syncthreads();
      gu_finish<Q>(red[0], 0, it, row0, I, h, tok, use_tab, a, xe_s);
      // row group 1 (set b) -> row group 3
      gu_partial<Q, NBL>(gb, ub, xf, red[1]);
      gb = wrow(it, 3, blk_gate(ex, it.e));
      ub = wrow(it, 3, blk_up(ex, it.e));
      __syncthreads();
      gu_finish<Q>(red[1], 1, it, row0 + 16, I, h, tok, use_tab, a, xe_s);
    }
    // row group R - 2 (set a) -> the next item's row group 0
    gu_partial<Q, NBL>(ga, ua, xf, red[0]);
    if (more) {
      ga = wrow(nx, 0, blk_gate(ex, nx.e));
      ua = wrow(nx, 0, blk_up(ex, nx.e));
    }
    __syncthreads();
    gu_finish<Q>(red[0], R - 2, it, row0 + 16 * (R - 2), I, h, tok, use_tab, a, xe_s);
    // row group R - 1 (set b) -> the next item's row group 1
    gu_partial<Q, NBL>(gb, ub, xf, red[1]);
    if (more) {
      gb = wrow(nx, 1, blk_gate(ex, nx.e));
      ub = wrow(nx, 1, blk_up(ex, nx.e));
    }
    __syncthreads();
    gu_finish<Q>(red[1], R - 1, it, row0 + 16 * (R - 1), I, h, tok, use_tab, a, xe_s);
    if (!more) break;
    new_group = nx.e != it.e || nx.tg != it.tg;
    item = next;
    it = nx;
  }
}

// --- down -------------------------------------------------------------------

// One 16-row x 16-token down tile over all of K on bf16 operands (h is
// bf16); two accumulators (step parity) keep consecutive MFMAs independent.
template <int Q, int NBL>
__device__ inline floatx4_t dn_tile(const WRow<NBL>& wd, const uint16_t* hrow, int kb0) {
  floatx4_t acc0 = {}, acc1 = {};
#pragma unroll
  for (int b = 0; b < NBL; ++b) {
    bf16x8_t xf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xf[kk] = *reinterpret_cast<const bf16x8_t*>(hrow + 32 * (kb0 + b) + 8 * kk);
    if constexpr (Q == 3) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const WByteWord sd = wbyte_word(wd.c[2 * b + w], wd.hi[b], wd.dm[b], w);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag_byte_bf(sd, 0), xf[2 * w], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag_byte_bf(sd, 1), xf[2 * w + 1], acc1, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      const WStage sd = wstage_block<Q>(wd.c[2 * b], wd.c[2 * b + 1], wd.hi[b], wd.dm[b]);
#pragma unroll
      for (int kk = 0; kk < 4; kk += 2) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag_bf<Q>(sd, kk), xf[kk], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag_bf<Q>(sd, kk + 1), xf[kk + 1], acc1, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  return acc0 + acc1;
}

__device__ inline void dn_store(const FfnArgs& a, int H, int slot, int row, float g, floatx4_t v) {
  const size_t o = (size_t)slot * H + row;
  if (a.o) {
    *reinterpret_cast<float4*>(a.o + o) = make_float4(g * v[0], g * v[1], g * v[2], g * v[3]);
  } else {
    *reinterpret_cast<uint2*>(a.ob + o) =
        make_uint2(f32_to_bf16_bits(g * v[0]) | (f32_to_bf16_bits(g * v[1]) << 16),
                   f32_to_bf16_bits(g * v[2]) | (f32_to_bf16_bits(g * v[3]) << 16));
  }
}

// NBL = I / 128 (lane groups c cover all of K). Each thread carries HC
// 16-byte chunks of the item's 16 h rows.
template <int Q, int NBL>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(6)))
void bat_down(Experts ex, FfnArgs a) {
  static_assert(kDnRows == 1 || kDnRows == 2, "one or two row groups per wave");
  constexpr int kRow = kBMaxI + 8;  // LDS row of h (halves), padded against bank conflicts
  constexpr int I_ = 128 * NBL;
  constexpr int HC = 16 * (I_ / 8) / kBThreads;  // h chunks per thread (I / 256)
  static_assert(HC >= 1, "I >= 256");
  __shared__ BatMap bm;
  extern __shared__ int bat_dyn[];  // base, off (bat_map_bytes)
  __shared__ float gtab[kBTabDn];
  __shared__ __attribute__((aligned(16))) uint16_t hs[2][16 * kRow];
  const int H = ex.H, E_tot = ex.E_tot;
  const int A = a.T * (a.k + ex.has_shared);
  const bool use_tab = A <= kBTabDn;
  int* base = bat_dyn;
  int* off = bat_dyn + E_tot + 2;
  // the gate table is filled after the first item's loads are in flight (below)
  batmap_init<false>(bm, base, off, a, E_tot, false, A, [](int, int) {});
  const int NC = H / (16 * kDnRows * kBWaves);
  const int n_items = __builtin_amdgcn_readfirstlane(bm.n * NC);  // uniform: scalar branches
  // runs of consecutive items in (expert, token group, chunk) order, as in
  // the gate/up kernel: a token group's h rows stay in LDS for its run
  int item, item_end;
  bat_run(n_items, item, item_end);
  if (item >= item_end) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, r16 = lane & 15;
  const int kb0 = NBL * c;
  const uint4* h4 = static_cast<const uint4*>(a.h);
  // the lane's row inside the item's chunk, and its first block
  const uint32_t lane_blk = (uint32_t)((16 * kDnRows * wave + r16) * (I_ / 32) + kb0);
  auto wrow = [&](const BatItem& it, int j) {
    const size_t ubase = blk_down(ex, it.e) + (size_t)(16 * kDnRows * kBWaves * it.chunk + 16 * j) * (I_ / 32);
    return load_wrow_at<Q, NBL>(ex, ubase, lane_blk);
  };
  // h chunk q = tid + 512 u of the item: token row q / (I / 8), chunk q % (I / 8)
  auto hload = [&](const BatItem& it, uint4 (&hv)[HC]) {
#pragma unroll
    for (int u = 0; u < HC; ++u) {
      const int q = tid + kBThreads * u, r = q / (I_ / 8), col = q % (I_ / 8);
      const int m = 16 * it.tg + r;
      hv[u] = m < it.M ? h4[(size_t)(it.slot0 + m) * (I_ / 8) + col] : make_uint4(0, 0, 0, 0);
    }
  };

  BatItem it = bat_item_seq(base, off, E_tot, NC, item);
  WRow<NBL> w0 = wrow(it, 0), w1;
  if constexpr (kDnRows == 2) w1 = wrow(it, 1);
  uint4 hv[HC];
  hload(it, hv);
  // routing gate of every slot (perm, then gates: two dependent loads), read
  // while the first item's loads are in flight; the loop's first barrier
  // publishes it
  if (use_tab)
    for (int s = tid; s < A; s += kBThreads) gtab[s] = gate_of(a, s);
  int buf = 0, done = 0;
  bool new_group = true;
  for (;;) {
    set_prio_by_progress(done++);
    if (new_group) {
#pragma unroll
      for (int u = 0; u < HC; ++u) {
        const int q = tid + kBThreads * u, r = q / (I_ / 8), col = q % (I_ / 8);
        *reinterpret_cast<uint4*>(&hs[buf][r * kRow + 8 * col]) = hv[u];
      }
      __syncthreads();  // hs[buf] complete; hs[buf ^ 1] no longer read
    }
    const int next = item + 1;
    const bool more = next < item_end;
    BatItem nx = it;
    if (more) nx = bat_item_seq(base, off, E_tot, NC, next);
    const bool next_group = more && (nx.e != it.e || nx.tg != it.tg);
    if (next_group) hload(nx, hv);
    const int m = 16 * it.tg + r16, slot = it.slot0 + m;
    const bool live = m < it.M;
    const float g = live ? (use_tab ? gtab[slot] : gate_of(a, slot)) : 0.f;
    const uint16_t* hrow = &hs[buf][r16 * kRow];
    const int row0 = 16 * kDnRows * (kBWaves * it.chunk + wave) + 4 * c;
    const floatx4_t o0 = dn_tile<Q, NBL>(w0, hrow, kb0);
    if (more) w0 = wrow(nx, 0);
    if constexpr (kDnRows == 2) {
      const floatx4_t o1 = dn_tile<Q, NBL>(w1, hrow, kb0);
      if (more) w1 = wrow(nx, 1);
      if (live) dn_store(a, H, slot, row0 + 16, g, o1);
    }
    if (live) dn_store(a, H, slot, row0, g, o0);
    if (!more) break;
    if (next_group) buf ^= 1;
    new_group = next_group;
    item = next;
    it = nx;
  }
}


template <int Q>
hipError_t launch_bat_q(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const long A = (long)a.T * (a.k + ex.has_shared);
  // token groups: sum over touched experts of ceil(M / 16) <= A / 16 + touched, and <= A
  const long touched = A < ex.E_tot ? A : ex.E_tot;
  const long groups = A / 16 + touched < A ? A / 16 + touched : A;
  // resident workgroups per CU: gate/up 2 (registers), down 3 (LDS, with the
  // map of a layer of up to ~1,000 experts)
  const long cap_gu = 2L * device_cus(), cap_dn = 3L * device_cus();
  const long gu_items = groups * (ex.I / (16 * kGuRows));
  const long dn_items = groups * (ex.H / (16 * kDnRows * kBWaves));
  const dim3 ggu((unsigned)(gu_items < cap_gu ? gu_items : cap_gu));
  const dim3 gdn((unsigned)(dn_items < cap_dn ? dn_items : cap_dn));
  const size_t map = bat_map_bytes(ex.E_tot);
  if (!a.xs_ready) {
    const int xg = (a.T + 3) / 4 < 1024 ? (a.T + 3) / 4 : 1024;  // a wave per token row
    MOE_LAUNCH("bat_xs", s, bat_xs, dim3(xg), dim3(256), 0, s,
               xs_job(ex.qtype, ex.H, a.x, a.xdtype, a.T, a.x16, a.xe));
  }
  switch (ex.H / 1024) {
    case 1: MOE_LAUNCH("bat_gateup", s, (bat_gateup<Q, 1>), ggu, dim3(kBThreads), map, s, ex, a); break;
    case 2: MOE_LAUNCH("bat_gateup", s, (bat_gateup<Q, 2>), ggu, dim3(kBThreads), map, s, ex, a); break;
    default: return hipErrorInvalidValue;
  }
  switch (ex.I / 128) {
    case 2: MOE_LAUNCH("bat_down", s, (bat_down<Q, 2>), gdn, dim3(kBThreads), map, s, ex, a); break;
    case 4: MOE_LAUNCH("bat_down", s, (bat_down<Q, 4>), gdn, dim3(kBThreads), map, s, ex, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

bool batch_supported(int H, int I) {
  return (H == 1024 || H == 2048) && (I == 256 || I == 512) && H % (16 * kDnRows * kBWaves) == 0 &&
         I % (16 * kGuRows) == 0 && I <= kBMaxI;
}

XsJob xs_job(int q, int H, const void* x, int xdtype, int T, uint16_t* x16, int32_t* xe) {
  return XsJob{x, xdtype != 0, q, H, T, q < 0 ? nullptr : reinterpret_cast<uint4*>(x16), xe};
}

hipError_t launch_batch(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  return ex.qtype == 3 ? launch_bat_q<3>(ex, a, s) : launch_bat_q<2>(ex, a, s);
}

}  // namespace moe

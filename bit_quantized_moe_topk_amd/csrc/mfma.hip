// Prefill tiles of the expert FFN on gfx950 matrix cores.
//
// An expert with many assignments multiplies a gathered block of its tokens'
// activations by its dequantised weights: gate and up share one activation
// tile and SwiGLU runs in the epilogue; the down projection folds the routing
// gate into its epilogue. The pages' prompt path likewise multiplies quantised
// experts in large chunks without first expanding them to FP16 in memory
// ("Strata - the details", "Faster prompts"). Here weights are expanded only
// in registers, right before v_mfma_f32_32x32x16_f16 (gate/up: fp16 weights
// and activations, each token row scaled by a power of two into fp16 range)
// or v_mfma_f32_32x32x16_bf16 (down: bf16 weights and h) consumes them.
//
// Workgroup tile: kBM = 128 assignments x NW * 64 weight rows, K in stages of
// 64 (two quantisation blocks), NW = 8 waves (4 for narrow matrices), two
// per SIMD. Each wave owns 64 weight rows for all 128 assignments: it loads
// its own weight blocks and dequantises them straight into MFMA operand
// registers (w = d*q + m, one fp16 or bf16 rounding), so weights never touch LDS. The
// activation tile is gathered through the grouping permutation by all waves
// into double-buffered LDS and read by every wave.
// K order: stage s of S = K/64 holds blocks s (lane half 0) and S + s (lane
// half 1); within a 16-wide MFMA step kk, lane half h covers weights
// 8 kk .. 8 kk + 7 of its block. So each lane dequantises one whole block per
// weight row per stage, and its blocks for stages s, s + 1 are adjacent in
// memory (one 16-byte code load per two stages).
//
// The grid is persistent. Work items are (expert tile, N tile) with the N
// tiles of one expert tile adjacent; consecutive items go to workgroups of one
// XCD, so the activation rows they share stay in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "deq16.h"
#include "gemv.h"
#include "sched.h"
#include "batch_x.h"

namespace moe {
namespace {

constexpr int kBM = 128;          // assignments per tile
constexpr int kBK = 64;           // K per stage
// Activation stage in LDS: kBM rows of 64 halves (128 B), the eight 16-byte
// chunks of row m stored at chunk position q ^ ((m >> 1) & 7). A fragment
// read takes one logical chunk of 32 consecutive rows; 16 lanes at a time
// are served from the 64 banks (256 bytes, two rows' worth), and with this
// placement the 16 rows of such a group (8 even, 8 odd, each set on its own
// half of the banks) hit every bank once. No padding rows, so a wave's
// direct global-to-LDS load still fills 8 whole rows.
constexpr int kRow = 64;
// Epilogue staging per wave (16-bit outputs): down, 64 assignments x 64 rows
// (stride 72); gate/up, 128 assignments x 32 rows (stride 40).
constexpr int kStage = 128 * 40;

// Direct global-to-LDS load of 16 bytes per lane: lane l's bytes land at
// lds_wave + 16 l (lds_wave must be the same for the whole wave).
__device__ inline void lds_load16(const uint4* src, uint4* lds_wave) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave, 16, 0, 0);
}

// Two consecutive quantisation blocks of one weight row (the blocks a lane
// needs for two consecutive stages): codes, third bits (Q3), d and m.
struct WPair {
  uint4 c;   // block 0: c.x, c.y; block 1: c.z, c.w
  uint2 hi;  // Q3 third bits of blocks 0, 1
  uint2 dm;  // fp16 d | m << 16 of blocks 0, 1
};

template <int Q>
__device__ inline WPair load_wpair(const Experts& ex, size_t blk) {
  WPair w;
  w.c = *reinterpret_cast<const uint4*>(ex.codes + blk * 8);
  w.dm = *reinterpret_cast<const uint2*>(ex.dm + blk * 2);
  w.hi = Q == 3 ? *reinterpret_cast<const uint2*>(ex.hi + blk * 4) : make_uint2(0, 0);
  return w;
}

template <int Q>
__device__ inline WStage wstage(const WPair& w, int b) {
  return wstage_block<Q>(b ? w.c.z : w.c.x, b ? w.c.w : w.c.y, b ? w.hi.y : w.hi.x,
                         b ? w.dm.y : w.dm.x);
}

// One stage of an MFMA wave over NI 32-row activation groups: activation
// fragments are read one MFMA step ahead and each step's weight operands are
// dequantised while the previous step's MFMAs run. BF: bf16 operands (the
// down projection, whose activation operand h is bf16), else fp16.
template <int Q, bool BF>
__device__ inline auto wop(const WStage& w, int kk) {
  if constexpr (BF) return wfrag_bf<Q>(w, kk);
  else return wfrag<Q>(w, kk);
}

template <int NI, int Q, bool BF>
__device__ inline void stage_mma(const _Float16* xb, const WStage (&w)[2],
                                 float16_t (&acc)[4][2]) {
  typedef typename std::conditional<BF, bf16x8_t, half8_t>::type op_t;
  const int lane = threadIdx.x & 63;
  // row 32 i + lane % 32, logical chunk 4 h + kk (h = lane / 32), swizzled
  const _Float16* ap = xb + (lane & 31) * kRow;
  const int hq = 4 * (lane >> 5), sw = (lane >> 1) & 7;  // ((row >> 1) & 7) of row lane % 32
  auto afrag = [](const _Float16* p) { return *reinterpret_cast<const op_t*>(p); };
  op_t af[2][NI], bf[2][2];
#pragma unroll
  for (int i = 0; i < NI; ++i) af[0][i] = afrag(ap + 32 * i * kRow + 8 * (hq ^ sw));
#pragma unroll
  for (int j = 0; j < 2; ++j) bf[0][j] = wop<Q, BF>(w[j], 0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = kk & 1, n = c ^ 1;
    if (kk < 3) {
#pragma unroll
      for (int i = 0; i < NI; ++i) af[n][i] = afrag(ap + 32 * i * kRow + 8 * ((hq + kk + 1) ^ sw));
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[n][j] = wop<Q, BF>(w[j], kk + 1);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (BF)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[c][j], af[c][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[c][j], af[c][i], acc[i][j], 0, 0, 0);
      }
  }
}

// Tile map of one launch, built in LDS by every workgroup. Tiles are ordered
// by cost class — tiles that fill all four 32-row groups first, then tiles of
// two groups, then of one (Q2; Q3 runs every tile in full) — and within a
// class by expert, M block and output tile.
struct TileMap {
  int b4[MOE_MAX_E_DEV + 2];  // exclusive prefix of each expert's four-group tiles
  int b2[MOE_MAX_E_DEV + 2];  // of its two-group tile (0 or 1)
  int b1[MOE_MAX_E_DEV + 2];  // of its one-group tile (0 or 1)
  int wsum[16];
  int n4, n2, n1;
};

// CLASSES = false keeps one class: every tile in expert order.
template <int Q, bool CLASSES>
__device__ inline void tilemap_init(TileMap& tm, const int32_t* __restrict__ counts, int E_tot,
                                    int gmax) {
  for (int e = threadIdx.x; e < E_tot; e += blockDim.x) {
    const int M = counts[e];
    int c4 = 0, c2 = 0, c1 = 0;
    if (M > gmax) {
      const int r = M % kBM;
      c4 = M / kBM;
      if (CLASSES && Q == 2 && r > 0 && r <= 32) c1 = 1;
      else if (CLASSES && Q == 2 && r > 32 && r <= 64) c2 = 1;
      else if (r > 0) c4 += 1;
    }
    tm.b4[e] = c4;
    tm.b2[e] = c2;
    tm.b1[e] = c1;
  }
  __syncthreads();
  const int n4 = block_exclusive_scan(tm.b4, E_tot, tm.wsum);
  const int n2 = block_exclusive_scan(tm.b2, E_tot, tm.wsum);
  const int n1 = block_exclusive_scan(tm.b1, E_tot, tm.wsum);
  if (threadIdx.x == 0) {
    tm.b4[E_tot] = n4;
    tm.b2[E_tot] = n2;
    tm.b1[E_tot] = n1;
    tm.n4 = n4;
    tm.n2 = n2;
    tm.n1 = n1;
  }
  __syncthreads();
}

// Items are dealt to the workgroups round by round; with SERP, in serpentine
// order (round r runs positions forward when r is even, backward when odd),
// so the cheap partial tiles at the end of the class order even out the
// per-workgroup work. Within a round, consecutive items share an XCD
// (workgroup g runs on XCD g % 8) when the grid is a multiple of 8.
__device__ inline int deal_pos() {
  const int g = blockIdx.x, G = gridDim.x;
  return (G % 8) ? g : (g % 8) * (G / 8) + g / 8;
}
template <bool SERP>
__device__ inline int item_of(int r) {
  const int G = gridDim.x, p = deal_pos();
  return r * G + ((SERP && (r & 1)) ? G - 1 - p : p);
}
template <bool SERP>
__device__ inline int items_of_workgroup(int n_items) {
  const int G = gridDim.x, R = n_items / G, rem = n_items % G, p = deal_pos();
  return R + (rem > 0 && ((SERP && (R & 1)) ? G - 1 - p : p) < rem ? 1 : 0);
}

struct TileInfo {
  int e, nt, M, slot0;
};

// Wave-uniform description of work item `item` (values read from LDS are
// moved to scalar registers).
__device__ inline TileInfo tile_info(const TileMap& tm, const int* offs, int E_tot, int n_nt,
                                     int item) {
  const int ti = item / n_nt;
  int e, blk;
  if (ti < tm.n4) {
    e = workmap_find(tm.b4, E_tot, ti);
    blk = ti - tm.b4[e];
  } else {
    e = ti < tm.n4 + tm.n2 ? workmap_find(tm.b2, E_tot, ti - tm.n4)
                           : workmap_find(tm.b1, E_tot, ti - tm.n4 - tm.n2);
    blk = (offs[e + 1] - offs[e]) / kBM;  // the expert's last, partial M block
  }
  TileInfo t;
  t.e = __builtin_amdgcn_readfirstlane(e);
  t.nt = item % n_nt;
  const int m0 = blk * kBM;
  t.M = __builtin_amdgcn_readfirstlane(min(kBM, offs[e + 1] - offs[e] - m0));
  t.slot0 = __builtin_amdgcn_readfirstlane(offs[e] + m0);
  return t;
}

// Output rows of one workgroup tile: gate/up: 32 NW rows of I from each of
// gate and up; down: 64 NW rows of H.
template <bool DOWN, int NW>
constexpr int tile_rows() { return DOWN ? 64 * NW : 32 * NW; }

// DOWN = false: gate/up + SwiGLU -> h (bf16, grouped order, [A][I], each
//               group of four rows of I in the MFMA K order); fp16 operands,
//               each token's activations scaled by 2^-e (xe).
// DOWN = true : gate * (W_d h) -> per-slot outputs; bf16 operands.
//
// NW waves, each owning 64 weight rows (gate/up: 32 gate + 32 up rows, so
// SwiGLU is local) for all kBM activation rows of the tile. Every wave also
// loads a share of the activation tile. Loads follow the stage sequence of all
// of the workgroup's tiles through two cursors, so they run on across tile
// boundaries: activations two stages ahead of their LDS stores (stage g lives
// in LDS buffer g & 1), weight blocks one stage pair ahead. One barrier per
// stage.
template <int Q, bool DOWN, int NW, bool TILED>
__global__ __launch_bounds__(64 * NW) void mfma_tiles(Experts ex, FfnArgs a) {
  constexpr int NT = 64 * NW;                 // threads
  constexpr int CH = kBM * (kBK / 8) / NT;    // 16-byte activation chunks per thread per stage
  __shared__ __attribute__((aligned(16))) _Float16 xs0[kBM * kRow];  // even stages
  __shared__ __attribute__((aligned(16))) _Float16 xs1[kBM * kRow];  // odd stages
  __shared__ __attribute__((aligned(16))) uint16_t ostage[NW][kStage];  // epilogue, per wave
  __shared__ TileMap wm;
  __shared__ int offs[MOE_MAX_E_DEV + 2];
  for (int e = threadIdx.x; e <= ex.E_tot; e += NT) offs[e] = a.offsets[e];
  // gate/up: cost classes dealt in serpentine order; down (four output tiles
  // per M block, whose outputs the combine reads next): expert order
  constexpr bool kClasses = !DOWN;
  tilemap_init<Q, kClasses>(wm, a.counts, ex.E_tot, a.gmax);
  const int K = DOWN ? ex.I : ex.H;
  const int n_nt = (DOWN ? ex.H : ex.I) / tile_rows<DOWN, NW>();
  const int n_items = (wm.n4 + wm.n2 + wm.n1) * n_nt;
  const int S = K / kBK;  // even: H % 256 == 0, I % 128 == 0
  const int n_my = items_of_workgroup<kClasses>(n_items);
  if (n_my == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const uint16_t* a16 = DOWN ? static_cast<const uint16_t*>(a.h) : a.x16;

  // ---- activation cursor: wave w fills rows 8 (CH w + u) .. + 7 of a stage
  // (u < CH) with one direct global-to-LDS load each: lane l lands at chunk
  // position l % 8 of row m = 8 (CH w + u) + l / 8, so it loads logical chunk
  // q = (l % 8) ^ ((m >> 1) & 7). Logical chunk q of stage s holds K column
  // 32 (s + S (q / 4)) + 8 (q % 4) (canonical planes) or 64 s + 8 q (tiled).
  const uint4* x4 = reinterpret_cast<const uint4*>(a16);
  uint32_t xoff[CH];      // next stage's source chunk in 16-byte units (~0u: row past M)
  int anext[CH];
  int xt = 0, xsg = 0;    // tile round and stage of the next activation load
  auto xrow = [&](int u) { return 8 * (CH * wave + u) + (lane >> 3); };
  auto xprep = [&](int r) {  // tile r's rows: permutation entries, not yet waited on
    const TileInfo t = tile_info(wm, offs, ex.E_tot, n_nt, item_of<kClasses>(r));
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int m = xrow(u);
      anext[u] = m >= t.M ? -1 : (DOWN ? t.slot0 + m : a.perm[t.slot0 + m]);
    }
  };
  auto xfin = [&]() {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      int r = anext[u];
      if (!DOWN && r >= 0) {
        r = token_of(r, a.T, a.k);
        r = (unsigned)r < (unsigned)a.T ? r : -1;
      }
      const int xq = (lane & 7) ^ ((xrow(u) >> 1) & 7);
      const int col = TILED ? 8 * xq : 32 * S * (xq >> 2) + 8 * (xq & 3);
      xoff[u] = r < 0 ? ~0u : (uint32_t)(((size_t)r * K + col) / 8);
    }
  };
  // One stage into buf. Rows past M are not loaded: their LDS rows keep
  // stale values, which only reach output rows the epilogue never stores.
  auto xdma = [&](_Float16* buf) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (xoff[u] != ~0u) {
        lds_load16(x4 + xoff[u], reinterpret_cast<uint4*>(buf) + 64 * (CH * wave + u));
        xoff[u] += TILED ? 8 : 4;  // the next stage
      }
    }
    if (++xsg == S) {
      xsg = 0;
      if (++xt < n_my) {
        xfin();
        if (xt + 1 < n_my) xprep(xt + 1);
      }
    }
  };

  // ---- weight cursor: rows wrow(j) + lane % 32 ----
  // canonical planes: blocks h S + stage; tiled copy: one 64-lane record per
  // (32-row group, stage pair), blocks 4p + h and 4p + 2 + h.
  int wt = 0, wp = 0;  // tile round and stage pair of the next weight load
  uint32_t wb[2];      // next pair's index in 16-byte code / 8-byte d,m units, per row j
  const uint4* c4 = reinterpret_cast<const uint4*>(TILED ? ex.t_codes : ex.codes);
  const uint2* dm2 = reinterpret_cast<const uint2*>(TILED ? ex.t_dm : ex.dm);
  const uint2* hi2 = reinterpret_cast<const uint2*>(TILED ? ex.t_hi : ex.hi);
  auto wsetup = [&](int r) {
    const TileInfo t = tile_info(wm, offs, ex.E_tot, n_nt, item_of<kClasses>(r));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row0 = t.nt * tile_rows<DOWN, NW>() + (DOWN ? 64 * wave + 32 * j : 32 * wave);
      const int mat = DOWN ? 2 : j;  // gate, up, down
      if (TILED) {
        const size_t rec = ((size_t)t.e * 3 + mat) * tiled_records(ex) + (size_t)(row0 / 32) * (S / 2);
        wb[j] = (uint32_t)(rec * 64 + lane);
      } else {
        const size_t base = DOWN ? blk_down(ex, t.e) : (j ? blk_up(ex, t.e) : blk_gate(ex, t.e));
        const size_t blk = base + (size_t)(row0 + (lane & 31)) * (K / 32) + h * S;
        wb[j] = (uint32_t)(blk / 2);  // blk is even
      }
    }
  };
  auto wload = [&](WPair (&w)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[j].c = c4[wb[j]];
      w[j].dm = dm2[wb[j]];
      w[j].hi = Q == 3 ? hi2[wb[j]] : make_uint2(0, 0);
      wb[j] += TILED ? 64 : 1;
    }
    if (++wp == S / 2) {
      wp = 0;
      if (++wt < n_my) wsetup(wt);
    }
  };

  const int total = n_my * S;
  xprep(0);
  xfin();
  if (n_my > 1) xprep(1);
  wsetup(0);
  WPair wq[2];           // the current stage pair's weight blocks
  xdma(xs0);             // stage 0
  wload(wq);             // stage pair 0, 1
  __syncthreads();       // waits for the LDS writes of stage 0

  int g = 0;  // global stage index
  // One tile whose assignments fill LIVE 32-row activation groups; MFMAs of
  // the empty groups are left out.
  auto tile = [&](auto live_c, const TileInfo& t) {
    constexpr int LIVE = decltype(live_c)::value;
    const int wrow0 = t.nt * tile_rows<DOWN, NW>() + (DOWN ? 64 : 32) * wave;
    // per assignment of this lane: the routing gate (down) or the exponent
    // of its token's activation row (gate/up), fetched early
    float gpre[LIVE];
    int epre[LIVE];
#pragma unroll
    for (int i = 0; i < LIVE; ++i) {
      const int mm = 32 * i + (lane & 31);
      gpre[i] = DOWN && mm < t.M ? gate_of(a, t.slot0 + mm) : 0.f;
      epre[i] = 0;
      if (!DOWN && mm < t.M) {
        const int tk = token_of(a.perm[t.slot0 + mm], a.T, a.k);
        epre[i] = (unsigned)tk < (unsigned)a.T ? a.xe[tk] : 0;
      }
    }
    float16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = float16_t{};
    for (int s = 0; s < S; s += 2, g += 2) {
      // even stage g: xs0, weight block 0 of the pair; stage g + 1 streams
      // into xs1 (its last readers passed the previous barrier)
      WStage w[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) w[j] = wstage<Q>(wq[j], 0);
      xdma(xs1);                     // stage g + 1 (total is even)
      stage_mma<LIVE, Q, DOWN>(xs0, w, acc);
      __syncthreads();               // also waits for stage g + 1's LDS writes
      // odd stage g + 1: xs1, weight block 1
#pragma unroll
      for (int j = 0; j < 2; ++j) w[j] = wstage<Q>(wq[j], 1);
      if (g + 2 < total) {
        wload(wq);                   // stage pair g + 2, g + 3
        xdma(xs0);                   // stage g + 2
      }
      stage_mma<LIVE, Q, DOWN>(xs1, w, acc);
      if (s + 2 < S) __syncthreads();
    }
    // ---- epilogue ----
    // acc[i][j][v]: weight row wrow0 (+ 32 j for down) + 8 (v / 4) + 4 h + v % 4,
    //               activation row 32 i + lane % 32.
    // 16-bit outputs go through this wave's LDS staging area so that each
    // assignment's row segment is written with full 16-byte stores.
    uint16_t* stg = ostage[wave];
    if (DOWN && a.o) {
#pragma unroll
      for (int i = 0; i < LIVE; ++i) {
        const int mm = 32 * i + (lane & 31);
        if (mm >= t.M) continue;
        const size_t orow = (size_t)(t.slot0 + mm) * ex.H + wrow0;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(a.o + orow + 32 * j + 8 * q + 4 * h) =
                make_float4(gpre[i] * acc[i][j][4 * q], gpre[i] * acc[i][j][4 * q + 1],
                            gpre[i] * acc[i][j][4 * q + 2], gpre[i] * acc[i][j][4 * q + 3]);
      }
    } else if (DOWN) {
      // two passes of 64 assignments x 64 rows (bf16, row stride 72)
#pragma unroll
      for (int ip = 0; ip < (LIVE + 1) / 2; ++ip) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * ip + ii;
          if (i >= LIVE) break;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float g = gpre[i];
              const uint32_t b0 = f32_to_bf16_bits(g * acc[i][j][4 * q]);
              const uint32_t b1 = f32_to_bf16_bits(g * acc[i][j][4 * q + 1]);
              const uint32_t b2 = f32_to_bf16_bits(g * acc[i][j][4 * q + 2]);
              const uint32_t b3 = f32_to_bf16_bits(g * acc[i][j][4 * q + 3]);
              *reinterpret_cast<uint2*>(stg + (32 * ii + (lane & 31)) * 72 + 32 * j + 8 * q + 4 * h) =
                  make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < 8; ++it) {  // 8 assignments x 8 chunks of 16 bytes per step
          const int tk = (lane >> 3) + 8 * it, mm = 64 * ip + tk;
          if (mm < t.M) {
            const uint4 v = *reinterpret_cast<const uint4*>(stg + tk * 72 + 8 * (lane & 7));
            *reinterpret_cast<uint4*>(a.ob + (size_t)(t.slot0 + mm) * ex.H + wrow0 + 8 * (lane & 7)) = v;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    } else {
      // 128 assignments x 32 rows of h (bf16, row stride 40): the token's
      // exponent restores the true g and u before SwiGLU
#pragma unroll
      for (int i = 0; i < LIVE; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = silu_mul_x(acc[i][0][4 * q + u], acc[i][1][4 * q + u], epre[i]);
          *reinterpret_cast<uint2*>(stg + (32 * i + (lane & 31)) * 40 + 8 * q + 4 * h) =
              make_uint2(pack_bf16x2(v[0], v[2]), pack_bf16x2(v[1], v[3]));  // K order 0, 2, 1, 3
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 2 * LIVE; ++it) {  // 16 assignments x 4 chunks of 16 bytes per step
        const int mm = (lane >> 2) + 16 * it;
        if (mm < t.M) {
          const uint4 v = *reinterpret_cast<const uint4*>(stg + mm * 40 + 8 * (lane & 3));
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.h) + (size_t)(t.slot0 + mm) * ex.I +
                                    wrow0 + 8 * (lane & 3)) = v;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  };
  for (int r = 0; r < n_my; ++r) {
    const TileInfo t = tile_info(wm, offs, ex.E_tot, n_nt, item_of<kClasses>(r));
    // wave-uniform; Q3 keeps one variant (its third-bit plane leaves no
    // registers for more)
    if (Q == 2 && t.M <= 32) tile(std::integral_constant<int, 1>{}, t);
    else if (Q == 2 && t.M <= 64) tile(std::integral_constant<int, 2>{}, t);
    else tile(std::integral_constant<int, 4>{}, t);
  }
}

// x -> fp16 copy, the activation operand of the gate/up tiles, in the MFMA K
// order (each group of four stored as 0, 2, 1, 3), each token row scaled by
// 2^-e with its exponent e in xe.
__global__ __launch_bounds__(256) void x_to_f16(XsJob xj) {
  xs_write_rows(xj, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
}

// Writes the tiled copy: one thread per (expert, matrix, record, lane).
__global__ __launch_bounds__(256) void tile_weights(Experts ex, long n) {
  const size_t R = tiled_records(ex);
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int lane = (int)(i & 63);
    const size_t rec_all = (size_t)i >> 6;
    const size_t rec = rec_all % R;
    const int mat = (int)((rec_all / R) % 3);
    const int e = (int)(rec_all / (R * 3));
    const int K = mat == 2 ? ex.I : ex.H;
    const size_t P = K / 128;  // block quads per row
    const size_t g = rec / P, p = rec % P;
    const size_t row = 32 * g + (lane & 31);
    const size_t base = mat == 0 ? blk_gate(ex, e) : mat == 1 ? blk_up(ex, e) : blk_down(ex, e);
    const size_t b0 = base + row * (K / 32) + 4 * p + (lane >> 5), b1 = b0 + 2;
    const uint2* c = reinterpret_cast<const uint2*>(ex.codes);
    const uint32_t* dm = reinterpret_cast<const uint32_t*>(ex.dm);
    const uint2 c0 = c[b0], c1 = c[b1];
    reinterpret_cast<uint4*>(const_cast<uint8_t*>(ex.t_codes))[i] = make_uint4(c0.x, c0.y, c1.x, c1.y);
    reinterpret_cast<uint2*>(const_cast<uint16_t*>(ex.t_dm))[i] = make_uint2(dm[b0], dm[b1]);
    if (ex.qtype == 3) {
      const uint32_t* hi = reinterpret_cast<const uint32_t*>(ex.hi);
      reinterpret_cast<uint2*>(const_cast<uint8_t*>(ex.t_hi))[i] = make_uint2(hi[b0], hi[b1]);
    }
  }
}

template <int Q>
hipError_t launch_q(const Experts& ex, const FfnArgs& a, int grid, hipStream_t s) {
  if (!a.xs_ready) {
    const hipError_t xe = launch_x16(ex, a, s);
    if (xe != hipSuccess) return xe;
  }
  const bool g8 = ex.I % tile_rows<false, 8>() == 0, d8 = ex.H % tile_rows<true, 8>() == 0;
#define MOE_TILES(NAME, DOWN, NW)                                                              \
  do {                                                                                         \
    if (ex.t_codes)                                                                            \
      MOE_LAUNCH(NAME, s, (mfma_tiles<Q, DOWN, NW, true>), dim3(grid), dim3(64 * NW), 0, s, ex, \
                 a);                                                                           \
    else                                                                                       \
      MOE_LAUNCH(NAME, s, (mfma_tiles<Q, DOWN, NW, false>), dim3(grid), dim3(64 * NW), 0, s,   \
                 ex, a);                                                                       \
  } while (0)
  if (g8) MOE_TILES("mfma_gateup", false, 8);
  else MOE_TILES("mfma_gateup", false, 4);
  if (d8) MOE_TILES("mfma_down", true, 8);
  else MOE_TILES("mfma_down", true, 4);
#undef MOE_TILES
  return hipGetLastError();
}

}  // namespace

hipError_t launch_x16(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const int xg = (a.T + 3) / 4 < 2048 ? (a.T + 3) / 4 : 2048;  // a wave per token row
  MOE_LAUNCH("x_to_f16", s, x_to_f16, dim3(xg), dim3(256), 0, s,
             xs_job(0, ex.H, a.x, a.xdtype, a.T, a.x16, a.xe));
  return hipGetLastError();
}

hipError_t launch_tile_weights(const Experts& ex, hipStream_t s) {
  const long n = (long)ex.E_tot * 3 * (long)tiled_records(ex) * 64;
  const int grid = (int)(n / 256 + 1 < 8192 ? n / 256 + 1 : 8192);
  MOE_LAUNCH("tile_weights", s, tile_weights, dim3(grid), dim3(256), 0, s, ex, n);
  return hipGetLastError();
}

bool mfma_supported(int H, int I) {
  return H % tile_rows<true, 4>() == 0 && I % tile_rows<false, 4>() == 0;
}

hipError_t launch_mfma(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const long A = (long)a.T * (a.k + ex.has_shared);
  const long max_tiles = A / kBM + ex.E_tot + 1;
  const long max_items = max_tiles * (ex.H / tile_rows<true, 4>() > ex.I / tile_rows<false, 4>()
                                          ? ex.H / tile_rows<true, 4>()
                                          : ex.I / tile_rows<false, 4>());
  static int cus[64] = {0};  // compute units per device, read once
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  const int grid = (int)(max_items < cus[dev] ? max_items : cus[dev]);
  return ex.qtype == 3 ? launch_q<3>(ex, a, grid, s) : launch_q<2>(ex, a, grid, s);
}

}  // namespace moe

// Prefill tiles of the expert FFN on gfx950 matrix cores.
//
// An expert with many assignments multiplies a gathered block of its tokens'
// activations by its dequantised weights: gate and up share one activation
// tile and SwiGLU runs in the epilogue; the down projection folds the routing
// gate into its epilogue. The pages' prompt path likewise multiplies quantised
// experts in large chunks without first expanding them to FP16 in memory
// ("Strata - the details", "Faster prompts"). Here each weight tile is
// expanded only in LDS, once per workgroup tile, and fed to
// v_mfma_f32_32x32x16_f16.
//
// Workgroup tile: kBM = 128 assignments x kBN = 256 weight rows (gate/up: 128
// rows of I from each of gate and up; down: 256 rows of H), K in stages of 64
// (two quantisation blocks). Eight waves split by role, two per SIMD:
//   waves 0..3 (MFMA): each a 64 x 128 sub-tile, 8 MFMAs per 16 of K;
//   waves 4..7 (load): gather the next stage's activation rows through the
//     grouping permutation, load and dequantise the next stage's weight rows
//     (w = d*q + m, one fp16 rounding), and write both to the other LDS buffer.
// One barrier per stage hands a buffer from the loaders to the MFMA waves.
//
// The grid is persistent. Work items are (expert tile, N tile) with the N
// tiles of one expert tile adjacent; consecutive items go to workgroups of one
// XCD, so the activation rows they share stay in that XCD's L2.
#include "common.h"
#include "gemv.h"
#include "sched.h"

namespace moe {
namespace {

constexpr int kBM = 128;          // assignments per tile
constexpr int kBN = 256;          // weight rows per tile
constexpr int kBK = 64;           // K per stage
constexpr int kRow = 72;          // LDS row stride in halves (64 + 8 pad: 144 B)
constexpr int kMThreads = 512;    // 4 MFMA waves + 4 loader waves
constexpr int kLoadT = 256;       // loader threads
constexpr int kDepth = 4;         // stages a loader has in flight (even)

struct TileLds {
  _Float16 x[2][kBM * kRow];
  _Float16 w[2][kBN * kRow];
};

// --- dequantisation -------------------------------------------------------
// Code pair -> fp16 pair: OR the codes into the mantissa of 1024 (exact
// 1024 + q), subtract 1024 (exact), then one fused d*q + m.
__device__ inline uint32_t deq_pair(uint32_t t, half2_t d2, half2_t m2) {
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2_t q = __builtin_bit_cast(half2_t, t | 0x64006400u) - k1024;
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, d2, m2));
}

// 16 two-bit codes (code j at bits 2j of c) -> 8 fp16 pairs in natural order.
// Byte j of c holds codes 4j..4j+3; byte j of c >> 2 holds 4j+1..4j+3. A byte
// permute puts byte j of each in the two halves; masks pick codes (4j, 4j+1)
// from bits 0-1 and (4j+2, 4j+3) from bits 4-5. hq: the third code bits
// (Q3), bit j = code j's bit 2.
template <int Q>
__device__ inline void deq_word(uint32_t c, uint32_t hq, half2_t d2, half2_t m2, uint32_t* out) {
  const uint32_t s = c >> 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t r = __builtin_amdgcn_perm(s, c, 0x0C000C00u | ((4u + j) << 16) | (uint32_t)j);
    uint32_t t0 = r & 0x00030003u, t1 = (r >> 4) & 0x00030003u;
    if (Q == 3) {
      const uint32_t h = hq >> (4 * j);
      t0 |= ((h & 1u) << 2) | ((h & 2u) << 17);
      t1 |= (h & 4u) | ((h & 8u) << 15);
    }
    out[2 * j] = deq_pair(t0, d2, m2);
    out[2 * j + 1] = deq_pair(t1, d2, m2);
  }
}

// Two consecutive blocks of one weight row (64 weights) -> 64 fp16 in LDS.
template <int Q>
__device__ inline void deq_stage(uint4 c, uint2 hi, uint2 dm, _Float16* dst) {
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t dmb = b ? dm.y : dm.x;
    const half2_t d2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dmb, dmb, 0x01000100u));
    const half2_t m2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dmb, dmb, 0x03020302u));
    const uint32_t c0 = b ? c.z : c.x, c1 = b ? c.w : c.y;
    const uint32_t h = Q == 3 ? (b ? hi.y : hi.x) : 0u;
    uint32_t o[16];
    deq_word<Q>(c0, h, d2, m2, o);
    deq_word<Q>(c1, h >> 16, d2, m2, o + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d4[4 * b + i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
}

// --- loader role ------------------------------------------------------------
// Per stage a loader thread fetches 4 activation chunks (rows xrow + 32 i,
// 8 halves at column 8 * xq) and one weight row's two blocks.
struct Stage {
  uint4 x[4];
  uint4 c;
  uint2 hi, dm;
};

template <int Q>
__device__ inline void load_stage(const Experts& ex, const uint16_t* __restrict__ a16, int lda,
                                  const int (&arow)[4], int xq, size_t wblk, int k0, Stage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (arow[i] >= 0)
      st.x[i] = *reinterpret_cast<const uint4*>(a16 + (size_t)arow[i] * lda + k0 + 8 * xq);
    else
      st.x[i] = make_uint4(0, 0, 0, 0);
  }
  const size_t blk = wblk + k0 / 32;
  st.c = *reinterpret_cast<const uint4*>(ex.codes + blk * 8);
  st.dm = *reinterpret_cast<const uint2*>(ex.dm + blk * 2);
  st.hi = Q == 3 ? *reinterpret_cast<const uint2*>(ex.hi + blk * 4) : make_uint2(0, 0);
}

template <int Q>
__device__ inline void store_stage(const Stage& st, int tl, _Float16* xs, _Float16* ws) {
  const int xrow = tl >> 3, xq = tl & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(xs + (xrow + 32 * i) * kRow + 8 * xq) = st.x[i];
  deq_stage<Q>(st.c, st.hi, st.dm, ws + tl * kRow);
}

// --- MFMA role --------------------------------------------------------------
__device__ inline half8_t frag(const _Float16* p) { return *reinterpret_cast<const half8_t*>(p); }

// One stage for an MFMA wave: weight rows brow[j] + lane%32 (the MFMA's row
// operand) times activation rows 64 mh + 32 i + lane%32 (its column operand);
// the 32-row half i = 1 is skipped when it lies at or past M.
__device__ inline void mma_stage(const _Float16* xs, const _Float16* ws, int mh, bool live1,
                                 const int (&brow)[4], float16_t (&acc)[2][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 16) {
    const int kc = kk + 8 * (lane >> 5);
    half8_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag(ws + (brow[j] + (lane & 31)) * kRow + kc);
    const half8_t a0 = frag(xs + (64 * mh + (lane & 31)) * kRow + kc);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a0, acc[0][j], 0, 0, 0);
    if (live1) {
      const half8_t a1 = frag(xs + (64 * mh + 32 + (lane & 31)) * kRow + kc);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a1, acc[1][j], 0, 0, 0);
    }
  }
}

// Logical item of this workgroup in round r: consecutive items share an XCD
// (workgroup g runs on XCD g % 8) when the grid is a multiple of 8.
__device__ inline long item_of(long r) {
  const int g = blockIdx.x, G = gridDim.x;
  if (G % 8) return r * G + g;
  return r * G + (g % 8) * (G / 8) + g / 8;
}

struct TileInfo {
  int e, nt, M, slot0;
};

__device__ inline TileInfo tile_info(const WorkMap& wm, const int* offs, int E_tot, int n_nt,
                                     long item) {
  int tl;
  TileInfo t;
  t.e = workmap_tile(wm, E_tot, (int)(item / n_nt), tl);
  t.nt = (int)(item % n_nt);
  const int m0 = tl * kBM;
  t.M = min(kBM, offs[t.e + 1] - offs[t.e] - m0);
  t.slot0 = offs[t.e] + m0;
  return t;
}

// DOWN = false: gate/up + SwiGLU -> h (fp16, grouped order, [A][I]).
// DOWN = true : gate * (W_d h) -> per-slot outputs.
//
// Loader waves run a flat sequence of (tile, stage) loads kDepth stages ahead
// of the LDS stores (kDepth register sets; stage i lands in LDS buffer i & 1);
// the grouping permutation entries of the next tile are fetched a tile ahead.
template <int Q, bool DOWN>
__global__ __launch_bounds__(kMThreads) void mfma_tiles(Experts ex, FfnArgs a) {
  __shared__ __attribute__((aligned(16))) TileLds L;
  __shared__ WorkMap wm;
  __shared__ int offs[MOE_MAX_E_DEV + 2];
  for (int e = threadIdx.x; e <= ex.E_tot; e += blockDim.x) offs[e] = a.offsets[e];
  workmap_init(wm, a.counts, ex.E_tot, a.gmax, kBM);
  const int K = DOWN ? ex.I : ex.H;
  const int n_nt = DOWN ? ex.H / kBN : ex.I / (kBN / 2);
  const long n_items = (long)wm.n_tiles * n_nt;
  const int S = K / kBK;  // even: H % 256 == 0, I % 128 == 0
  const long first = item_of(0);
  const int n_my = first < n_items ? (int)((n_items - first + gridDim.x - 1) / gridDim.x) : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (tid >= kMThreads - kLoadT) {
    // ---- loader ----
    const int tl = tid - (kMThreads - kLoadT), xr = tl >> 3, xq = tl & 7;
    const uint16_t* a16 = DOWN ? static_cast<const uint16_t*>(a.h) : a.x16;
    int arow[4], nxt[4];
    size_t wblk = 0;
    TileInfo tn{};
    auto prep = [&](int r) {  // tile r's info and permutation entries, not yet waited on
      tn = tile_info(wm, offs, ex.E_tot, n_nt, item_of(r));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = xr + 32 * i;
        nxt[i] = m >= tn.M ? -1 : (DOWN ? tn.slot0 + m : a.perm[tn.slot0 + m]);
      }
    };
    auto fin = [&]() {  // make the prepared tile the one being loaded
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = nxt[i];
        if (!DOWN && r >= 0) {
          r = token_of(r, a.T, a.k);
          r = (unsigned)r < (unsigned)a.T ? r : -1;
        }
        arow[i] = r;
      }
      if (DOWN) {
        wblk = blk_down(ex, tn.e) + (size_t)(tn.nt * kBN + tl) * (ex.I / 32);
      } else {
        const int row = tn.nt * (kBN / 2) + (tl & (kBN / 2 - 1));
        wblk = (tl < kBN / 2 ? blk_gate(ex, tn.e) : blk_up(ex, tn.e)) + (size_t)row * (ex.H / 32);
      }
    };
    int lr = 0, ls = 0;  // tile round and stage of the next load
    if (n_my > 0) {
      prep(0);
      fin();
      if (n_my > 1) prep(1);
    }
    auto next_load = [&](Stage& st) {
      load_stage<Q>(ex, a16, K, arow, xq, wblk, ls * kBK, st);
      if (++ls == S) {
        ls = 0;
        if (++lr < n_my) {
          fin();
          if (lr + 1 < n_my) prep(lr + 1);
        }
      }
    };
    const int total = n_my * S;
    Stage st[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (d < total) next_load(st[d]);
    for (int i = 0; i < total; i += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        if (i + d < total) {
          store_stage<Q>(st[d], tl, L.x[d & 1], L.w[d & 1]);
          if (i + d + kDepth < total) next_load(st[d]);
          __syncthreads();
        }
      }
    }
    return;
  }

  // ---- MFMA waves ----
  const int mh = wave & 1, nq = wave >> 1;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = DOWN ? 128 * nq + 32 * j : (j < 2 ? 64 * nq + 32 * j : 128 + 64 * nq + 32 * (j - 2));
  for (int r = 0; r < n_my; ++r) {
    const TileInfo t = tile_info(wm, offs, ex.E_tot, n_nt, item_of(r));
    float16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = float16_t{};
    const bool live = 64 * mh < t.M, live1 = 64 * mh + 32 < t.M;
    for (int s = 0; s < S; s += 2) {
      __syncthreads();
      if (live) mma_stage(L.x[0], L.w[0], mh, live1, brow, acc);
      __syncthreads();
      if (live) mma_stage(L.x[1], L.w[1], mh, live1, brow, acc);
    }
    if (!live) continue;
    // acc[i][j][v]: weight row brow[j] + 8 (v / 4) + 4 (lane / 32) + v % 4,
    //               activation row 64 mh + 32 i + lane % 32
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int mm = 64 * mh + 32 * i + (lane & 31);
      if (mm >= t.M) continue;
      const int slot = t.slot0 + mm;
      if (DOWN) {
        const float gt = gate_of(a, slot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const size_t off = (size_t)slot * ex.H + t.nt * kBN + brow[j] + 8 * q + 4 * (lane >> 5);
            const float v0 = gt * acc[i][j][4 * q], v1 = gt * acc[i][j][4 * q + 1];
            const float v2 = gt * acc[i][j][4 * q + 2], v3 = gt * acc[i][j][4 * q + 3];
            if (a.o) {
              *reinterpret_cast<float4*>(a.o + off) = make_float4(v0, v1, v2, v3);
            } else {
              *reinterpret_cast<uint2*>(a.ob + off) =
                  make_uint2(f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16),
                             f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16));
            }
          }
        }
      } else {
        _Float16* h = static_cast<_Float16*>(a.h) + (size_t)slot * ex.I + t.nt * (kBN / 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = silu_mul(acc[i][j][4 * q + u], acc[i][j + 2][4 * q + u]);
            *reinterpret_cast<uint2*>(h + brow[j] + 8 * q + 4 * (lane >> 5)) =
                make_uint2(pack_half2(v[0], v[1]), pack_half2(v[2], v[3]));
          }
        }
      }
    }
  }
}

// x -> fp16 copy, the activation operand of the gate/up tiles.
template <bool XF32>
__global__ __launch_bounds__(256) void x_to_f16(const void* __restrict__ x, long n8,
                                                uint16_t* __restrict__ x16) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    uint32_t o[4];
    if (XF32) {
      const float4* src = static_cast<const float4*>(x) + 2 * i;
      const float4 f0 = src[0], f1 = src[1];
      o[0] = pack_half2(f0.x, f0.y);
      o[1] = pack_half2(f0.z, f0.w);
      o[2] = pack_half2(f1.x, f1.y);
      o[3] = pack_half2(f1.z, f1.w);
    } else {
      const uint4 v = static_cast<const uint4*>(x)[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = pack_half2(bf16_lo(w[j]), bf16_hi(w[j]));
    }
    reinterpret_cast<uint4*>(x16)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <int Q>
hipError_t launch_q(const Experts& ex, const FfnArgs& a, int grid, hipStream_t s) {
  const long n8 = (long)a.T * ex.H / 8;
  const int xg = (int)(n8 / 256 + 1 < 2048 ? n8 / 256 + 1 : 2048);
  if (a.xdtype == 0)
    MOE_LAUNCH("x_to_f16", s, x_to_f16<true>, dim3(xg), dim3(256), 0, s, a.x, n8, a.x16);
  else
    MOE_LAUNCH("x_to_f16", s, x_to_f16<false>, dim3(xg), dim3(256), 0, s, a.x, n8, a.x16);
  MOE_LAUNCH("mfma_gateup", s, (mfma_tiles<Q, false>), dim3(grid), dim3(kMThreads), 0, s, ex, a);
  MOE_LAUNCH("mfma_down", s, (mfma_tiles<Q, true>), dim3(grid), dim3(kMThreads), 0, s, ex, a);
  return hipGetLastError();
}

}  // namespace

bool mfma_supported(int H, int I) { return H % kBN == 0 && I % (kBN / 2) == 0; }

hipError_t launch_mfma(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const long A = (long)a.T * (a.k + ex.has_shared);
  const long max_tiles = A / kBM + ex.E_tot + 1;
  const long max_items = max_tiles * (ex.H / kBN > ex.I / (kBN / 2) ? ex.H / kBN : ex.I / (kBN / 2));
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int grid = (int)(max_items < cus ? max_items : cus);
  return ex.qtype == 3 ? launch_q<3>(ex, a, grid, s) : launch_q<2>(ex, a, grid, s);
}

}  // namespace moe

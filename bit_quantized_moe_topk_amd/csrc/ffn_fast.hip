// Fast mode of the expert FFN on gfx950.
//
// Decode shape (an expert holding 1..4 of the step's assignments): the layer is
// bound by streaming the packed weights ("Strata - the details", section "Other
// GPUs": the GPU share of the work scales with memory bandwidth). The GEMV
// kernels read every touched weight once with coalesced loads and never expand
// it: the 2-bit (or 3-bit) code becomes an exact bf16 value (128 + q) by
// setting mantissa bits, v_dot2 multiplies code pairs by bf16 activation pairs
// in fp32, and the block affine map is applied once per block and token:
//     sum_k (d q_k + m) x_k = d * (sum_k (128 + q_k) x_k - 128 S) + m * S,
// S = sum_k x_k over the block.
//
// Prefill shape (more assignments per expert): tiles of 64 assignments x 64
// output rows run on v_mfma_f32_32x32x16_f16. Each K step dequantises a weight
// tile to fp16 (w = d*q + m, one rounding) into LDS and gathers the tile's
// activation rows (through the grouping permutation) into LDS as fp16; gate and
// up tiles share the activation fragment and SwiGLU runs in the epilogue. The
// pages' prompt path likewise multiplies quantised experts without expanding
// them to FP16 in memory first ("Faster prompts").
//
// Lane layout of every kernel is stated where it is used.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)

__device__ inline float half_lo(uint32_t v) { return half_bits_to_f32((uint16_t)(v & 0xFFFFu)); }
__device__ inline float half_hi(uint32_t v) { return half_bits_to_f32((uint16_t)(v >> 16)); }
__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ inline int token_of(int asg, int T, int k) { return asg < T * k ? asg / k : asg - T * k; }

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------------------
// Activations of one 32-wide block as 16 bf16 pairs in code-pair order:
// pair (w*8 + s) = (x[16w + s], x[16w + s + 8]), w in {0,1}, s in 0..7,
// which is the order in which code pairs are extracted from a code word
// (codes 16w+s and 16w+s+8 sit 16 bits apart). Also returns S = sum of x.
struct XBlock {
  uint32_t p[16];
  float S;
};

// v[i] holds bf16 elements 2i (low half) and 2i+1 (high half), i < 16.
__device__ inline void make_pairs(const uint32_t v[16], XBlock& xb) {
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) S += bf16_lo(v[i]) + bf16_hi(v[i]);
  xb.S = S;
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t a = v[8 * w + s / 2], b = v[8 * w + 4 + s / 2];
      xb.p[8 * w + s] = (s & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
}

__device__ inline void load_xblock_bf16(const uint16_t* src, XBlock& xb) {
  uint32_t v[16];
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = s4[i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
  make_pairs(v, xb);
}

__device__ inline void load_xblock_f32(const float* src, XBlock& xb) {
  uint32_t v[16];
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 q = s4[i];
    v[2 * i] = f32_to_bf16_bits(q.x) | (f32_to_bf16_bits(q.y) << 16);
    v[2 * i + 1] = f32_to_bf16_bits(q.z) | (f32_to_bf16_bits(q.w) << 16);
  }
  make_pairs(v, xb);
}

// Packed block: 2 code words (+ the high-bit word for Q3) and the (d, m) word.
struct QBlock {
  uint32_t c0, c1, hi, dm;
};

template <int Q>
__device__ inline QBlock load_qblock(const Experts& ex, size_t blk) {
  QBlock b;
  const uint2 c = *reinterpret_cast<const uint2*>(ex.codes + blk * 8);
  b.c0 = c.x;
  b.c1 = c.y;
  b.dm = *reinterpret_cast<const uint32_t*>(ex.dm + blk * 2);
  b.hi = Q == 3 ? *reinterpret_cast<const uint32_t*>(ex.hi + blk * 4) : 0u;
  return b;
}

// sum_k q_k x_k + 128 S  (the chain starts at -128 S so the result is sum q x)
template <int Q>
__device__ inline float block_dot(const QBlock& b, const XBlock& xb) {
  float D = -128.0f * xb.S;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t cw = w ? b.c1 : b.c0;
    uint32_t r2 = 0;
    if (Q == 3) {
      const uint32_t hw = b.hi >> (16 * w);
      r2 = ((hw & 0xFFu) | ((hw & 0xFF00u) << 8)) << 2;  // code 16w+s -> bit s+2, +8 -> bit s+18
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t pr = ((cw >> (2 * s)) & 0x00030003u) | kMagic;
      if (Q == 3) pr |= (r2 >> s) & 0x00040004u;
      D = dot2(pr, xb.p[8 * w + s], D);
    }
  }
  return D;
}

template <int Q>
__device__ inline float block_term(const QBlock& b, const XBlock& xb) {
  return half_lo(b.dm) * block_dot<Q>(b, xb) + half_hi(b.dm) * xb.S;
}

template <int W>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Decode GEMV, gate + up + SwiGLU.
// Lane l works on block (l % BPR) of row (l / BPR) of a group of 64/BPR rows.
// A workgroup takes RC consecutive rows of I for one expert; its 4 waves take
// ROWS_W rows each, in PASSES passes of 64/BPR rows.
template <int BPR, int Q, bool XF32>
__global__ __launch_bounds__(kThreads) void gemv_gateup(Experts ex, FfnArgs a) {
  constexpr int RPI = 64 / BPR;
  constexpr int ROWS_W = RPI > 4 ? RPI : 4;
  constexpr int PASSES = ROWS_W / RPI;
  constexpr int RC = 4 * ROWS_W;
  const SchedView sv = sched_view(a.sched, ex.E_tot);
  const int n_items = sv.hdr[0] * (ex.I / RC);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk_in_row = lane % BPR, row_in_grp = lane / BPR;
  uint16_t* h = static_cast<uint16_t*>(a.h);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int e = sv.gemv[item / (ex.I / RC)];
    const int r0 = (item % (ex.I / RC)) * RC + wave * ROWS_W;
    const int M = a.counts[e];
    const int slot0 = a.offsets[e];
    XBlock xb[kGemvMaxTokens];
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; ++m) {
      if (m < M) {
        int t = token_of(a.perm[slot0 + m], a.T, a.k);
        t = (unsigned)t < (unsigned)a.T ? t : 0;
        const size_t off = (size_t)t * ex.H + 32 * blk_in_row;
        if (XF32) load_xblock_f32(static_cast<const float*>(a.x) + off, xb[m]);
        else load_xblock_bf16(static_cast<const uint16_t*>(a.x) + off, xb[m]);
      }
    }
    QBlock qg[PASSES], qu[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = r0 + p * RPI + row_in_grp;
      qg[p] = load_qblock<Q>(ex, blk_gate(ex, e) + (size_t)row * BPR + blk_in_row);
      qu[p] = load_qblock<Q>(ex, blk_up(ex, e) + (size_t)row * BPR + blk_in_row);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = r0 + p * RPI + row_in_grp;
#pragma unroll
      for (int m = 0; m < kGemvMaxTokens; ++m) {
        if (m < M) {
          const float g = group_sum<BPR>(block_term<Q>(qg[p], xb[m]));
          const float u = group_sum<BPR>(block_term<Q>(qu[p], xb[m]));
          if (blk_in_row == 0)
            h[(size_t)(slot0 + m) * ex.I + row] = (uint16_t)f32_to_bf16_bits(silu_mul(g, u));
        }
      }
    }
  }
}

// Decode GEMV, down projection with the gate folded in: o[slot] = gate * Wd h.
// Lane layout as above with BPR = I/32; a workgroup takes 64 rows of H.
template <int BPR, int Q>
__global__ __launch_bounds__(kThreads) void gemv_down(Experts ex, FfnArgs a) {
  constexpr int RPI = 64 / BPR;
  constexpr int ROWS_W = RPI > 16 ? RPI : 16;
  constexpr int PASSES = ROWS_W / RPI;
  constexpr int RC = 4 * ROWS_W;
  const SchedView sv = sched_view(a.sched, ex.E_tot);
  const int n_items = sv.hdr[0] * (ex.H / RC);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk_in_row = lane % BPR, row_in_grp = lane / BPR;
  const uint16_t* h = static_cast<const uint16_t*>(a.h);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int e = sv.gemv[item / (ex.H / RC)];
    const int r0 = (item % (ex.H / RC)) * RC + wave * ROWS_W;
    const int M = a.counts[e];
    const int slot0 = a.offsets[e];
    XBlock xb[kGemvMaxTokens];
    float gate[kGemvMaxTokens];
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; ++m) {
      if (m < M) {
        load_xblock_bf16(h + (size_t)(slot0 + m) * ex.I + 32 * blk_in_row, xb[m]);
        const int asg = a.perm[slot0 + m];
        gate[m] = asg < a.T * a.k ? a.gates[asg] : 1.0f;
      }
    }
    QBlock qd[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = r0 + p * RPI + row_in_grp;
      qd[p] = load_qblock<Q>(ex, blk_down(ex, e) + (size_t)row * BPR + blk_in_row);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = r0 + p * RPI + row_in_grp;
#pragma unroll
      for (int m = 0; m < kGemvMaxTokens; ++m) {
        if (m < M) {
          const float v = group_sum<BPR>(block_term<Q>(qd[p], xb[m]));
          if (blk_in_row == 0) a.o[(size_t)(slot0 + m) * ex.H + row] = gate[m] * v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA tiles.
constexpr int kTN = 64;      // output rows per tile
constexpr int kTK = 64;      // K per step (two blocks)
constexpr int kLdsRow = 72;  // fp16 elements per LDS row (64 + 8 pad: 144 B stride)

__device__ inline uint32_t pack_half2(float lo, float hi) {
  const half2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Dequantise one 32-weight block to fp16 and store it at dst (LDS, 64 bytes).
template <int Q>
__device__ inline void deq_block_to_lds(const QBlock& b, _Float16* dst) {
  const float d = half_lo(b.dm), m = half_hi(b.dm);
  uint32_t out[16];
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    const uint32_t cw = j < 16 ? b.c0 : b.c1;
    int q0 = (cw >> (2 * (j & 15))) & 3, q1 = (cw >> (2 * ((j + 1) & 15))) & 3;
    if (Q == 3) {
      q0 |= ((b.hi >> j) & 1) << 2;
      q1 |= ((b.hi >> (j + 1)) & 1) << 2;
    }
    out[j / 2] = pack_half2(fmaf(d, (float)q0, m), fmaf(d, (float)q1, m));
  }
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d4[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

__device__ inline half8_t lds_frag(const _Float16* base) {
  return *reinterpret_cast<const half8_t*>(base);
}

// Gate + up + SwiGLU. Workgroup tile: 64 assignments x 64 rows of I (gate and
// up: 128 weight rows). Wave w: assignments 32*(w&1).., rows 32*(w>>1)..
template <int Q, bool XF32>
__global__ __launch_bounds__(kThreads) void mfma_gateup(Experts ex, FfnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[kTileM * kLdsRow];
  __shared__ __attribute__((aligned(16))) _Float16 ws[2 * kTN * kLdsRow];
  const SchedView sv = sched_view(a.sched, ex.E_tot);
  const int n_nt = ex.I / kTN;
  const int n_items = sv.hdr[1] * n_nt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int th = wave & 1, rh = wave >> 1;
  _Float16* hbuf = static_cast<_Float16*>(a.h);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile = sv.tiles[item / n_nt];
    const int n0 = (item % n_nt) * kTN;
    const int e = tile >> 16, m0 = (tile & 0xFFFF) * kTileM;
    const int M = a.counts[e] - m0;
    const int slot0 = a.offsets[e] + m0;
    // loader roles
    const int xr = tid >> 2, xq = tid & 3;  // x: row xr, 16 K-elements at 16*xq
    int tok = -1;
    if (xr < M) {
      tok = token_of(a.perm[slot0 + xr], a.T, a.k);
      if ((unsigned)tok >= (unsigned)a.T) tok = -1;
    }
    const int wr = tid >> 1, wb = tid & 1;  // w: weight row wr (0..127), block wb
    const size_t wblk0 = (wr < kTN ? blk_gate(ex, e) : blk_up(ex, e)) +
                         (size_t)(n0 + (wr & (kTN - 1))) * (ex.H / 32) + wb;
    float16_t acc_g = {}, acc_u = {};
    for (int k0 = 0; k0 < ex.H; k0 += kTK) {
      // global -> registers
      uint32_t xv[8];
      if (tok >= 0) {
        if (XF32) {
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) +
                                                              (size_t)tok * ex.H + k0 + 16 * xq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 f = src[i];
            xv[2 * i] = pack_half2(f.x, f.y);
            xv[2 * i + 1] = pack_half2(f.z, f.w);
          }
        } else {
          const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) +
                                                            (size_t)tok * ex.H + k0 + 16 * xq);
          const uint4 q0 = src[0], q1 = src[1];
          const uint32_t r[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[i] = pack_half2(bf16_lo(r[i]), bf16_hi(r[i]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = 0u;
      }
      const QBlock qb = load_qblock<Q>(ex, wblk0 + k0 / 32);
      __syncthreads();  // previous step's fragments consumed
      {
        uint4* dst = reinterpret_cast<uint4*>(xs + xr * kLdsRow + 16 * xq);
        dst[0] = make_uint4(xv[0], xv[1], xv[2], xv[3]);
        dst[1] = make_uint4(xv[4], xv[5], xv[6], xv[7]);
      }
      deq_block_to_lds<Q>(qb, ws + wr * kLdsRow + 32 * wb);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kTK; kk += 16) {
        const int kc = kk + 8 * (lane >> 5);
        const half8_t af = lds_frag(xs + (32 * th + (lane & 31)) * kLdsRow + kc);
        const half8_t bg = lds_frag(ws + (32 * rh + (lane & 31)) * kLdsRow + kc);
        const half8_t bu = lds_frag(ws + (kTN + 32 * rh + (lane & 31)) * kLdsRow + kc);
        acc_g = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bg, acc_g, 0, 0, 0);
        acc_u = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bu, acc_u, 0, 0, 0);
      }
    }
    // epilogue: acc[i] -> assignment 8*(i/4) + 4*(lane/32) + i%4, row lane%32
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mm = 32 * th + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (mm < M) {
        const int row = n0 + 32 * rh + (lane & 31);
        hbuf[(size_t)(slot0 + mm) * ex.I + row] = (_Float16)silu_mul(acc_g[i], acc_u[i]);
      }
    }
  }
}

// Down projection, o[slot] = gate * Wd h. Tile: 64 assignments x 64 rows of H.
template <int Q>
__global__ __launch_bounds__(kThreads) void mfma_down(Experts ex, FfnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[kTileM * kLdsRow];
  __shared__ __attribute__((aligned(16))) _Float16 ws[kTN * kLdsRow];
  const SchedView sv = sched_view(a.sched, ex.E_tot);
  const int n_nt = ex.H / kTN;
  const int n_items = sv.hdr[1] * n_nt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int th = wave & 1, rh = wave >> 1;
  const _Float16* hbuf = static_cast<const _Float16*>(a.h);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile = sv.tiles[item / n_nt];
    const int n0 = (item % n_nt) * kTN;
    const int e = tile >> 16, m0 = (tile & 0xFFFF) * kTileM;
    const int M = a.counts[e] - m0;
    const int slot0 = a.offsets[e] + m0;
    const int xr = tid >> 2, xq = tid & 3;
    const int wr = (tid >> 1) & (kTN - 1), wb = tid & 1;  // threads >= 128 mirror; only < 128 store
    const size_t wblk0 = blk_down(ex, e) + (size_t)(n0 + wr) * (ex.I / 32) + wb;
    float16_t acc = {};
    for (int k0 = 0; k0 < ex.I; k0 += kTK) {
      uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
      if (xr < M) {
        const uint4* src = reinterpret_cast<const uint4*>(hbuf + (size_t)(slot0 + xr) * ex.I + k0 + 16 * xq);
        x0 = src[0];
        x1 = src[1];
      }
      QBlock qb;
      if (tid < 2 * kTN) qb = load_qblock<Q>(ex, wblk0 + k0 / 32);
      __syncthreads();
      {
        uint4* dst = reinterpret_cast<uint4*>(xs + xr * kLdsRow + 16 * xq);
        dst[0] = x0;
        dst[1] = x1;
      }
      if (tid < 2 * kTN) deq_block_to_lds<Q>(qb, ws + wr * kLdsRow + 32 * wb);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kTK; kk += 16) {
        const int kc = kk + 8 * (lane >> 5);
        const half8_t af = lds_frag(xs + (32 * th + (lane & 31)) * kLdsRow + kc);
        const half8_t bf = lds_frag(ws + (32 * rh + (lane & 31)) * kLdsRow + kc);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mm = 32 * th + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (mm < M) {
        const int slot = slot0 + mm;
        const int asg = a.perm[slot];
        const float gate = asg < a.T * a.k ? a.gates[asg] : 1.0f;
        a.o[(size_t)slot * ex.H + n0 + 32 * rh + (lane & 31)] = gate * acc[i];
      }
    }
  }
}

inline int grid_for(long max_items, int cap) {
  return (int)(max_items < cap ? (max_items > 0 ? max_items : 1) : cap);
}

template <int Q, bool XF32>
hipError_t launch_q(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const int A = a.T * (a.k + ex.has_shared);
  const long max_gemv = A < ex.E_tot ? A : ex.E_tot;
  const long max_tiles = A / kTileM + ex.E_tot + 1;
  const int bpr_h = ex.H / 32, bpr_i = ex.I / 32;
  // decode GEMV (only when the shapes fit the lane layouts; otherwise the
  // scheduler sends every expert to the MFMA tiles)
#define GU(B) hipLaunchKernelGGL((gemv_gateup<B, Q, XF32>), dim3(grid_for(max_gemv * (ex.I / (4 * (64 / B > 4 ? 64 / B : 4))), 2048)), dim3(kThreads), 0, s, ex, a)
#define DN(B) hipLaunchKernelGGL((gemv_down<B, Q>), dim3(grid_for(max_gemv * (ex.H / (4 * (64 / B > 16 ? 64 / B : 16))), 2048)), dim3(kThreads), 0, s, ex, a)
  switch (bpr_h) {
    case 4: GU(4); break;
    case 8: GU(8); break;
    case 16: GU(16); break;
    case 32: GU(32); break;
    case 64: GU(64); break;
    default: break;
  }
  hipLaunchKernelGGL((mfma_gateup<Q, XF32>), dim3(grid_for(max_tiles * (ex.I / kTN), 4096)),
                     dim3(kThreads), 0, s, ex, a);
  switch (bpr_i) {
    case 4: DN(4); break;
    case 8: DN(8); break;
    case 16: DN(16); break;
    case 32: DN(32); break;
    case 64: DN(64); break;
    default: break;
  }
#undef GU
#undef DN
  hipLaunchKernelGGL((mfma_down<Q>), dim3(grid_for(max_tiles * (ex.H / kTN), 4096)),
                     dim3(kThreads), 0, s, ex, a);
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

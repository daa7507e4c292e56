// Router product in front of the top-k: logits[t][e] = x[t] . w[e] (+ bias[e]).
//
// The pages keep each layer's router on the GPU and route every token to the
// experts its router scores highest ("Strata - the details", "How it works";
// Strata README, "How does it work?"). The router matrix is bf16 [E][H] (row e
// belongs to expert e); x is f32 or bf16 [T][H]; logits are f32 [T][E]. Every
// product of two bf16 values is exact in f32; sums are f32 in a fixed order,
// so the logits are reproducible run to run.
//
//   router_dot  (few tokens, or f32 x): one wave per (expert, 4-token block);
//               the tokens' rows in LDS, lanes split H in 4-element chunks, a
//               fixed-order DPP sum. Bound: reading the router (2 MB at H
//               2048, E 512) and its latency.
//   router_mfma (bf16 x, many tokens, E a multiple of 128): 128-token x
//               128-expert tiles on v_mfma_f32_32x32x16_bf16, K in stages of
//               64 through LDS (rows XOR-swizzled by 16-byte chunk), loads two
//               stages ahead. Bound: MFMA.
#include "common.h"
#include "gemv.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kDotTok = 4;   // tokens per router_dot workgroup
constexpr int kDotMaxH = 4096;

// One workgroup per (4 experts, 4 tokens): the tokens' rows go to LDS once
// (f32 for either input dtype), each wave streams one expert row with all of
// its loads in flight, and lanes split H in 4-element chunks.
template <bool XF32>
__global__ __launch_bounds__(256) void router_dot(const void* __restrict__ x, int T, int H,
                                                  const uint16_t* __restrict__ w,
                                                  const float* __restrict__ bias, int E,
                                                  float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float xs[kDotTok * kDotMaxH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = min(blockIdx.x * 4 + wave, E - 1);  // clamped waves compute, never store
  const int t0 = blockIdx.y * kDotTok;
  const int n4 = H / 256;  // 4-element chunks per lane
  const uint2* wr = reinterpret_cast<const uint2*>(w + (size_t)e * H);
  constexpr int kMaxN4 = kDotMaxH / 256;
  uint2 wv[kMaxN4];
#pragma unroll
  for (int i = 0; i < kMaxN4; ++i)
    if (i < n4) wv[i] = wr[lane + 64 * i];
  for (int c = tid; c < kDotTok * H / 4; c += 256) {  // rows past T repeat the last row
    const int j = c / (H / 4), q = c % (H / 4);
    const int t = min(t0 + j, T - 1);
    float4 f;
    if (XF32) {
      f = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * H)[q];
    } else {
      const uint2 u = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)t * H)[q];
      f = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    reinterpret_cast<float4*>(xs)[c] = f;
  }
  __syncthreads();
  float acc[kDotTok] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMaxN4; ++i) {
    if (i < n4) {
      const float w0 = bf16_lo(wv[i].x), w1 = bf16_hi(wv[i].x), w2 = bf16_lo(wv[i].y), w3 = bf16_hi(wv[i].y);
#pragma unroll
      for (int j = 0; j < kDotTok; ++j) {
        const float4 f = reinterpret_cast<const float4*>(xs + j * H)[lane + 64 * i];
        acc[j] = fmaf(f.w, w3, fmaf(f.z, w2, fmaf(f.y, w1, fmaf(f.x, w0, acc[j]))));
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int j = 0; j < kDotTok; ++j) {
    const float s = wave_sum(acc[j]);
    if (lane == 0 && t0 + j < T && blockIdx.x * 4 + wave < E) logits[(size_t)(t0 + j) * E + e] = s + b;
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kRT = 128;  // tokens per tile
constexpr int kRE = 128;  // experts per tile
constexpr int kRK = 64;   // K per stage (8 chunks of 16 bytes per row)
constexpr int kRThreads = 512;

// Tile rows (token or expert) of 128 bytes; chunk q of row m at q ^ (m & 7).
__device__ inline int swz(int m, int q) { return m * 8 + (q ^ (m & 7)); }

// 8 waves: wave w owns tokens 32 (w % 4) .. + 31 and experts 64 (w / 4) .. + 63
// of the tile (two 32 x 32 accumulators). Stage loads run two stages ahead in
// registers (two sets, alternating), LDS is double-buffered, one barrier per
// stage.
__global__ __launch_bounds__(kRThreads) void router_mfma(const uint16_t* __restrict__ x, int T,
                                                         int H, const uint16_t* __restrict__ w,
                                                         const float* __restrict__ bias, int E,
                                                         float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint4 xs[2][kRT * 8];
  __shared__ __attribute__((aligned(16))) uint4 ws[2][kRE * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tt = blockIdx.x * kRT, ee = blockIdx.y * kRE;
  const int wm = wave & 3, wn = wave >> 2;
  const int S = H / kRK;
  // chunk c = tid + 512 u (u = 0, 1) of each operand -> row c / 8, chunk c % 8.
  // Two register sets of named variables, even stages in the a set and odd
  // stages in the b set (arrays or structs of them end up in scratch memory).
  const int m0 = tid >> 3, m1 = (tid + kRThreads) >> 3, q = tid & 7;
  const uint4* xr0 = reinterpret_cast<const uint4*>(x + (size_t)min(tt + m0, T - 1) * H) + q;
  const uint4* xr1 = reinterpret_cast<const uint4*>(x + (size_t)min(tt + m1, T - 1) * H) + q;
  const uint4* wr0 = reinterpret_cast<const uint4*>(w + (size_t)(ee + m0) * H) + q;
  const uint4* wr1 = reinterpret_cast<const uint4*>(w + (size_t)(ee + m1) * H) + q;
  const int s0 = swz(m0, q), s1 = swz(m1, q);
  constexpr int kStep = kRK / 8;  // uint4 per row per stage
  uint4 ax0, ax1, aw0, aw1, bx0, bx1, bw0, bw1;
  floatx16_t acc0 = {}, acc1 = {};  // experts 64 wn + 0..31, 64 wn + 32..63
  const int am = 32 * wm + (lane & 31), h = lane >> 5;
  const int bn0 = 64 * wn + (lane & 31), bn1 = bn0 + 32;
  auto compute = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {  // K 16 kk .. 16 kk + 15: lane half h takes chunk 2 kk + h
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xs[b][swz(am, 2 * kk + h)]);
      const bf16x8_t v0 = __builtin_bit_cast(bf16x8_t, ws[b][swz(bn0, 2 * kk + h)]);
      const bf16x8_t v1 = __builtin_bit_cast(bf16x8_t, ws[b][swz(bn1, 2 * kk + h)]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v1, acc1, 0, 0, 0);
    }
  };
#define ROUTER_LOAD(P, st) \
  P##x0 = xr0[(st) * kStep]; P##x1 = xr1[(st) * kStep]; P##w0 = wr0[(st) * kStep]; P##w1 = wr1[(st) * kStep];
#define ROUTER_STORE(P, b) \
  xs[b][s0] = P##x0; xs[b][s1] = P##x1; ws[b][s0] = P##w0; ws[b][s1] = P##w1;
  ROUTER_LOAD(a, 0)
  if (S > 1) { ROUTER_LOAD(b, 1) }
  ROUTER_STORE(a, 0)
  __syncthreads();
  for (int s = 0; s < S; s += 2) {
    // even stage s: buffer 0; the a set is free for stage s + 2
    if (s + 2 < S) { ROUTER_LOAD(a, s + 2) }
    compute(0);
    if (s + 1 < S) {
      ROUTER_STORE(b, 1)
      __syncthreads();
      // odd stage s + 1: buffer 1; the b set is free for stage s + 3
      if (s + 3 < S) { ROUTER_LOAD(b, s + 3) }
      compute(1);
      if (s + 2 < S) {
        ROUTER_STORE(a, 0)
        __syncthreads();
      }
    }
  }
#undef ROUTER_LOAD
#undef ROUTER_STORE
  // acc0/acc1[v]: token 8 (v / 4) + 4 h + v % 4 of the wave's 32, expert lane % 32 of its block
  const int e0 = ee + bn0, e1 = ee + bn1;
  const float b0 = bias ? bias[e0] : 0.f, b1 = bias ? bias[e1] : 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = tt + 32 * wm + 8 * (v >> 2) + 4 * h + (v & 3);
    if (t < T) {
      logits[(size_t)t * E + e0] = acc0[v] + b0;
      logits[(size_t)t * E + e1] = acc1[v] + b1;
    }
  }
}

// Router product and top-k in one launch (bf16 x, E = 256 NT): workgroup b
// takes tokens 32 b .. 32 b + 31 against every expert, so the selection of
// each of its tokens needs no other workgroup. K runs in stages of 32: the
// stage's router rows (E x 64 bytes) and token rows (32 x 64 bytes) come into
// LDS by direct global-to-LDS loads (each wave instruction fills 16 whole
// rows), four buffers with three stages in flight ahead of the one computed
// (a stage's loads take longer than its products), the 16-byte piece p of
// row r at position p ^ ((r >> 2) & 3) so that the 16 rows of a fragment
// read's lane group cover the 64 banks once. Wave w computes experts 32 NT w .. + 32 NT - 1 on
// v_mfma_f32_32x32x16_bf16 (router rows as A, tokens as B). Then the tiles go
// to LDS (rows padded to E + 1 floats: the 32 token columns of a write fall
// on different banks) and each wave selects for four tokens: bias added, the
// logits written out (coalesced) when asked for, top-k and gates as topk.h.
constexpr int kRtTok = 32;     // tokens per workgroup
constexpr int kRtKS = 32;      // K per stage (64 bytes per row)
constexpr int kRtThreads = 512;

__device__ inline int rt_pos(int r, int p) { return 4 * r + (p ^ ((r >> 2) & 3)); }  // 16-byte units

// The four stages' buffers are separate LDS arrays, and the loop is unrolled
// by four so that each step names its arrays: a read of one buffer then need
// wait only for that buffer's loads (the compiler still adds a full wait in
// some steps). Measured at 8,192 tokens: 65 us against 38 us for router_mfma
// followed by topk_kernel, which the layer calls use (every workgroup here
// reads the whole router matrix: four times the cache traffic).
template <int NT>
__global__ __launch_bounds__(kRtThreads) void router_topk(const uint16_t* __restrict__ x, int T, int H,
                                                          const uint16_t* __restrict__ w,
                                                          const float* __restrict__ bias, int E, int k,
                                                          float* __restrict__ logits, int32_t* __restrict__ idx,
                                                          float* __restrict__ gates) {
  constexpr int kE = 256 * NT;
  constexpr int kWStage = kE * 4;          // 16-byte units of a router stage
  constexpr int kXStage = kRtTok * 4;      // of a token stage
  constexpr int kHalf = (kRtTok / 2) * (kE + 1);  // floats of half the logits tile
  constexpr int kWUnits = (kHalf * 4 > kWStage * 16) ? (kHalf + 3) / 4 : kWStage;
  __shared__ __attribute__((aligned(16))) uint4 w0[kWUnits], w1[kWUnits], w2[kWStage], w3[kWStage];
  __shared__ __attribute__((aligned(16))) uint4 x0[kXStage], x1[kXStage], x2[kXStage], x3[kXStage];
  __shared__ TopkScratch tks[kRtThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int t0 = blockIdx.x * kRtTok;
  const int S = H / kRtKS;  // a multiple of 8 (H % 256 == 0)
  // loads: LDS unit u = position of (row r, piece p); the lane that fills unit
  // u reads the global piece that belongs there
  auto fill = [&](int s, uint4* ws, uint4* xs) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < kWStage / kRtThreads; ++v) {
      const int u0 = v * kRtThreads + 64 * wave;  // the wave's 64 consecutive units
      const int u = u0 + lane, r = u >> 2, pos = u & 3, p = pos ^ ((r >> 2) & 3);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(w + (size_t)r * H + kRtKS * s) + p,
                                       (__attribute__((address_space(3))) void*)(ws + u0), 16, 0, 0);
    }
    if (wave < kXStage / 64) {
      const int u0 = 64 * wave;
      const int u = u0 + lane, r = u >> 2, pos = u & 3, p = pos ^ ((r >> 2) & 3);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const uint4*>(x + (size_t)min(t0 + r, T - 1) * H + kRtKS * s) + p,
          (__attribute__((address_space(3))) void*)(xs + u0), 16, 0, 0);
    }
  };
  floatx16_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = floatx16_t{};
  auto compute = [&](const uint4* ws, const uint4* xs) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {  // 16 K each: lane half h takes piece 2 kk + h
      const bf16x8_t xv = __builtin_bit_cast(bf16x8_t, xs[rt_pos(i, 2 * kk + h)]);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int r = 32 * (NT * wave + j) + i;
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ws[rt_pos(r, 2 * kk + h)]),
                                                         xv, acc[j], 0, 0, 0);
      }
    }
  };
  // loads per stage and wave: 2 NT router pieces, plus one token piece for
  // the first two waves; a step waits until at most the two later stages'
  // loads are outstanding (vmcnt counts this wave's loads in order), except
  // near the end, where fewer are
  static_assert(kWStage / kRtThreads == 2 * NT && kXStage / 64 == 2, "stage load counts");
  const bool xw = wave < 2;
  auto wait_for = [&](int s) __attribute__((always_inline)) {
    if (s + 2 < S) {
      if (NT == 2) { if (xw) __builtin_amdgcn_s_waitcnt(0x0F70 | 10); else __builtin_amdgcn_s_waitcnt(0x0F70 | 8); }
      else { if (xw) __builtin_amdgcn_s_waitcnt(0x0F70 | 6); else __builtin_amdgcn_s_waitcnt(0x0F70 | 4); }
    } else if (s + 1 < S) {
      if (NT == 2) { if (xw) __builtin_amdgcn_s_waitcnt(0x0F70 | 5); else __builtin_amdgcn_s_waitcnt(0x0F70 | 4); }
      else { if (xw) __builtin_amdgcn_s_waitcnt(0x0F70 | 3); else __builtin_amdgcn_s_waitcnt(0x0F70 | 2); }
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    // every wave's pieces of stage s are in; the buffer refilled next was last
    // read in the previous step. A plain s_barrier: __syncthreads()'s fence
    // would wait for every load in flight, the later stages' too (the memory
    // clobber keeps the compiler from moving LDS reads across it)
    asm volatile("s_barrier" ::: "memory");
  };
  fill(0, w0, x0);
  fill(1, w1, x1);
  fill(2, w2, x2);
  for (int s = 0; s < S; s += 4) {
    wait_for(s);
    if (s + 3 < S) fill(s + 3, w3, x3);
    compute(w0, x0);
    wait_for(s + 1);
    if (s + 4 < S) fill(s + 4, w0, x0);
    compute(w1, x1);
    wait_for(s + 2);
    if (s + 5 < S) fill(s + 5, w1, x1);
    compute(w2, x2);
    wait_for(s + 3);
    if (s + 6 < S) fill(s + 6, w2, x2);
    compute(w3, x3);
  }
  __syncthreads();  // every wave is done with the stages: w0, w1 take the logits tile
  // acc[j][v]: expert 32 (NT wave + j) + 8 (v / 4) + 4 h + v % 4, token i
  float* lt = reinterpret_cast<float*>(i < 16 ? w0 : w1) + (i & 15) * (kE + 1);
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) lt[32 * (NT * wave + j) + 8 * (v >> 2) + 4 * h + (v & 3)] = acc[j][v];
  __syncthreads();
  constexpr int kPer = kE / 64;
#pragma unroll 1
  for (int u = 0; u < kRtTok / (kRtThreads / 64); ++u) {
    const int tl = wave * (kRtTok / (kRtThreads / 64)) + u, t = t0 + tl;
    if (t >= T) break;
    const float* row = reinterpret_cast<const float*>(tl < 16 ? w0 : w1) + (tl & 15) * (kE + 1);
    float raw[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = lane + 64 * q;
      raw[q] = e < E ? row[e] + (bias ? bias[e] : 0.f) : 0.f;
      if (logits && e < E) logits[(size_t)t * E + e] = raw[q];
    }
    topk_select<kPer>(raw, E, k, idx + (size_t)t * k, gates + (size_t)t * k, &tks[wave]);
  }
}

}  // namespace

bool router_topk_supported(int xdtype, int H, int E, int k) {
  return xdtype != 0 && H % 256 == 0 && H <= kDotMaxH && (E == 256 || E == 512) && k >= 1 && k <= 64;
}

hipError_t launch_router_topk(const void* x, int T, int H, const uint16_t* w, const float* bias, int E,
                              int k, float* logits, int32_t* idx, float* gates, hipStream_t s) {
  const dim3 grid((T + kRtTok - 1) / kRtTok);
  if (E == 512)
    MOE_LAUNCH("router_topk", s, router_topk<2>, grid, dim3(kRtThreads), 0, s,
               static_cast<const uint16_t*>(x), T, H, w, bias, E, k, logits, idx, gates);
  else
    MOE_LAUNCH("router_topk", s, router_topk<1>, grid, dim3(kRtThreads), 0, s,
               static_cast<const uint16_t*>(x), T, H, w, bias, E, k, logits, idx, gates);
  return hipGetLastError();
}

bool router_supported(int H, int E) { return H >= 256 && H % 256 == 0 && H <= kDotMaxH && E >= 1; }

hipError_t launch_router(const void* x, int xdtype, int T, int H, const uint16_t* w,
                         const float* bias, int E, float* logits, hipStream_t s) {
  if (xdtype != 0 && T >= kRouterMfmaMinT && E % kRE == 0) {
    MOE_LAUNCH("router_mfma", s, router_mfma, dim3((T + kRT - 1) / kRT, E / kRE), dim3(kRThreads), 0, s,
               static_cast<const uint16_t*>(x), T, H, w, bias, E, logits);
  } else {
    const dim3 grid((E + 3) / 4, (T + kDotTok - 1) / kDotTok);
    if (xdtype == 0)
      MOE_LAUNCH("router_dot", s, router_dot<true>, grid, dim3(256), 0, s, x, T, H, w, bias, E, logits);
    else
      MOE_LAUNCH("router_dot", s, router_dot<false>, grid, dim3(256), 0, s, x, T, H, w, bias, E, logits);
  }
  return hipGetLastError();
}

}  // namespace moe

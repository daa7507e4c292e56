// Per-token top-k selection with softmax gates on one 64-wide wavefront
// (header-only; used by the top-k kernel and the fused route + group kernel).
//
// The router scores every expert of the layer for each token and keeps the 10
// best of 512 ("Strata - the details", "How it works"; the Strata README,
// "How does it work?"). Each lane holds ceil(E/64) logits, expert lane + 64*i
// in slot i, as order-preserving 32-bit codes. A round finds the largest code
// with a DPP max over the wave, then the lowest expert index holding it with a
// DPP min (ties go to the lower index); the owning lane retires that slot.
#pragma once

#include "common.h"

namespace moe {

// Monotone map float -> uint32: larger float, larger code. -0 folds to +0 so
// the two tie; NaN maps to 1 (below -inf, whose code is 0x007FFFFF); 0 marks a
// retired or padding slot.
__device__ inline uint32_t orderable(float v) {
  if (v != v) return 1u;
  const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float from_orderable(uint32_t o) {
  if (o <= 1u) return __uint_as_float(0x7FC00000u);
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ inline uint32_t dpp(uint32_t v, int ctrl) {
  switch (ctrl) {  // the control word must be a compile-time constant
    case 0xB1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
    case 0x4E: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
    case 0x141: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
  }
}

// Max (or min) over the 64 lanes, returned in every lane: quad swaps, half-row
// and row mirrors reduce each 16-lane row; four lane reads combine the rows.
template <bool MAX>
__device__ inline uint32_t wave_reduce(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, dpp(v, 0xB1));   // quad_perm [1,0,3,2]
  v = op(v, dpp(v, 0x4E));   // quad_perm [2,3,0,1]
  v = op(v, dpp(v, 0x141));  // row_half_mirror
  v = op(v, dpp(v, 0x140));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// Sum over the 64 lanes in a fixed order, returned in every lane (DPP within
// each 16-lane row, then the four row sums in lane order).
__device__ inline float wave_sum(float v) {
  v += __uint_as_float(dpp(__float_as_uint(v), 0xB1));
  v += __uint_as_float(dpp(__float_as_uint(v), 0x4E));
  v += __uint_as_float(dpp(__float_as_uint(v), 0x141));
  v += __uint_as_float(dpp(__float_as_uint(v), 0x140));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// LDS scratch of one wave for topk_token.
struct alignas(16) TopkScratch {
  uint32_t head[64];  // every lane's best code
  uint64_t cand[64];  // compacted candidates: code << 32 | (~expert)
};

// Selects the k best experts of logits row l (E entries) into idx_t[0..k) in
// rank order and their gates into g_t[0..k); also into lds_idx when not null.
// Every lane of the wave calls it; sc is this wave's own LDS scratch.
//
// Threshold pass (k <= 64): the k-th largest of the 64 lane maxima, tau, is at
// most the k-th largest code overall (k distinct experts reach it), so every
// selected expert has a code >= tau, and few others do. Those candidates are
// compacted into LDS; each ranks itself by counting the candidates that beat
// it (larger code, or equal code and lower index), and rank r < k lands in
// slot r. When more than 64 codes reach tau (heavy ties), or k > 64, rounds
// take over: each finds the largest remaining code with a DPP max and the
// lowest index holding it, and retires it.
//
// topk_load fetches a row (lane + 64 i for slot i, all loads back to back,
// clamped address, no branch, so their latencies overlap); topk_select works
// on a fetched row, so a caller can have several rows in flight at once.
template <int PER_LANE>
__device__ inline void topk_load(const float* __restrict__ l, int E, float (&raw)[PER_LANE]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) raw[i] = l[min(lane + 64 * i, E - 1)];
}

template <int PER_LANE>
__device__ inline void topk_select(const float (&raw)[PER_LANE], int E, int k, int32_t* idx_t,
                                   float* g_t, TopkScratch* sc, int32_t* lds_idx = nullptr) {
  const int lane = threadIdx.x & 63;
  // padding slots get code 0
  uint32_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) key[i] = lane + 64 * i < E ? orderable(raw[i]) : 0u;

  if (k <= 64) {
    uint32_t head = key[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) head = key[i] > head ? key[i] : head;
    sc->head[lane] = head;
    sc->cand[lane] = 0ull;  // padding for the unrolled rank loop: beats nothing
    __builtin_amdgcn_wave_barrier();
    int gt = 0;
    const uint4* h4 = reinterpret_cast<const uint4*>(sc->head);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 h = h4[j];
      gt += (h.x > head) + (h.y > head) + (h.z > head) + (h.w > head);
    }
    const uint32_t tau = wave_reduce<false>(gt < k ? head : 0xFFFFFFFFu);
    int n = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) n += __popcll(__ballot(key[i] >= tau));
    if (n <= 64) {
      int base = 0;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const bool c = key[i] >= tau;
        const uint64_t m = __ballot(c);
        if (c)
          sc->cand[base + __popcll(m & lanemask_lt())] =
              ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(lane + 64 * i);
        base += __popcll(m);
      }
      __builtin_amdgcn_wave_barrier();
      const uint64_t mine = sc->cand[lane];
      int rank = 0;
      const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(sc->cand);
      for (int c = 0; c < n; c += 4) {
        const ulonglong2 a = c2[c >> 1], b = c2[(c >> 1) + 1];
        rank += (a.x > mine) + (a.y > mine) + (b.x > mine) + (b.y > mine);
      }
      const bool sel = lane < n && rank < k;
      const int e = (int)~(uint32_t)mine;
      const uint32_t code = (uint32_t)(mine >> 32);
      const uint64_t first = __ballot(lane < n && rank == 0);
      const float top =
          from_orderable(__builtin_amdgcn_readlane(code, __ffsll((unsigned long long)first) - 1));
      const float ej = sel ? expf(from_orderable(code) - top) : 0.f;
      const float sum = wave_sum(ej);
      if (sel) {
        idx_t[rank] = e;
        if (lds_idx) lds_idx[rank] = e;
        g_t[rank] = ej / sum;
      }
      __builtin_amdgcn_wave_barrier();  // scratch free for the wave's next call
      return;
    }
  }

  uint32_t my_v = 0u;  // code of the selected logit of rank `lane` (and lane + 64*r)
  for (int j = 0; j < k; ++j) {
    uint32_t bv = key[0];
    int bs = 0;
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i)
      if (key[i] > bv) {  // strict: the lower slot (lower index) keeps ties
        bv = key[i];
        bs = i;
      }
    const uint32_t wv = wave_reduce<true>(bv);
    const uint64_t holders = __ballot(bv == wv);
    int e;
    if (__popcll(holders) == 1) {
      const int src = __ffsll((unsigned long long)holders) - 1;
      e = src + 64 * __builtin_amdgcn_readlane(bs, src);
    } else {
      const uint32_t cand = bv == wv ? (uint32_t)(lane + 64 * bs) : 0xFFFFFFFFu;
      e = (int)wave_reduce<false>(cand);
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        if (i == (e >> 6)) key[i] = 0u;
    }
    if (lane == (j & 63)) {
      idx_t[j] = e;
      if (lds_idx) lds_idx[j] = e;
      if (j < 64) my_v = wv;
      else g_t[j] = from_orderable(wv);  // past 64 ranks: kept in memory by this lane
    }
  }
  // gates: softmax over the selected logits, relative to the largest
  const float top = from_orderable(__builtin_amdgcn_readlane(my_v, 0));
  const float ej = lane < k ? expf(from_orderable(my_v) - top) : 0.f;
  float sum = ej;
  for (int j = 64 + lane; j < k; j += 64) sum += expf(g_t[j] - top);  // k > 64 only
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane < k) g_t[lane] = ej / sum;
  for (int j = 64 + lane; j < k; j += 64) g_t[j] = expf(g_t[j] - top) / sum;
}

template <int PER_LANE>
__device__ inline void topk_token(const float* __restrict__ l, int E, int k, int32_t* idx_t,
                                  float* g_t, TopkScratch* sc, int32_t* lds_idx = nullptr) {
  float raw[PER_LANE];
  topk_load<PER_LANE>(l, E, raw);
  topk_select<PER_LANE>(raw, E, k, idx_t, g_t, sc, lds_idx);
}

}  // namespace moe

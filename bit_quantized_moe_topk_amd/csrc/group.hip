// Stable grouping of token-to-expert assignments by expert (counting sort).
//
// Prefill multiplies each expert once for all the tokens routed to it in a
// chunk ("Strata - the details", "Faster prompts"), which needs the chunk's
// assignments grouped by expert. The grouping here is a stable counting sort
// on the flat assignment id t*k + j:
//   1. every wave owns a segment of kSeg consecutive ids and counts its experts;
//   2. an exclusive scan over (expert, segment) in expert-major order gives each
//      segment the first output slot of each of its experts;
//   3. every wave walks its segment in id order, 64 ids at a time; lanes holding
//      the same expert find each other with one ballot per key bit, take ranks
//      by lane order, and the group's last lane advances the expert's counter.
// Order inside an expert is therefore ascending id, identical on every run.
// Small inputs run all three steps in one workgroup; large ones in 3 launches.
#include "common.h"
#include "batch_x.h"
#include "sched.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kSeg = 1024;  // assignment ids per wave segment

__device__ inline int key_bits(int E) { return E <= 1 ? 0 : 32 - __builtin_clz((unsigned)(E - 1)); }

// The expert ids of up to KB chunks of 64 consecutive assignment ids, loaded
// before any is used so that one memory round trip covers them all (ids past
// f1 read as -1). Large inputs take KB = 16; the one-workgroup kernels take
// fewer, since their code runs once per launch from a cold instruction cache
// and every unrolled chunk costs fetch time.
constexpr int kBatch = 16;
constexpr int kBatchSmall = 2;  // group_fused: ids come from global memory
template <int KB>
__device__ inline void load_chunks(const int32_t* __restrict__ idx, int base, int f1, int (&e)[KB]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < KB; ++u) {
    const int f = base + 64 * u + lane;
    e[u] = f < f1 ? idx[f] : -1;
  }
}

// Count the experts of ids [f0, f1) into hist[e * stride] (LDS, zeroed by caller).
template <int KB = kBatch>
__device__ inline void wave_count(const int32_t* __restrict__ idx, int f0, int f1, int E,
                                  int* hist, int stride) {
  for (int base = f0; base < f1; base += 64 * KB) {
    int ev[KB];
    load_chunks<KB>(idx, base, f1, ev);
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (ev[u] >= 0 && ev[u] < E) atomicAdd(&hist[ev[u] * stride], 1);
  }
}

// Stable scatter of ids [f0, f1) using the running counters cnt[e * stride].
template <int KB = kBatch>
__device__ inline void wave_scatter(const int32_t* __restrict__ idx, int f0, int f1, int E,
                                    int* cnt, int stride, int32_t* __restrict__ perm,
                                    int32_t* __restrict__ slot_of) {
  const int lane = threadIdx.x & 63;
  const int nbits = key_bits(E);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = f0; b0 < f1; b0 += 64 * KB) {
    int ev[KB];
    load_chunks<KB>(idx, b0, f1, ev);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int f = b0 + 64 * u + lane;
      const int e = ev[u];
      const bool ok = e >= 0 && e < E;
      uint64_t mask = __ballot(ok);
      if (mask == 0) continue;  // a chunk past the range: nothing to rank
      for (int b = 0; b < nbits; ++b) {
        const bool bit = ok && ((e >> b) & 1);
        const uint64_t bal = __ballot(bit);
        mask &= bit ? bal : ~bal;
      }
      if (ok) {
        const int rank = __popcll(mask & below);
        const int n = __popcll(mask);
        const int pos = cnt[e * stride] + rank;
        perm[pos] = f;
        slot_of[f] = pos;
        if (rank == n - 1) cnt[e * stride] = pos + 1;
      }
    }
  }
}

__device__ inline void write_offsets(const int* base, int nseg, int E, int T, int k, int has_shared,
                                     int32_t* counts, int32_t* offsets) {
  const int AR = T * k;
  for (int e = threadIdx.x; e <= E + 1; e += blockDim.x) {
    if (e < E) offsets[e] = base[e * nseg];
    else if (e == E) offsets[E] = AR;
    else offsets[E + 1] = AR + (has_shared ? T : 0);
  }
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    if (e < E) counts[e] = (e + 1 < E ? base[(e + 1) * nseg] : AR) - base[e * nseg];
    else counts[E] = has_shared ? T : 0;
  }
}

// Identity slots of the shared expert, tokens t0, t0 + ts, ... (the caller's
// threads split them).
__device__ inline void write_shared(int T, int k, int has_shared, int32_t* perm, int32_t* slot_of,
                                    int t0, int ts) {
  if (!has_shared) return;
  const int AR = T * k;
  for (int t = t0; t < T; t += ts) {
    perm[AR + t] = AR + t;
    slot_of[AR + t] = AR + t;
  }
}

// All three steps in one workgroup: one wave per segment of seg_len ids
// (nseg <= 16 segments; lds holds E * nseg + 16 ints).
__device__ inline void group_one_wg(const int32_t* __restrict__ idx, int T, int k, int E, int has_shared,
                                    int nseg, int seg_len, int32_t* counts, int32_t* offsets,
                                    int32_t* perm, int32_t* slot_of, int* lds) {
  int* hist = lds;
  int* tmp = lds + E * nseg;
  const int AR = T * k;
  for (int i = threadIdx.x; i < E * nseg; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int seg = threadIdx.x >> 6;
  const int f0 = min(AR, seg * seg_len), f1 = min(AR, f0 + seg_len);
  if (seg < nseg) wave_count<kBatchSmall>(idx, f0, f1, E, hist + seg, nseg);
  __syncthreads();
  block_exclusive_scan(hist, E * nseg, tmp);
  write_offsets(hist, nseg, E, T, k, has_shared, counts, offsets);
  __syncthreads();  // the bases are read above before the scatter advances them
  if (seg < nseg) wave_scatter<kBatchSmall>(idx, f0, f1, E, hist + seg, nseg, perm, slot_of);
  write_shared(T, k, has_shared, perm, slot_of, threadIdx.x, blockDim.x);
}

// group_one_wg in the first workgroup; workgroups past the first, when the
// launch has them, write the small-batch activation layout (xj) meanwhile.
__global__ __launch_bounds__(1024) void group_fused(const int32_t* __restrict__ idx, int T, int k,
                                                    int E, int has_shared, int nseg, int seg_len,
                                                    int32_t* counts, int32_t* offsets,
                                                    int32_t* perm, int32_t* slot_of, XsJob xj) {
  if (blockIdx.x > 0) {
    const int wpb = blockDim.x >> 6;
    xs_write_rows(xj, (blockIdx.x - 1) * wpb + (threadIdx.x >> 6), (gridDim.x - 1) * wpb);
    return;
  }
  extern __shared__ int lds[];  // [E * nseg] bases, then [16] wave totals
  group_one_wg(idx, T, k, E, has_shared, nseg, seg_len, counts, offsets, perm, slot_of, lds);
}

// Top-k and grouping in one workgroup for small batches (a decode verify
// window, a few of them batched): every wave selects experts for its tokens
// into global memory and into LDS, then the workgroup groups the LDS copy as
// group_fused does, one wave per segment of seg_len ids.
template <int PER_LANE>
__global__ __launch_bounds__(1024) void route_group_small(const float* __restrict__ logits, int T,
                                                          int E, int k, int has_shared, int nseg,
                                                          int seg_len, int32_t* idx, float* gates,
                                                          int32_t* counts, int32_t* offsets,
                                                          int32_t* perm, int32_t* slot_of) {
  extern __shared__ int lds[];  // [T*k] expert ids, [E * nseg] bases, [16] wave totals
  __shared__ TopkScratch sc[16];
  int* lidx = lds;
  int* hist = lds + T * k;
  int* wsum = hist + E * nseg;
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int t = wv; t < T; t += nw)
    topk_token<PER_LANE>(logits + (size_t)t * E, E, k, idx + (size_t)t * k, gates + (size_t)t * k,
                         &sc[wv], lidx + t * k);
  for (int i = threadIdx.x; i < E * nseg; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int AR = T * k;
  const int f0 = min(AR, wv * seg_len), f1 = min(AR, f0 + seg_len);
  if (wv < nseg) wave_count<1>(lidx, f0, f1, E, hist + wv, nseg);
  __syncthreads();
  block_exclusive_scan(hist, E * nseg, wsum);
  write_offsets(hist, nseg, E, T, k, has_shared, counts, offsets);
  __syncthreads();  // the bases are read above before the scatter advances them
  if (wv < nseg) wave_scatter<1>(lidx, f0, f1, E, hist + wv, nseg, perm, slot_of);
  write_shared(T, k, has_shared, perm, slot_of, threadIdx.x, blockDim.x);
}

// Large inputs, step 1: per-segment counts into hist[seg * E + e] (global,
// segment-major so that every step's accesses are coalesced).
// Workgroups from nb on write the activation copy (xj) meanwhile.
__global__ __launch_bounds__(256) void group_count(const int32_t* __restrict__ idx, int T, int k,
                                                   int E, int has_shared, int nseg, int* hist,
                                                   int32_t* perm, int32_t* slot_of, int nb, XsJob xj) {
  if ((int)blockIdx.x >= nb) {
    xs_write_rows(xj, (blockIdx.x - nb) * 4 + (threadIdx.x >> 6), (gridDim.x - nb) * 4);
    return;
  }
  extern __shared__ int lds[];  // [4][E]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* h = lds + w * E;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  const int AR = T * k;
  const int seg = blockIdx.x * 4 + w;
  if (seg < nseg) {
    const int f0 = seg * kSeg, f1 = min(AR, f0 + kSeg);
    wave_count(idx, f0, f1, E, h, 1);
  }
  __syncthreads();
  if (seg < nseg)
    for (int e = lane; e < E; e += 64) hist[(size_t)seg * E + e] = h[e];
  write_shared(T, k, has_shared, perm, slot_of, blockIdx.x * blockDim.x + threadIdx.x, nb * blockDim.x);
}

// Step 2: one workgroup turns hist into exclusive bases in (expert, segment)
// order. Two threads per expert take the first and second half of its
// segments (a segment's counts are adjacent, so the workgroup's loads
// coalesce), 16 loads in flight each; a block scan over the expert totals in
// LDS gives each expert's first slot, and each thread rewrites its half of
// the column as running bases.
__global__ __launch_bounds__(1024) void group_scan(int T, int k, int E, int has_shared, int nseg,
                                                   int* hist, int32_t* counts, int32_t* offsets) {
  __shared__ int tot[MOE_MAX_E_DEV + 1];
  __shared__ int part[2][MOE_MAX_E_DEV];  // per expert: the halves' sums
  __shared__ int wsum[16];
  const int tid = threadIdx.x, NT = blockDim.x;
  constexpr int U = 16;
  const int mid = nseg / 2;
  // half-column sums
  for (int i = tid; i < 2 * E; i += NT) {
    const int e = i % E, hf = i / E;
    const int s0 = hf ? mid : 0, s1 = hf ? nseg : mid;
    int sum = 0;
    for (int s = s0; s < s1; s += U) {  // every round a full batch of loads (the tail predicated)
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = s + u < s1 ? hist[(size_t)(s + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) sum += v[u];
    }
    part[hf][e] = sum;
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) tot[e] = part[0][e] + part[1][e];
  __syncthreads();
  block_exclusive_scan(tot, E, wsum);
  const int AR = T * k;
  for (int e = tid; e <= E + 1; e += NT) {
    if (e < E) offsets[e] = tot[e];
    else if (e == E) offsets[E] = AR;
    else offsets[E + 1] = AR + (has_shared ? T : 0);
  }
  for (int e = tid; e <= E; e += NT) {
    if (e < E) counts[e] = (e + 1 < E ? tot[e + 1] : AR) - tot[e];
    else counts[E] = has_shared ? T : 0;
  }
  // running bases: the second half starts after the first half's sum
  for (int i = tid; i < 2 * E; i += NT) {
    const int e = i % E, hf = i / E;
    const int s0 = hf ? mid : 0, s1 = hf ? nseg : mid;
    int run = tot[e] + (hf ? part[0][e] : 0);
    for (int s = s0; s < s1; s += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = s + u < s1 ? hist[(size_t)(s + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s + u < s1) hist[(size_t)(s + u) * E + e] = run;
        run += v[u];
      }
    }
  }
}

// Step 3: per-segment stable scatter from the scanned bases. One workgroup
// per segment; its four waves take consecutive quarters of the segment, count
// their experts, and start from the segment's base plus the earlier quarters'
// counts, so the order stays ascending within every expert.
__global__ __launch_bounds__(256) void group_scatter(const int32_t* __restrict__ idx, int T, int k,
                                                     int E, int nseg, const int* hist,
                                                     int32_t* perm, int32_t* slot_of) {
  extern __shared__ int lds[];  // [4][E] quarter counts, then bases
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = blockIdx.x;
  const int AR = T * k;
  const int f0 = seg * kSeg, f1 = min(AR, f0 + kSeg);
  const int g0 = min(f1, f0 + w * (kSeg / 4)), g1 = min(f1, g0 + kSeg / 4);
  int* cnt = lds + w * E;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  wave_count<kSeg / 256>(idx, g0, g1, E, cnt, 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = hist[(size_t)seg * E + e];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lds[q * E + e];
      lds[q * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  wave_scatter<kSeg / 256>(idx, g0, g1, E, cnt, 1, perm, slot_of);
}

inline int nseg_of(int T, int k) { return (T * k + kSeg - 1) / kSeg; }
// One workgroup when its LDS (bases + wave totals) stays within 64 KiB.
inline bool use_fused(int T, int k, int E) {
  const int n = nseg_of(T, k);
  return n <= 16 && (size_t)E * n + 16 <= 16384;
}

// One token per wave (at most 16): past that, the top-k kernel (a wave per
// token over many workgroups) and group_fused take less time than waves
// selecting several tokens in turn.
inline bool small_route_group(int T, int k, int E) {
  return T <= 16 && T * k <= kSeg &&
         (size_t)(T * k + E + 16) * sizeof(int) + 16 * sizeof(TopkScratch) <= 65536;
}

// Segments for a one-workgroup grouping of A ids: as many as there are waves
// (at most max_seg), of a multiple of 64 ids each, while E ints of bases per
// segment fit in lds_ints; returns the segment count and sets seg_len.
inline int small_segments(int A, int E, int max_seg, size_t lds_ints, int& seg_len) {
  int n = (A + 63) / 64;
  if (n > max_seg) n = max_seg;
  while (n > 1 && (size_t)E * n > lds_ints) --n;
  if (n < 1) n = 1;
  seg_len = ((A + n - 1) / n + 63) / 64 * 64;
  if (seg_len < 64) seg_len = 64;
  return (A + seg_len - 1) / seg_len;
}

template <int P>
hipError_t launch_rg(const float* logits, int T, int E, int k, int has_shared, int32_t* idx,
                     float* gates, int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* slot_of, hipStream_t s) {
  const int waves = T < 16 ? T : 16;
  const size_t budget = (65536 - 16 * sizeof(TopkScratch)) / sizeof(int) - (size_t)T * k - 16;
  int seg_len = 64;
  const int nseg = small_segments(T * k, E, waves, budget, seg_len);
  const size_t lds = ((size_t)T * k + (size_t)E * nseg + 16) * sizeof(int);
  MOE_LAUNCH("route_group", s, route_group_small<P>, dim3(1), dim3(64 * waves), lds, s, logits, T,
             E, k, has_shared, nseg, seg_len, idx, gates, counts, offsets, perm, slot_of);
  return hipGetLastError();
}

}  // namespace

size_t group_scratch_bytes(int T, int k, int E) {
  if (use_fused(T, k, E)) return 0;
  return (size_t)E * nseg_of(T, k) * sizeof(int);
}

hipError_t launch_group(const int32_t* idx, int T, int k, int E, int has_shared, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* slot_of, void* scratch,
                        hipStream_t s, const XsJob* xj, bool* xs_done) {
  const int nseg = nseg_of(T, k);
  if (xs_done) *xs_done = false;
  if (use_fused(T, k, E)) {
    int seg_len = kSeg;
    const int nf = small_segments(T * k, E, 16, 16384 - 16, seg_len);
    const size_t lds = ((size_t)E * nf + 16) * sizeof(int);
    const int threads = 64 * (nf > 0 ? nf : 1);
    XsJob job{};
    int grid = 1;
    if (xj && xj->xs && xj->T > 0) {
      job = *xj;
      const long g = (xj->T + threads / 64 - 1) / (threads / 64);  // a wave per token row
      grid = 1 + (int)(g < 256 ? g : 256);
      if (xs_done) *xs_done = true;
    }
    MOE_LAUNCH("group_fused", s, group_fused, dim3(grid), dim3(threads), lds, s, idx, T, k, E, has_shared, nf,
               seg_len, counts, offsets, perm, slot_of, job);
    return hipGetLastError();
  }
  int* hist = static_cast<int*>(scratch);
  const int blocks = (nseg + 3) / 4;
  const size_t lds = (size_t)4 * E * sizeof(int);
  XsJob job{};
  int grid = blocks;
  if (xj && xj->xs && xj->T > 0) {
    job = *xj;
    const long g = (xj->T + 3) / 4;  // a wave per token row
    grid += (int)(g < 1024 ? g : 1024);
    if (xs_done) *xs_done = true;
  }
  MOE_LAUNCH("group_count", s, group_count, dim3(grid), dim3(256), lds, s, idx, T, k, E, has_shared, nseg,
                     hist, perm, slot_of, blocks, job);
  MOE_LAUNCH("group_scan", s, group_scan, dim3(1), dim3(1024), 0, s, T, k, E, has_shared, nseg, hist,
                     counts, offsets);
  MOE_LAUNCH("group_scatter", s, group_scatter, dim3(nseg), dim3(256), lds, s, idx, T, k, E, nseg, hist,
                     perm, slot_of);
  return hipGetLastError();
}

hipError_t launch_route_group(const float* logits, int T, int E, int k, int has_shared, int32_t* idx,
                              float* gates, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* slot_of, void* scratch, hipStream_t s, const XsJob* xj,
                              bool* xs_done) {
  if (xs_done) *xs_done = false;
  if (small_route_group(T, k, E)) {
    const int per = (E + 63) / 64;
    if (per <= 1) return launch_rg<1>(logits, T, E, k, has_shared, idx, gates, counts, offsets, perm, slot_of, s);
    if (per <= 2) return launch_rg<2>(logits, T, E, k, has_shared, idx, gates, counts, offsets, perm, slot_of, s);
    if (per <= 4) return launch_rg<4>(logits, T, E, k, has_shared, idx, gates, counts, offsets, perm, slot_of, s);
    if (per <= 8) return launch_rg<8>(logits, T, E, k, has_shared, idx, gates, counts, offsets, perm, slot_of, s);
    if (per <= 16) return launch_rg<16>(logits, T, E, k, has_shared, idx, gates, counts, offsets, perm, slot_of, s);
    return launch_rg<32>(logits, T, E, k, has_shared, idx, gates, counts, offsets, perm, slot_of, s);
  }
  hipError_t e = launch_topk(logits, T, E, k, idx, gates, s);
  if (e != hipSuccess) return e;
  return launch_group(idx, T, k, E, has_shared, counts, offsets, perm, slot_of, scratch, s, xj, xs_done);
}

}  // namespace moe

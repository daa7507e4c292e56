// Device-side work map for the FFN kernels (header-only).
//
// There is no scheduler kernel and no host round trip: every workgroup loads
// the grouping's per-expert counts into LDS once, turns them into two prefix
// sums, and maps each of its item numbers to work by binary search:
//   GEMV experts: 1 .. gmax assignments, one unit per expert;
//   MFMA tiles  : experts with more than gmax assignments, ceil(M / tile_m)
//                 token tiles each.
// Only experts that a token picked get work, as in the pages' prefill, which
// multiplies only the routed experts ("Strata - the details", "Faster
// prompts"; the routed-stream entry of the StrataPool README's credits).
#pragma once

#include "common.h"

namespace moe {

__device__ inline int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Block-wide exclusive scan of data[0..n) in place (LDS or global); returns the
// total. Each thread scans a contiguous run; runs are combined with one wave
// scan per wave and one pass over the (at most 16) wave totals. All threads of
// the block must call it; blockDim.x is a multiple of 64, at most 1024.
__device__ inline int block_exclusive_scan(int* data, int n, int* wsum /* LDS, >= 16 */) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + nt - 1) / nt;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += data[i];
  const int incl = wave_inclusive_scan(s);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int w = 0; w < (nt >> 6); ++w) {
    if (w < wv) wbase += wsum[w];
    total += wsum[w];
  }
  int run = wbase + incl - s;
  for (int i = lo; i < hi; ++i) {
    const int v = data[i];
    data[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Work map of one FFN launch, built in LDS by every workgroup.
struct WorkMap {
  int gbase[MOE_MAX_E_DEV + 2];  // exclusive prefix of "is a GEMV expert"
  int tbase[MOE_MAX_E_DEV + 2];  // exclusive prefix of MFMA tile counts
  int wsum[16];
  int n_gemv, n_tiles;
};

__device__ inline void workmap_init(WorkMap& wm, const int32_t* __restrict__ counts, int E_tot,
                                    int gmax, int tile_m = kTileM) {
  for (int e = threadIdx.x; e < E_tot; e += blockDim.x) {
    const int M = counts[e];
    wm.gbase[e] = (M >= 1 && M <= gmax) ? 1 : 0;
    wm.tbase[e] = M > gmax ? (M + tile_m - 1) / tile_m : 0;
  }
  __syncthreads();
  const int ng = block_exclusive_scan(wm.gbase, E_tot, wm.wsum);
  const int nt = block_exclusive_scan(wm.tbase, E_tot, wm.wsum);
  if (threadIdx.x == 0) {
    wm.gbase[E_tot] = ng;
    wm.tbase[E_tot] = nt;
    wm.n_gemv = ng;
    wm.n_tiles = nt;
  }
  __syncthreads();
}

// The last e in [0, E_tot) with base[e] <= target (base non-decreasing).
__device__ inline int workmap_find(const int* base, int E_tot, int target) {
  int lo = 0, hi = E_tot;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (base[mid] <= target) lo = mid;
    else hi = mid;
  }
  return lo;
}

// GEMV expert number `target` (0 <= target < n_gemv).
__device__ inline int workmap_gemv(const WorkMap& wm, int E_tot, int target) {
  return workmap_find(wm.gbase, E_tot, target);
}

// MFMA tile number `target` (0 <= target < n_tiles): its expert and tile index.
__device__ inline int workmap_tile(const WorkMap& wm, int E_tot, int target, int& tile) {
  const int e = workmap_find(wm.tbase, E_tot, target);
  tile = target - wm.tbase[e];
  return e;
}

}  // namespace moe

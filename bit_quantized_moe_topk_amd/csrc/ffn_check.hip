// fp32 check mode of the expert FFN: every weight dequantised to fp32
// (w = d*q + m, one rounding-free product since d*q fits in 24 bits), fp32 FMA
// accumulation in ascending K order, fp32 h and o. Slow on purpose; it is the
// parity mode the fast path is measured against on the GPU.
//
// Expert = gate, up and down rows ("Strata - the details", "Low-RAM mode
// without experts.bin"); h = silu(gate . x) * (up . x); o = down . h.
#include "common.h"
#include "sched.h"

namespace moe {
namespace {

constexpr int kCkRows = 32;  // output rows per tile
constexpr int kThreads = 256;


// Dequantise weight j (0..31) of block `blk` to fp32.
__device__ inline float deq(const Experts& ex, size_t blk, int j) {
  const uint8_t c = ex.codes[blk * 8 + (j >> 2)];
  int q = (c >> (2 * (j & 3))) & 3;
  if (ex.qtype == 3) q |= ((ex.hi[blk * 4 + (j >> 3)] >> (j & 7)) & 1) << 2;
  const float d = half_bits_to_f32(ex.dm[blk * 2]);
  const float m = half_bits_to_f32(ex.dm[blk * 2 + 1]);
  return d * (float)q + m;
}

__device__ inline int token_of(int a, int T, int k) { return a < T * k ? a / k : a - T * k; }

__device__ inline float load_x(const void* x, int xdtype, size_t i) {
  if (xdtype == 0) return static_cast<const float*>(x)[i];
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[i] << 16);
}

// Tile: kTileM assignments of one expert x kCkRows rows of gate and of up.
// Thread: token lane tm = tid / 4 (0..63), rows rq*8 .. rq*8+7 (rq = tid % 4).
__global__ __launch_bounds__(kThreads) void ck_gateup(Experts ex, FfnArgs a) {
  __shared__ WorkMap wm;
  workmap_init(wm, a.counts, ex.E_tot, 0);
  __shared__ float xs[kTileM][33];
  __shared__ float wg[kCkRows][33];
  __shared__ float wu[kCkRows][33];
  const int n_rt = ex.I / kCkRows;
  const int tid = threadIdx.x;
  const int tm = tid >> 2, rq = tid & 3;
  float* h = static_cast<float*>(a.h);
  for (int item = blockIdx.x; item < wm.n_tiles * n_rt; item += gridDim.x) {
    int tl;
    const int e = workmap_tile(wm, ex.E_tot, item / n_rt, tl);
    const int r0 = (item % n_rt) * kCkRows;
    const int m0 = tl * kTileM;
    const int M = a.counts[e] - m0;  // assignments left in this expert
    const int slot0 = a.offsets[e] + m0;
    // token of each of the tile's rows (loaded cooperatively below)
    const int my_slot = slot0 + tm;
    int my_tok = tm < M ? token_of(a.perm[my_slot], a.T, a.k) : -1;
    if ((unsigned)my_tok >= (unsigned)a.T) my_tok = -1;
    float g[8], u[8];
    for (int i = 0; i < 8; ++i) g[i] = u[i] = 0.f;
    for (int kb = 0; kb < ex.H / 32; ++kb) {
      __syncthreads();
      // x tile: thread (tm, rq) loads 8 of token tm's 32 values
      for (int j = 0; j < 8; ++j) {
        const int c = rq * 8 + j;
        xs[tm][c] = my_tok >= 0 ? load_x(a.x, a.xdtype, (size_t)my_tok * ex.H + kb * 32 + c) : 0.f;
      }
      // weight tiles: 64 rows (32 gate + 32 up) x 32 weights; thread -> row tid/4, 8 weights
      {
        const int rr = tid >> 2, j0 = (tid & 3) * 8;
        const bool is_up = rr >= kCkRows;
        const int row = r0 + (rr & (kCkRows - 1));
        const size_t blk = (is_up ? blk_up(ex, e) : blk_gate(ex, e)) + (size_t)row * (ex.H / 32) + kb;
        for (int j = 0; j < 8; ++j) {
          const float w = deq(ex, blk, j0 + j);
          if (is_up) wu[rr - kCkRows][j0 + j] = w;
          else wg[rr][j0 + j] = w;
        }
      }
      __syncthreads();
      for (int c = 0; c < 32; ++c) {
        const float xv = xs[tm][c];
        for (int i = 0; i < 8; ++i) {
          g[i] = fmaf(wg[rq * 8 + i][c], xv, g[i]);
          u[i] = fmaf(wu[rq * 8 + i][c], xv, u[i]);
        }
      }
    }
    if (tm < M) {
      for (int i = 0; i < 8; ++i) {
        const float s = g[i] / (1.0f + expf(-g[i]));
        h[(size_t)my_slot * ex.I + r0 + rq * 8 + i] = s * u[i];
      }
    }
  }
}

// Tile: kTileM assignments x kCkRows output rows of down; K = I.
__global__ __launch_bounds__(kThreads) void ck_down(Experts ex, FfnArgs a) {
  __shared__ WorkMap wm;
  workmap_init(wm, a.counts, ex.E_tot, 0);
  __shared__ float hs[kTileM][33];
  __shared__ float wd[kCkRows][33];
  const int n_rt = ex.H / kCkRows;
  const int tid = threadIdx.x;
  const int tm = tid >> 2, rq = tid & 3;
  const float* h = static_cast<const float*>(a.h);
  for (int item = blockIdx.x; item < wm.n_tiles * n_rt; item += gridDim.x) {
    int tl;
    const int e = workmap_tile(wm, ex.E_tot, item / n_rt, tl);
    const int r0 = (item % n_rt) * kCkRows;
    const int m0 = tl * kTileM;
    const int M = a.counts[e] - m0;
    const int my_slot = a.offsets[e] + m0 + tm;
    float acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int kb = 0; kb < ex.I / 32; ++kb) {
      __syncthreads();
      for (int j = 0; j < 8; ++j) {
        const int c = rq * 8 + j;
        hs[tm][c] = tm < M ? h[(size_t)my_slot * ex.I + kb * 32 + c] : 0.f;
      }
      if (tid < 128) {
        const int rr = tid >> 2, j0 = (tid & 3) * 8;
        const size_t blk = blk_down(ex, e) + (size_t)(r0 + rr) * (ex.I / 32) + kb;
        for (int j = 0; j < 8; ++j) wd[rr][j0 + j] = deq(ex, blk, j0 + j);
      }
      __syncthreads();
      for (int c = 0; c < 32; ++c) {
        const float hv = hs[tm][c];
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wd[rq * 8 + i][c], hv, acc[i]);
      }
    }
    if (tm < M) {
      const int asg = a.perm[my_slot];
      const float gate = asg < a.T * a.k ? a.gates[asg] : 1.0f;
      for (int i = 0; i < 8; ++i) a.o[(size_t)my_slot * ex.H + r0 + rq * 8 + i] = gate * acc[i];
    }
  }
}

inline int grid_for(int max_items) { return max_items < 4096 ? (max_items > 0 ? max_items : 1) : 4096; }

}  // namespace

hipError_t launch_ffn_check(const Experts& ex, const FfnArgs& a, hipStream_t s) {
  const int A = a.T * (a.k + ex.has_shared);
  const int max_tiles = A / kTileM + ex.E_tot + 1;
  MOE_LAUNCH("ck_gateup", s, ck_gateup, dim3(grid_for(max_tiles * (ex.I / kCkRows))), dim3(kThreads), 0, s,
                     ex, a);
  MOE_LAUNCH("ck_down", s, ck_down, dim3(grid_for(max_tiles * (ex.H / kCkRows))), dim3(kThreads), 0, s,
                     ex, a);
  return hipGetLastError();
}

}  // namespace moe

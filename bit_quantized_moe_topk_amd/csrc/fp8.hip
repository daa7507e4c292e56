// Gate/up + SwiGLU of one expert over a batch of tokens on the FP8 matrix
// cores: a measured variant, not the layer path (the layer's prefill runs the
// fp16 tiles of mfma.hip).
//
// The pages' prompt kernels moved to 8-bit integer tensor cores ("Strata -
// the details", "Speed (measured)"). The gfx950 analogue is the f8f6f4
// matrix-core family, whose block scales are powers of two. The block scale
// d of a 32-weight block is not a power of two, so it cannot ride in them.
// The variant keeps both operands exact instead:
//   * the codes q (0..3 for Q2, 0..7 for Q3) are exact E4M3 values (A);
//   * each token row of x is scaled by its own power of two 2^-e (largest
//     |x| in [128, 256)) and split into hi = e4m3(x 2^-e) and
//     lo = e4m3(x 2^-e - hi), which together hold a bf16 value to ~2^-8 (B);
//   * one product per 32-weight block: the A lanes of the other block of the
//     instruction's 64 K values are zero, so P = sum over the block of q x
//     (hi and lo accumulate into the same P), and an fp32 epilogue adds
//     d P + m S (S = the block's sum of x) into the row's total;
//   * g and u are scaled back by 2^e, then SwiGLU.
// Every product of two E4M3 values is exact in fp32; the error is the fp32
// accumulation, the hi + lo split and the E4M3 rounding of x's tiny entries.
//
// Two preparation kernels write the operands: fp8_codes (the expert's gate
// and up codes as E4M3 bytes, [2 I][H]) and fp8_x (hi, lo [T][H], block sums
// S [T][H / 32], exponents e [T]).
#include "batch_x.h"
#include "common.h"
#include "gemv.h"
#include "topk.h"

namespace moe {
namespace {

typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kF8Threads = 256;  // 4 waves, 32 tokens each, the same 32 rows
constexpr int kF8Rows = 32;      // rows of I per workgroup (gate and up)
constexpr int kF8Tok = 128;      // tokens per workgroup
constexpr int kF8MaxH = 2048;  // (d, m) of the workgroup's rows as fp32 in LDS: 32 KB

// E4M3 bytes of the integers 0..7.
__device__ inline uint32_t e4m3_of_code(uint32_t q) {
  // 0, 1, 2, 3, 4, 5, 6, 7 -> 0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E
  return q == 0 ? 0u : (q == 1 ? 0x38u : (q < 4 ? 0x40u + 4u * (q - 2) : 0x48u + 2u * (q - 4)));
}

// One 32-weight block of gate or up (row r of the matrix) -> 32 E4M3 bytes.
template <int Q>
__global__ __launch_bounds__(256) void fp8_codes(Experts ex, int expert, uint8_t* __restrict__ q8) {
  const int bpr = ex.H / 32;
  const size_t nblk = (size_t)2 * ex.I * bpr;  // gate rows, then up rows
  for (size_t b = blockIdx.x * 256 + threadIdx.x; b < nblk; b += (size_t)gridDim.x * 256) {
    const size_t src = blk_gate(ex, expert) + b;  // up rows follow gate rows in the planes
    const uint2 c = *reinterpret_cast<const uint2*>(ex.codes + src * 8);
    const uint32_t hb = Q == 3 ? *reinterpret_cast<const uint32_t*>(ex.hi + src * 4) : 0u;
    uint32_t out[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {  // weights 4w .. 4w + 3
      const uint32_t cw = w < 4 ? c.x : c.y;
      uint32_t v = 0;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int j = 4 * w + n;
        uint32_t q = (cw >> (2 * (j % 16))) & 3u;
        if (Q == 3) q |= ((hb >> j) & 1u) << 2;
        v |= e4m3_of_code(q) << (8 * n);
      }
      out[w] = v;
    }
    uint4* dst = reinterpret_cast<uint4*>(q8 + b * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
}

// One wave per token row: e from the row's largest |x|, then per 8 values the
// hi and lo bytes and, per 32-value block, S = the sum of hi + lo (as the
// matrix cores see x, in the scaled units).
__global__ __launch_bounds__(256) void fp8_x(const uint16_t* __restrict__ x, int T, int H,
                                             uint8_t* __restrict__ xh, uint8_t* __restrict__ xl,
                                             float* __restrict__ S, int32_t* __restrict__ xe) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int e = row_exp(row_absmax(x, 1, H, t)) - 5;  // largest |x| 2^-e in [128, 256)
  if (lane == 0) xe[t] = e;
  const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  for (int c = lane; c < H / 8; c += 64) {  // 8 values; a block is 4 consecutive c
    const uint4 u = row[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t hi2[2] = {0u, 0u}, lo2[2] = {0u, 0u};
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = __builtin_ldexpf(bf16_lo(w[p]), -e), b = __builtin_ldexpf(bf16_hi(w[p]), -e);
      const uint32_t hp = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
      const float ha = __builtin_amdgcn_cvt_f32_fp8((int)hp, 0), hb = __builtin_amdgcn_cvt_f32_fp8((int)hp, 1);
      const uint32_t lp = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a - ha, b - hb, 0, false) & 0xFFFFu;
      const float la = __builtin_amdgcn_cvt_f32_fp8((int)lp, 0), lb = __builtin_amdgcn_cvt_f32_fp8((int)lp, 1);
      s += (ha + la) + (hb + lb);
      hi2[p / 2] |= hp << (16 * (p % 2));
      lo2[p / 2] |= lp << (16 * (p % 2));
    }
    reinterpret_cast<uint2*>(xh + (size_t)t * H)[c] = make_uint2(hi2[0], hi2[1]);
    reinterpret_cast<uint2*>(xl + (size_t)t * H)[c] = make_uint2(lo2[0], lo2[1]);
    // the block's sum: 4 consecutive lanes (c % 4), in lane order
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if ((c & 3) == 0) S[(size_t)t * (H / 32) + c / 4] = s;
  }
}

// Workgroup (rt, tt): rows 32 rt .. 32 rt + 31 of gate and up, tokens
// 128 tt .. 128 tt + 127 (wave w: 32 of them). Per K step of 64 (two blocks):
// lane (i, g) = (lane % 32, lane / 32) holds row i's 32 codes of block
// 2 s + g (A) and token i's 32 hi and lo bytes of that block (B); for each
// block and matrix, P = A_masked . hi + A_masked . lo on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales), then acc += d P + m S.
// (d, m) of the workgroup's rows sit in LDS as fp32 pairs [matrix][block][row]
// (every lane of a half reads the same rows: broadcasts). Measured on one
// expert over 8,192 tokens it runs at about half the rate of the fp16 tiles:
// the per-block epilogue (two fp32 FMAs per output and block), not the
// matrix cores, bounds it; keeping the next step's operands or all four
// products of a step in flight, and placing a token tile's row tiles on one
// XCD, each measured slower.
__global__ __launch_bounds__(kF8Threads) void fp8_gateup(Experts ex, int expert, int T,
                                                          const uint8_t* __restrict__ q8,
                                                          const uint8_t* __restrict__ xh,
                                                          const uint8_t* __restrict__ xl,
                                                          const float* __restrict__ S,
                                                          const int32_t* __restrict__ xe,
                                                          float* __restrict__ h) {
  __shared__ float2 dm_s[2][kF8MaxH / 32][kF8Rows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = ex.H, I = ex.I, nbk = H / 32;
  const int r0 = blockIdx.x * kF8Rows;
  const int t0 = blockIdx.y * kF8Tok + wave * 32;
  for (int i = tid; i < 2 * nbk * kF8Rows; i += kF8Threads) {
    const int mat = i / (nbk * kF8Rows), rem = i % (nbk * kF8Rows), r = rem % kF8Rows, b = rem / kF8Rows;
    const size_t blk = (mat ? blk_up(ex, expert) : blk_gate(ex, expert)) + (size_t)(r0 + r) * nbk + b;
    const uint32_t v = *reinterpret_cast<const uint32_t*>(ex.dm + blk * 2);
    dm_s[mat][b][r] = make_float2(half_lo(v), half_hi(v));
  }
  __syncthreads();
  const int i = lane & 31, g = lane >> 5;
  const int tok = min(t0 + i, T - 1);
  const uint8_t* ag = q8 + (size_t)(r0 + i) * H + 32 * g;            // gate row
  const uint8_t* au = q8 + (size_t)(I + r0 + i) * H + 32 * g;        // up row
  const uint8_t* bh = xh + (size_t)tok * H + 32 * g;
  const uint8_t* bl = xl + (size_t)tok * H + 32 * g;
  // this lane's output column (token) and rows 8 (v / 4) + 4 g + v % 4
  const float* Sj = S + (size_t)tok * nbk;
  floatx16_t acc_g = {}, acc_u = {};
  auto ld = [](const uint8_t* p) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
    int8v_t v;
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
    return v;
  };
  const int8v_t zero = {};
  for (int k0 = 0; k0 < H; k0 += 64) {
    const int8v_t vg = ld(ag + k0), vu = ld(au + k0), vh = ld(bh + k0), vl = ld(bl + k0);
    const float s0 = Sj[k0 / 32], s1 = Sj[k0 / 32 + 1];
#pragma unroll
    for (int gb = 0; gb < 2; ++gb) {  // block 2 s + gb: the A lanes of the other block are zero
      const int b = k0 / 32 + gb;
      const float sb = gb ? s1 : s0;
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        const int8v_t a = g == gb ? (mat ? vu : vg) : zero;
        floatx16_t p = {};
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, vh, p, 0, 0, 0, 127, 0, 127);
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, vl, p, 0, 0, 0, 127, 0, 127);
        // p[v]: row 8 (v / 4) + 4 g + v % 4, this lane's token
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 da = *reinterpret_cast<const float4*>(&dm_s[mat][b][8 * q + 4 * g]);
          const float4 db = *reinterpret_cast<const float4*>(&dm_s[mat][b][8 * q + 4 * g + 2]);
          const float d[4] = {da.x, da.z, db.x, db.z}, m[4] = {da.y, da.w, db.y, db.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (mat)
              acc_u[4 * q + r] = fmaf(d[r], p[4 * q + r], fmaf(m[r], sb, acc_u[4 * q + r]));
            else
              acc_g[4 * q + r] = fmaf(d[r], p[4 * q + r], fmaf(m[r], sb, acc_g[4 * q + r]));
          }
        }
      }
    }
  }
  const int t = t0 + i;
  if (t < T) {
    const float sc = __builtin_ldexpf(1.f, xe[t]);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = r0 + 8 * (v / 4) + 4 * g + v % 4;
      const float gv = acc_g[v] * sc, uv = acc_u[v] * sc;
      h[(size_t)t * I + r] = gv / (1.f + __expf(-gv)) * uv;
    }
  }
}

}  // namespace

size_t fp8_gateup_workspace_bytes(const Experts& ex, int T) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al((size_t)2 * ex.I * ex.H) + 2 * al((size_t)T * ex.H) + al(sizeof(float) * (size_t)T * (ex.H / 32)) +
         al(sizeof(int32_t) * (size_t)T);
}

bool fp8_gateup_supported(const Experts& ex) {
  return ex.H % 64 == 0 && ex.H <= kF8MaxH && ex.I % kF8Rows == 0;
}

hipError_t launch_fp8_gateup(const Experts& ex, int expert, const uint16_t* x, int T, float* h,
                             void* ws, hipStream_t s) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  uint8_t* q8 = reinterpret_cast<uint8_t*>(p);   p += al((size_t)2 * ex.I * ex.H);
  uint8_t* xh = reinterpret_cast<uint8_t*>(p);   p += al((size_t)T * ex.H);
  uint8_t* xl = reinterpret_cast<uint8_t*>(p);   p += al((size_t)T * ex.H);
  float* S = reinterpret_cast<float*>(p);        p += al(sizeof(float) * (size_t)T * (ex.H / 32));
  int32_t* xe = reinterpret_cast<int32_t*>(p);
  const size_t nblk = (size_t)2 * ex.I * (ex.H / 32);
  const dim3 gq((unsigned)((nblk + 255) / 256));
  if (ex.qtype == 3)
    MOE_LAUNCH("fp8_codes", s, fp8_codes<3>, gq, dim3(256), 0, s, ex, expert, q8);
  else
    MOE_LAUNCH("fp8_codes", s, fp8_codes<2>, gq, dim3(256), 0, s, ex, expert, q8);
  MOE_LAUNCH("fp8_x", s, fp8_x, dim3((T + 3) / 4), dim3(256), 0, s, x, T, ex.H, xh, xl, S, xe);
  MOE_LAUNCH("fp8_gateup", s, fp8_gateup, dim3(ex.I / kF8Rows, (T + kF8Tok - 1) / kF8Tok),
             dim3(kF8Threads), 0, s, ex, expert, T, q8, xh, xl, S, xe, h);
  return hipGetLastError();
}

}  // namespace moe

// Decode GEMV building blocks on gfx950 (header-only).
//
// A code q (2 or 3 bits) becomes the exact bf16 value 128 + q by OR-ing it into
// the mantissa of 128; v_dot2 multiplies pairs of such values by bf16
// activation pairs, and the block affine map is applied once per block and
// token:
//     sum_k (d q_k + m) x_k = d * (D - 128 S) + m * S,
// D = sum of the dot2 terms, S = sum of the block's activations. The codes are
// never expanded: every product is exact and the sums are fp32.
#pragma once

#include "common.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));

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

// SwiGLU of a token whose activations entered the matrix cores scaled by
// 2^-e (row_exp): the true g = 2^e gs and u = 2^e us are exact in fp32.
__device__ inline float silu_mul_x(float gs, float us, int e) {
  return silu_mul(__builtin_ldexpf(gs, e), __builtin_ldexpf(us, e));
}

// Power-of-two exponent that brings a token row into fp16 for the matrix
// cores: with amax its largest |x|, amax * 2^-e lies in [4, 8), so every bf16
// value of the row converts exactly (bf16's 8-bit significand fits fp16's 11)
// unless it is below 2^-12 of the row's largest, where fp16 turns subnormal;
// fp32 rows round once, as any fp16 conversion does. All-zero and non-finite
// rows keep e = 0.
__device__ inline int row_exp(float amax) {
  if (!(amax > 0.f) || !(amax <= 3.4028235e38f)) return 0;
  return __builtin_amdgcn_frexp_expf(amax) - 3;  // amax = f 2^E, f in [0.5, 1)
}

// Largest value of v over the 64 lanes of the wave (every lane gets it).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Activations of one 32-wide block, as 16 bf16 pairs in code-pair order:
// pair (8w + s) = (x[16w + s], x[16w + s + 8]), the order in which code pairs
// come out of a code word (codes 16w+s and 16w+s+8 sit 16 bits apart), plus
// S = sum of the 32 values (taken with v_dot2 against (1, 1): exact products,
// fp32 sum).
struct XB {
  uint32_t p[16];
  float S;
};

constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

// v[i] holds bf16 elements 2i (low half) and 2i+1 (high half), i < 16.
template <int Q>
__device__ inline void make_xb(const uint32_t v[16], XB& xb) {
  float S = 0.f;
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t a = v[8 * w + s / 2], b = v[8 * w + 4 + s / 2];
      // low half from a, high half from b: halves 0 (s even) or 1 (s odd)
      const uint32_t pr = __builtin_amdgcn_perm(b, a, (s & 1) ? 0x07060302u : 0x05040100u);
      xb.p[8 * w + s] = pr;
      S = dot2(pr, kOnes, S);
    }
  xb.S = S;
}

template <int Q>
__device__ inline void load_xb_bf16(const uint16_t* src, XB& xb) {
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
  make_xb<Q>(v, xb);
}

template <int Q>
__device__ inline void load_xb_f32(const float* src, XB& xb) {
  uint32_t v[16];
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 q = s4[i];
    v[2 * i] = f32_to_bf16_bits(q.x) | (f32_to_bf16_bits(q.y) << 16);
    v[2 * i + 1] = f32_to_bf16_bits(q.z) | (f32_to_bf16_bits(q.w) << 16);
  }
  make_xb<Q>(v, xb);
}

__device__ inline void zero_xb(XB& xb) {
#pragma unroll
  for (int i = 0; i < 16; ++i) xb.p[i] = 0u;
  xb.S = 0.f;
}

// Packed block: two code words, the high-bit word (Q3) and the (d, m) word.
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

// The 16 code pairs of a block as bf16 pairs (128 + q, 128 + q'): pair
// (8w + s) holds codes 16w+s and 16w+s+8 of code word w.
template <int Q>
__device__ inline void decode_pairs(const QBlock& b, uint32_t (&pr)[16]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t cw = w ? b.c1 : b.c0;
    uint32_t r2 = 0;
    if (Q == 3) {
      const uint32_t hw = b.hi >> (16 * w);
      r2 = ((hw & 0xFFu) | ((hw & 0xFF00u) << 8)) << 2;  // code 16w+s -> bit s+2, +8 -> s+18
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t v = ((cw >> (2 * s)) & 0x00030003u) | kMagic;
      if (Q == 3) v |= (r2 >> s) & 0x00040004u;
      pr[8 * w + s] = v;
    }
  }
}

// sum_k (d q_k + m) x_k for one block and MP tokens: the code pairs are
// decoded once and multiplied into every token's chain.
template <int Q, int MP>
__device__ inline void block_values(const QBlock& b, const XB (&xb)[MP], float (&out)[MP]) {
  uint32_t pr[16];
  decode_pairs<Q>(b, pr);
  const float d = half_lo(b.dm), m = half_hi(b.dm);
#pragma unroll
  for (int i = 0; i < MP; ++i) {
    float D = -128.0f * xb[i].S;
#pragma unroll
    for (int p = 0; p < 16; ++p) D = dot2(pr[p], xb[i].p[p], D);
    out[i] = d * D + m * xb[i].S;
  }
}

// ---------------------------------------------------------------------------
// Batched sum of N values per lane over the lanes that differ in bits < 2*O.
// Halving steps (top lane bit first) hand half of the values to the partner
// and keep the other half; once one value is left, butterfly steps finish the
// sum. On return the lane holds max(1, N / (2*O)) fully summed values whose
// first index is jbase.
template <int N, int O>
struct LaneReduce {
  __device__ static void run(float* v, int lane, int& jbase) {
    if constexpr (O >= 1) {
      if constexpr (N > 1) {
        constexpr int H = N / 2;
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          const float send = up ? v[i] : v[i + H];
          const float keep = up ? v[i + H] : v[i];
          v[i] = keep + __shfl_xor(send, O, 64);
        }
        if (up) jbase += H;
        LaneReduce<H, O / 2>::run(v, lane, jbase);
      } else {
        v[0] += __shfl_xor(v[0], O, 64);
        LaneReduce<1, O / 2>::run(v, lane, jbase);
      }
    }
  }
};

// fp32 pair -> packed fp16 pair (round to nearest even).
__device__ inline uint32_t pack_half2(float lo, float hi) {
  const half2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

typedef float float2v_t __attribute__((ext_vector_type(2)));

// Two floats -> a bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v_t){lo, hi}, bf16x2_t));
}

// Gate-scaled expert output of one assignment slot and output row.
__device__ inline void emit(const Experts& ex, const FfnArgs& a, int slot, int row, float val) {
  if (a.o) a.o[(size_t)slot * ex.H + row] = val;
  else a.ob[(size_t)slot * ex.H + row] = (uint16_t)f32_to_bf16_bits(val);
}

__device__ inline float gate_of(const FfnArgs& a, int slot) {
  const int asg = a.perm[slot];
  return asg < a.T * a.k ? a.gates[asg] : 1.0f;
}

}  // namespace moe

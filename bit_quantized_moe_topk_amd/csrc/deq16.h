// Block dequantisation to fp16 matrix-core operands (header-only; used by the
// prefill tiles and the decode window's matrix-core kernels).
#pragma once

#include "common.h"
#include "gemv.h"

namespace moe {

// --- dequantisation -------------------------------------------------------
// Code pair -> fp16 pair: OR the codes into the mantissa of 1024 (exact
// 1024 + q), subtract 1024 (exact), then one fused d*q + m.
__device__ inline uint32_t deq_pair(uint32_t t, half2_t d2, half2_t m2) {
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2_t q = __builtin_bit_cast(half2_t, t | 0x64006400u) - k1024;
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, d2, m2));
}

// MFMA K order inside each group of four weights: positions 0, 1, 2, 3 hold
// weights 0, 2, 1, 3. Both operands follow it: the fp16 activation copy and the
// SwiGLU output are stored that way, so each products' sum is unchanged.
//
// Q2 operands: byte j of e = c & 0x33333333 holds codes 4j (low nibble) and
// 4j + 2 (high nibble), and byte j of o = (c >> 2) & 0x33333333 holds codes
// 4j + 1 and 4j + 3, each as an FP4 E2M1 value q / 2. One scaled conversion
// (scale 2) turns a byte into the exact fp16 pair (q, q'), then one fused
// d*q + m rounds once.
//
// Q3 operands: a byte permute puts byte j of c and of c >> 2 in the two halves
// of a word; masks pick codes (4j, 4j + 1) from bits 0-1 and (4j + 2, 4j + 3)
// from bits 4-5, OR in the third bits, and OR-ing into the mantissa of 1024
// gives 1024 + q exactly; subtracting 1024 and one fused d*q + m follow, and a
// final permute brings the pairs into the K order above.
struct WStage {
  uint32_t w0, w1, w2, w3;  // Q2: e, o of code words 0, 1; Q3: codes 0, 1, third bits
  half2_t d2, m2;
  float d, m;               // the same scales for the bf16 operands
};

// Per-row operand state of one block: its two code words (Q2: as e, o
// nibble planes), third bits and broadcast d, m.
template <int Q>
__device__ inline WStage wstage_block(uint32_t c0, uint32_t c1, uint32_t hi, uint32_t dm) {
  WStage st;
  if (Q == 2) {
    st.w0 = c0 & 0x33333333u;
    st.w1 = (c0 >> 2) & 0x33333333u;
    st.w2 = c1 & 0x33333333u;
    st.w3 = (c1 >> 2) & 0x33333333u;
  } else {
    st.w0 = c0;
    st.w1 = c1;
    st.w2 = hi;
    st.w3 = 0u;
  }
  st.d2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x01000100u));
  st.m2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x03020302u));
  st.d = half_lo(dm);
  st.m = half_hi(dm);
  return st;
}

// Byte j of w as two FP4 E2M1 values, times 2, in fp16 (j is a constant after
// unrolling; the instruction takes it as an immediate).
__device__ inline half2_t fp4x2_to_f16(uint32_t w, int j) {
  switch (j) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 3);
  }
}

// Weights 8 kk .. 8 kk + 7 of the block (in the K order above) as an MFMA operand.
template <int Q>
__device__ inline half8_t wfrag(const WStage& w, int kk) {
  uint32_t o[4];
  if (Q == 2) {
    const uint32_t e = kk < 2 ? w.w0 : w.w2, od = kk < 2 ? w.w1 : w.w3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * (kk & 1) + u;
      const half2_t qa = fp4x2_to_f16(e, j), qb = fp4x2_to_f16(od, j);
      o[2 * u] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qa, w.d2, w.m2));
      o[2 * u + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qb, w.d2, w.m2));
    }
  } else {
    const uint32_t cw = kk < 2 ? w.w0 : w.w1, hq = kk < 2 ? w.w2 : w.w2 >> 16;
    const uint32_t s = cw >> 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t j = 2 * (kk & 1) + u;  // byte of cw: codes 4j .. 4j + 3
      const uint32_t r = __builtin_amdgcn_perm(s, cw, 0x0C000C00u | ((4u + j) << 16) | j);
      uint32_t t0 = r & 0x00030003u, t1 = (r >> 4) & 0x00030003u;
      const uint32_t hb = hq >> (4 * j);
      t0 |= ((hb & 1u) << 2) | ((hb & 2u) << 17);
      t1 |= (hb & 4u) | ((hb & 8u) << 15);
      const uint32_t p01 = deq_pair(t0, w.d2, w.m2), p23 = deq_pair(t1, w.d2, w.m2);
      o[2 * u] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);      // weights 0, 2
      o[2 * u + 1] = __builtin_amdgcn_perm(p23, p01, 0x07060302u);  // weights 1, 3
    }
  }
  return __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// --- bf16 operands (the down projection) ----------------------------------
// The same weights, positions and K order as wfrag, as bf16: each code comes
// out of the FP4 conversion (Q2) or as a small integer (Q3) in fp32, d*q + m
// is one fp32 fma (d*q is exact), and the pair is rounded once to bf16.
__device__ inline float2v_t fp4x2_to_f32(uint32_t w, int j) {
  switch (j) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 2.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 2.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 2.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 2.0f, 3);
  }
}

__device__ inline uint32_t deq_bf16x2(float qa, float qb, float d, float m) {
  return pack_bf16x2(__builtin_fmaf(qa, d, m), __builtin_fmaf(qb, d, m));
}

template <int Q>
__device__ inline bf16x8_t wfrag_bf(const WStage& w, int kk) {
  uint32_t o[4];
  if (Q == 2) {
    const uint32_t e = kk < 2 ? w.w0 : w.w2, od = kk < 2 ? w.w1 : w.w3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * (kk & 1) + u;
      const float2v_t qa = fp4x2_to_f32(e, j), qb = fp4x2_to_f32(od, j);
      o[2 * u] = deq_bf16x2(qa.x, qa.y, w.d, w.m);
      o[2 * u + 1] = deq_bf16x2(qb.x, qb.y, w.d, w.m);
    }
  } else {
    const uint32_t cw = kk < 2 ? w.w0 : w.w1, hq = kk < 2 ? w.w2 : w.w2 >> 16;
    const uint32_t s = cw >> 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t j = 2 * (kk & 1) + u;
      const uint32_t r = __builtin_amdgcn_perm(s, cw, 0x0C000C00u | ((4u + j) << 16) | j);
      uint32_t t0 = r & 0x00030003u, t1 = (r >> 4) & 0x00030003u;
      const uint32_t hb = hq >> (4 * j);
      t0 |= ((hb & 1u) << 2) | ((hb & 2u) << 17);
      t1 |= (hb & 4u) | ((hb & 8u) << 15);
      // t0: codes 4j, 4j + 1 in its two halves; t1: codes 4j + 2, 4j + 3
      o[2 * u] = deq_bf16x2((float)(t0 & 0xFFu), (float)(t1 & 0xFFu), w.d, w.m);      // weights 0, 2
      o[2 * u + 1] = deq_bf16x2((float)(t0 >> 16), (float)(t1 >> 16), w.d, w.m);      // weights 1, 3
    }
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// --- Q3 through the FP8 conversion ----------------------------------------
// A byte holding a code q <= 15 is the OCP E4M3 value q * 2^-9 (subnormal
// below 8, exponent 1 from 8 on), so the scaled FP8 -> fp16 conversion with
// scale 2^9 (a power of two) gives q exactly, two bytes per instruction. One
// code word (16 codes, 2 bits each) and its half of the third-bit plane make
// four byte words: byte b of word s holds code 4 b + s, its two low bits
// shifted down from the code word and its third bit taken from a copy of the
// plane spread one nibble per byte. One fused d*q + m per pair then rounds
// once. About two VALU instructions per weight, against three and a half for
// separate FP4 conversions of the low and third bits.
//
// K order of this form (both operands follow it): position i of operand half
// h of a word holds weight 4 (i & 3) + 2 h + (i >> 2), i.e. weights
// 0, 4, 8, 12, 1, 5, 9, 13 for h = 0 and 2, 6, 10, 14, 3, 7, 11, 15 for h = 1.
struct WByteWord {
  uint32_t b[4];
  half2_t d2, m2;
  float d, m;
};

__device__ inline WByteWord wbyte_word(uint32_t c, uint32_t hi, uint32_t dm, int w) {
  // third bits of codes 16 w .. 16 w + 15: nibble b into byte b
  uint32_t x = __builtin_amdgcn_perm(hi, hi, w ? 0x0C030C02u : 0x0C010C00u);
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  WByteWord r;
  r.b[0] = (c & 0x03030303u) | ((x << 2) & 0x04040404u);
  r.b[1] = ((c >> 2) & 0x03030303u) | ((x << 1) & 0x04040404u);
  r.b[2] = ((c >> 4) & 0x03030303u) | (x & 0x04040404u);
  r.b[3] = ((c >> 6) & 0x03030303u) | ((x >> 1) & 0x04040404u);
  r.d2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x01000100u));
  r.m2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x03020302u));
  r.d = half_lo(dm);
  r.m = half_hi(dm);
  return r;
}

// Operand half h of the word: byte words 2 h and 2 h + 1, low bytes (codes s,
// s + 4) then high bytes (s + 8, s + 12) of each.
__device__ inline half8_t wfrag_byte(const WByteWord& w, int h) {
  uint32_t o[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t bw = w.b[2 * h + u];
    const half2_t ql = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bw, 512.0f, false);
    const half2_t qh = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bw, 512.0f, true);
    o[2 * u] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(ql, w.d2, w.m2));
    o[2 * u + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qh, w.d2, w.m2));
  }
  return __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// The same as bf16 (positions as wfrag_byte): the scaled FP8 -> fp32
// conversion gives two exact codes, then one fp32 fma each and one bf16
// rounding per pair.
__device__ inline bf16x8_t wfrag_byte_bf(const WByteWord& w, int h) {
  uint32_t o[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t bw = w.b[2 * h + u];
    const float2v_t ql = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bw, 512.0f, false);
    const float2v_t qh = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bw, 512.0f, true);
    o[2 * u] = deq_bf16x2(ql.x, ql.y, w.d, w.m);
    o[2 * u + 1] = deq_bf16x2(qh.x, qh.y, w.d, w.m);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// --- raw weight rows -------------------------------------------------------
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// NBL consecutive quantisation blocks of one weight row as loaded from the
// canonical planes: two code words, the third-bit word (Q3) and the fp16 pair
// (d, m) per block.
template <int NBL>
struct WRow {
  uint32_t c[2 * NBL], hi[NBL], dm[NBL];
};

// The same with the block index split into a wave-uniform part (ubase, kept
// in scalar registers) and a 32-bit per-lane part, so that no 64-bit per-lane
// address stays live between loads.
template <int Q, int NBL>
__device__ inline WRow<NBL> load_wrow_at(const Experts& ex, size_t ubase, uint32_t lane_blk) {
  const uint8_t* cb = ex.codes + ubase * 8;
  const uint16_t* db = ex.dm + ubase * 2;
  const uint8_t* hb = Q == 3 ? ex.hi + ubase * 4 : nullptr;
  WRow<NBL> w;
  if (NBL == 1) {
    const uint2 c = *reinterpret_cast<const uint2*>(cb + 8 * lane_blk);
    w.c[0] = c.x;
    w.c[1] = c.y;
    w.dm[0] = *reinterpret_cast<const uint32_t*>(db + 2 * lane_blk);
    if (Q == 3) w.hi[0] = *reinterpret_cast<const uint32_t*>(hb + 4 * lane_blk);
  } else {
#pragma unroll
    for (int i = 0; i < NBL; i += 2) {
      const uint4 c = *reinterpret_cast<const uint4*>(cb + 8 * (lane_blk + i));
      w.c[2 * i] = c.x;
      w.c[2 * i + 1] = c.y;
      w.c[2 * i + 2] = c.z;
      w.c[2 * i + 3] = c.w;
      const uint2 dm = *reinterpret_cast<const uint2*>(db + 2 * (lane_blk + i));
      w.dm[i] = dm.x;
      w.dm[i + 1] = dm.y;
      if (Q == 3) {
        const uint2 h = *reinterpret_cast<const uint2*>(hb + 4 * (lane_blk + i));
        w.hi[i] = h.x;
        w.hi[i + 1] = h.y;
      }
    }
  }
  if (Q != 3)
#pragma unroll
    for (int i = 0; i < NBL; ++i) w.hi[i] = 0u;
  return w;
}

template <int Q, int NBL>
__device__ inline WRow<NBL> load_wrow(const Experts& ex, size_t blk) {
  WRow<NBL> w;
  if (NBL == 1) {
    const uint2 c = *reinterpret_cast<const uint2*>(ex.codes + blk * 8);
    w.c[0] = c.x;
    w.c[1] = c.y;
    w.dm[0] = *reinterpret_cast<const uint32_t*>(ex.dm + blk * 2);
    if (Q == 3) w.hi[0] = *reinterpret_cast<const uint32_t*>(ex.hi + blk * 4);
  } else {
#pragma unroll
    for (int i = 0; i < NBL; i += 2) {
      const uint4 c = *reinterpret_cast<const uint4*>(ex.codes + (blk + i) * 8);
      w.c[2 * i] = c.x;
      w.c[2 * i + 1] = c.y;
      w.c[2 * i + 2] = c.z;
      w.c[2 * i + 3] = c.w;
      const uint2 dm = *reinterpret_cast<const uint2*>(ex.dm + (blk + i) * 2);
      w.dm[i] = dm.x;
      w.dm[i + 1] = dm.y;
      if (Q == 3) {
        const uint2 h = *reinterpret_cast<const uint2*>(ex.hi + (blk + i) * 4);
        w.hi[i] = h.x;
        w.hi[i + 1] = h.y;
      }
    }
  }
  if (Q != 3)
#pragma unroll
    for (int i = 0; i < NBL; ++i) w.hi[i] = 0u;
  return w;
}

}  // namespace moe

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

// The same times 8 (E2M1 0.5 becomes 4).
__device__ inline half2_t fp4x2_to_f16_x8(uint32_t w, int j) {
  switch (j) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 8.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 8.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 8.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 8.0f, 3);
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

// --- Q3 through the FP4 conversion ----------------------------------------
// A 3-bit code is q = q_lo + 4 q_hi. The two low bits take the Q2 path above
// (an FP4 conversion with scale 2 gives q_lo exactly); the third bits, spread
// to the same nibble positions (byte j of a word's e plane holds codes 4j,
// 4j + 2 in its two nibbles, the o plane codes 4j + 1, 4j + 3), go through the
// FP4 conversion with scale 8, which turns nibble 0b0001 (E2M1 0.5) into an
// exact 4. One exact fp16 add gives q, then one fused d*q + m rounds once, as
// in wfrag<3>, for far fewer VALU instructions than assembling 3-bit fields.
struct WSplit {
  uint32_t e0, o0, e1, o1;      // low bits of code words 0, 1 as E2M1 nibbles (Q2 planes)
  uint32_t he0, ho0, he1, ho1;  // third bits at the same nibble positions
  half2_t d2, m2;
};

// Bits 2i of x (i = 0..7) in the bytes sel picks, moved to bit 4i of the
// result: a byte permute, then two shift-or-mask steps.
__device__ inline uint32_t spread_even(uint32_t x, uint32_t sel) {
  x = __builtin_amdgcn_perm(x, x, sel);
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  return (x | (x << 2)) & 0x33333333u;
}

__device__ inline WSplit wsplit_block(uint32_t c0, uint32_t c1, uint32_t hi, uint32_t dm) {
  WSplit st;
  st.e0 = c0 & 0x33333333u;
  st.o0 = (c0 >> 2) & 0x33333333u;
  st.e1 = c1 & 0x33333333u;
  st.o1 = (c1 >> 2) & 0x33333333u;
  const uint32_t ev = hi & 0x55555555u, od = (hi >> 1) & 0x55555555u;
  st.he0 = spread_even(ev, 0x0C010C00u);  // third bits of codes 0 .. 15
  st.ho0 = spread_even(od, 0x0C010C00u);
  st.he1 = spread_even(ev, 0x0C030C02u);  // codes 16 .. 31
  st.ho1 = spread_even(od, 0x0C030C02u);
  st.d2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x01000100u));
  st.m2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x03020302u));
  return st;
}

// The planes of one code word w (0: codes 0 .. 15, 1: codes 16 .. 31), for
// callers short of registers: weights 8 kk .. 8 kk + 7 for kk = 2 w, 2 w + 1.
struct WSplitWord {
  uint32_t e, o, he, ho;
  half2_t d2, m2;
};

__device__ inline WSplitWord wsplit_word(uint32_t c, uint32_t hi, uint32_t dm, int w) {
  WSplitWord st;
  st.e = c & 0x33333333u;
  st.o = (c >> 2) & 0x33333333u;
  const uint32_t sel = w ? 0x0C030C02u : 0x0C010C00u;
  st.he = spread_even(hi & 0x55555555u, sel);
  st.ho = spread_even((hi >> 1) & 0x55555555u, sel);
  st.d2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x01000100u));
  st.m2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dm, dm, 0x03020302u));
  return st;
}

// Weights 8 kk .. 8 kk + 7 of the block, kk = 2 w + half.
__device__ inline half8_t wfrag_word(const WSplitWord& w, int half) {
  uint32_t o[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = 2 * half + u;
    const half2_t qa = fp4x2_to_f16(w.e, j) + fp4x2_to_f16_x8(w.he, j);
    const half2_t qb = fp4x2_to_f16(w.o, j) + fp4x2_to_f16_x8(w.ho, j);
    o[2 * u] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qa, w.d2, w.m2));
    o[2 * u + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qb, w.d2, w.m2));
  }
  return __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// Weights 8 kk .. 8 kk + 7 of the block in the K order above.
__device__ inline half8_t wfrag_split(const WSplit& w, int kk) {
  const uint32_t e = kk < 2 ? w.e0 : w.e1, od = kk < 2 ? w.o0 : w.o1;
  const uint32_t he = kk < 2 ? w.he0 : w.he1, ho = kk < 2 ? w.ho0 : w.ho1;
  uint32_t o[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = 2 * (kk & 1) + u;
    const half2_t qa = fp4x2_to_f16(e, j) + fp4x2_to_f16_x8(he, j);
    const half2_t qb = fp4x2_to_f16(od, j) + fp4x2_to_f16_x8(ho, j);
    o[2 * u] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qa, w.d2, w.m2));
    o[2 * u + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qb, w.d2, w.m2));
  }
  return __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
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

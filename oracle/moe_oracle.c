/*
 * moe_oracle.c -- plain, slow CPU oracle for the routed MoE FFN layer over
 * block-quantized expert weights.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code. It shares nothing with the
 * HIP library: no headers, no helpers, no tables.
 *
 * What the layer computes (sources are the Strata pages):
 *   - per token, a router scores every expert and the token is sent to the 10
 *     best of a layer's 512 ("Strata - the details", "How it works": routers and
 *     shared experts live on the GPU; the Strata README, "How does it work?":
 *     each word needs only 10 of the experts; "Which model?": 10 active per
 *     token);
 *   - each expert is three matrices, its gate, up and down rows ("Strata - the
 *     details", "Low-RAM mode without experts.bin"), held as 2-bit (Q2_0) or
 *     3-bit packs ("Speed (measured)", "Which model?");
 *   - shared experts run for every token ("How it works").
 * The pages leave the arithmetic open; the plain readings used here are:
 *   route : the k largest logits, ties to the lower expert index, ranked in
 *           descending order; gates are a softmax over the k selected logits
 *           (the same as a softmax over all E renormalised over the top k);
 *   group : a stable counting sort of the assignments t*k+j by expert;
 *   dequant: w = d*q + m per 32-weight block, d and m fp16;
 *   FFN   : g = Wg x, u = Wu x, h = silu(g) * u, o = Wd h (SwiGLU);
 *   combine: y_t = sum_j gate[t,j] * o(idx[t,j], x_t) + o(shared, x_t).
 *
 * Accumulation is sequential in index order, in the type ORACLE_ACC (double by
 * default; the float build is the fp32 oracle). No blocking, no reordering.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_ACC
#define ORACLE_ACC double
#define ORACLE_SUFFIX f64
#define ORACLE_COMMON 1
#endif

#define CAT2(a, b) a##_##b
#define CAT(a, b) CAT2(a, b)
#define NAME(f) CAT(f, ORACLE_SUFFIX)

typedef ORACLE_ACC acc_t;

/* ------------------------------------------------------------------------ */
/* Scalar conversions, written from the IEEE-754 binary16 / bfloat16 formats. */

#ifdef ORACLE_COMMON
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);               /* zero or subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* 1.frac * 2^(expo-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}
#else
double oracle_half_to_double(uint16_t h);
double oracle_bf16_to_double(uint16_t b);
#endif

/* ------------------------------------------------------------------------ */
/* Routing and grouping do not depend on the accumulation type. */

#ifdef ORACLE_COMMON
/* Is expert a (logit va) ranked before expert b (logit vb)?  Larger logit first,
 * equal logits (IEEE equality, so +0 == -0) to the lower index, NaN after every
 * number. */
static int ranks_before(float va, int a, float vb, int b)
{
    int na = isnan(va), nb = isnan(vb);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb;              /* a is a number, b is NaN */
    }
    if (va > vb) return 1;
    if (va < vb) return 0;
    return a < b;
}

/* Top-k selection and gates for every token.
 * logits [T][E] f32; idx [T][k] int32 in rank order; gates [T][k] f32. */
void oracle_route(const float *logits, int T, int E, int k, int32_t *idx, float *gates)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * k + j] = best;
        }
        /* softmax over the selected logits, relative to the largest one */
        double top = l[idx[(size_t)t * k]];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp((double)l[idx[(size_t)t * k + j]] - top);
        for (int j = 0; j < k; ++j)
            gates[(size_t)t * k + j] = (float)(exp((double)l[idx[(size_t)t * k + j]] - top) / sum);
    }
    free(taken);
}

/* Stable counting sort of the assignments by expert.
 * Routed assignment (t, j) has flat id t*k + j; with a shared expert, token t's
 * shared assignment has flat id T*k + t and lands in group E.
 * counts [E+1], offsets [E+2], perm [A], slot_of [A], A = T*(k + has_shared).
 * Every idx entry must lie in [0, E). */
void oracle_group(const int32_t *idx, int T, int k, int E, int has_shared,
                  int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *slot_of)
{
    int A_routed = T * k;
    for (int e = 0; e <= E; ++e) counts[e] = 0;
    for (int f = 0; f < A_routed; ++f) counts[idx[f]] += 1;
    counts[E] = has_shared ? T : 0;
    offsets[0] = 0;
    for (int e = 0; e <= E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    for (int f = 0; f < A_routed; ++f) {          /* ascending flat id: stable */
        int e = idx[f];
        int pos = offsets[e] + fill[e]++;
        perm[pos] = f;
        slot_of[f] = pos;
    }
    if (has_shared)
        for (int t = 0; t < T; ++t) {
            perm[A_routed + t] = A_routed + t;
            slot_of[A_routed + t] = A_routed + t;
        }
    free(fill);
}
#endif /* ORACLE_COMMON */

/* ------------------------------------------------------------------------ */
/* Dequantisation of one row of K weights (K/32 blocks), in acc_t.
 * codes: 8 bytes per block, weight j at byte j/4, bits 2*(j%4);
 * hi (Q3 only): 4 bytes per block, weight j's third bit at byte j/8, bit j%8;
 * dm: (d, m) fp16 bit patterns per block.  w = d*q + m. */
static void dequant_row(int qtype, const uint8_t *codes, const uint8_t *hi,
                        const uint16_t *dm, int K, acc_t *w)
{
    for (int b = 0; b < K / 32; ++b) {
        acc_t d = (acc_t)oracle_half_to_double(dm[2 * b]);
        acc_t m = (acc_t)oracle_half_to_double(dm[2 * b + 1]);
        for (int j = 0; j < 32; ++j) {
            int q = (codes[8 * b + j / 4] >> (2 * (j % 4))) & 3;
            if (qtype == 3) q |= ((hi[4 * b + j / 8] >> (j % 8)) & 1) << 2;
            w[32 * b + j] = d * (acc_t)q + m;
        }
    }
}

void NAME(oracle_dequant_row)(int qtype, const uint8_t *codes, const uint8_t *hi,
                              const uint16_t *dm, int K, acc_t *w)
{
    dequant_row(qtype, codes, hi, dm, K, w);
}

static acc_t silu(acc_t z)
{
    return z / ((acc_t)1 + (acc_t)exp(-(double)z));
}

/* One expert on one token.
 * Expert planes: blocks numbered gate rows, then up rows, then down rows.
 * x [H] -> o [H].  g, u, h [I] are written when non-NULL (for inspection). */
void NAME(oracle_expert_forward)(int qtype, int H, int I,
                                 const uint8_t *codes, const uint8_t *hi, const uint16_t *dm,
                                 const acc_t *x, acc_t *o, acc_t *g_out, acc_t *u_out,
                                 acc_t *h_out)
{
    size_t bpr_gu = (size_t)H / 32;        /* blocks per gate/up row */
    size_t bpr_d = (size_t)I / 32;         /* blocks per down row */
    size_t up0 = (size_t)I * bpr_gu;       /* first block of the up matrix */
    size_t dn0 = 2 * up0;                  /* first block of the down matrix */
    acc_t *wrow = (acc_t *)malloc(sizeof(acc_t) * (size_t)(H > I ? H : I));
    acc_t *h = (acc_t *)malloc(sizeof(acc_t) * (size_t)I);
    for (int r = 0; r < I; ++r) {
        size_t bg = (size_t)r * bpr_gu, bu = up0 + (size_t)r * bpr_gu;
        dequant_row(qtype, codes + 8 * bg, hi ? hi + 4 * bg : NULL, dm + 2 * bg, H, wrow);
        acc_t g = 0;
        for (int c = 0; c < H; ++c) g += wrow[c] * x[c];
        dequant_row(qtype, codes + 8 * bu, hi ? hi + 4 * bu : NULL, dm + 2 * bu, H, wrow);
        acc_t u = 0;
        for (int c = 0; c < H; ++c) u += wrow[c] * x[c];
        h[r] = silu(g) * u;
        if (g_out) g_out[r] = g;
        if (u_out) u_out[r] = u;
        if (h_out) h_out[r] = h[r];
    }
    for (int r = 0; r < H; ++r) {
        size_t bd = dn0 + (size_t)r * bpr_d;
        dequant_row(qtype, codes + 8 * bd, hi ? hi + 4 * bd : NULL, dm + 2 * bd, I, wrow);
        acc_t s = 0;
        for (int c = 0; c < I; ++c) s += wrow[c] * h[c];
        o[r] = s;
    }
    free(h);
    free(wrow);
}

/* The layer for a subset of tokens.
 * xdtype 0: x is float [T][H]; 1: x is bf16 bits [T][H].
 * idx, gates [T][k]; planes of E + has_shared experts, each NB = 3*H*I/32 blocks.
 * rows [nrows] are token ids; y [nrows][H] in acc_t.
 * nthreads > 0 sets the OpenMP team size (tokens are independent). */
void NAME(oracle_layer_rows)(int qtype, int T, int H, int E, int I, int k, int has_shared,
                             int xdtype, const void *x, const int32_t *idx, const float *gates,
                             const uint8_t *codes, const uint8_t *hi, const uint16_t *dm,
                             const int32_t *rows, int nrows, acc_t *y, int nthreads)
{
    (void)T;
    size_t nb = (size_t)3 * H * I / 32;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int r = 0; r < nrows; ++r) {
        int t = rows[r];
        acc_t *xt = (acc_t *)malloc(sizeof(acc_t) * (size_t)H);
        acc_t *o = (acc_t *)malloc(sizeof(acc_t) * (size_t)H);
        acc_t *yt = y + (size_t)r * H;
        for (int c = 0; c < H; ++c) {
            if (xdtype == 0) xt[c] = (acc_t)((const float *)x)[(size_t)t * H + c];
            else xt[c] = (acc_t)oracle_bf16_to_double(((const uint16_t *)x)[(size_t)t * H + c]);
            yt[c] = 0;
        }
        int n_terms = k + (has_shared ? 1 : 0);
        for (int j = 0; j < n_terms; ++j) {
            int e = j < k ? idx[(size_t)t * k + j] : E;
            acc_t gate = j < k ? (acc_t)gates[(size_t)t * k + j] : (acc_t)1;
            NAME(oracle_expert_forward)(qtype, H, I, codes + (size_t)e * nb * 8,
                                        hi ? hi + (size_t)e * nb * 4 : NULL,
                                        dm + (size_t)e * nb * 2, xt, o, NULL, NULL, NULL);
            for (int c = 0; c < H; ++c) yt[c] += gate * o[c];
        }
        free(o);
        free(xt);
    }
}

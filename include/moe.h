/*
 * moe.h -- C ABI of the routed mixture-of-experts FFN layer over block-quantized
 * expert weights, for one AMD Instinct MI355X (gfx950).
 *
 * The layer is the one the Strata pages describe: a router scores the 512
 * experts of a layer and each token is sent to the 10 best; shared experts run
 * for every token ("Strata - the details", section "How it works"; the Strata
 * README, "How does it work?"); every expert is three matrices, its gate, up and
 * down rows ("Strata - the details", "Low-RAM mode without experts.bin"), stored
 * as 2-bit or 3-bit block-quantized packs ("Speed (measured)", "Which model?").
 * It runs over decode verify windows of a few tokens ("How it works":
 * speculation) and over prefill chunks of up to 8,192 tokens ("Faster prompts").
 *
 * Conventions shared by every call
 *   - Every buffer pointer is a DEVICE pointer (HBM), unless a comment says
 *     otherwise. The caller allocates and owns every buffer; the library never
 *     allocates device memory and keeps no pointer after a call returns, except
 *     the weight planes a moe_experts handle refers to.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls validate their arguments on the host, enqueue kernels on `stream`
 *     and return without synchronising. Results are ready when the stream is.
 *   - Return value: MOE_OK, or a negative moe_status. Argument errors are
 *     detected on the host before anything is enqueued; nothing is written then.
 *     MOE_ERR_HIP means a kernel launch failed (hipGetLastError); faults inside
 *     a kernel surface at the caller's next synchronisation of the stream.
 *   - Element counts are int32; sizes in bytes are size_t.
 *   - No compute call keeps global state (the opt-in launch profiler below is
 *     the one exception); calls on different streams may run concurrently as
 *     long as they do not share output or workspace buffers.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* a size, pointer or enum is out of range     */
#define MOE_ERR_UNSUPPORTED (-2) /* valid, but outside what the kernels handle */
#define MOE_ERR_WORKSPACE (-3)   /* workspace smaller than the *_size() query  */
#define MOE_ERR_HIP (-4)         /* a HIP runtime call or launch failed         */

/* ---- enums -------------------------------------------------------------- */
#define MOE_F32 0  /* activations x and output y are float32               */
#define MOE_BF16 1 /* activations x and output y are bfloat16 (uint16 bits) */

#define MOE_Q2 2 /* 2-bit codes, w = d*q + m, q in 0..3, 32-weight blocks */
#define MOE_Q3 3 /* 3-bit codes, w = d*q + m, q in 0..7, 32-weight blocks */

/* FFN compute modes.
 * MOE_FAST: matrix cores with fp32 accumulation. Gate/up: weights dequantised
 *   to fp16 (one rounding of d*q + m) times the activations in fp16, each token
 *   row first scaled by its own power of two 2^-e (its largest |x| lands in
 *   [4, 8)), which is exact for bf16 rows; the epilogue multiplies g and u by
 *   2^e again before SwiGLU. h = silu(g) * u is rounded to bf16. Down: weights
 *   dequantised to bf16 times bf16 h. y is rounded to the activation dtype.
 *   So neither x nor h is limited to fp16's range: every finite bf16 or fp32
 *   activation row is handled at its own scale (values below 2^-12 of their
 *   row's largest turn fp16-subnormal and lose low bits). Some experts of
 *   batches of up to 256 tokens run an exact-code dot on bf16 activations
 *   instead. Expected agreement with an exact evaluation: a few 1e-3 relative
 *   L2 per token row.
 * MOE_CHECK_F32: every step in fp32 on the vector ALUs (parity mode); y is
 *   always float32. Agreement about 1e-6. */
#define MOE_FAST 0
#define MOE_CHECK_F32 2

/* ---- limits ------------------------------------------------------------- */
#define MOE_MAX_E 2048 /* routed experts per layer */

/* ---- routing ------------------------------------------------------------ */

/* Router scores in front of the top-k: the product of each token's hidden
 * state with every expert's router row ("Strata - the details", "How it
 * works": routers stay on the GPU and pick the experts that score highest).
 *   logits[t][e] = sum_h x[t][h] * w[e][h] (+ bias[e] when bias != NULL)
 * x: [T][H], float32 (xdtype MOE_F32) or bf16 (MOE_BF16), 16-byte aligned.
 * w: [E][H] bf16 (row e = expert e's router row), 16-byte aligned.
 * bias: [E] float32 or NULL.  logits: [T][E] float32.
 * Products of bf16 values are exact in float32; sums are float32 in a fixed
 * order (reproducible run to run; with bf16 x, at least 256 tokens and E a
 * multiple of 128 the order is the matrix cores', else a lane split of H).
 * Requires H % 256 == 0, H <= 4096, 1 <= E <= MOE_MAX_E, T >= 0 (T == 0: no
 * launch). The result feeds moe_route_topk, moe_route_group or moe_layer. */
int moe_router_logits(const void *x, int32_t xdtype, int32_t T, int32_t H, const uint16_t *w,
                      const float *bias, int32_t E, float *logits, void *stream);

/* Top-k expert selection and gates, per token.
 *
 * Per token t (the router step of "How it works"; 10 of 512 experts per token):
 *   idx[t][0..k-1]  = the k experts with the largest logits, in descending rank;
 *                     equal logits (IEEE equality, +0 == -0) go to the lower
 *                     expert index; NaN ranks below every number.
 *   gates[t][j]     = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0), l_j the
 *                     logit of idx[t][j]: a softmax over the selected logits,
 *                     equal to a softmax over all E renormalised over the top k.
 * logits: [T][E] float32, row-major.  idx: [T][k] int32.  gates: [T][k] float32.
 * Requires 1 <= E <= MOE_MAX_E, 1 <= k <= E, T >= 0 (T == 0: no launch).
 * Gates are finite when the selected logits are finite. */
int moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *idx,
                   float *gates, void *stream);

/* ---- grouping ----------------------------------------------------------- */

/* Workspace bytes moe_group needs for these sizes (device memory, any content). */
size_t moe_group_workspace_size(int32_t T, int32_t k, int32_t E);

/* Stable grouping of the token-to-expert assignments by expert (a counting sort;
 * the pages' prefill groups the chunk's tokens per expert before the expert
 * matrices run: "Faster prompts").
 *
 * Assignment ids: routed assignment (t, j) has id t*k + j; with has_shared, the
 * shared expert's assignment of token t has id T*k + t and belongs to group E.
 * A = T*(k + has_shared) assignments in all.
 *   counts [E+1]  : assignments per expert (counts[E] = T with a shared expert, else 0)
 *   offsets[E+2]  : exclusive prefix sum of counts; offsets[E+1] = A
 *   perm   [A]    : the assignment ids of group e at perm[offsets[e] .. offsets[e+1]),
 *                   in ascending id order (so ascending token order)
 *   slot_of[A]    : inverse of perm: perm[slot_of[a]] == a
 * idx [T][k] int32, every entry in [0, E). Entries outside that range are not
 * detected; the kernels stay in bounds and skip them, and the affected outputs
 * are unspecified.
 * ws: device scratch of at least moe_group_workspace_size(T, k, E) bytes. */
int moe_group(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t has_shared,
              int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *slot_of, void *ws,
              size_t ws_bytes, void *stream);

/* Top-k routing followed by the grouping, in one call: the same results as
 * moe_route_topk then moe_group (idx, gates, counts, offsets, perm, slot_of as
 * defined there). Small batches (T <= 16 and T*k <= 1024, e.g. decode verify
 * windows) run as one workgroup in a single launch; larger ones run the two
 * steps' kernels back to back. ws: at least moe_group_workspace_size(T, k, E)
 * bytes. T == 0 writes the empty grouping (counts, offsets) only. */
int moe_route_group(const float *logits, int32_t T, int32_t E, int32_t k, int32_t has_shared,
                    int32_t *idx, float *gates, int32_t *counts, int32_t *offsets, int32_t *perm,
                    int32_t *slot_of, void *ws, size_t ws_bytes, void *stream);

/* ---- experts ------------------------------------------------------------ */

/* An immutable description of one layer's packed experts. The handle is a small
 * host object; it refers to the caller's device planes, which must stay alive
 * and unchanged until moe_experts_destroy.
 *
 * Packed layout (fixed by this library; the pages publish none):
 *   experts 0..E-1 routed, then the shared expert (index E) when has_shared;
 *   each expert holds NB = 3*H*I/32 blocks of 32 weights: its gate matrix [I][H],
 *   then up [I][H], then down [H][I], each row-major with blocks along a row.
 *   codes: NB * 8 bytes per expert. Weight j (0..31) of a block is in byte j/4 at
 *          bits 2*(j%4) (the low two bits of the code for Q3).
 *   hi   : Q3 only, NB * 4 bytes per expert; bit j of the block's little-endian
 *          32-bit word is bit 2 of code j. Pass NULL for Q2.
 *   dm   : NB * 2 uint16 per expert: fp16 bits of d, then of m, per block.
 *   Weight value: w = d*q + m.
 * Plane bases must be 16-byte aligned. Requires H a multiple of 256 and I a
 * multiple of 128 (the matrix-core tile: 256 output rows of the down
 * projection, 128 rows each of gate and up), 1 <= E <= MOE_MAX_E; other
 * shapes return MOE_ERR_UNSUPPORTED. The decode GEMV kernels cover H/32 and
 * I/32 in {4, 8, 16, 32, 64}; other shapes run every expert on the
 * matrix-core tiles. */
typedef struct moe_experts moe_experts;

int moe_experts_create(moe_experts **out, int32_t qtype, int32_t E, int32_t has_shared,
                       int32_t H, int32_t I, const void *codes, const void *hi,
                       const void *dm);
int moe_experts_destroy(moe_experts *ex);

/* Optional second copy of the weights, in the order in which the prefill
 * matrix-core tiles read them, so that every wave's weight loads are
 * contiguous (the canonical planes give one 16-byte piece per weight row).
 * The pages' prompt path likewise runs on quantised expert data in kernel-
 * friendly form ("Strata - the details", "Faster prompts"); the arrangement
 * here is this library's own.
 *
 * moe_experts_tiled_size: bytes of the copy (the same as the codes, hi and dm
 *   planes together), or 0 for a null handle.
 * moe_experts_attach_tiled: enqueues on `stream` a device kernel that writes
 *   the copy into buf (device memory owned by the caller, at least
 *   moe_experts_tiled_size bytes, 16-byte aligned) from the canonical planes,
 *   and records buf in the handle; from then on moe_ffn_q and moe_layer run
 *   their matrix-core tiles on it (same results up to fp32 summation order).
 *   buf == NULL detaches. The caller keeps buf alive and unchanged until it
 *   detaches or destroys the handle, and must not call this while other calls
 *   on the handle are in flight on other streams.
 * Layout of the copy: codes [E_tot][3 matrices][R][64 lanes][16 bytes], then
 *   dm [E_tot][3][R][64][4 uint16], then (Q3) hi [E_tot][3][R][64][8 bytes],
 *   R = H*I/4096 records per matrix: for 32-row group g (rows 32g..32g+31 of
 *   the matrix) and block quad p (blocks 4p..4p+3 of each row), record
 *   g * (K/128) + p (K = the matrix's row length) holds for lane l the blocks
 *   4p + l/32 and 4p + 2 + l/32 of row 32g + l%32.
 * Errors: MOE_ERR_INVALID_ARG for a null handle, a misaligned buf or
 *   bytes below the size; MOE_ERR_HIP if the kernel launch fails. */
size_t moe_experts_tiled_size(const moe_experts *ex);
int moe_experts_attach_tiled(moe_experts *ex, void *buf, size_t bytes, void *stream);

/* ---- expert FFN and combine ---------------------------------------------- */

/* Workspace bytes moe_ffn_q needs for T tokens, k experts per token, `mode`,
 * including room for the grouping when the caller does not pass one. */
size_t moe_ffn_q_workspace_size(const moe_experts *ex, int32_t T, int32_t k, int32_t mode);

/* The routed expert FFN with gate-weighted combine, for T tokens.
 *
 * For every token t (expert = gate/up/down rows, "Low-RAM mode without
 * experts.bin"; shared experts for every token, "How it works"):
 *   o(e, x) = Wd_e . ( silu(Wg_e . x) * (Wu_e . x) ),   silu(z) = z / (1 + e^-z)
 *   y[t]    = sum_{j<k} gates[t][j] * o(idx[t][j], x[t])  +  o(shared, x[t])
 * with every weight dequantised as w = d*q + m from the handle's planes.
 *
 * x     : [T][H], dtype xdtype (MOE_F32 or MOE_BF16).
 * idx   : [T][k] int32 in [0, E); gates: [T][k] float32 (any values).
 * counts/offsets/perm/slot_of: a grouping of idx exactly as moe_group writes
 *         it, or all four NULL to have it computed inside `ws`.
 * y     : [T][H]; dtype xdtype in MOE_FAST, float32 in MOE_CHECK_F32.
 * ws    : device scratch of at least moe_ffn_q_workspace_size(ex, T, k, mode).
 * T == 0 is valid and launches nothing.
 *
 * Execution (fast mode; results agree within the FFN tolerance whichever form
 * runs): below 256 tokens with H 1024 or 2048 and I 256 or 512, every touched
 * expert runs on the small-batch matrix-core kernels (work items of expert,
 * output rows and 16 of its tokens); other batches below 256 tokens run
 * experts with 1..4 assignments on the GEMV kernels and the rest on the
 * matrix-core tiles; from 256 tokens on every expert runs on the tiles. */
int moe_ffn_q(const void *x, int32_t xdtype, int32_t T, const moe_experts *ex,
              const int32_t *idx, const float *gates, int32_t k, const int32_t *counts,
              const int32_t *offsets, const int32_t *perm, const int32_t *slot_of, void *y,
              int32_t mode, void *ws, size_t ws_bytes, void *stream);

/* ---- whole layer ---------------------------------------------------------- */

/* Workspace bytes moe_layer needs (device scratch). */
size_t moe_layer_workspace_size(const moe_experts *ex, int32_t T, int32_t k, int32_t mode);

/* The whole routed MoE layer in one call: top-k routing of `logits` ([T][E]
 * f32), the grouping, the expert FFN and the combine, writing idx and gates
 * ([T][k]) and y ([T][H]). Results match moe_route_group followed by
 * moe_ffn_q within the FFN tolerance (idx and gates identically).
 *
 * A decode verify window ("Strata - the details", "How it works": the drafted
 * tokens are checked in one pass) is fast mode with T <= 4, k <= 64 and H/32,
 * I/32 in {4..64}. With H a multiple of 1024 up to 4096, I 256 or 512,
 * E <= 512, T k <= 64 and T k + T (with a shared expert; T k without) at most
 * 32768 / I - 1 (the routed rows of h that the down rows hold at once: 63 at
 * I = 512, so k <= 14 at T = 4) it runs as ONE kernel: every workgroup routes the
 * window itself; the first workgroups compute gate/up rows, the others down
 * rows once counters at the head of `ws` show every gate/up row released; y is
 * reproducible run to run. Other windows run as two kernels (gate/up, then
 * down); other calls run moe_route_group then moe_ffn_q inside the workspace.
 *
 * ws: at least moe_layer_workspace_size(ex, T, k, mode) bytes. Its first 8192
 * bytes (the head) must be zero before the first call that uses it (a
 * zero-filled allocation). The one-kernel window keeps counters there that
 * count over all calls on the workspace; every call leaves them in a state the
 * next call can start from, also when a wait timed out; no other form of the
 * call writes the head, so one zeroed workspace serves every shape. Calls that
 * overlap in time must not share a workspace. A head whose first 128 bytes are
 * not zero shows as NaN in the window's y; a down row that waits longer than
 * about 0.2 s for the gate/up rows gives up and becomes NaN. Bytes 128..131 of
 * the head may hold a shorter bound on that wait, in ticks of the 100 MHz wall
 * clock (0 = the default); this exists for testing the timeout path. */
int moe_layer(const float *logits, const void *x, int32_t xdtype, int32_t T, const moe_experts *ex,
              int32_t k, int32_t *idx, float *gates, void *y, int32_t mode, void *ws,
              size_t ws_bytes, void *stream);

/* Router product and top-k in one launch, for many bf16 tokens: the logits of
 * moe_router_logits (written to `logits` [T][E] when not NULL) and their top-k
 * and gates as moe_route_topk ("Strata - the details", "How it works": the
 * router picks the experts that score highest), with no logits round trip
 * through memory between the two. x: [T][H] bf16 (xdtype MOE_BF16), w: [E][H]
 * bf16, both 16-byte aligned; bias: [E] float32 or NULL; idx, gates: [T][k].
 * The logits are f32 sums of exact bf16 products (matrix cores, a fixed
 * order), so idx and gates are exactly moe_route_topk of the logits written.
 * Each workgroup takes 32 tokens against every expert, so it reads the whole
 * router matrix from cache: measured at 8,192 tokens x 512 experts x 2,048 it
 * takes about 1.7 times as long as moe_router_logits followed by
 * moe_route_topk (which read the matrix once per 128 tokens); the layer calls
 * use those two.
 * Requires H % 256 == 0, H <= 4096, E 256 or 512, 1 <= k <= 64 (else
 * MOE_ERR_UNSUPPORTED); T == 0: no launch. */
int moe_router_topk(const void *x, int32_t xdtype, int32_t T, int32_t H, const uint16_t *w,
                    const float *bias, int32_t E, int32_t k, int32_t *idx, float *gates, float *logits,
                    void *stream);

/* ---- whole layer from hidden states --------------------------------------- */

/* Workspace bytes moe_layer_hidden needs: moe_layer's plus room for the
 * logits ([T][E] float32). */
size_t moe_layer_hidden_workspace_size(const moe_experts *ex, int32_t T, int32_t k, int32_t mode);

/* The layer from the tokens' hidden states: the router product
 * (moe_router_logits: logits[t][e] = x[t] . w_router[e] (+ bias[e]); "Strata -
 * the details", "How it works": each layer's router runs on the GPU in front
 * of its experts), then moe_layer on those logits. x: [T][H] as for moe_layer
 * (also the router's input); w_router: [E][H] bf16 (16-byte aligned); bias:
 * [E] float32 or NULL; logits: [T][E] float32 output, or NULL to keep them in
 * the workspace. idx, gates, y, mode and the workspace head as moe_layer; ws at
 * least moe_layer_hidden_workspace_size bytes.
 *
 * A decode window that moe_layer runs as one kernel runs here as one kernel
 * too: its first E / 16 workgroups compute the logits (an f32 sum of H
 * products per entry, in a fixed order) and store them; the other workgroups
 * wait for them through counters in the head (bounded like the window's other
 * wait; a wait that runs out makes y NaN and idx 0 .. k-1) and route from
 * them. Other calls launch the router product and then moe_layer (for many
 * tokens that is faster than moe_router_topk's single launch, see there). In
 * every form idx and gates are the top-k of the logits written.
 * Requires what moe_router_logits requires of H and E (else
 * MOE_ERR_UNSUPPORTED); other errors as moe_layer. */
int moe_layer_hidden(const void *x, int32_t xdtype, int32_t T, const uint16_t *w_router,
                     const float *bias, const moe_experts *ex, int32_t k, int32_t *idx, float *gates,
                     void *y, float *logits, int32_t mode, void *ws, size_t ws_bytes, void *stream);

/* ---- one expert's gate/up on the FP8 matrix cores (measured variant) -------- */

/* Workspace bytes moe_expert_gateup_fp8 needs for T tokens. */
size_t moe_expert_gateup_fp8_workspace_size(const moe_experts *ex, int32_t T);

/* h[t][r] = silu(g) * u of expert `expert` (0 .. E + has_shared - 1) for every
 * token row of x ([T][H] bf16, 16-byte aligned), g and u its gate and up
 * products: the analogue of the pages' 8-bit tensor-core prompt kernels
 * ("Strata - the details", "Speed (measured)") on the gfx950 FP8 matrix
 * cores, kept as a measured variant beside the layer's fp16 prefill tiles.
 * The codes enter the matrix cores as exact E4M3 values; each token row is
 * scaled by a power of two and split into two E4M3 parts (hi + lo, about 8
 * significant bits together); one product per 32-weight block, and d and m are
 * applied per block in fp32. h: [T][I] float32. Requires H % 64 == 0,
 * H <= 4096 and I % 32 == 0 (else MOE_ERR_UNSUPPORTED). ws: at least
 * moe_expert_gateup_fp8_workspace_size bytes (no zeroing needed); it holds the
 * E4M3 operands. Other errors as moe_ffn_q. */
int moe_expert_gateup_fp8(const void *x, int32_t T, const moe_experts *ex, int32_t expert, float *h,
                          void *ws, size_t ws_bytes, void *stream);

/* ---- whole layer without allocation --------------------------------------- */

/* Bytes of the library's own scratch array per GPU (moe_layer_static). */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)

/* moe_layer for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The same computation, results and kernels as moe_layer
 * (same arguments without ws/ws_bytes); the workspace is a 16 MiB array inside
 * the library, one per GPU, held until the process ends. The first call on a
 * device resolves that device's array and enqueues a small kernel on `stream`
 * that zeroes its first 8192 bytes; no call allocates or frees anything.
 * Calls whose moe_layer_workspace_size exceeds MOE_STATIC_SCRATCH_BYTES return
 * MOE_ERR_WORKSPACE before launching anything (decode windows and batches of a
 * few dozen tokens fit; 1,024-token prefill chunks do not). Every call on a GPU
 * uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results; serialise them.
 * Returns MOE_ERR_HIP if the device's array cannot be resolved. */
int moe_layer_static(const float *logits, const void *x, int32_t xdtype, int32_t T,
                     const moe_experts *ex, int32_t k, int32_t *idx, float *gates, void *y,
                     int32_t mode, void *stream);

/* ---- launch profiling ------------------------------------------------------ */

/* A measurement aid for the caller's own timing (per-kernel GPU durations).
 * moe_profile_begin: from now on every kernel the library launches carries
 *   two HIP events attached to its dispatch on its launch stream, which record
 *   the start and end of the kernel's execution, for up to max_launches
 *   launches (later launches are not recorded). Clears earlier records.
 *   Creates the events on first use (host-side objects, no device memory).
 * moe_profile_end: stops recording, waits for the recorded events and sums the
 *   elapsed time per kernel name.
 * moe_profile_count / moe_profile_get: the summary, one entry per kernel name:
 *   name (static string owned by the library), launches, total milliseconds.
 * The profiling state is process-global and not thread-safe; it is off unless
 * moe_profile_begin is called. */
int moe_profile_begin(int32_t max_launches);
int moe_profile_end(void);
int32_t moe_profile_count(void);
int moe_profile_get(int32_t i, const char **name, int32_t *launches, double *total_ms);

/* A static, human-readable description of a status code (host string). */
const char *moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

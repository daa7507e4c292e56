// Host implementation of the C ABI declared in include/moe.h: argument checks,
// workspace layout and kernel dispatch. Nothing here allocates device memory.
#include <mutex>
#include <new>

#include "../../include/moe.h"
#include "common.h"
#include "batch_x.h"

using moe::Experts;

struct moe_experts {
  Experts d;
};

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte layout of the moe_ffn_q workspace.
//   grouping (used when the caller passes none) | h [A][I] | x16 [T][H] |
//   xe [T] | o [A][H]
// h: fp32 in check mode, bf16 in fast mode. x16: the fp16 activation copy of
// the matrix-core kernels, xe its per-token exponents. o: gate-scaled expert
// outputs per assignment, fp32 in check mode and for few tokens, bf16
// otherwise.
struct FfnLayout {
  size_t counts, offsets, perm, slot_of, group, h, x16, xe, o, total;
  bool o_f32;
};

FfnLayout ffn_layout(const Experts& ex, int T, int k, int mode) {
  FfnLayout L{};
  const size_t A = (size_t)T * (k + ex.has_shared);
  size_t off = 0;
  L.counts = off;  off = align_up(off + sizeof(int32_t) * (ex.E + 1));
  L.offsets = off; off = align_up(off + sizeof(int32_t) * (ex.E + 2));
  L.perm = off;    off = align_up(off + sizeof(int32_t) * A);
  L.slot_of = off; off = align_up(off + sizeof(int32_t) * A);
  L.group = off;   off = align_up(off + moe::group_scratch_bytes(T, k, ex.E));
  L.h = off;       off = align_up(off + (mode == MOE_CHECK_F32 ? 4 : 2) * A * (size_t)ex.I);
  L.x16 = off;     off = align_up(off + (mode == MOE_CHECK_F32 ? 0 : 2) * (size_t)T * ex.H);
  L.xe = off;      off = align_up(off + (mode == MOE_CHECK_F32 ? 0 : sizeof(int32_t)) * (size_t)T);
  L.o_f32 = mode == MOE_CHECK_F32 || T <= moe::kF32SlotMaxTokens;
  L.o = off;       off = align_up(off + (L.o_f32 ? 4 : 2) * A * (size_t)ex.H);
  L.total = off;
  return L;
}

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, type or mode";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_router_logits(const void* x, int32_t xdtype, int32_t T, int32_t H, const uint16_t* w,
                      const float* bias, int32_t E, float* logits, void* stream) {
  if (T < 0 || H < 1 || E < 1 || (xdtype != MOE_F32 && xdtype != MOE_BF16)) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_E || !moe::router_supported(H, E)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * E > 0x7FFFFFFFLL || (long long)T * H > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w || !logits || !aligned16(x) || !aligned16(w)) return MOE_ERR_INVALID_ARG;
  return status_of(moe::launch_router(x, xdtype, T, H, w, bias, E, logits,
                                      static_cast<hipStream_t>(stream)));
}

int moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* idx, float* gates,
                   void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_E) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * E > 0x7FFFFFFFLL || (long long)T * k > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !idx || !gates) return MOE_ERR_INVALID_ARG;
  return status_of(moe::launch_topk(logits, T, E, k, idx, gates, static_cast<hipStream_t>(stream)));
}

size_t moe_group_workspace_size(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_E) return 0;
  return moe::group_scratch_bytes(T, k, E);
}

int moe_group(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t has_shared,
              int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_of, void* ws,
              size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || E < 1 || (has_shared != 0 && has_shared != 1)) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_E) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * (k + has_shared) > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!idx || !perm || !slot_of)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::group_scratch_bytes(T, k, E);
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE;
  return status_of(moe::launch_group(idx, T, k, E, has_shared, counts, offsets, perm, slot_of, ws,
                                     static_cast<hipStream_t>(stream)));
}

int moe_route_group(const float* logits, int32_t T, int32_t E, int32_t k, int32_t has_shared,
                    int32_t* idx, float* gates, int32_t* counts, int32_t* offsets, int32_t* perm,
                    int32_t* slot_of, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || (has_shared != 0 && has_shared != 1))
    return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_E) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * E > 0x7FFFFFFFLL || (long long)T * (k + has_shared) > 0x7FFFFFFFLL)
    return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !idx || !gates || !perm || !slot_of)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::group_scratch_bytes(T, k, E);
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return status_of(moe::launch_group(idx, T, k, E, has_shared, counts, offsets, perm,
                                                 slot_of, ws, s));
  return status_of(moe::launch_route_group(logits, T, E, k, has_shared, idx, gates, counts, offsets,
                                           perm, slot_of, ws, s));
}

int moe_experts_create(moe_experts** out, int32_t qtype, int32_t E, int32_t has_shared, int32_t H,
                       int32_t I, const void* codes, const void* hi, const void* dm) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  if (qtype != MOE_Q2 && qtype != MOE_Q3) return MOE_ERR_INVALID_ARG;
  if (E < 1 || (has_shared != 0 && has_shared != 1) || H < 64 || I < 64) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_E) return MOE_ERR_UNSUPPORTED;
  if (!moe::mfma_supported(H, I)) return MOE_ERR_UNSUPPORTED;
  if (!codes || !dm || (qtype == MOE_Q3) != (hi != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(dm) || (hi && !aligned16(hi))) return MOE_ERR_INVALID_ARG;
  moe_experts* ex = new (std::nothrow) moe_experts();
  if (!ex) return MOE_ERR_INVALID_ARG;
  ex->d.qtype = qtype;
  ex->d.E = E;
  ex->d.has_shared = has_shared;
  ex->d.E_tot = E + has_shared;
  ex->d.H = H;
  ex->d.I = I;
  ex->d.nb = (size_t)3 * H * I / 32;
  ex->d.codes = static_cast<const uint8_t*>(codes);
  ex->d.hi = static_cast<const uint8_t*>(hi);
  ex->d.dm = static_cast<const uint16_t*>(dm);
  *out = ex;
  return MOE_OK;
}

int moe_experts_destroy(moe_experts* ex) {
  delete ex;
  return MOE_OK;
}

size_t moe_experts_tiled_size(const moe_experts* ex) {
  if (!ex) return 0;
  const moe::Experts& d = ex->d;
  return (size_t)d.E_tot * d.nb * (8 + 4 + (d.qtype == MOE_Q3 ? 4 : 0));
}

int moe_experts_attach_tiled(moe_experts* ex, void* buf, size_t bytes, void* stream) {
  if (!ex) return MOE_ERR_INVALID_ARG;
  moe::Experts& d = ex->d;
  if (!buf) {
    d.t_codes = nullptr;
    d.t_dm = nullptr;
    d.t_hi = nullptr;
    return MOE_OK;
  }
  if (!aligned16(buf) || bytes < moe_experts_tiled_size(ex)) return MOE_ERR_INVALID_ARG;
  const size_t nblk = (size_t)d.E_tot * d.nb;
  uint8_t* base = static_cast<uint8_t*>(buf);
  moe::Experts t = d;
  t.t_codes = base;
  t.t_dm = reinterpret_cast<const uint16_t*>(base + nblk * 8);
  t.t_hi = d.qtype == MOE_Q3 ? base + nblk * 12 : nullptr;
  const hipError_t e = moe::launch_tile_weights(t, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return MOE_ERR_HIP;
  d = t;
  return MOE_OK;
}

size_t moe_ffn_q_workspace_size(const moe_experts* ex, int32_t T, int32_t k, int32_t mode) {
  if (!ex || T < 0 || k < 1 || k > ex->d.E) return 0;
  if (mode != MOE_FAST && mode != MOE_CHECK_F32) return 0;
  return ffn_layout(ex->d, T, k, mode).total;
}

}  // extern "C"

namespace {

// Fast mode below 256 tokens on shapes the small-batch kernels cover.
inline bool batch_path(const Experts& d, int T, int mode) {
  return mode == MOE_FAST && T < moe::kGemvBatchLimit && moe::batch_supported(d.H, d.I);
}

// GEMV token limit of fast mode outside the small-batch path: from a few
// hundred tokens on, experts with few assignments ride in the persistent
// matrix-core grid, where their weight reads overlap the other tiles'
// arithmetic; a separate GEMV pass would run on its own.
inline int gemv_max(const Experts& d, int T) {
  const bool small_batch = T < moe::kGemvBatchLimit || !moe::mfma_supported(d.H, d.I);
  return moe::gemv_supported(d.H, d.I) && small_batch ? moe::kGemvMaxTokens : 0;
}

// The fp16 activation copy the FFN's matrix-core kernels read, as the Q of an
// XsJob: the small-batch layout (2, 3), the prefill tiles' copy (0), or none
// (-1: check mode, or GEMV kernels only).
inline int x16_kind(const Experts& d, int T, int mode) {
  if (mode != MOE_FAST) return -1;
  if (batch_path(d, T, mode)) return d.qtype;
  return T > gemv_max(d, T) ? 0 : -1;
}

// moe_ffn_q; xs_ready: the workspace's x16 already holds the small-batch
// activation layout (written by the caller's grouping launch).
int ffn_q_impl(const void* x, int32_t xdtype, int32_t T, const moe_experts* ex, const int32_t* idx,
               const float* gates, int32_t k, const int32_t* counts, const int32_t* offsets,
               const int32_t* perm, const int32_t* slot_of, void* y, int32_t mode, void* ws,
               size_t ws_bytes, void* stream, bool xs_ready) {
  if (!ex || T < 0 || k < 1 || k > ex->d.E) return MOE_ERR_INVALID_ARG;
  if (xdtype != MOE_F32 && xdtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_FAST && mode != MOE_CHECK_F32) return MOE_ERR_INVALID_ARG;
  const Experts& d = ex->d;
  const long long A = (long long)T * (k + d.has_shared);
  if (A > 0x7FFFFFFFLL || A * d.H > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  const int given = (counts != nullptr) + (offsets != nullptr) + (perm != nullptr) + (slot_of != nullptr);
  if (given != 0 && given != 4) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !idx || !gates || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(d, T, k, mode);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  moe::FfnArgs a{};
  a.x = x;
  a.xdtype = xdtype;
  a.T = T;
  a.k = k;
  a.idx = idx;
  a.gates = gates;
  a.y = y;
  a.h = at(ws, L.h);
  a.x16 = reinterpret_cast<uint16_t*>(at(ws, L.x16));
  a.xe = reinterpret_cast<int32_t*>(at(ws, L.xe));
  a.xs_ready = xs_ready;
  if (given == 4) {
    a.counts = counts;
    a.offsets = offsets;
    a.perm = perm;
    a.slot_of = slot_of;
  } else {
    int32_t* c = reinterpret_cast<int32_t*>(at(ws, L.counts));
    int32_t* o = reinterpret_cast<int32_t*>(at(ws, L.offsets));
    int32_t* p = reinterpret_cast<int32_t*>(at(ws, L.perm));
    int32_t* so = reinterpret_cast<int32_t*>(at(ws, L.slot_of));
    // the fp16 activation copy rides in the grouping launch
    const int kind = x16_kind(d, T, mode);
    const moe::XsJob xj = moe::xs_job(kind, d.H, x, xdtype, T, a.x16, a.xe);
    bool xs_done = false;
    hipError_t e = moe::launch_group(idx, T, k, d.E, d.has_shared, c, o, p, so, at(ws, L.group), s,
                                     kind >= 0 ? &xj : nullptr, &xs_done);
    if (e != hipSuccess) return MOE_ERR_HIP;
    a.xs_ready = xs_done;
    a.counts = c;
    a.offsets = o;
    a.perm = p;
    a.slot_of = so;
  }
  a.out_f32 = mode == MOE_CHECK_F32 || xdtype == MOE_F32;
  if (L.o_f32) a.o = reinterpret_cast<float*>(at(ws, L.o));
  else a.ob = reinterpret_cast<uint16_t*>(at(ws, L.o));
  hipError_t e;
  if (mode == MOE_CHECK_F32) {
    e = moe::launch_ffn_check(d, a, s);
  } else {
    if (batch_path(d, T, mode)) {
      e = moe::launch_batch(d, a, s);
    } else {
      a.gmax = gemv_max(d, T);
      e = moe::launch_ffn_fast(d, a, s);
    }
  }
  if (e == hipSuccess) e = moe::launch_combine(d, a, s);
  return status_of(e);
}

}  // namespace

extern "C" {

int moe_ffn_q(const void* x, int32_t xdtype, int32_t T, const moe_experts* ex, const int32_t* idx,
              const float* gates, int32_t k, const int32_t* counts, const int32_t* offsets,
              const int32_t* perm, const int32_t* slot_of, void* y, int32_t mode, void* ws,
              size_t ws_bytes, void* stream) {
  return ffn_q_impl(x, xdtype, T, ex, idx, gates, k, counts, offsets, perm, slot_of, y, mode, ws,
                    ws_bytes, stream, false);
}

// ---- whole layer -----------------------------------------------------------

namespace {
struct LayerLayout {
  bool window;
  size_t counts, offsets, perm, slot_of, group, ffn, total;
};

LayerLayout layer_layout(const Experts& d, int T, int k, int mode) {
  LayerLayout L{};
  L.window = mode == MOE_FAST && moe::window_supported(d, T, k);
  if (L.window) {
    L.total = align_up(moe::window_workspace_bytes(d, T, k));
    return L;
  }
  const size_t A = (size_t)T * (k + d.has_shared);
  size_t off = moe::kWinSyncBytes;  // kept zero for the decode window's counters
  L.counts = off;  off = align_up(off + sizeof(int32_t) * (d.E + 1));
  L.offsets = off; off = align_up(off + sizeof(int32_t) * (d.E + 2));
  L.perm = off;    off = align_up(off + sizeof(int32_t) * (A ? A : 1));
  L.slot_of = off; off = align_up(off + sizeof(int32_t) * (A ? A : 1));
  L.group = off;   off = align_up(off + moe::group_scratch_bytes(T, k, d.E));
  L.ffn = off;     off = align_up(off + ffn_layout(d, T, k, mode).total);
  L.total = off;
  return L;
}
}  // namespace

size_t moe_layer_workspace_size(const moe_experts* ex, int32_t T, int32_t k, int32_t mode) {
  if (!ex || T < 0 || k < 1 || k > ex->d.E) return 0;
  if (mode != MOE_FAST && mode != MOE_CHECK_F32) return 0;
  return layer_layout(ex->d, T, k, mode).total;
}

int moe_layer(const float* logits, const void* x, int32_t xdtype, int32_t T, const moe_experts* ex,
              int32_t k, int32_t* idx, float* gates, void* y, int32_t mode, void* ws, size_t ws_bytes,
              void* stream) {
  if (!ex || T < 0 || k < 1 || k > ex->d.E) return MOE_ERR_INVALID_ARG;
  if (xdtype != MOE_F32 && xdtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_FAST && mode != MOE_CHECK_F32) return MOE_ERR_INVALID_ARG;
  const Experts& d = ex->d;
  const long long A = (long long)T * (k + d.has_shared);
  if ((long long)T * d.E > 0x7FFFFFFFLL || A > 0x7FFFFFFFLL || A * d.H > (1LL << 40))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !x || !idx || !gates || !y || !aligned16(x) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  const LayerLayout L = layer_layout(d, T, k, mode);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.window)
    return status_of(moe::launch_window(logits, T, k, d, x, xdtype, idx, gates, y,
                                        xdtype == MOE_F32, ws, s));
  int32_t* c = reinterpret_cast<int32_t*>(at(ws, L.counts));
  int32_t* o = reinterpret_cast<int32_t*>(at(ws, L.offsets));
  int32_t* p = reinterpret_cast<int32_t*>(at(ws, L.perm));
  int32_t* so = reinterpret_cast<int32_t*>(at(ws, L.slot_of));
  // the FFN's fp16 activation copy rides in the routing's grouping launch
  const FfnLayout F = ffn_layout(d, T, k, mode);
  const int kind = x16_kind(d, T, mode);
  const moe::XsJob xj = moe::xs_job(kind, d.H, x, xdtype, T, reinterpret_cast<uint16_t*>(at(ws, L.ffn + F.x16)),
                                    reinterpret_cast<int32_t*>(at(ws, L.ffn + F.xe)));
  bool xs_done = false;
  const hipError_t e = moe::launch_route_group(logits, T, d.E, k, d.has_shared, idx, gates, c, o, p, so,
                                               at(ws, L.group), s, kind >= 0 ? &xj : nullptr,
                                               &xs_done);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return ffn_q_impl(x, xdtype, T, ex, idx, gates, k, c, o, p, so, y, mode, at(ws, L.ffn),
                    ws_bytes - L.ffn, stream, xs_done);
}

// ---- router product + top-k in one launch ----------------------------------------

int moe_router_topk(const void* x, int32_t xdtype, int32_t T, int32_t H, const uint16_t* w,
                    const float* bias, int32_t E, int32_t k, int32_t* idx, float* gates, float* logits,
                    void* stream) {
  if (T < 0 || H < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (xdtype != MOE_F32 && xdtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!moe::router_topk_supported(xdtype, H, E, k)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * E > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w || !idx || !gates || !aligned16(x) || !aligned16(w)) return MOE_ERR_INVALID_ARG;
  return status_of(moe::launch_router_topk(x, T, H, w, bias, E, k, logits, idx, gates,
                                           static_cast<hipStream_t>(stream)));
}

// ---- whole layer from hidden states -------------------------------------------


size_t moe_layer_hidden_workspace_size(const moe_experts* ex, int32_t T, int32_t k, int32_t mode) {
  const size_t base = moe_layer_workspace_size(ex, T, k, mode);
  if (!base) return 0;
  return base + align_up(sizeof(uint64_t) * (size_t)T * ex->d.E);  // tagged (window) or plain logits
}

int moe_layer_hidden(const void* x, int32_t xdtype, int32_t T, const uint16_t* w_router,
                     const float* bias, const moe_experts* ex, int32_t k, int32_t* idx, float* gates,
                     void* y, float* logits, int32_t mode, void* ws, size_t ws_bytes, void* stream) {
  if (!ex || T < 0 || k < 1 || k > ex->d.E) return MOE_ERR_INVALID_ARG;
  if (xdtype != MOE_F32 && xdtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_FAST && mode != MOE_CHECK_F32) return MOE_ERR_INVALID_ARG;
  const Experts& d = ex->d;
  if (!moe::router_supported(d.H, d.E)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * d.E > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !idx || !gates || !y || !aligned16(x) || !aligned16(y) || !aligned16(w_router))
    return MOE_ERR_INVALID_ARG;
  const LayerLayout L = layer_layout(d, T, k, mode);
  if (!ws || ws_bytes < moe_layer_hidden_workspace_size(ex, T, k, mode)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.window && moe::window_hidden_supported(d, T, k))
    return status_of(moe::launch_window_hidden(logits, reinterpret_cast<uint64_t*>(at(ws, L.total)),
                                               w_router, bias, T, k, d, x, xdtype, idx, gates, y,
                                               xdtype == MOE_F32, ws, s));
  float* lg = logits ? logits : reinterpret_cast<float*>(at(ws, L.total));
  if (moe::launch_router(x, xdtype, T, d.H, w_router, bias, d.E, lg, s) != hipSuccess) return MOE_ERR_HIP;
  return moe_layer(lg, x, xdtype, T, ex, k, idx, gates, y, mode, ws, L.total, stream);
}

// ---- one expert's gate/up on the FP8 matrix cores (measured variant) ----------

size_t moe_expert_gateup_fp8_workspace_size(const moe_experts* ex, int32_t T) {
  if (!ex || T < 0) return 0;
  return moe::fp8_gateup_workspace_bytes(ex->d, T);
}

int moe_expert_gateup_fp8(const void* x, int32_t T, const moe_experts* ex, int32_t expert, float* h,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!ex || T < 0 || expert < 0 || expert >= ex->d.E_tot) return MOE_ERR_INVALID_ARG;
  if (!moe::fp8_gateup_supported(ex->d)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * ex->d.H > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !h || !aligned16(x)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe::fp8_gateup_workspace_bytes(ex->d, T)) return MOE_ERR_WORKSPACE;
  return status_of(moe::launch_fp8_gateup(ex->d, expert, static_cast<const uint16_t*>(x), T, h, ws,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- whole layer without allocation ------------------------------------------

namespace {

// Scratch of moe_layer_static: one array per GPU the library runs on, kept
// until the process ends. In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_static_once[kMaxDevices];
void* g_static_ptr[kMaxDevices];
hipError_t g_static_err[kMaxDevices];

// Zeroes the head of the scratch (the decode window's counters) once at set-up.
__global__ __launch_bounds__(256) void zero_head(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// The calling thread's current device's scratch address, resolved (and its
// head zeroed on `s`) on the first call for that device.
int static_scratch(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::call_once(g_static_once[dev], [&]() {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p) {
      hipLaunchKernelGGL(zero_head, dim3(8), dim3(256), 0, s, static_cast<uint32_t*>(p),
                         (int)(moe::kWinSyncBytes / sizeof(uint32_t)));
      e = hipGetLastError();
    } else if (e == hipSuccess) {
      e = hipErrorInvalidSymbol;
    }
    g_static_err[dev] = e;
    g_static_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  if (g_static_err[dev] != hipSuccess || !g_static_ptr[dev]) return MOE_ERR_HIP;
  *out = g_static_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_static(const float* logits, const void* x, int32_t xdtype, int32_t T,
                     const moe_experts* ex, int32_t k, int32_t* idx, float* gates, void* y,
                     int32_t mode, void* stream) {
  if (!ex || T < 0 || k < 1 || k > ex->d.E) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_FAST && mode != MOE_CHECK_F32) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (layer_layout(ex->d, T, k, mode).total > kStaticBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = static_scratch(static_cast<hipStream_t>(stream), &ws);
  if (st != MOE_OK) return st;
  return moe_layer(logits, x, xdtype, T, ex, k, idx, gates, y, mode, ws, kStaticBytes, stream);
}

}  // extern "C"

// coli.cpp -- the C ABI of libcoli.so (declared in include/coli.h).
//
// Host side only: validates every argument before the first launch (fail
// closed: on error nothing is written), carves the caller's workspace, and
// enqueues the HIP kernels on the caller's stream.  No allocation, no
// synchronisation, no global mutable state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "coli.h"
#include "kernels.h"

using namespace coli;

namespace {

inline bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}
inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
inline int dev_status(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_EDEVICE; }

bool layer_shape_ok(int H, int I, int E, int K) {
  return H >= 64 && H <= COLI_MAX_DIM && H % 64 == 0 && I >= 64 && I <= COLI_MAX_DIM &&
         I % 64 == 0 && E >= 1 && E <= COLI_MAX_EXPERTS && K >= 1 && K <= E;
}

// Workspace carve-up (byte offsets, each section 256-byte aligned).
struct WsLayout {
  size_t logits, idx, gates, counts, offsets, perm, unique, n_unique, chunk, h, slot;
  size_t xp, sx, sh;                          // prefill only
  size_t slotmap;                             // decode only
  size_t xdig, xcorr, nxsc, hn;               // decode, single-token path
  size_t bxp, bxs, bhf, bh16, bhs, bslot;     // decode batch path
  size_t total;
};
WsLayout ws_layout(int H, int I, int E, int K, int T, coli_mode mode) {
  WsLayout w;
  const size_t TK = size_t(T) * K;
  size_t o = 0;
  w.logits = o; o += align256(size_t(T) * E * 4);
  w.idx = o; o += align256(TK * 4);
  w.gates = o; o += align256(TK * 4);
  w.counts = o; o += align256(size_t(E) * 4);
  w.offsets = o; o += align256(size_t(E + 1) * 4);
  w.perm = o; o += align256(TK * 4);
  w.unique = o; o += align256(size_t(E) * 4);
  w.n_unique = o; o += 256;
  size_t chunk = permute_chunk_ints(T, E);
  if (chunk < size_t(E) + 2) chunk = size_t(E) + 2;
  w.chunk = o; o += align256(chunk * 4);
  w.xp = w.sx = w.sh = 0;
  w.h = w.slot = w.slotmap = 0;
  w.xdig = w.xcorr = w.nxsc = w.hn = 0;
  w.bxp = w.bxs = w.bhf = w.bh16 = w.bhs = w.bslot = 0;
  if (mode == COLI_PREFILL) {
    const PrefillLayout pl = prefill_layout(H, I);
    w.xp = o; o += align256(size_t(T) * pl.HP * 2);
    w.sx = o; o += align256(size_t(T) * pl.CSX * 2);
    w.h = o; o += align256((TK + T) * size_t(pl.IP) * 2);
    w.sh = o; o += align256((TK + T) * size_t(pl.CSI) * 2);
    w.slot = o; o += align256((TK + T) * size_t(H) * 2);
  } else {
    const size_t units = TK < size_t(E) ? TK : size_t(E);
    w.slotmap = o; o += align256(units * size_t(T) * 4);
    const size_t GH = size_t(groups_of(H));
    w.xdig = o; o += align256(size_t(T) * GH * 256);
    w.xcorr = o; o += align256(size_t(T) * GH * 16);
    w.nxsc = o; o += align256(size_t(T) * 4);
    w.hn = o; o += align256((units + 1) * size_t(I) * 4);
    const PrefillLayout pl = prefill_layout(H, I);
    const size_t R = TK + T;
    w.bxp = o; o += align256(2 * size_t(T) * pl.HP * 2);
    w.bxs = o; o += align256(size_t(T) * 4);
    w.bhf = o; o += align256(R * size_t(I) * 4);
    w.bh16 = o; o += align256(2 * R * size_t(pl.IP) * 2);
    w.bhs = o; o += align256(R * 4);
    w.bslot = o; o += align256(R * size_t(H) * 4);
  }
  w.total = o;
  return w;
}

Routing carve(uint8_t *ws, const WsLayout &w) {
  Routing r;
  r.logits = reinterpret_cast<float *>(ws + w.logits);
  r.idx = reinterpret_cast<int32_t *>(ws + w.idx);
  r.gates = reinterpret_cast<float *>(ws + w.gates);
  r.counts = reinterpret_cast<int32_t *>(ws + w.counts);
  r.offsets = reinterpret_cast<int32_t *>(ws + w.offsets);
  r.perm = reinterpret_cast<int32_t *>(ws + w.perm);
  r.unique = reinterpret_cast<int32_t *>(ws + w.unique);
  r.n_unique = reinterpret_cast<int32_t *>(ws + w.n_unique);
  r.chunk = reinterpret_cast<int32_t *>(ws + w.chunk);
  return r;
}

}  // namespace

extern "C" {

const char *coli_strerror(int status) {
  switch (status) {
    case COLI_OK: return "ok";
    case COLI_EINVAL: return "invalid argument (NULL pointer or bad value)";
    case COLI_ESHAPE: return "dimension out of range";
    case COLI_EALIGN: return "pointer not aligned as required";
    case COLI_EDTYPE: return "dtype not supported here";
    case COLI_EWORKSPACE: return "workspace missing or too small";
    case COLI_EDEVICE: return "HIP runtime reported a launch error";
    default: return "unknown status";
  }
}

size_t coli_int4_g64_packed_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 1) return 0;
  return size_t(rows) * size_t(groups_of(cols)) * 32;
}

size_t coli_int4_g64_scale_count(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 1) return 0;
  return size_t(rows) * size_t(groups_of(cols));
}

int coli_quant_int4_g64(const float *w, int64_t rows, int64_t cols, uint8_t *packed,
                        float *scales, int32_t *status, void *stream) {
  if ((!w || !packed || !scales) && rows != 0) return COLI_EINVAL;
  if (rows < 0 || cols < 1 || (rows > 0 && cols > (int64_t(1) << 40) / rows))
    return COLI_ESHAPE;
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(scales, 4) ||
      (status && !aligned(status, 4)))
    return COLI_EALIGN;
  if (rows == 0) return COLI_OK;
  return dev_status(
      launch_quant_int4_g64(w, rows, cols, packed, scales, status, as_stream(stream)));
}

int coli_router_topk(const void *x, coli_dtype x_dtype, int T, int H, const void *w_router,
                     coli_dtype w_dtype, int E, const float *bias, int K, int32_t *topk_idx,
                     float *topk_gate, float *logits, void *stream) {
  if (!w_router) return COLI_EINVAL;
  if ((!x || !topk_idx || !topk_gate || !logits) && T != 0) return COLI_EINVAL;
  if (T < 0 || T > COLI_MAX_TOKENS || H < 8 || H > COLI_MAX_DIM || H % 8 || E < 1 ||
      E > COLI_MAX_EXPERTS || K < 1 || K > E)
    return COLI_ESHAPE;
  if ((x_dtype != COLI_F32 && x_dtype != COLI_BF16) ||
      (w_dtype != COLI_F32 && w_dtype != COLI_BF16))
    return COLI_EDTYPE;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(topk_idx, 4) ||
      !aligned(topk_gate, 4) || !aligned(logits, 4) || (bias && !aligned(bias, 4)))
    return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_router_logits(x, x_dtype == COLI_BF16, T, H, w_router,
                                      w_dtype == COLI_BF16, E, bias, logits, s);
  if (e != hipSuccess) return COLI_EDEVICE;
  return dev_status(launch_topk(logits, T, E, K, topk_idx, topk_gate, s));
}

size_t coli_expert_permute_workspace_bytes(int T, int E) {
  if (T < 0 || T > COLI_MAX_TOKENS || E < 1 || E > COLI_MAX_EXPERTS) return 0;
  return permute_chunk_ints(T, E) * 4;
}

int coli_expert_permute(const int32_t *topk_idx, int T, int K, int E, int32_t *counts,
                        int32_t *offsets, int32_t *perm, int32_t *unique, int32_t *n_unique,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (!counts || !offsets || !unique || !n_unique) return COLI_EINVAL;
  if ((!topk_idx || !perm) && T > 0) return COLI_EINVAL;
  if (T < 0 || T > COLI_MAX_TOKENS || E < 1 || E > COLI_MAX_EXPERTS || K < 1 || K > E)
    return COLI_ESHAPE;
  if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(perm, 4) || !aligned(unique, 4) || !aligned(n_unique, 4) ||
      (workspace && !aligned(workspace, 4)))
    return COLI_EALIGN;
  const size_t need = permute_chunk_ints(T, E) * 4;
  if (need && (!workspace || workspace_bytes < need)) return COLI_EWORKSPACE;
  Routing r;
  std::memset(&r, 0, sizeof(r));
  r.idx = const_cast<int32_t *>(topk_idx);
  r.counts = counts;
  r.offsets = offsets;
  r.perm = perm;
  r.unique = unique;
  r.n_unique = n_unique;
  r.chunk = reinterpret_cast<int32_t *>(workspace);
  return dev_status(launch_topk_permute(r, T, E, K, 0, as_stream(stream)));
}

size_t coli_expert_blob_bytes(int H, int I) {
  if (H < 1 || H > COLI_MAX_DIM || I < 1 || I > COLI_MAX_DIM) return 0;
  return blob_layout(H, I).bytes;
}

int coli_expert_views(const uint8_t *blob, int H, int I, coli_q4 *gate, coli_q4 *up,
                      coli_q4 *down) {
  if (!blob || !gate || !up || !down) return COLI_EINVAL;
  if (H < 1 || H > COLI_MAX_DIM || I < 1 || I > COLI_MAX_DIM) return COLI_ESHAPE;
  const BlobLayout b = blob_layout(H, I);
  gate->q = blob + b.gq;
  gate->s = reinterpret_cast<const float *>(blob + b.gs);
  up->q = blob + b.uq;
  up->s = reinterpret_cast<const float *>(blob + b.us);
  down->q = blob + b.dq;
  down->s = reinterpret_cast<const float *>(blob + b.ds);
  return COLI_OK;
}

int coli_expert_finish(uint8_t *blob, int H, int I, void *stream) {
  if (!blob) return COLI_EINVAL;
  if (H < 1 || H > COLI_MAX_DIM || I < 1 || I > COLI_MAX_DIM) return COLI_ESHAPE;
  if (!aligned(blob, 256)) return COLI_EALIGN;
  return dev_status(launch_expert_finish(blob, blob_layout(H, I), H, I, as_stream(stream)));
}

size_t coli_moe_workspace_bytes(const coli_moe_layer *L, int T, coli_mode mode) {
  if (!L || !layer_shape_ok(L->H, L->I, L->E, L->K)) return 0;
  if (mode != COLI_DECODE && mode != COLI_PREFILL) return 0;
  const int tmax = mode == COLI_DECODE ? COLI_MAX_DECODE_T : COLI_MAX_TOKENS;
  if (T < 0 || T > tmax) return 0;
  return ws_layout(L->H, L->I, L->E, L->K, T, mode).total;
}

namespace {

int moe_forward_impl(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                     int32_t *topk_idx_out, float *topk_gate_out, void *workspace,
                     size_t workspace_bytes, void *stream, hipEvent_t *ev) {
  if (!L || !L->w_router || !L->experts || !L->shared) return COLI_EINVAL;
  if ((!x || !y) && T != 0) return COLI_EINVAL;
  if (mode != COLI_DECODE && mode != COLI_PREFILL) return COLI_EINVAL;
  if (!layer_shape_ok(L->H, L->I, L->E, L->K)) return COLI_ESHAPE;
  const int tmax = mode == COLI_DECODE ? COLI_MAX_DECODE_T : COLI_MAX_TOKENS;
  if (T < 0 || T > tmax) return COLI_ESHAPE;
  if (L->router_dtype != COLI_F32 && L->router_dtype != COLI_BF16) return COLI_EDTYPE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(L->w_router, 16) ||
      !aligned(L->experts, 256) || !aligned(L->shared, 256) ||
      (L->router_bias && !aligned(L->router_bias, 4)) ||
      (topk_idx_out && !aligned(topk_idx_out, 4)) ||
      (topk_gate_out && !aligned(topk_gate_out, 4)))
    return COLI_EALIGN;
  const WsLayout w = ws_layout(L->H, L->I, L->E, L->K, T, mode);
  if (!workspace || workspace_bytes < w.total) return COLI_EWORKSPACE;
  if (!aligned(workspace, 256)) return COLI_EALIGN;
  if (T == 0) return COLI_OK;

  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  Routing r = carve(ws, w);
  if (topk_idx_out) r.idx = topk_idx_out;
  if (topk_gate_out) r.gates = topk_gate_out;
  LayerDev d;
  d.H = L->H;
  d.I = L->I;
  d.E = L->E;
  d.K = L->K;
  d.experts = L->experts;
  d.shared = L->shared;
  d.lay = blob_layout(L->H, L->I);
  hipStream_t s = as_stream(stream);
  const int wbf = L->router_dtype == COLI_BF16;

  hipError_t e;
  if (mode == COLI_PREFILL && ev) (void)hipEventRecord(ev[0], s);
  if (mode == COLI_DECODE) {
    int32_t *slotmap = reinterpret_cast<int32_t *>(ws + w.slotmap);
    if (narrow_supported(d, T)) {
      NarrowBufs nb;
      nb.xdig = reinterpret_cast<int8_t *>(ws + w.xdig);
      nb.xcorr = reinterpret_cast<int32_t *>(ws + w.xcorr);
      nb.xsc = reinterpret_cast<float *>(ws + w.nxsc);
      nb.hn = reinterpret_cast<float *>(ws + w.hn);
      // one kernel per stage: the events are stamped by the launches
      e = launch_router_narrow(reinterpret_cast<const float *>(x), T, L->H, L->w_router, wbf,
                               L->E, L->router_bias, r.logits, nb, s, ev ? ev[0] : nullptr,
                               ev ? ev[1] : nullptr);
      if (e != hipSuccess) return COLI_EDEVICE;
      return dev_status(launch_ffn_narrow(d, nb, r.logits, r.idx, r.gates,
                                          reinterpret_cast<float *>(y), s, ev ? ev + 2 : nullptr));
    }
    BatchBufs bb;
    bb.xp = reinterpret_cast<uint16_t *>(ws + w.bxp);
    bb.xs = reinterpret_cast<float *>(ws + w.bxs);
    bb.hf = reinterpret_cast<float *>(ws + w.bhf);
    bb.h16 = reinterpret_cast<uint16_t *>(ws + w.bh16);
    bb.hs = reinterpret_cast<float *>(ws + w.bhs);
    bb.slot = reinterpret_cast<float *>(ws + w.bslot);
    if (ev) (void)hipEventRecord(ev[0], s);
    // the router launch also writes x's staged rows for the batch GEMM
    e = launch_router_logits(x, 0, T, L->H, L->w_router, wbf, L->E, L->router_bias, r.logits, s,
                             bb.xp, bb.xs, prefill_layout(L->H, L->I).HP);
    if (e != hipSuccess) return COLI_EDEVICE;
    e = launch_route_decode(r, T, L->E, L->K, slotmap, s);
    if (e != hipSuccess) return COLI_EDEVICE;
    if (ev) (void)hipEventRecord(ev[1], s);
    e = launch_ffn_batch(d, reinterpret_cast<const float *>(x), T, r, bb,
                         reinterpret_cast<float *>(y), s, ev ? ev + 2 : nullptr, true);
    return dev_status(e);
  }
  if (wbf) {
    // the staged-x region is free until the activation conversion: it holds the
    // router's K-split partial sums
    const PrefillLayout pl = prefill_layout(L->H, L->I);
    e = launch_router_topk_mfma(reinterpret_cast<const uint16_t *>(x), T, L->H,
                                reinterpret_cast<const uint16_t *>(L->w_router), L->E,
                                L->router_bias, L->K, r.logits, r.idx, r.gates,
                                reinterpret_cast<float *>(ws + w.xp),
                                size_t(T) * pl.HP * 2, s);
    if (e != hipSuccess) return COLI_EDEVICE;
    e = launch_topk_permute(r, T, L->E, L->K, 0, s);
  } else {
    e = launch_router_logits(x, 1, T, L->H, L->w_router, 0, L->E, L->router_bias, r.logits, s);
    if (e != hipSuccess) return COLI_EDEVICE;
    e = launch_topk_permute(r, T, L->E, L->K, 1, s);
  }
  if (e != hipSuccess) return COLI_EDEVICE;
  if (ev) (void)hipEventRecord(ev[1], s);
  PrefillBufs pb;
  pb.xp = reinterpret_cast<uint16_t *>(ws + w.xp);
  pb.sx = reinterpret_cast<uint16_t *>(ws + w.sx);
  pb.h = reinterpret_cast<uint16_t *>(ws + w.h);
  pb.sh = reinterpret_cast<uint16_t *>(ws + w.sh);
  pb.slot = reinterpret_cast<uint16_t *>(ws + w.slot);
  e = launch_ffn_prefill(d, reinterpret_cast<const uint16_t *>(x), T, r, pb,
                         reinterpret_cast<uint16_t *>(y), s, ev ? ev + 2 : nullptr);
  return dev_status(e);
}

}  // namespace

int coli_moe_forward(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                     int32_t *topk_idx_out, float *topk_gate_out, void *workspace,
                     size_t workspace_bytes, void *stream) {
  return moe_forward_impl(L, mode, x, T, y, topk_idx_out, topk_gate_out, workspace,
                          workspace_bytes, stream, nullptr);
}

int coli_moe_forward_timed(const coli_moe_layer *L, coli_mode mode, const void *x, int T,
                           void *y, int32_t *topk_idx_out, float *topk_gate_out,
                           void *workspace, size_t workspace_bytes, void *stream, void **events,
                           int n_events) {
  const int need = 2 * (mode == COLI_PREFILL ? 5 : 3);
  if (!events || n_events < need) return COLI_EINVAL;
  for (int i = 0; i < need; ++i)
    if (!events[i]) return COLI_EINVAL;
  return moe_forward_impl(L, mode, x, T, y, topk_idx_out, topk_gate_out, workspace,
                          workspace_bytes, stream, reinterpret_cast<hipEvent_t *>(events));
}

int coli_rmsnorm_f32(const float *x, float *y, int T, int H, float eps, void *stream) {
  if (((!x || !y) && T != 0) || !(eps >= 0.0f) || !std::isfinite(eps)) return COLI_EINVAL;
  if (T < 0 || T > COLI_MAX_TOKENS || H < 1 || H > COLI_MAX_DIM) return COLI_ESHAPE;
  if (!aligned(x, 4) || !aligned(y, 4)) return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  return dev_status(launch_rmsnorm_f32(x, y, T, H, eps, as_stream(stream)));
}

}  // extern "C"

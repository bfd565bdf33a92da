// coli.cpp -- the C ABI of libcoli.so (declared in include/coli.h).
//
// Host side only: validates every argument before the first launch (fail
// closed: on error nothing is written), carves the caller's workspace, and
// enqueues the HIP kernels on the caller's stream.  No allocation, no
// synchronisation, no global mutable state.  (coli_moe_forward_noalloc, in
// noalloc.hip, adds a per-device address cache for its static scratch.)
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
  return H >= 1 && H <= COLI_MAX_DIM && I >= 1 && I <= COLI_MAX_DIM && E >= 1 &&
         E <= COLI_MAX_EXPERTS && K >= 1 && K <= E;
}

// Tokens of one decode sub-batch: longer decode calls run in sub-batches.
inline int decode_chunk_t(int T) { return T < COLI_MAX_DECODE_T ? T : COLI_MAX_DECODE_T; }

// Whether every buffer offset of a forward of T tokens fits 31 bits (the
// kernels address their buffers through 32-bit buffer-resource offsets whose
// top bit masks lanes).
bool offsets_ok(int H, int I, int K, int T, coli_mode mode) {
  const size_t blob = blob_layout(H, I).bytes;
  if (mode == COLI_PREFILL) return prefill_offsets_ok(H, I, K, T, blob);
  return batch_offsets_ok(H, I, K, decode_chunk_t(T), blob);
}

// Workspace carve-up (byte offsets, each section 256-byte aligned).
struct WsLayout {
  size_t logits, idx, gates, counts, offsets, perm, unique, n_unique, chunk, h, slot;
  size_t xp, sx, sh, xe;                      // prefill only
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
  size_t chunk = permute_chunk_ints(T, K, E);
  if (chunk < size_t(E) + 2) chunk = size_t(E) + 2;
  w.chunk = o; o += align256(chunk * 4);
  w.xp = w.sx = w.sh = w.xe = 0;
  w.h = w.slot = 0;
  w.xdig = w.xcorr = w.nxsc = w.hn = 0;
  w.bxp = w.bxs = w.bhf = w.bh16 = w.bhs = w.bslot = 0;
  if (mode == COLI_PREFILL) {
    const PrefillLayout pl = prefill_layout(H, I);
    w.xp = o; o += align256(size_t(T) * pl.HP * 2);
    w.sx = o; o += align256(size_t(T) * pl.CSX * 2);
    w.h = o; o += align256((TK + T) * size_t(pl.IP) * 2);
    w.sh = o; o += align256((TK + T) * size_t(pl.CSI) * 2);
    w.slot = o; o += align256((TK + T) * size_t(prefill_slot_stride(H)) * 2);
    w.xe = o; o += align256(size_t(T) * 4);
  } else {
    const size_t units = TK < size_t(E) ? TK : size_t(E);
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
    w.bslot = o; o += align256(R * size_t(batch_slot_stride(H)) * 4);
  }
  w.total = o;
  return w;
}

Routing carve(uint8_t *ws, const WsLayout &w) {
  Routing r;
  r.usage = nullptr;
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
    case COLI_ESCRATCH: return "request larger than the no-alloc scratch array";
    case COLI_EUSAGE: return "routing history refused (geometry, version or identity)";
    case COLI_EIO: return "routing history file could not be read or written";
    case COLI_EFORMAT: return "no single registry format has these byte counts";
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

}  // extern "C"

namespace {

int router_topk_impl(const void *x, coli_dtype x_dtype, int T, int H, const void *w_router,
                     coli_dtype w_dtype, int E, const float *bias, int K, coli_scoring scoring,
                     int32_t *topk_idx, float *topk_gate, float *logits, void *stream) {
  if (!w_router) return COLI_EINVAL;
  if ((!x || !topk_idx || !topk_gate) && T != 0) return COLI_EINVAL;
  if (scoring != COLI_SCORE_SOFTMAX && scoring != COLI_SCORE_SIGMOID) return COLI_EINVAL;
  if (T < 0 || T > COLI_MAX_TOKENS || H < 1 || H > COLI_MAX_DIM || E < 1 ||
      E > COLI_MAX_EXPERTS || K < 1 || K > E)
    return COLI_ESHAPE;
  if ((x_dtype != COLI_F32 && x_dtype != COLI_BF16) ||
      (w_dtype != COLI_F32 && w_dtype != COLI_BF16))
    return COLI_EDTYPE;
  const uintptr_t xa = x_dtype == COLI_BF16 ? 2 : 4, wa = w_dtype == COLI_BF16 ? 2 : 4;
  if (!aligned(x, xa) || !aligned(w_router, wa) || !aligned(topk_idx, 4) ||
      !aligned(topk_gate, 4) || (logits && !aligned(logits, 4)) || (bias && !aligned(bias, 4)))
    return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  hipStream_t s = as_stream(stream);
  const int xb = x_dtype == COLI_BF16, wb = w_dtype == COLI_BF16;
  const bool sig = scoring == COLI_SCORE_SIGMOID;
  const Scoring sc{sig ? 1 : 0, sig ? bias : nullptr};
  const float *lbias = sig ? nullptr : bias;  // the bias added to the logits
  if (!logits)
    return dev_status(launch_router_topk_fused(x, xb, T, H, w_router, wb, E, K, lbias, sc,
                                               topk_idx, topk_gate, s));
  hipError_t e = router_vec_ok(x, xb, H, w_router, wb)
                     ? launch_router_logits(x, xb, T, H, w_router, wb, E, lbias, logits, s)
                     : launch_router_any(x, xb, T, H, w_router, wb, E, lbias, logits, s);
  if (e != hipSuccess) return COLI_EDEVICE;
  return dev_status(launch_topk(logits, T, E, K, topk_idx, topk_gate, sc, s));
}

}  // namespace

extern "C" {

int coli_router_topk(const void *x, coli_dtype x_dtype, int T, int H, const void *w_router,
                     coli_dtype w_dtype, int E, const float *bias, int K, int32_t *topk_idx,
                     float *topk_gate, float *logits, void *stream) {
  return router_topk_impl(x, x_dtype, T, H, w_router, w_dtype, E, bias, K, COLI_SCORE_SOFTMAX,
                          topk_idx, topk_gate, logits, stream);
}

int coli_router_topk_scored(const void *x, coli_dtype x_dtype, int T, int H,
                            const void *w_router, coli_dtype w_dtype, int E, const float *bias,
                            int K, coli_scoring scoring, int32_t *topk_idx, float *topk_gate,
                            float *logits, void *stream) {
  return router_topk_impl(x, x_dtype, T, H, w_router, w_dtype, E, bias, K, scoring, topk_idx,
                          topk_gate, logits, stream);
}

size_t coli_expert_permute_workspace_bytes(int T, int K, int E) {
  if (T < 0 || T > COLI_MAX_TOKENS || E < 1 || E > COLI_MAX_EXPERTS || K < 1 || K > E) return 0;
  return permute_chunk_ints(T, K, E) * 4;
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
  const size_t need = permute_chunk_ints(T, K, E) * 4;
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

int coli_quant_int4_g64_many(const float *const *w, uint8_t *const *packed, float *const *scales,
                             int n, int64_t rows, int64_t cols, int32_t *status, void *stream) {
  if (!w || !packed || !scales) return COLI_EINVAL;
  if (n < 0 || n > 65535 || rows < 0 || cols < 1 || rows > (int64_t(1) << 31) ||
      cols > (int64_t(1) << 31))
    return COLI_ESHAPE;
  if (!aligned(w, 8) || !aligned(packed, 8) || !aligned(scales, 8) ||
      (status && !aligned(status, 4)))
    return COLI_EALIGN;
  if (n == 0 || rows == 0) return COLI_OK;
  return dev_status(launch_quant_int4_g64_many(w, packed, scales, n, rows, cols, status,
                                               as_stream(stream)));
}

int coli_quant_expert(uint8_t *blob, int H, int I, const float *w_gate, const float *w_up,
                      const float *w_down, int32_t *status, void *stream) {
  if (!blob || !w_gate || !w_up || !w_down) return COLI_EINVAL;
  if (H < 1 || H > COLI_MAX_DIM || I < 1 || I > COLI_MAX_DIM) return COLI_ESHAPE;
  if (!aligned(blob, 256) || !aligned(w_gate, 4) || !aligned(w_up, 4) || !aligned(w_down, 4) ||
      (status && !aligned(status, 4)))
    return COLI_EALIGN;
  const BlobLayout b = blob_layout(H, I);
  hipStream_t s = as_stream(stream);
  const struct {
    const float *w;
    int rows, cols;
    size_t q, sc;
  } m[3] = {{w_gate, I, H, b.gq, b.gs}, {w_up, I, H, b.uq, b.us}, {w_down, H, I, b.dq, b.ds}};
  for (const auto &x : m) {
    const hipError_t e = launch_quant_int4_g64(x.w, x.rows, x.cols, blob + x.q,
                                               reinterpret_cast<float *>(blob + x.sc), status, s);
    if (e != hipSuccess) return COLI_EDEVICE;
  }
  return dev_status(launch_expert_finish(blob, b, H, I, s));
}

size_t coli_moe_workspace_bytes(const coli_moe_layer *L, int T, coli_mode mode) {
  if (!L || !layer_shape_ok(L->H, L->I, L->E, L->K)) return 0;
  if (mode != COLI_DECODE && mode != COLI_PREFILL) return 0;
  if (T < 0 || T > COLI_MAX_TOKENS) return 0;
  if (!offsets_ok(L->H, L->I, L->K, T, mode)) return 0;
  const int tl = mode == COLI_DECODE ? decode_chunk_t(T) : T;
  return ws_layout(L->H, L->I, L->E, L->K, tl, mode).total;
}

}  // extern "C"

namespace {

// Argument checks shared by the forward entry points (no launch).  On success
// *lay holds the workspace carve-up for the call.
int forward_checks(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                   int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                   WsLayout *lay) {
  if (!L || !L->w_router || !L->experts || !L->shared) return COLI_EINVAL;
  if ((!x || !y) && T != 0) return COLI_EINVAL;
  if (mode != COLI_DECODE && mode != COLI_PREFILL) return COLI_EINVAL;
  if (L->scoring != COLI_SCORE_SOFTMAX && L->scoring != COLI_SCORE_SIGMOID) return COLI_EINVAL;
  if (!layer_shape_ok(L->H, L->I, L->E, L->K)) return COLI_ESHAPE;
  if (T < 0 || T > COLI_MAX_TOKENS) return COLI_ESHAPE;
  if (!offsets_ok(L->H, L->I, L->K, T, mode)) return COLI_ESHAPE;
  if (L->router_dtype != COLI_F32 && L->router_dtype != COLI_BF16) return COLI_EDTYPE;
  if (!aligned(x, 16) || !aligned(y, 16) ||
      !aligned(L->w_router, L->router_dtype == COLI_BF16 ? 2 : 4) ||
      !aligned(L->experts, 256) || !aligned(L->shared, 256) ||
      (L->router_bias && !aligned(L->router_bias, 4)) ||
      (L->slot_map && !aligned(L->slot_map, 4)) || (L->usage && !aligned(L->usage, 8)) ||
      (topk_idx_out && !aligned(topk_idx_out, 4)) ||
      (topk_gate_out && !aligned(topk_gate_out, 4)) || (status && !aligned(status, 4)))
    return COLI_EALIGN;
  const int tl = mode == COLI_DECODE ? decode_chunk_t(T) : T;
  *lay = ws_layout(L->H, L->I, L->E, L->K, tl, mode);
  return COLI_OK;
}

// The device view of a layer for one call.
LayerDev layer_dev(const coli_moe_layer *L, int32_t *status, const Scoring &sc) {
  LayerDev d;
  d.H = L->H;
  d.I = L->I;
  d.E = L->E;
  d.K = L->K;
  d.experts = L->experts;
  d.shared = L->shared;
  d.lay = blob_layout(L->H, L->I);
  d.tag = finish_tag(L->H, L->I);
  d.status = status;
  d.sc = sc;
  d.slot_map = L->slot_map;
  d.usage = reinterpret_cast<unsigned long long *>(L->usage);
  return d;
}

// Buffers of one call inside the workspace.
struct CallBufs {
  Routing r;
  NarrowBufs nb;
  BatchBufs bb;
  PrefillBufs pb;
};
CallBufs carve_call(const coli_moe_layer *L, uint8_t *ws, const WsLayout &w,
                    int32_t *topk_idx_out, float *topk_gate_out) {
  CallBufs c;
  c.r = carve(ws, w);
  if (topk_idx_out) c.r.idx = topk_idx_out;
  if (topk_gate_out) c.r.gates = topk_gate_out;
  const bool sig = L->scoring == COLI_SCORE_SIGMOID;
  c.r.sc = Scoring{sig ? 1 : 0, sig ? L->router_bias : nullptr};
  c.r.usage = reinterpret_cast<unsigned long long *>(L->usage);
  c.nb.xdig = reinterpret_cast<int8_t *>(ws + w.xdig);
  c.nb.xcorr = reinterpret_cast<int32_t *>(ws + w.xcorr);
  c.nb.xsc = reinterpret_cast<float *>(ws + w.nxsc);
  c.nb.hn = reinterpret_cast<float *>(ws + w.hn);
  c.bb.xp = reinterpret_cast<uint16_t *>(ws + w.bxp);
  c.bb.xs = reinterpret_cast<float *>(ws + w.bxs);
  c.bb.hf = reinterpret_cast<float *>(ws + w.bhf);
  c.bb.h16 = reinterpret_cast<uint16_t *>(ws + w.bh16);
  c.bb.hs = reinterpret_cast<float *>(ws + w.bhs);
  c.bb.slot = reinterpret_cast<float *>(ws + w.bslot);
  c.pb.xp = reinterpret_cast<uint16_t *>(ws + w.xp);
  c.pb.sx = reinterpret_cast<uint16_t *>(ws + w.sx);
  c.pb.h = reinterpret_cast<uint16_t *>(ws + w.h);
  c.pb.sh = reinterpret_cast<uint16_t *>(ws + w.sh);
  c.pb.slot = reinterpret_cast<uint16_t *>(ws + w.slot);
  c.pb.xe = reinterpret_cast<int *>(ws + w.xe);
  return c;
}

// The route part: logits, top-K, gates, the batch union (DECODE: T <= 256).
// fused_topk: the single-token path leaves the top-K to its gate/up kernel.
int route_launch(const coli_moe_layer *L, coli_mode mode, const void *x, int T,
                 const CallBufs &c, const LayerDev &d, hipStream_t s, hipEvent_t *ev,
                 bool fused_topk) {
  const Routing &r = c.r;
  const int wbf = L->router_dtype == COLI_BF16;
  const float *lbias = r.sc.sigmoid ? nullptr : L->router_bias;  // bias added to the logits
  hipError_t e;
  if (mode == COLI_DECODE) {
    if (narrow_supported(d, T)) {
      // one kernel per stage: the events are stamped by the launches
      e = launch_router_narrow(reinterpret_cast<const float *>(x), T, L->H, L->w_router, wbf,
                               L->E, lbias, r.logits, c.nb, s, ev ? ev[0] : nullptr,
                               ev ? ev[1] : nullptr);
      if (e != hipSuccess) return COLI_EDEVICE;
      if (fused_topk) return COLI_OK;
      // two-phase: the top-K and the union now, for the caller to read
      return dev_status(launch_topk_permute(r, T, L->E, L->K, 1, s));
    }
    if (ev) (void)hipEventRecord(ev[0], s);
    // the vector router launch also writes x's staged rows for the batch GEMM
    if (router_vec_ok(x, 0, L->H, L->w_router, wbf))
      e = launch_router_logits(x, 0, T, L->H, L->w_router, wbf, L->E, lbias, r.logits, s, c.bb.xp,
                               c.bb.xs, prefill_layout(L->H, L->I).HP);
    else
      e = launch_router_any(x, 0, T, L->H, L->w_router, wbf, L->E, lbias, r.logits, s);
    if (e != hipSuccess) return COLI_EDEVICE;
    e = launch_route_decode(r, T, L->E, L->K, s);
    if (e != hipSuccess) return COLI_EDEVICE;
    if (ev) (void)hipEventRecord(ev[1], s);
    return COLI_OK;
  }
  if (ev) (void)hipEventRecord(ev[0], s);
  if (wbf && L->H % 32 == 0 && router_vec_ok(x, 1, L->H, L->w_router, 1)) {
    // the staged-x region is free until the activation conversion: it holds the
    // router's K-split partial sums
    const PrefillLayout pl = prefill_layout(L->H, L->I);
    e = launch_router_mfma(reinterpret_cast<const uint16_t *>(x), T, L->H,
                           reinterpret_cast<const uint16_t *>(L->w_router), L->E, lbias,
                           r.logits, reinterpret_cast<float *>(c.pb.xp),
                           size_t(T) * pl.HP * 2, s);
  } else if (router_vec_ok(x, 1, L->H, L->w_router, wbf)) {
    e = launch_router_logits(x, 1, T, L->H, L->w_router, wbf, L->E, lbias, r.logits, s);
  } else {
    e = launch_router_any(x, 1, T, L->H, L->w_router, wbf, L->E, lbias, r.logits, s);
  }
  if (e != hipSuccess) return COLI_EDEVICE;
  e = launch_topk_permute(r, T, L->E, L->K, 1, s);
  if (e != hipSuccess) return COLI_EDEVICE;
  if (ev) (void)hipEventRecord(ev[1], s);
  return COLI_OK;
}

// The experts part: the FFNs and the combine from the routing in the workspace.
int experts_launch(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                   const CallBufs &c, const LayerDev &d, hipStream_t s, hipEvent_t *ev,
                   bool pre_routed) {
  const Routing &r = c.r;
  if (mode == COLI_DECODE) {
    if (narrow_supported(d, T))
      return dev_status(launch_ffn_narrow(d, c.nb, r.logits, r.idx, r.gates,
                                          reinterpret_cast<float *>(y), s, ev ? ev + 2 : nullptr,
                                          pre_routed));
    // the vector router staged x's rows in the route part
    const bool staged = router_vec_ok(x, 0, L->H, L->w_router, L->router_dtype == COLI_BF16);
    return dev_status(launch_ffn_batch(d, reinterpret_cast<const float *>(x), T, r, c.bb,
                                       reinterpret_cast<float *>(y), s, ev ? ev + 2 : nullptr,
                                       staged));
  }
  return dev_status(launch_ffn_prefill(d, reinterpret_cast<const uint16_t *>(x), T, r, c.pb,
                                       reinterpret_cast<uint16_t *>(y), s,
                                       ev ? ev + 2 : nullptr));
}

// One forward of T tokens (DECODE: T <= COLI_MAX_DECODE_T) with every
// argument already checked.
int forward_launch(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                   int32_t *topk_idx_out, float *topk_gate_out, int32_t *status, uint8_t *ws,
                   const WsLayout &w, hipStream_t s, hipEvent_t *ev) {
  const CallBufs c = carve_call(L, ws, w, topk_idx_out, topk_gate_out);
  const LayerDev d = layer_dev(L, status, c.r.sc);
  const int rc = route_launch(L, mode, x, T, c, d, s, ev, true);
  if (rc != COLI_OK) return rc;
  return experts_launch(L, mode, x, T, y, c, d, s, ev, false);
}

}  // namespace

namespace coli {
int forward_arg_check(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                      int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                      size_t *ws_need) {
  WsLayout w;
  const int rc = forward_checks(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, &w);
  *ws_need = rc == COLI_OK ? w.total : 0;
  return rc;
}
}  // namespace coli

namespace {

int moe_forward_impl(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                     int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                     void *workspace, size_t workspace_bytes, void *stream, hipEvent_t *ev) {
  WsLayout w;
  const int rc = forward_checks(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, &w);
  if (rc != COLI_OK) return rc;
  if (!workspace || workspace_bytes < w.total) return COLI_EWORKSPACE;
  if (!aligned(workspace, 256)) return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  hipStream_t s = as_stream(stream);
  if (mode == COLI_PREFILL || T <= COLI_MAX_DECODE_T)
    return forward_launch(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, ws, w, s, ev);
  // decode of more than 256 tokens: consecutive 256-token sub-batches, each
  // reading its experts once
  const size_t H = size_t(L->H), K = size_t(L->K);
  for (int t0 = 0; t0 < T; t0 += COLI_MAX_DECODE_T) {
    const int n = T - t0 < COLI_MAX_DECODE_T ? T - t0 : COLI_MAX_DECODE_T;
    const int r2 = forward_launch(
        L, mode, reinterpret_cast<const float *>(x) + size_t(t0) * H, n,
        reinterpret_cast<float *>(y) + size_t(t0) * H,
        topk_idx_out ? topk_idx_out + size_t(t0) * K : nullptr,
        topk_gate_out ? topk_gate_out + size_t(t0) * K : nullptr, status, ws, w, s, nullptr);
    if (r2 != COLI_OK) return r2;
  }
  return COLI_OK;
}

}  // namespace

extern "C" {

int coli_moe_forward(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                     int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return moe_forward_impl(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, workspace,
                          workspace_bytes, stream, nullptr);
}

int coli_moe_forward_timed(const coli_moe_layer *L, coli_mode mode, const void *x, int T,
                           void *y, int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                           void *workspace, size_t workspace_bytes, void *stream, void **events,
                           int n_events) {
  const int need = 2 * (mode == COLI_PREFILL ? 5 : 3);
  if (!events || n_events < need) return COLI_EINVAL;
  for (int i = 0; i < need; ++i)
    if (!events[i]) return COLI_EINVAL;
  if (mode == COLI_DECODE && T > COLI_MAX_DECODE_T) return COLI_ESHAPE;
  return moe_forward_impl(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, workspace,
                          workspace_bytes, stream, reinterpret_cast<hipEvent_t *>(events));
}

}  // extern "C"

namespace {

// Checks, workspace and carve-up shared by the two-phase entry points.
int two_phase_setup(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                    int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                    void *workspace, size_t workspace_bytes, WsLayout *w) {
  const int rc = forward_checks(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, w);
  if (rc != COLI_OK) return rc;
  if (mode == COLI_DECODE && T > COLI_MAX_DECODE_T) return COLI_ESHAPE;
  if (!workspace || workspace_bytes < w->total) return COLI_EWORKSPACE;
  if (!aligned(workspace, 256)) return COLI_EALIGN;
  return COLI_OK;
}

}  // namespace

extern "C" {

int coli_moe_route(const coli_moe_layer *L, coli_mode mode, const void *x, int T,
                   int32_t *topk_idx_out, float *topk_gate_out, int32_t *unique_out,
                   int32_t *n_unique_out, void *workspace, size_t workspace_bytes,
                   void *stream) {
  WsLayout w;
  // y is not written by this call: the checks take x in its place
  int rc = two_phase_setup(L, mode, x, T, const_cast<void *>(x), topk_idx_out, topk_gate_out,
                           nullptr, workspace, workspace_bytes, &w);
  if (rc != COLI_OK) return rc;
  if (!aligned(unique_out, 4) || !aligned(n_unique_out, 4)) return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  hipStream_t s = as_stream(stream);
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  const CallBufs c = carve_call(L, ws, w, topk_idx_out, topk_gate_out);
  const LayerDev d = layer_dev(L, nullptr, c.r.sc);
  rc = route_launch(L, mode, x, T, c, d, s, nullptr, false);
  if (rc != COLI_OK) return rc;
  if (unique_out || n_unique_out)
    return dev_status(launch_copy_union(c.r, L->E, unique_out, n_unique_out, s));
  return COLI_OK;
}

int coli_moe_experts(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                     int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                     void *workspace, size_t workspace_bytes, void *stream) {
  WsLayout w;
  const int rc = two_phase_setup(L, mode, x, T, y, topk_idx_out, topk_gate_out, status,
                                 workspace, workspace_bytes, &w);
  if (rc != COLI_OK) return rc;
  if (T == 0) return COLI_OK;
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  const CallBufs c = carve_call(L, ws, w, topk_idx_out, topk_gate_out);
  const LayerDev d = layer_dev(L, status, c.r.sc);
  return experts_launch(L, mode, x, T, y, c, d, as_stream(stream), nullptr, true);
}

}  // extern "C"

namespace {

// Workspace of the sibling-format forward: the routing sections of the decode
// layout, then h [units][T][I] and the per-unit outputs [units][T][H].
struct FmtWs {
  WsLayout w;
  size_t h, part, total;
};
FmtWs fmt_ws(const coli_moe_layer *L, int T) {
  FmtWs f;
  f.w = ws_layout(L->H, L->I, L->E, L->K, T, COLI_DECODE);
  const size_t units = size_t(L->E < T * L->K ? L->E : T * L->K) + 1;
  f.h = align256(f.w.total);
  f.part = f.h + align256(units * T * L->I * 4);
  f.total = f.part + align256(units * T * L->H * 4);
  return f;
}

int fmt_forward_checks(const coli_moe_layer *L, int fmt, const void *x, int T, void *y,
                       int32_t *topk_idx_out, float *topk_gate_out, int32_t *status) {
  WsLayout w;
  const int rc = forward_checks(L, COLI_DECODE, x, T, y, topk_idx_out, topk_gate_out, status, &w);
  if (rc != COLI_OK) return rc;
  if (!fmt_layer_supported(fmt) || L->slot_map) return COLI_EINVAL;
  if (T != 0 && !fmt_layer_shape_ok(fmt, L->H, L->I, T)) return COLI_ESHAPE;
  return COLI_OK;
}

}  // namespace

extern "C" {

size_t coli_moe_fmt_workspace_bytes(const coli_moe_layer *L, int fmt, int T) {
  if (!L || !layer_shape_ok(L->H, L->I, L->E, L->K) || !fmt_layer_supported(fmt)) return 0;
  if (T < 1 || !fmt_layer_shape_ok(fmt, L->H, L->I, T)) return 0;
  return fmt_ws(L, T).total;
}

int coli_moe_forward_fmt(const coli_moe_layer *L, int fmt, const float *x, int T, float *y,
                         int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                         void *workspace, size_t workspace_bytes, void *stream) {
  int rc = fmt_forward_checks(L, fmt, x, T, y, topk_idx_out, topk_gate_out, status);
  if (rc != COLI_OK) return rc;
  if (T == 0) return COLI_OK;
  const FmtWs f = fmt_ws(L, T);
  if (!workspace || workspace_bytes < f.total) return COLI_EWORKSPACE;
  if (!aligned(workspace, 256)) return COLI_EALIGN;
  hipStream_t s = as_stream(stream);
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  Routing r = carve(ws, f.w);
  if (topk_idx_out) r.idx = topk_idx_out;
  if (topk_gate_out) r.gates = topk_gate_out;
  const bool sig = L->scoring == COLI_SCORE_SIGMOID;
  r.sc = Scoring{sig ? 1 : 0, sig ? L->router_bias : nullptr};
  r.usage = reinterpret_cast<unsigned long long *>(L->usage);
  const float *lbias = sig ? nullptr : L->router_bias;
  const int wbf = L->router_dtype == COLI_BF16;
  hipError_t e = router_vec_ok(x, 0, L->H, L->w_router, wbf)
                     ? launch_router_logits(x, 0, T, L->H, L->w_router, wbf, L->E, lbias,
                                            r.logits, s)
                     : launch_router_any(x, 0, T, L->H, L->w_router, wbf, L->E, lbias,
                                         r.logits, s);
  if (e != hipSuccess) return COLI_EDEVICE;
  e = launch_route_decode(r, T, L->E, L->K, s);
  if (e != hipSuccess) return COLI_EDEVICE;
  FmtLayer fl;
  fl.fmt = fmt;
  fl.H = L->H;
  fl.I = L->I;
  fl.E = L->E;
  fl.K = L->K;
  fl.experts = L->experts;
  fl.shared = L->shared;
  fl.blob_bytes = fmt_blob_layout(fmt, L->H, L->I, fl.q_off, fl.s_off);
  return dev_status(launch_fmt_experts(fl, r, x, T, reinterpret_cast<float *>(ws + f.h),
                                       reinterpret_cast<float *>(ws + f.part), y, status, s));
}

int coli_rmsnorm_f32(const float *x, float *y, int T, int H, float eps, void *stream) {
  if (((!x || !y) && T != 0) || !(eps >= 0.0f) || !std::isfinite(eps)) return COLI_EINVAL;
  if (T < 0 || T > COLI_MAX_TOKENS || H < 1 || H > COLI_MAX_DIM) return COLI_ESHAPE;
  if (!aligned(x, 4) || !aligned(y, 4)) return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  return dev_status(launch_rmsnorm_f32(x, y, T, H, eps, as_stream(stream)));
}

}  // extern "C"

// kernels.h -- internal launchers of libcoli (not part of the C ABI).
//
// Every launcher enqueues on `stream` and returns hipGetLastError() of its
// launches.  Shapes have been validated by the caller (coli.cpp); each
// launcher only re-derives grid sizes from them.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "coli.h"

// lanes of a wave hold ceil(E/64) router logits each
#define COLI_MAX_PER_LANE (COLI_MAX_EXPERTS / 64)
// decode mode accumulates the combine of up to this many tokens on chip
#define COLI_MAX_DECODE_T 256

namespace coli {

// ---- shared layout arithmetic -------------------------------------------
inline int64_t groups_of(int64_t cols) { return (cols + 63) / 64; }
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Offsets of the six sections of an expert blob (see coli.h).
struct BlobLayout {
  size_t gq, uq, dq, gs, us, ds;
  size_t gsT, usT, dsT;  // the scales again, group-major ([G][rows]; coli_expert_finish)
  size_t gsB, usB, dsB;  // and blocked by 8 rows ([ceil(rows/8)][G][8]; coli_expert_finish)
  size_t tag;            // 16-byte finish tag (coli_expert_finish; checked by the decode paths)
  size_t bytes;
  int64_t GH, GI;  // groups per row of gate/up (input H) and of down (input I)
};
inline BlobLayout blob_layout(int H, int I) {
  BlobLayout b;
  b.GH = groups_of(H);
  b.GI = groups_of(I);
  size_t o = 0;
  b.gq = o; o += align256(size_t(I) * b.GH * 32);
  b.uq = o; o += align256(size_t(I) * b.GH * 32);
  b.dq = o; o += align256(size_t(H) * b.GI * 32);
  b.gs = o; o += align256(size_t(I) * b.GH * 4);
  b.us = o; o += align256(size_t(I) * b.GH * 4);
  b.ds = o; o += align256(size_t(H) * b.GI * 4);
  b.gsT = o; o += align256(size_t(I) * b.GH * 4);
  b.usT = o; o += align256(size_t(I) * b.GH * 4);
  b.dsT = o; o += align256(size_t(H) * b.GI * 4);
  b.gsB = o; o += align256(size_t((I + 7) / 8) * 8 * b.GH * 4);
  b.usB = o; o += align256(size_t((I + 7) / 8) * 8 * b.GH * 4);
  b.dsB = o; o += align256(size_t((H + 7) / 8) * 8 * b.GI * 4);
  b.tag = o; o += 256;
  b.bytes = o;
  return b;
}

// Scoring of the router.  softmax (sigmoid == 0): the logits are the keys and
// the gates are the softmax over the selected logits.  sigmoid (page "Colibrì
// 深度解析", section 十一: one expert group, sigmoid scores, selection without
// an auxiliary loss): score s = 1 / (1 + e^-l), key = s + bias[e] (the bias
// only steers the selection), gates = the selected scores over their sum.
struct Scoring {
  int sigmoid;
  const float *bias;  // selection bias [E] (sigmoid only; NULL = 0)
};

// Device-side view of the routing products, all inside the workspace.
struct Routing {
  float *logits;     // [T, E]
  int32_t *idx;      // [T, K]
  float *gates;      // [T, K]
  int32_t *counts;   // [E]
  int32_t *offsets;  // [E + 1]
  int32_t *perm;     // [T*K]
  int32_t *unique;   // [E]
  int32_t *n_unique; // [1]
  int32_t *chunk;    // [n_chunks * E] per-chunk counts / bases (large T)
  Scoring sc;        // how the top-K scores the logits
  unsigned long long *usage;  // [E] routing-history counters to add the counts to, or NULL
};


// Single-token decode buffers (inside the workspace).  xdig: x as four int8
// digit planes, [T][GH][4 planes][64] in "A order" (see ffn_narrow.hip), value
// = digits * xsc[t]; xcorr [T][GH][4]: -8 * (sum of the group's digits) per
// plane; xsc [T]: 2^-e, NaN if the token holds a non-finite value; hn
// [units][I]: h' = gate_weight * SiLU(gate) * up in fp32, units in top-K order
// then the shared expert.
struct NarrowBufs {
  int8_t *xdig;
  int32_t *xcorr;
  float *xsc;
  float *hn;
};
#define COLI_NARROW_MAX_K 16

// The finish tag of a blob of shape (H, I): written last by
// coli_expert_finish, compared by every kernel that reads the derived scale
// copies ('COLI', 'FIN1', H, I).
inline uint4 finish_tag(int H, int I) {
  uint4 t;
  t.x = 0x494C4F43u;
  t.y = 0x314E4946u;
  t.z = uint32_t(H);
  t.w = uint32_t(I);
  return t;
}

// One layer as the kernels see it.
struct LayerDev {
  int H, I, E, K;
  const uint8_t *experts;
  const uint8_t *shared;
  BlobLayout lay;
  uint4 tag;        // finish_tag(H, I)
  int32_t *status;  // optional device flag: COLI_STATUS_* bits OR-ed in
  Scoring sc;       // router scoring (the fused single-token top-K)
  const int32_t *slot_map;  // expert -> cache slot of `experts`, or NULL (identity)
  unsigned long long *usage;  // routing-history counters [E] (the fused top-K adds), or NULL
};

// Blob of routed expert e.  With a slot map, e's blob is its slot; an expert
// without a slot sets `missing` and gets the shared blob's address in its place
// (valid memory to read), and its outputs are to be poisoned by the caller.
__device__ inline const uint8_t *expert_blob(const LayerDev &L, int e, bool &missing) {
  const int s = L.slot_map ? L.slot_map[e] : e;
  missing = s < 0;
  return s < 0 ? L.shared : L.experts + size_t(s) * L.lay.bytes;
}

// Device side of the status flag: OR bits into *status (if any) from one lane.
__device__ inline void raise_status(int32_t *status, int bits) {
  if (status) atomicOr(status, bits);
}

// ---- coli.cpp ----------------------------------------------------------
// The host-side argument checks of coli_moe_forward (no launch, no HIP call);
// on COLI_OK *ws_need is the workspace the call needs.
int forward_arg_check(const coli_moe_layer *L, coli_mode mode, const void *x, int T, void *y,
                      int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                      size_t *ws_need);

// ---- quant.hip ----------------------------------------------------------
hipError_t launch_quant_int4_g64(const float *w, int64_t rows, int64_t cols,
                                 uint8_t *packed, float *scales,
                                 int32_t *status, hipStream_t s);
// n matrices of one shape [rows, cols] in one launch; the pointer arrays are
// device memory.
hipError_t launch_quant_int4_g64_many(const float *const *w, uint8_t *const *packed,
                                      float *const *scales, int n, int64_t rows, int64_t cols,
                                      int32_t *status, hipStream_t s);

// ---- route.hip ----------------------------------------------------------
// logits[t, e] = x[t] . Wr[e] + b[e]; x fp32 (x_bf16 = 0) or bf16.
// xp, xs (optional, fp32 x only): the decode batch's staged hi/lo rows of x
// ([2T][HP] fp16, stage_rows.h) and row scales, written by extra blocks of the
// same launch.
hipError_t launch_router_logits(const void *x, int x_bf16, int T, int H,
                                const void *wr, int w_bf16, int E,
                                const float *bias, float *logits, hipStream_t s,
                                uint16_t *xp = nullptr, float *xs = nullptr, int HP = 0);
// Prefill router logits: bf16 x and bf16 Wr through MFMA (H % 32 == 0).
// part: scratch for the K-split partial sums (part_bytes; a smaller split is
// used when S * T * E floats do not fit).
hipError_t launch_router_mfma(const uint16_t *x, int T, int H, const uint16_t *wr, int E,
                              const float *bias, float *logits, float *part, size_t part_bytes,
                              hipStream_t s);
// Logits for any H and row alignment (element loads).
hipError_t launch_router_any(const void *x, int x_bf16, int T, int H, const void *wr,
                             int w_bf16, int E, const float *bias, float *logits,
                             hipStream_t s);
// Whether the 16-byte-load router kernels take these operands.
bool router_vec_ok(const void *x, int x_bf16, int H, const void *wr, int w_bf16);
// Logits and top-K per token in one launch, the logits kept on chip.
hipError_t launch_router_topk_fused(const void *x, int x_bf16, int T, int H, const void *wr,
                                    int w_bf16, int E, int K, const float *logit_bias,
                                    Scoring sc, int32_t *idx, float *gates, hipStream_t s);
// top-K + gates from logits, one wave per token.
hipError_t launch_topk(const float *logits, int T, int E, int K, int32_t *idx,
                       float *gates, Scoring sc, hipStream_t s);
// top-K + gates from logits (do_topk), then the batch-union permute.  For
// T * K above a small threshold the permute uses r.chunk,
// permute_chunk_ints() ints of scratch.
hipError_t launch_topk_permute(const Routing &r, int T, int E, int K,
                               int do_topk, hipStream_t s);
// Decode: one block does top-K, the permute and the per-unit M-chunk prefix
// (r.chunk, chunks of 32 tokens, the shared unit last).  Requires
// T <= COLI_MAX_DECODE_T.
hipError_t launch_route_decode(const Routing &r, int T, int E, int K, hipStream_t s);
size_t permute_chunk_ints(int T, int K, int E);
// ---- formats.hip: a layer whose experts are in a sibling format ----------
constexpr int kFmtLayerMaxT = 4;
struct FmtLayer {
  int fmt, H, I, E, K;
  const uint8_t *experts, *shared;
  size_t blob_bytes;
  size_t q_off[3], s_off[3];  // gate, up, down sections of a blob
};
// Blob sections of one expert in fmt (gate.q | up.q | down.q | gate.s | up.s |
// down.s, 256-byte aligned); returns the blob bytes, 0 for an unsupported fmt.
size_t fmt_blob_layout(int fmt, int H, int I, size_t q_off[3], size_t s_off[3]);
bool fmt_layer_supported(int fmt);
bool fmt_layer_shape_ok(int fmt, int H, int I, int T);
// The experts part of the layer from the routing in r: h = SiLU(gate) * up *
// gate weight per (unit, token) -> h [units][T][I]; per-unit down outputs ->
// part [units][T][H]; y [T][H] = their sum in unit order.
hipError_t launch_fmt_experts(const FmtLayer &L, const Routing &r, const float *x, int T,
                              float *h, float *part, float *y, int32_t *status, hipStream_t s);
// ---- ffn_mx.hip: an MXFP4 layer's experts on the scaled matrix cores ------
// Whether the gate/up takes this call (MXFP4, T <= 2, H % 256 == 0 and
// H <= 8192, I % 8 == 0, at most 40 units, x 16-byte aligned), and the down
// (T == 1, I % 256 == 0, units x ceil(I / 2048) <= 18, H <= 8192).
bool mx_gateup_ok(const FmtLayer &L, const float *x, int T);
bool mx_down_ok(const FmtLayer &L, int T);
// h [units][T][I] as launch_fmt_experts defines it.
hipError_t launch_mx_gateup(const FmtLayer &L, const Routing &r, const float *x, int T, float *h,
                            hipStream_t s);
// One token: y [H] from h [units][I] (status: COLI_STATUS_NONFINITE for a
// non-finite output).
hipError_t launch_mx_down(const FmtLayer &L, const Routing &r, const float *h, float *y,
                          int32_t *status, hipStream_t s);

// Copy the batch union (r.unique [E], r.n_unique) to caller buffers (either
// may be NULL).
hipError_t launch_copy_union(const Routing &r, int E, int32_t *unique, int32_t *n_unique,
                             hipStream_t s);
// Single-token decode router: logits [T, E] and x as digit planes (nb.xdig,
// nb.xcorr, nb.xsc).  Requires H % 256 == 0, T <= 4.
// start/stop: optional events stamped at the kernel's start and end.
hipError_t launch_router_narrow(const float *x, int T, int H, const void *wr, int w_bf16,
                                int E, const float *bias, float *logits,
                                const NarrowBufs &nb, hipStream_t s, hipEvent_t start = nullptr,
                                hipEvent_t stop = nullptr);

// ---- ffn_narrow.hip -----------------------------------------------------
// Whether the single-token int8 matrix-core path covers this layer and T.
bool narrow_supported(const LayerDev &L, int T);
// Top-K of the token (from logits; idx/gates written), gate/up -> nb.hn, down
// -> y.  ev: optional (NULL or 4: start and stop of the gate/up kernel, of the
// down kernel, stamped by the kernel launches themselves).
// pre_routed: idx/gates already hold the token's top-K (the gate/up kernel then
// reads them instead of selecting).
hipError_t launch_ffn_narrow(const LayerDev &L, const NarrowBufs &nb, const float *logits,
                             int32_t *idx, float *gates, float *y, hipStream_t s,
                             hipEvent_t *ev, bool pre_routed = false);

// ---- ffn_prefill.hip ----------------------------------------------------
// Row strides (elements) of the prefill activation buffers: staged x and h
// rows are padded to whole 256-column blocks; group-sum rows hold a hi/lo
// fp16 pair per group, padded to whole 16-group blocks.
struct PrefillLayout {
  int HP, IP, CSX, CSI;
};
PrefillLayout prefill_layout(int H, int I);
// Prefill buffers (inside the workspace): xp [T, HP] fp16, sx [T, CSX],
// h [T*K + T, IP] fp16, sh [T*K + T, CSI], slot [T*K + T, SP] fp16
// (SP = prefill_slot_stride(H)), xe [T] the per-token activation exponents.
struct PrefillBufs {
  uint16_t *xp, *sx, *h, *sh, *slot;
  int *xe;
};
// ev: optional stage events (NULL or 8: start and stop of prep + tiles, gate/up,
// down, combine).
hipError_t launch_ffn_prefill(const LayerDev &L, const uint16_t *x, int T, const Routing &r,
                              const PrefillBufs &b, uint16_t *y, hipStream_t s, hipEvent_t *ev);
// Whether every prefill buffer offset fits the 31 bits of a buffer resource.
bool prefill_offsets_ok(int H, int I, int K, int T, size_t blob_bytes);
int prefill_slot_stride(int H);

// Decode batch (1 < T <= 256) on the same grouped-GEMM weight stream:
// xp: x as staged fp16 hi/lo rows [2T][HP] (hi rows first), xs [T] row scales;
// hf: h = SiLU(gate) * up fp32 [T*K + T][I]; h16 [2 (T*K + T)][IP], hs: its
// staged hi/lo rows and scales; slot [T*K + T][H] fp32 gate-scaled outputs.
struct BatchBufs {
  uint16_t *xp;
  float *xs;
  float *hf;
  uint16_t *h16;
  float *hs;
  float *slot;
};
// r: routing with 32-token M-chunk prefix (launch_route_decode).  ev: optional
// (NULL or 4: start and stop of the gate/up step, of the down step).
// x_staged: xp / xs already hold x's staged rows (launch_router_logits did them).
hipError_t launch_ffn_batch(const LayerDev &L, const float *x, int T, const Routing &r,
                            const BatchBufs &b, float *y, hipStream_t s, hipEvent_t *ev,
                            bool x_staged = false);
// Whether every decode-batch buffer offset fits the 31 bits of a buffer resource.
bool batch_offsets_ok(int H, int I, int K, int T, size_t blob_bytes);
// Row stride (floats) of the decode batch's per-slot outputs.
int batch_slot_stride(int H);

// Group-major copies of a blob's three scale sections (gs -> gsT etc.).
hipError_t launch_expert_finish(uint8_t *blob, const BlobLayout &lay, int H, int I,
                                hipStream_t s);

// ---- rmsnorm.hip --------------------------------------------------------
hipError_t launch_rmsnorm_f32(const float *x, float *y, int T, int H,
                              float eps, hipStream_t s);

}  // namespace coli

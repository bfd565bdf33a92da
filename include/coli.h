/*
 * coli.h -- C ABI of libcoli.so: the routed-expert MoE layer with int4-g64
 * planar experts, on one AMD MI355X (gfx950).
 *
 * The layer (sources cited by page title and section):
 *   route   -- page "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
 *              section 十一: the router picks the top-k experts of each token;
 *              gates are the normalised values the layer applies (page
 *              "colibrì 路由遥测全解析", section 分离计数与追踪).
 *   union   -- page "Colibrì 深度解析", section 四: positions of a batch routed
 *              to one expert are grouped so that the expert is read once.
 *   experts -- page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
 *              section 权重转换: int4 grouped weights, group 64, one fp32 scale
 *              per group, q = clip(rint(w/s), -8, 7) stored as unsigned q+8,
 *              planar nibbles (byte k of a 64-group: element k in the low
 *              nibble, element k+32 in the high nibble); the expert FFN reads
 *              these bytes directly.  An expert's gate, up and down matrices
 *              sit side by side (page "Colibrì 深度解析", section 四).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, unless a
 *     comment says "host".  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t passed
 *     as void*, NULL = the default stream) and is asynchronous.
 *   - Fail closed (the pages' guard convention, page "Colibrì 深度解析",
 *     section 十五, and page "colibrì 路由遥测全解析", section 测试与 CI 保障):
 *     every argument check runs on the host before the first launch; on any
 *     error the call returns a negative status and writes nothing.
 *   - A launch failure reported by the HIP runtime returns COLI_EDEVICE.
 *   - Row-major layouts throughout.  Calls are reentrant: the library has no
 *     global mutable state besides the per-device address of the no-alloc
 *     scratch array (coli_moe_forward_noalloc); concurrent calls must not
 *     share output or workspace buffers.
 *   - Data conditions found on the device (non-finite values, an operand out
 *     of range, an unfinished expert blob) are OR-ed into an optional device
 *     status flag; they never change the return value.
 */
#ifndef COLI_H
#define COLI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    COLI_OK = 0,
    COLI_EINVAL = -1,     /* NULL pointer or invalid enum / parameter value */
    COLI_ESHAPE = -2,     /* a dimension is out of its valid range */
    COLI_EALIGN = -3,     /* a pointer is not aligned as required */
    COLI_EDTYPE = -4,     /* dtype not supported for this call / mode */
    COLI_EWORKSPACE = -5, /* workspace NULL or smaller than required */
    COLI_EDEVICE = -6,    /* the HIP runtime reported a launch error */
    COLI_ESCRATCH = -7,   /* the call needs more than the no-alloc scratch holds */
    COLI_EUSAGE = -8,     /* a routing history refused (geometry, version, identity) */
    COLI_EIO = -9,        /* a routing history file could not be read or written */
    COLI_EFORMAT = -10    /* no registry format, or more than one, has the byte
                             counts given to coli_resolve_fmt */
};

typedef enum { COLI_F32 = 0, COLI_BF16 = 1 } coli_dtype;
typedef enum { COLI_DECODE = 0, COLI_PREFILL = 1 } coli_mode;

/* How the router turns logits into a selection and gates.
 *   SOFTMAX: the K largest logits (an optional bias is added to the logits);
 *            gates = softmax over the K selected logits.
 *   SIGMOID: the router of page "Colibrì 深度解析", section 十一 (one expert
 *            group, sigmoid scores, selection without an auxiliary loss):
 *            score s_e = 1 / (1 + exp(-l_e)) of the raw logit; the K largest
 *            keys s_e + b_e are selected, where the optional bias b only
 *            steers the selection; gates = the selected scores divided by
 *            their sum.  The returned logits are the raw ones. */
typedef enum { COLI_SCORE_SOFTMAX = 0, COLI_SCORE_SIGMOID = 1 } coli_scoring;

/* Bits of the optional device status flag of coli_moe_forward (OR-ed in by
 * the kernels; the caller clears the flag).  Device-side data conditions are
 * reported here, never through the return value. */
#define COLI_STATUS_NONFINITE 1   /* y holds a non-finite value (a non-finite
                                     x or weight reached it) */
#define COLI_STATUS_RANGE 2       /* PREFILL: an fp16 operand (h or a
                                     per-slot output, after the per-token
                                     scaling) exceeded 65504; y is unreliable */
#define COLI_STATUS_UNFINISHED 4  /* DECODE: an expert blob the call read has
                                     no finish tag (coli_expert_finish was not
                                     run on it); that expert's outputs, and so
                                     y of its tokens, are NaN */
#define COLI_STATUS_NOT_RESIDENT 8 /* a routed expert has no slot in the
                                     layer's slot_map (-1); its outputs, and so
                                     y of its tokens, are NaN */

#define COLI_GROUP 64           /* elements per quantisation group */
#define COLI_MAX_EXPERTS 1024   /* upper bound for E (and K) */
#define COLI_MAX_DIM 65536      /* upper bound for H and I */
#define COLI_MAX_TOKENS 65536   /* upper bound for T */

/* Human-readable text for a status code (static storage, never NULL). */
const char *coli_strerror(int status);

/* ---------------------------------------------------------------------- */
/* int4-g64 planar format (page "从源码开始...", section 权重转换)          */
/* ---------------------------------------------------------------------- */

/* Bytes of packed nibbles for a [rows, cols] matrix: rows * ceil(cols/64) * 32.
 * Returns 0 for rows < 0 or cols < 1 (no valid matrix). */
size_t coli_int4_g64_packed_bytes(int64_t rows, int64_t cols);

/* Number of fp32 scales for a [rows, cols] matrix: rows * ceil(cols/64). */
size_t coli_int4_g64_scale_count(int64_t rows, int64_t cols);

/*
 * Quantise and pack one fp32 matrix W [rows, cols] (row-major).
 *   packed [rows][ceil(cols/64)*32] u8  (16-byte aligned)
 *   scales [rows][ceil(cols/64)]    f32
 * Per row and per 64-group g along the columns (the last group is zero
 * padded when cols is not a multiple of 64):
 *   amax = max |w|, s = fl32(amax / 7) (IEEE fp32 divide),
 *   q = clip(rint_half_even(fl32(w / s)), -8, 7), u = q + 8,
 *   byte g*32+k = u[g*64+k] | u[g*64+k+32] << 4.
 * A group whose scale is 0 stores nibbles 8.  A group holding NaN or Inf
 * stores nibbles 8 and a NaN scale, and bit 0 of *status is OR-ed with 1
 * (status: optional device int32; NULL to skip).  The output is bit-exact:
 * same bytes and scale bits as the IEEE definition above.
 * w must be 4-byte aligned; 16-byte rows (cols % 4 == 0) take the fast path.
 * rows == 0 is a no-op (pointers may then be NULL).  Errors: EINVAL (NULL
 * w/packed/scales with rows > 0), ESHAPE
 * (rows < 0, cols < 1, rows*cols > 2^40), EALIGN.
 */
int coli_quant_int4_g64(const float *w, int64_t rows, int64_t cols,
                        uint8_t *packed, float *scales, int32_t *status,
                        void *stream);

/*
 * The same quantiser over n matrices of one shape [rows, cols] in one launch
 * (for whole layers: fewer launch tails than n calls).  w, packed, scales:
 * DEVICE arrays of n device pointers (8-byte aligned); each matrix follows the
 * rules and alignments of coli_quant_int4_g64 (an fp32 matrix that is not
 * 16-byte aligned takes element loads).  Bytes are identical to n separate
 * calls.  Errors: EINVAL (NULL arrays), ESHAPE (n outside [0, 65535], rows < 0,
 * cols < 1), EALIGN, EDEVICE.
 */
int coli_quant_int4_g64_many(const float *const *w, uint8_t *const *packed,
                             float *const *scales, int n, int64_t rows, int64_t cols,
                             int32_t *status, void *stream);

/* ---------------------------------------------------------------------- */
/* route (page "Colibrì 深度解析", section 十一)                           */
/* ---------------------------------------------------------------------- */

/*
 * Router logits and top-K with renormalised gates for T tokens.
 *   x        [T, H]  fp32 or bf16 (x_dtype), row-major, any H
 *   w_router [E, H]  fp32 or bf16 (w_dtype)
 *   bias     [E]     fp32, or NULL (SOFTMAX: added to the logits, so it
 *                    steers the selection and enters the gates; SIGMOID: the
 *                    selection bias of coli_scoring)
 *   logits   [T, E]  fp32 output, or NULL: the logits are then kept on chip
 *                    (one block per token) and not written
 *   topk_idx [T, K]  int32 output: the K selected expert ids of each token
 *                    in ascending id order
 *   topk_gate[T, K]  fp32 output, same order as topk_idx.  SOFTMAX: softmax
 *                    over the K selected logits (equal to the softmax over
 *                    all E restricted to the selected and renormalised to sum
 *                    1); SIGMOID: see coli_scoring.
 * Selection: the K largest keys (logits, or biased sigmoid scores); on equal
 * keys (-0 and +0 are equal) the lower id wins; NaN never wins.  A slot with no valid candidate
 * (every remaining key NaN) takes id k if free, else the lowest free id (page
 * "colibrì 路由遥测全解析", section 测试与 CI 保障); its gates are then
 * unspecified.
 * x and w_router must be 4-byte (fp32) or 2-byte (bf16) aligned; 16-byte
 * aligned rows with H % 8 == 0 take the vector kernels.
 * Errors: EINVAL, ESHAPE (T outside [0, MAX_TOKENS], H outside [1, MAX_DIM],
 * E outside [1, MAX_EXPERTS], K outside [1, E]), EDTYPE, EALIGN.
 * T == 0 is a no-op.
 */
int coli_router_topk(const void *x, coli_dtype x_dtype, int T, int H,
                     const void *w_router, coli_dtype w_dtype, int E,
                     const float *bias, int K, int32_t *topk_idx,
                     float *topk_gate, float *logits, void *stream);
/* coli_router_topk with the scoring chosen (coli_router_topk is
 * COLI_SCORE_SOFTMAX).  Errors: as coli_router_topk, plus EINVAL for an
 * unknown scoring. */
int coli_router_topk_scored(const void *x, coli_dtype x_dtype, int T, int H,
                            const void *w_router, coli_dtype w_dtype, int E,
                            const float *bias, int K, coli_scoring scoring,
                            int32_t *topk_idx, float *topk_gate, float *logits,
                            void *stream);

/*
 * Batch-union permute (page "Colibrì 深度解析", section 四).
 *   topk_idx [T, K] int32 input, ids in [0, E)
 *   counts   [E]    int32: pairs (t, slot) routed to each expert
 *   offsets  [E+1]  int32: exclusive running sum of counts
 *   perm     [T*K]  int32: the pair indices p = t*K + slot sorted stably by
 *                   expert id (expert e owns perm[offsets[e] .. offsets[e+1]))
 *   unique   [E]    int32: experts with count > 0, ascending; entries past
 *                   *n_unique are unspecified
 *   n_unique [1]    int32
 *   workspace: device scratch of coli_expert_permute_workspace_bytes(T, K, E)
 *              bytes (0 for T*K <= 2048; then workspace may be NULL).
 * Pairs whose id lies outside [0, E) are skipped (not counted, not placed);
 * offsets[E] is the number of pairs placed.  A row may name an expert more
 * than once: every pair is counted and placed.
 * Errors: EINVAL, ESHAPE, EALIGN, EWORKSPACE.  T == 0 writes zero counts,
 * zero offsets and n_unique = 0.
 */
size_t coli_expert_permute_workspace_bytes(int T, int K, int E);
int coli_expert_permute(const int32_t *topk_idx, int T, int K, int E,
                        int32_t *counts, int32_t *offsets, int32_t *perm,
                        int32_t *unique, int32_t *n_unique, void *workspace,
                        size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* the layer                                                               */
/* ---------------------------------------------------------------------- */

/* One quantised matrix: packed [rows][ceil(cols/64)*32] u8, scales
 * [rows][ceil(cols/64)] f32. */
typedef struct {
    const uint8_t *q;
    const float *s;
} coli_q4;

/*
 * A MoE layer.  Host struct; the pointers in it are device pointers.
 *   w_router [E, H] in router_dtype (fp32 or bf16); router_bias [E] or NULL.
 *   experts: E expert blobs laid end to end, each coli_expert_blob_bytes(H,I)
 *            bytes; shared: one blob of the same layout (the shared expert,
 *            applied to every token with weight 1).  Both 256-byte aligned.
 *   scoring: the router's coli_scoring (0, SOFTMAX, when left zero).
 *   slot_map: device int32 [E] or NULL.  NULL: expert e's blob is blob e of
 *            `experts`.  Otherwise `experts` holds cache slots and expert e's
 *            blob is slot slot_map[e] (see coli_cache); an expert routed while
 *            its entry is -1 gives NaN outputs and COLI_STATUS_NOT_RESIDENT.
 *   usage: device uint64 [E] or NULL.  When set, every forward (and
 *            coli_moe_route) adds to usage[e] the number of its (token, slot)
 *            routing decisions that chose expert e, inside its routing kernels
 *            (the counters of the .coli_usage history, page "colibrì 路由遥测
 *            全解析", section 历史文件 .coli_usage: point it at this layer's row of
 *            the counts coli_usage_save writes).  8-byte aligned.
 * H and I may be any value in [1, MAX_DIM]: a row whose length is not a
 * multiple of 64 ends in a zero-padded group (the quantiser pads it so).
 */
typedef struct {
    int H, I, E, K;
    const void *w_router;
    coli_dtype router_dtype;
    const float *router_bias;
    const uint8_t *experts;
    const uint8_t *shared;
    coli_scoring scoring;
    const int32_t *slot_map;
    uint64_t *usage;
} coli_moe_layer;

/*
 * Size of one expert blob.  Layout (each section starts on a 256-byte
 * boundary): gate.q [I][GH*32] | up.q [I][GH*32] | down.q [H][GI*32] |
 * gate.s [I][GH] | up.s [I][GH] | down.s [H][GI] | gate.sT [GH][I] |
 * up.sT [GH][I] | down.sT [GI][H] | gate.sB [I8/8][GH][8] |
 * up.sB [I8/8][GH][8] | down.sB [H8/8][GI][8] | tag [16 B], with GH = ceil(H/64),
 * GI = ceil(I/64), I8 and H8 = I and H rounded up to a multiple of 8.
 * gate/up are [I, H] (input dim H); down is [H, I].  The .sT sections hold
 * the same scales group-major, the .sB sections blocked by 8 rows
 * (sB[b][g][r] = s[8b + r][g], zero past the last row; see
 * coli_expert_finish); the tag section is written by coli_expert_finish.
 * Returns 0 if H or I is outside [1, MAX_DIM].
 */
size_t coli_expert_blob_bytes(int H, int I);

/*
 * Fill the blob's group-major scale sections (gate.sT, up.sT, down.sT) and
 * its 8-row blocked ones (gate.sB, up.sB, down.sB) from its row-major ones:
 * sT[g][o] = s[o][g] and sB[o/8][g][o%8] = s[o][g], bit for bit (the padding
 * rows of the last block are written as 0), then write the blob's finish tag,
 * in stream order after the copies.  Call it once the three matrices are in
 * the blob (quantised by coli_quant_int4_g64 into the coli_expert_views
 * pointers, or written from stored bytes), and again after any change to
 * them, before the blob is used by coli_moe_forward in DECODE mode: the decode
 * batch path (1 < T) reads the scales group-major (one cache line per 32 rows
 * and group), the single-token path blocked (one 8-row item's groups are
 * contiguous).  The PREFILL path reads the format's row-major scales only.
 * A DECODE forward that reads a blob without the tag gives NaN outputs for
 * that expert and raises COLI_STATUS_UNFINISHED (fail closed).
 * Asynchronous on `stream`.  The blob is the layout above, of [P2] 权重转换's
 * sections.  Errors: EINVAL (NULL), ESHAPE, EALIGN (blob not 256-byte
 * aligned), EDEVICE.
 */
int coli_expert_finish(uint8_t *blob, int H, int I, void *stream);

/*
 * Quantise one expert into the blob at `blob` and finish it: gate [I, H],
 * up [I, H] and down [H, I] fp32 (device, row-major, 4-byte aligned) go
 * through coli_quant_int4_g64 into the coli_expert_views sections, then
 * coli_expert_finish.  status: as coli_quant_int4_g64 (optional).
 * Errors: as those two calls; nothing is launched on an argument error.
 */
int coli_quant_expert(uint8_t *blob, int H, int I, const float *w_gate,
                      const float *w_up, const float *w_down, int32_t *status,
                      void *stream);

/* Views of the three matrices of the blob at `blob` (pure pointer
 * arithmetic on the host; nothing is read).  Errors: EINVAL, ESHAPE. */
int coli_expert_views(const uint8_t *blob, int H, int I, coli_q4 *gate,
                      coli_q4 *up, coli_q4 *down);

/* Workspace bytes coli_moe_forward needs for T tokens in `mode`
 * (0 if the layer's shape is invalid). */
size_t coli_moe_workspace_bytes(const coli_moe_layer *L, int T, coli_mode mode);

/*
 * One forward pass of the layer for T tokens:
 *   logits = x Wr^T (+ b), top-K with renormalised gates (as
 *     coli_router_topk_scored with L->scoring);
 *   batch-union permute (as coli_expert_permute);
 *   per selected (token, expert): h = SiLU(Wg x) * (Wu x), o = Wd h, with
 *     W = s * (u - 8) read from the planar bytes;
 *   y[t] = sum_k gate[t,k] * o[t,k] + Wd_sh (SiLU(Wg_sh x) * (Wu_sh x)).
 *   mode DECODE:  x, y fp32 [T, H]; fp32-class products on the matrix cores:
 *                 weights as the exact integers u - 8 with the fp32 group
 *                 scale applied per group, x and h split into fp16 hi + lo
 *                 parts under a power-of-two scale per row (T = 1 with H and
 *                 I multiples of 256: int8 digit planes), h and the per-slot
 *                 outputs held in fp32.  T > 256 runs as consecutive 256-token
 *                 batches (each reads its experts once).
 *   mode PREFILL: x, y bf16 [T, H], T <= COLI_MAX_TOKENS; grouped GEMMs on
 *                 the matrix cores with fp32 accumulation and fp16 operands:
 *                 each token's x is scaled by a power of two 2^-e (its
 *                 largest |x| then lies in [2, 4)) and its h by 2^-2e before
 *                 the fp16 conversion, weights s*(u-8) enter with s rounded
 *                 to fp16, per-slot outputs are fp16 before the fp32 combine,
 *                 which undoes the scaling.  Group scales must stay below 64.
 *   topk_idx_out, topk_gate_out: optional [T, K] copies of the routing.
 *   status: optional device int32 flag; COLI_STATUS_* bits are OR-ed in.
 *   workspace: device scratch of at least coli_moe_workspace_bytes bytes,
 *              256-byte aligned; its contents need no initialisation and are
 *              undefined afterwards.
 * Any H and I in [1, MAX_DIM].  Errors: EINVAL, ESHAPE (also when a buffer of
 * the call would pass 2^31 bytes, the limit of the kernels' buffer offsets;
 * coli_moe_workspace_bytes is then 0), EDTYPE, EALIGN (x, y 16-byte; blobs and
 * workspace 256-byte; status 4-byte), EWORKSPACE, EDEVICE.  Every check runs
 * before the first launch.  T == 0 is a no-op.
 */
int coli_moe_forward(const coli_moe_layer *L, coli_mode mode, const void *x,
                     int T, void *y, int32_t *topk_idx_out,
                     float *topk_gate_out, int32_t *status, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * coli_moe_forward with stage timestamps, for measurement.  events holds a
 * (start, stop) pair of hipEvent_t values (created by the caller with timing
 * enabled, passed as void*) per stage: events[2s] and events[2s + 1] bracket
 * stage s on `stream`.  Stages: DECODE 0 route (logits, top-K, permute),
 * 1 gate/up, 2 down + combine; PREFILL 0 route, 1 activation conversion and
 * tile list, 2 gate/up, 3 down, 4 combine.  Where a stage is a single kernel
 * (the single-token decode path) the pair is stamped by that kernel's own
 * launch, so elapsed(start, stop) is its execution time; elsewhere the events
 * are recorded on the stream before and after the stage's launches.
 * n_events must be at least 2 x the stage count (6 or 10).  Same work and
 * results as coli_moe_forward; DECODE takes T <= 256 here.
 * Errors: as coli_moe_forward, plus EINVAL for a NULL or short event array
 * and ESHAPE for DECODE with T > 256.
 */
int coli_moe_forward_timed(const coli_moe_layer *L, coli_mode mode,
                           const void *x, int T, void *y,
                           int32_t *topk_idx_out, float *topk_gate_out,
                           int32_t *status, void *workspace,
                           size_t workspace_bytes, void *stream, void **events,
                           int n_events);

/*
 * The forward in two calls, so that the caller can act on the routing before
 * the experts run: coli_moe_route does logits, top-K, gates and the batch
 * union (and, on the single-token path, x's digit planes), leaving them in the
 * workspace; coli_moe_experts then runs the expert FFNs and the combine from
 * that workspace.  Between the two the caller may read the batch's expert list
 * (unique_out, n_unique_out: optional device int32 [E] and [1], the unique
 * routed experts in ascending id order) and place the experts (coli_cache).
 * The pair gives the same results as coli_moe_forward when both calls take the
 * same L, mode, x, T and workspace (untouched in between).  DECODE takes
 * T <= 256 here.  Errors: as coli_moe_forward (ESHAPE for DECODE with
 * T > 256).
 */
int coli_moe_route(const coli_moe_layer *L, coli_mode mode, const void *x, int T,
                   int32_t *topk_idx_out, float *topk_gate_out,
                   int32_t *unique_out, int32_t *n_unique_out, void *workspace,
                   size_t workspace_bytes, void *stream);
int coli_moe_experts(const coli_moe_layer *L, coli_mode mode, const void *x, int T,
                     void *y, int32_t *topk_idx_out, float *topk_gate_out,
                     int32_t *status, void *workspace, size_t workspace_bytes,
                     void *stream);

/* ---------------------------------------------------------------------- */
/* expert placement (page "Colibrì 深度解析", section 三; page "为什么Colibrì  */
/* 越用越快", section 实时重固定REPIN)                                       */
/* ---------------------------------------------------------------------- */

/* 1 if an expert of heat `hot` may replace one of heat `cold`: hot > cold +
 * cold/4 + 4, computed in 64 bits (a saturated 32-bit heat stays put). */
int coli_tier_should_promote(uint32_t hot, uint32_t cold);
/* LFRU score: heat * 256 + recent, recent = 255 - age if the age
 * (clock - last, modulo 2^32) is below 255, else 0: one routing outweighs any
 * recency. */
uint64_t coli_tier_lfru_score(uint32_t heat, uint32_t last, uint32_t clock);

/*
 * An HBM cache of S expert blobs over host memory holding all E.  Host
 * memory owned by the caller; the functions below read and write it only.
 *   heat[E]      routings per expert (saturating), halved by coli_cache_decay
 *   last[E]      the clock of the expert's last admission
 *   slot_of[E]   the expert's slot, or -1
 *   expert_of[S] the slot's expert, or -1
 * 1 <= S <= E <= COLI_MAX_EXPERTS.
 */
typedef struct {
    int E, S;
    uint32_t clock;
    uint32_t *heat;
    uint32_t *last;
    int32_t *slot_of;
    int32_t *expert_of;
} coli_cache;

/* Zero the heat and clock, free every slot.  Errors: EINVAL, ESHAPE. */
int coli_cache_init(coli_cache *c);
/* Halve every heat (integer halving: the heat fades with time).  Errors:
 * EINVAL, ESHAPE. */
int coli_cache_decay(coli_cache *c);
/*
 * Admit the experts one batch needs (HOST ids `needed`, duplicates allowed):
 * the clock advances by one; each needed expert's heat grows by one and its
 * last becomes the clock; each needed expert without a slot takes a free slot
 * (lowest index first), else the slot of the resident the batch does not need
 * with the lowest LFRU score (ties: the lower id).  The loads to perform are
 * written to load_expert / load_slot (HOST, room for S each), *n_loads their
 * number, in the order the experts are first named.  Nothing changes on an
 * error: EINVAL (NULL, an id outside [0, E)), ESHAPE (the batch needs more
 * than S experts).
 */
int coli_cache_admit(coli_cache *c, const int32_t *needed, int n, int32_t *load_expert,
                     int32_t *load_slot, int *n_loads);
/*
 * REPIN: rank the non-resident experts by LFRU score (highest first) and the
 * residents (lowest first), pair them in that order and swap while the hot
 * one may replace the cold one (coli_tier_should_promote on their heats), at
 * most max_swaps times (the pages use 4).  Writes the swaps (HOST, room for
 * max_swaps each): the admitted expert, its slot, the evicted expert.
 * Errors: EINVAL, ESHAPE.
 */
int coli_cache_repin(coli_cache *c, int max_swaps, int32_t *load_expert, int32_t *load_slot,
                     int32_t *evicted, int *n_swaps);
/*
 * Copy the planned loads: blob load_expert[i] of host_blobs (PINNED host
 * memory, E blobs of blob_bytes) to slot load_slot[i] of `slots` (device, S
 * blobs), asynchronously on `stream` (hipMemcpyAsync, host to device).  The
 * ids are not checked against E and S (the caller's buffers): pass the lists
 * coli_cache_admit / coli_cache_repin wrote.  A slot must not be overwritten
 * while a kernel that reads it may still run: stage on the stream of the
 * forward, or order the streams.  Errors: EINVAL (NULL, negative id), ESHAPE,
 * EDEVICE.
 */
int coli_cache_stage(const uint8_t *host_blobs, uint8_t *slots, size_t blob_bytes,
                     const int32_t *load_expert, const int32_t *load_slot, int n_loads,
                     void *stream);
/* Upload c->slot_of to the device slot map (int32 [E]) on `stream`, for
 * coli_moe_layer.slot_map (hipMemcpyAsync, host to device: keep c->slot_of
 * unchanged until the stream has passed the copy).  Errors: EINVAL, ESHAPE,
 * EDEVICE. */
int coli_cache_slot_map(const coli_cache *c, int32_t *slot_map, void *stream);

/* ---------------------------------------------------------------------- */
/* sibling weight formats (page "从源码开始colibri纯C引擎的编译、权重转换与   */
/* .bin直映射实战", section 权重转换: the format registry, a tensor's format    */
/* inferred from its byte counts; page "Colibrì 深度解析", sections 八, 十    */
/* and 十五)                                                                  */
/* ---------------------------------------------------------------------- */

/* The registry's ordinals. */
typedef enum {
    COLI_FMT_F32 = 0,           /* 4 O I bytes, no scale array                   */
    COLI_FMT_INT8_ROW = 1,      /* O I bytes + one f32 per row                   */
    COLI_FMT_INT4_ROW = 2,      /* O ceil(I/2) bytes + one f32 per row           */
    COLI_FMT_INT2_ROW = 3,      /* O ceil(I/4) bytes + one f32 per row           */
    COLI_FMT_INT4_G64 = 4,      /* this library's int4-g64 planar format         */
    COLI_FMT_INT3_G64 = 5,      /* 24 bytes per 64 (three bit planes of u = q+4) */
                                /* + one f32 per 64: s = amax/3, q in [-4, 3]    */
    COLI_FMT_E8_IQ3 = 6,        /* layout not known here: never inferred         */
    COLI_FMT_MXFP4 = 7,         /* OCP MX: 16 bytes per 32 (E2M1 nibbles, element */
                                /* 2j low) + one E8M0 byte per 32                */
    COLI_FMT_FP8_E4M3_B128 = 8  /* OCP E4M3 bytes [O, I] + one f32 per 128x128   */
                                /* tile: s = amax/448                            */
} coli_fmt;

#define COLI_FMT_MAX_ROWS 1048576  /* O limit of the format calls               */
#define COLI_MATVEC_MAX_T 8

/* Weight and scale byte counts of an [O, I] tensor in `fmt` (HOST outputs).
 * Errors: EINVAL (NULL, fmt 6 or unknown), ESHAPE (O or I outside
 * [1, FMT_MAX_ROWS] x [1, MAX_DIM]). */
int coli_fmt_bytes(int fmt, int64_t O, int64_t I, uint64_t *weight_bytes,
                   uint64_t *scale_bytes);
/* The format whose byte counts are these, from the counts and [O, I] alone.
 * Returns the ordinal (>= 0) when exactly one format matches, else
 * COLI_EFORMAT (fail closed: some shapes give two formats the same counts,
 * e.g. int4-row and int4-g64 at I = 64); *candidates (optional, HOST) gets the
 * bit set of the matching ordinals.  ESHAPE for O or I out of range. */
int coli_resolve_fmt(int64_t O, int64_t I, uint64_t weight_bytes, uint64_t scale_bytes,
                     uint32_t *candidates);
/* Quantise fp32 w [O, I] (device) into `packed` / `scales` (device, sizes from
 * coli_fmt_bytes) in fmt 4, 5, 7 or 8, bit-exact to the rules above (round to
 * nearest even; zero-padded ragged groups and blocks; a group, block or tile
 * holding a non-finite value gets the NaN scale (E8M0 255), neutral codes and
 * status bit 1).  Alignment: w 4, packed 8 (int3) or 4, scales 4.  Errors:
 * EINVAL (NULL, other fmt), ESHAPE, EALIGN, EDEVICE. */
int coli_quant_fmt(int fmt, const float *w, int64_t O, int64_t I, void *packed,
                   void *scales, int32_t *status, void *stream);
/* Dequantising matrix-vector product for decode: y[t, o] = sum_i W^[o, i] x[t, i]
 * for t < T <= 8, W^ the dequantised [O, I] tensor in fmt 4, 5, 7 or 8 (fmt 4
 * with its row-major scales), x fp32 [T, I], y fp32 [T, O] (device), fp32
 * accumulation.  Limits: T * (I rounded up to the format's group) <= 24576;
 * fp8 rows a multiple of 16 bytes (I % 16 == 0).  Alignment: packed 16 (8 for
 * int3), scales, x and y 4.  Errors: EINVAL, ESHAPE, EALIGN, EDEVICE. */
int coli_matvec_fmt(int fmt, const void *packed, const void *scales, int64_t O, int64_t I,
                    const float *x, int T, float *y, void *stream);

/* A layer whose routed and shared experts are in a sibling format (fmt 4, 5,
 * 7 or 8), decode only.  One expert blob in fmt: gate.q | up.q | down.q |
 * gate.s | up.s | down.s (the coli_fmt_bytes arrays of gate [I, H], up [I, H]
 * and down [H, I]), each section 256-byte aligned; 0 for another fmt. */
size_t coli_fmt_blob_bytes(int fmt, int H, int I);
/* Quantise fp32 gate [I, H], up [I, H], down [H, I] (device) into a blob
 * (256-byte aligned) with coli_quant_fmt.  Errors: as coli_quant_fmt. */
int coli_quant_expert_fmt(int fmt, uint8_t *blob, int H, int I, const float *w_gate,
                          const float *w_up, const float *w_down, int32_t *status,
                          void *stream);
/* Workspace of coli_moe_forward_fmt (0 for an unsupported fmt or shape). */
size_t coli_moe_fmt_workspace_bytes(const coli_moe_layer *L, int fmt, int T);
/*
 * The layer a1-a6 with experts in fmt (L->experts: E blobs at a stride of
 * coli_fmt_blob_bytes, L->shared: one blob; L->slot_map must be NULL), DECODE:
 * x fp32 [T, H] -> y fp32 [T, H], T <= 4 with T * H and T * I (each rounded up
 * to the format's group) at most 24576.  The routing is the one of
 * coli_moe_forward (softmax or sigmoid scoring, ids and gates optional
 * outputs); per unique routed expert and the shared one: h = SiLU(W^g x) *
 * (W^u x) * gate weight, then W^d h, summed in unit order (fp32 products as in
 * coli_matvec_fmt).  Errors: as coli_moe_forward, plus EINVAL for another fmt
 * or a slot map, ESHAPE for T or H, I beyond those limits (fp8: H and I
 * multiples of 16).
 */
int coli_moe_forward_fmt(const coli_moe_layer *L, int fmt, const float *x, int T, float *y,
                         int32_t *topk_idx_out, float *topk_gate_out, int32_t *status,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as coli_moe_forward, with the workspace taken from a static device
 * array of COLI_NOALLOC_SCRATCH_BYTES inside the library (each GPU the library
 * runs on holds its own copy until the process ends).  The caller still passes
 * x, y and the optional outputs.  No hipMalloc, hipFree or other allocation;
 * the array's device address is looked up once per device, on the first call
 * made with that device current (the stream must belong to the current
 * device).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and give undefined results.
 * The workspace needs no initialisation, so nothing is cleared between calls.
 * Errors: as coli_moe_forward (argument errors take precedence), ESCRATCH when
 * coli_moe_workspace_bytes(L, T, mode) exceeds COLI_NOALLOC_SCRATCH_BYTES (32
 * MiB: the layer H=6144, I=2048, E=256, K=8 fits decode up to T = 74 and
 * prefill up to T = 206), EDEVICE if the address lookup fails.  T == 0 is a
 * no-op.
 */
#define COLI_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int coli_moe_forward_noalloc(const coli_moe_layer *L, coli_mode mode,
                             const void *x, int T, void *y,
                             int32_t *topk_idx_out, float *topk_gate_out,
                             int32_t *status, void *stream);

/* ---------------------------------------------------------------------- */
/* routing history (page "colibrì 路由遥测全解析：.coli_usage专家历史、       */
/* ROUTE_TRACE追踪流与route_trace.h统一格式")                               */
/* ---------------------------------------------------------------------- */

#define COLI_USAGE_VERSION 1

/*
 * Add one layer's routing decisions to device counters (section 历史文件: the
 * engine counts, per layer, which experts each routing decision chose):
 *   counts[layer][e] += number of (token, slot) pairs of topk_idx [T, K] with
 *   id e.  counts: device uint64 [n_layers][n_experts], 8-byte aligned, kept
 *   by the caller across calls.  Ids outside [0, n_experts) are not counted.
 * Integer atomics: exact and order independent.  Errors: EINVAL, ESHAPE,
 * EALIGN, EDEVICE.  T == 0 is a no-op.
 */
int coli_usage_count(const int32_t *topk_idx, int T, int K, int n_experts,
                     int layer, int n_layers, uint64_t *counts, void *stream);

/* The engine identity written in the history's "-2" record: the 32-bit
 * FNV-1a hash of the engine's name (the page's glm_moe_dsa is 3815245270). */
uint32_t coli_usage_engine_hash(const char *name);

/*
 * Write a routing history (host function; sections 历史文件, 头部记录为什么长这样,
 * 三条铁律, 空历史 = 零字节文件, COLI_USAGE_DECAY).  counts: HOST uint64
 * [n_layers][n_experts] (copied from the device counters by the caller).
 * The file, text, one record of exactly three numbers per line:
 *   -1 n_layers n_experts
 *   -2 COLI_USAGE_VERSION engine_hash
 *   layer expert count     (one per non-zero counter, ascending; counts above
 *                           2^32 - 1 are written as 2^32 - 1)
 * and nothing at all when every count is zero (a zero-byte file).  decay in
 * (0, 1): each count becomes round(count * decay), a non-zero count never
 * below 1; other values leave the counts as they are.  dropped: HOST
 * [n_layers] flags or NULL; a dropped layer's counts are never written.  The
 * file is written to "<path>.tmp.<pid>" and renamed over path; that
 * temporary path is built, and rejected with EINVAL if it does not fit 4096
 * bytes, before the file system is touched.  Errors: EINVAL, ESHAPE, EIO.
 */
int coli_usage_save(const char *path, const uint64_t *counts, int n_layers,
                    int n_experts, uint32_t engine_hash, double decay,
                    const uint8_t *dropped);

/*
 * Read a routing history into HOST counters (counts [n_layers][n_experts]
 * are added to; section 可信读取 and 仍然兼容读取的旧布局).  A zero-byte file
 * is an empty history.  Text files are read three numbers at a time: a "-1"
 * record must carry these dimensions and a "-2" record this format version
 * (both never relaxed) and engine_hash (relaxed when trusted != 0); records
 * with another negative layer are skipped; a record whose layer or expert is
 * out of range, or whose layer is dropped, is discarded.  Header-less legacy
 * files are accepted as they are.  A file starting with the magic "IKU1" is
 * the dense layout uint32 {magic, n_layers, n_experts} then uint32
 * [n_layers][n_experts], read only when engine_hash is that of "inkling" and
 * the dimensions match.  *accepted_total (optional) receives the sum of the
 * accepted counts only.  On EUSAGE the counters may hold part of the file.
 * Errors: EINVAL, ESHAPE, EIO (cannot open), EUSAGE (refused).
 */
int coli_usage_load(const char *path, uint64_t *counts, int n_layers,
                    int n_experts, uint32_t engine_hash, int trusted,
                    const uint8_t *dropped, uint64_t *accepted_total);

/*
 * RMSNorm with unit weight between stacked layers:
 *   y[t] = x[t] / sqrt(mean(x[t]^2) + eps), fp32 [T, H]; x == y allowed.
 * Errors: EINVAL (NULL, eps < 0 or not finite), ESHAPE, EALIGN (x or y not
 * 4-byte aligned).  T == 0 is a no-op.
 */
int coli_rmsnorm_f32(const float *x, float *y, int T, int H, float eps,
                     void *stream);

#ifdef __cplusplus
}
#endif
#endif /* COLI_H */

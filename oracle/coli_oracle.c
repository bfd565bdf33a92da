/*
 * coli_oracle.c -- the oracle: a plain, slow, fp64 CPU statement of the
 * routed-expert MoE layer with int4-g64 planar experts.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source, header, table or helper with
 * the HIP library: every definition below is written out again from the
 * pages, in the pages' order, with no blocking, fusion or reordering.
 *
 * Sources (cited by page title and section):
 *   [P1] "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
 *        section 四 (batch union: positions routed to one expert read it once)
 *        and section 十一 (the five token stages; "route" selects top-k).
 *   [P2] "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
 *        section 权重转换 (the int4 grouped quantiser: group 64, qmax 7,
 *        clip to [-8,7], rint, +8 offset, one f32 scale per group, and the
 *        planar nibble layout of the expert FFN: byte k of a 64-group holds
 *        element k low and element k+32 high).
 *   [P4] "colibrì 路由遥测全解析.coli_usage专家历史、ROUTE_TRACE追踪流与
 *        route_trace.h统一格式", sections 分离计数与追踪 / 追踪流ROUTE_TRACE
 *        (the gates applied are the normalised ones) and 测试与 CI 保障
 *        (router NaN guard: a slot with no valid candidate falls back to a
 *        deterministic index).
 *
 * Readings where the pages are silent (each one is listed in the design doc):
 *   - scale s = fl32(amax / 7); the quotient w/s is the IEEE fp32 quotient,
 *     rounded to fp32 before round-half-even;
 *   - a group whose scale is 0 stores all nibbles 8 and scale +0;
 *   - a group holding a NaN or Inf stores nibbles 8, a NaN scale, and sets
 *     bit 0 of the returned status;
 *   - a ragged last group is zero padded;
 *   - gates are softmax over all E restricted to the selected K and
 *     renormalised (which equals softmax over the K selected logits);
 *   - ties at the top-K boundary go to the lower expert id, NaN never wins,
 *     and the K ids are returned in ascending order;
 *   - h = SiLU(gate) * up, y = sum_k g_k Wd_k h_k + Wd_shared h_shared;
 *   - the sigmoid router with no auxiliary loss ([P1] 十一: one expert group,
 *     sigmoid scores, "noaux_tc" selection): score s_e = 1 / (1 + e^-l_e) of
 *     the raw logit; the selection key is s_e + b_e, where the per-expert bias
 *     b steers which experts are picked and nothing else; the gates are the
 *     selected scores divided by their sum; with a single group the group
 *     stage keeps every expert; no routed scaling factor (1).
 *
 * Arithmetic: everything is fp64 except where the quantiser must reproduce an
 * fp32 result exactly.  fp64 then fp32 rounding of a quotient of two fp32
 * values equals the correctly rounded fp32 quotient (53 >= 2*24 + 2), so the
 * scale and the quotient below are the IEEE fp32 values.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fopenmp -fPIC -shared.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GS 64 /* group size along the input dimension [P2 权重转换] */

/* ------------------------------------------------------------------ */
/* element conversions                                                 */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper 16 bits of an fp32 value; widening is exact. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* dtype codes used by the oracle's entry points: 0 = fp32, 1 = bf16,
 * 2 = fp64 (activations carried between stacked layers) */
static double load_elem(const void *base, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float *)base)[i];
    if (dtype == 2) return ((const double *)base)[i];
    return bf16_to_double(((const uint16_t *)base)[i]);
}

/* ------------------------------------------------------------------ */
/* quantiser and planar packer   [P2 权重转换]                         */
/* ------------------------------------------------------------------ */

int64_t orc_groups(int64_t cols) { return (cols + GS - 1) / GS; }

/*
 * Quantise one fp32 matrix W[rows][cols] to int4-g64 planar.
 *   packed: [rows][groups*32] bytes, scales: [rows][groups] fp32.
 * Per row and per 64-group along the columns:
 *   amax = max |w|;  s = fl32(amax / 7);
 *   q = clip(rint_half_even(fl32(w / s)), -8, 7);  u = q + 8;
 *   byte (g*32 + k) = u[k] | (u[k+32] << 4)   for k = 0..31.
 * Returns 1 if any element was NaN or Inf, else 0.
 */
int orc_quant_int4_g64(const float *w, int64_t rows, int64_t cols,
                       uint8_t *packed, float *scales) {
    const int64_t G = orc_groups(cols);
    int status = 0;
#pragma omp parallel for reduction(| : status) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < G; ++g) {
            float v[GS];
            int finite = 1;
            for (int j = 0; j < GS; ++j) {
                int64_t c = g * GS + j;
                v[j] = (c < cols) ? w[r * cols + c] : 0.0f; /* zero pad */
                if (!isfinite(v[j])) finite = 0;
            }
            unsigned u[GS];
            float s;
            if (!finite) {
                s = NAN;
                for (int j = 0; j < GS; ++j) u[j] = 8;
                status |= 1;
            } else {
                float amax = 0.0f;
                for (int j = 0; j < GS; ++j) {
                    float a = fabsf(v[j]);
                    if (a > amax) amax = a;
                }
                s = (float)((double)amax / 7.0);
                if (s == 0.0f) {
                    for (int j = 0; j < GS; ++j) u[j] = 8;
                } else {
                    for (int j = 0; j < GS; ++j) {
                        float quot = (float)((double)v[j] / (double)s);
                        double q = nearbyint((double)quot); /* half to even */
                        if (q < -8.0) q = -8.0;
                        if (q > 7.0) q = 7.0;
                        u[j] = (unsigned)((int)q + 8);
                    }
                }
            }
            scales[r * G + g] = s;
            uint8_t *dst = packed + r * (G * 32) + g * 32;
            for (int k = 0; k < 32; ++k)
                dst[k] = (uint8_t)(u[k] | (u[k + 32] << 4));
        }
    }
    return status;
}

/* The unsigned nibble of element (r, c) in a planar packed matrix. */
static unsigned nibble_at(const uint8_t *packed, int64_t G, int64_t r, int64_t c) {
    int64_t g = c / GS, j = c % GS;
    uint8_t b = packed[r * (G * 32) + g * 32 + (j % 32)];
    return (j < 32) ? (b & 0x0Fu) : (b >> 4);
}

/* Dequantise exactly: What[r][c] = s[r][c/64] * (u[r][c] - 8), in fp64. */
void orc_dequant_int4_g64(const uint8_t *packed, const float *scales,
                          int64_t rows, int64_t cols, double *out) {
    const int64_t G = orc_groups(cols);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (double)scales[r * G + c / GS] *
                                ((double)nibble_at(packed, G, r, c) - 8.0);
}

/* ------------------------------------------------------------------ */
/* router logits and top-K with renormalised gates  [P1 十一] [P4]      */
/* ------------------------------------------------------------------ */

/* logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]   (fp64, h ascending) */
void orc_router_logits(const void *x, int x_dtype, int T, int H,
                       const void *wr, int w_dtype, int E, const float *bias,
                       double *logits) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += load_elem(x, x_dtype, (size_t)t * H + h) *
                       load_elem(wr, w_dtype, (size_t)e * H + h);
            if (bias) acc += (double)bias[e];
            logits[(size_t)t * E + e] = acc;
        }
}

/*
 * Select K of E logits per token by K rounds of argmax.  A round takes the
 * largest logit not yet taken; NaN never wins, and on equal values the lower
 * id wins because the scan is ascending with a strict comparison.  A round
 * with no valid candidate (every remaining logit NaN) takes id `round` if
 * that id is still free, else the lowest free id [P4 测试与 CI 保障].
 * The ids are returned in ascending order; the gates are
 * exp(l_i - m) / sum_j exp(l_j - m) over the selected set, m = their max.
 * Returns the number of rounds that used the fallback (0 for valid input).
 */
int orc_topk(const double *logits, int T, int E, int K, int32_t *idx,
             double *gates) {
    int fallbacks = 0;
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int round = 0; round < K; ++round) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e] || isnan(l[e])) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            if (best < 0) {
                ++fallbacks;
                if (round < E && !taken[round]) best = round;
                else
                    for (int e = 0; e < E; ++e)
                        if (!taken[e]) { best = e; break; }
            }
            taken[best] = 1;
        }
        int n = 0;
        for (int e = 0; e < E; ++e)
            if (taken[e]) idx[(size_t)t * K + n++] = e;
        double m = -INFINITY;
        for (int i = 0; i < K; ++i) {
            double v = l[idx[(size_t)t * K + i]];
            if (v > m) m = v;
        }
        double z = 0.0;
        for (int i = 0; i < K; ++i) z += exp(l[idx[(size_t)t * K + i]] - m);
        for (int i = 0; i < K; ++i)
            gates[(size_t)t * K + i] = exp(l[idx[(size_t)t * K + i]] - m) / z;
    }
    free(taken);
    return fallbacks;
}

/*
 * The sigmoid router of [P1] 十一 ("n_group=1 sigmoid + noaux_tc"), per token:
 *   1. score s_e = 1 / (1 + exp(-l_e)) for every expert (l: raw logits);
 *   2. one expert group (n_group = 1): the group stage keeps all E experts;
 *   3. key k_e = s_e + b_e (b: the selection bias, zero if NULL); take the K
 *      largest keys by K rounds of argmax with the same rules as orc_topk
 *      (strict >, so ties go to the lower id; NaN never wins; the [P4]
 *      fallback for a round with no valid candidate);
 *   4. ids in ascending order; gate_i = s_i / sum_{j selected} s_j (the bias
 *      does not enter the gates).
 * Returns the number of fallback rounds (0 for valid input).
 */
int orc_topk_sigmoid(const double *logits, int T, int E, int K, const float *bias,
                     int32_t *idx, double *gates) {
    int fallbacks = 0;
    char *taken = (char *)malloc((size_t)E);
    double *s = (double *)malloc(sizeof(double) * (size_t)E);
    double *key = (double *)malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e) {
            s[e] = 1.0 / (1.0 + exp(-l[e]));
            key[e] = s[e] + (bias ? (double)bias[e] : 0.0);
        }
        memset(taken, 0, (size_t)E);
        for (int round = 0; round < K; ++round) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e] || isnan(key[e])) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            if (best < 0) {
                ++fallbacks;
                if (round < E && !taken[round]) best = round;
                else
                    for (int e = 0; e < E; ++e)
                        if (!taken[e]) { best = e; break; }
            }
            taken[best] = 1;
        }
        int n = 0;
        for (int e = 0; e < E; ++e)
            if (taken[e]) idx[(size_t)t * K + n++] = e;
        double z = 0.0;
        for (int i = 0; i < K; ++i) z += s[idx[(size_t)t * K + i]];
        for (int i = 0; i < K; ++i)
            gates[(size_t)t * K + i] = s[idx[(size_t)t * K + i]] / z;
    }
    free(taken); free(s); free(key);
    return fallbacks;
}

/* ------------------------------------------------------------------ */
/* batch-union permute  [P1 四]                                        */
/* ------------------------------------------------------------------ */

/*
 * counts[e] = number of (token, slot) pairs routed to expert e;
 * offsets[0..E] = exclusive running sum of counts;
 * perm[offsets[e] ..] = the pair indices p = t*K + slot routed to e, in
 * increasing p (a stable sort of p by expert id);
 * unique[0..n) = the experts with counts > 0, ascending.  Returns n.
 */
int orc_permute(const int32_t *idx, int T, int K, int E, int32_t *counts,
                int32_t *offsets, int32_t *perm, int32_t *unique) {
    const int P = T * K;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < P; ++p) counts[idx[p]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int p = 0; p < P; ++p) perm[fill[idx[p]]++] = p;
    free(fill);
    int n = 0;
    for (int e = 0; e < E; ++e)
        if (counts[e] > 0) unique[n++] = e;
    return n;
}

/* ------------------------------------------------------------------ */
/* one expert's FFN on dequantised weights  [P2 权重转换]               */
/* ------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * For n input vectors x[n][H] (fp64):
 *   gate = Wg x, up = Wu x  (Wg, Wu: [I][H]);  h = SiLU(gate) * up;
 *   out = Wd h  (Wd: [H][I]).
 * The weights are the exact dequantised values s * (u - 8), read nibble by
 * nibble from the planar bytes.  h_out (n x I) may be NULL.
 */
void orc_expert_ffn(const uint8_t *gq, const float *gs, const uint8_t *uq,
                    const float *us, const uint8_t *dq, const float *ds,
                    int H, int I, const double *x, int n, double *out,
                    double *h_out) {
    const int64_t GH = orc_groups(H), GI = orc_groups(I);
    double *h = (double *)malloc(sizeof(double) * (size_t)n * (size_t)I);
#pragma omp parallel for collapse(2) schedule(static)
    for (int j = 0; j < n; ++j)
        for (int o = 0; o < I; ++o) {
            double g = 0.0, u = 0.0;
            for (int k = 0; k < H; ++k) {
                double xv = x[(size_t)j * H + k];
                g += (double)gs[o * GH + k / GS] *
                     ((double)nibble_at(gq, GH, o, k) - 8.0) * xv;
                u += (double)us[o * GH + k / GS] *
                     ((double)nibble_at(uq, GH, o, k) - 8.0) * xv;
            }
            h[(size_t)j * I + o] = silu(g) * u;
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int j = 0; j < n; ++j)
        for (int r = 0; r < H; ++r) {
            double acc = 0.0;
            for (int o = 0; o < I; ++o)
                acc += (double)ds[r * GI + o / GS] *
                       ((double)nibble_at(dq, GI, r, o) - 8.0) *
                       h[(size_t)j * I + o];
            out[(size_t)j * H + r] = acc;
        }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)n * (size_t)I);
    free(h);
}

/* ------------------------------------------------------------------ */
/* the whole layer                                                     */
/* ------------------------------------------------------------------ */

/*
 * One quantised expert as the oracle holds it: three planar matrices.
 * gate, up: [I][H]; down: [H][I].
 */
typedef struct {
    const uint8_t *gq; const float *gs;
    const uint8_t *uq; const float *us;
    const uint8_t *dq; const float *ds;
} orc_expert;

/*
 * y[t] = sum_k gates[t][k] * FFN_{idx[t][k]}(x[t]) + FFN_shared(x[t]).
 * The routing (logits, top-K, gates) is computed here from x, Wr and b:
 * scoring 0 is the softmax router (b added to the logits, orc_topk),
 * scoring 1 the sigmoid router (b steers the selection, orc_topk_sigmoid).
 * experts[0..E) are the routed experts (an entry may have NULL pointers if
 * no token selects it; the call then returns -1 if one is selected);
 * shared is the shared expert, applied with weight 1.
 * Terms are added in ascending slot order, then the shared term.
 */
int orc_moe_forward(const void *x, int x_dtype, int T, int H, int I, int E,
                    int K, const void *wr, int w_dtype, const float *bias,
                    int scoring, const orc_expert *experts,
                    const orc_expert *shared, double *y, int32_t *idx,
                    double *gates) {
    double *logits = (double *)malloc(sizeof(double) * (size_t)T * (size_t)E);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    int rc = 0;
    if (scoring == 0) {
        /* softmax router: the bias is part of the logits */
        orc_router_logits(x, x_dtype, T, H, wr, w_dtype, E, bias, logits);
        orc_topk(logits, T, E, K, idx, gates);
    } else {
        /* sigmoid router: raw logits; the bias enters the selection only */
        orc_router_logits(x, x_dtype, T, H, wr, w_dtype, E, NULL, logits);
        orc_topk_sigmoid(logits, T, E, K, bias, idx, gates);
    }
    for (int t = 0; t < T && rc == 0; ++t) {
        for (int h = 0; h < H; ++h) xd[h] = load_elem(x, x_dtype, (size_t)t * H + h);
        double *yt = y + (size_t)t * H;
        for (int h = 0; h < H; ++h) yt[h] = 0.0;
        for (int k = 0; k < K; ++k) {
            const orc_expert *ex = &experts[idx[(size_t)t * K + k]];
            if (!ex->gq || !ex->uq || !ex->dq) { rc = -1; break; }
            orc_expert_ffn(ex->gq, ex->gs, ex->uq, ex->us, ex->dq, ex->ds, H, I,
                           xd, 1, o, NULL);
            double g = gates[(size_t)t * K + k];
            for (int h = 0; h < H; ++h) yt[h] += g * o[h];
        }
        if (rc) break;
        orc_expert_ffn(shared->gq, shared->gs, shared->uq, shared->us,
                       shared->dq, shared->ds, H, I, xd, 1, o, NULL);
        for (int h = 0; h < H; ++h) yt[h] += o[h];
    }
    free(logits); free(xd); free(o);
    return rc;
}

/* ------------------------------------------------------------------ */
/* RMSNorm between stacked layers (unit weight, no residual)           */
/* ------------------------------------------------------------------ */

/* out[t] = y[t] / sqrt(mean(y[t]^2) + eps) */
void orc_rmsnorm(const double *y, int T, int H, double eps, double *out) {
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int h = 0; h < H; ++h) ss += y[(size_t)t * H + h] * y[(size_t)t * H + h];
        double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int h = 0; h < H; ++h) out[(size_t)t * H + h] = y[(size_t)t * H + h] * r;
    }
}

/* number of OpenMP threads the oracle's parallel loops use */
int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

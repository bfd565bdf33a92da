// route.hip -- router logits, top-K with renormalised gates, batch-union
// permute.
//
// Route step: page "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
// section 十一 (the router selects the top-k experts per token); gates are the
// normalised values applied by the layer (page "colibrì 路由遥测全解析",
// section 分离计数与追踪); NaN guard (same page, section 测试与 CI 保障).
// Batch union: page "Colibrì 深度解析", section 四.
//
// Kernels
//   router_logits_kernel  GEMV-shaped logits for small T (decode): one block
//                         per (RW expert rows, TT tokens), its waves split H,
//                         16-byte loads of the router rows, fp32 FMA.
//   router_mfma_lds       logits for large T (prefill), H % 64 == 0: bf16 x bf16 ->
//                         fp32 on v_mfma_f32_16x16x32_bf16, 128 x 64 tiles staged
//                         through LDS, K split over grid.z with a fixed-order
//                         partial sum (router_sum_parts).
//   router_mfma_kernel    the same for H % 32 == 0, operands loaded straight from
//                         global memory (both operands are K-contiguous).
//   topk_kernel           one wave per token: K rounds of wave argmax.
//   topk_permute_small    one block: top-K for all tokens, then the permute
//                         (decode: one launch for the whole route stage).
//   permute_count/scan/place  the permute for large T in three launches:
//                         per-chunk (256 pairs) expert bitmaps, a scan over
//                         chunks, then stable placement by bitmap popcounts.
//   router_logits_any     logits for any H and any row alignment (scalar
//                         loads), the fallback of the vector kernels.
//   router_topk_fused     logits of one token kept in LDS, then its top-K:
//                         the router when the caller wants no logits array.
#include <hip/hip_ext.h>

#include "kernels.h"
#include "stage_rows.h"
#include "wave.h"

namespace coli {
namespace {

constexpr int kWave = 64;

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// Load 8 consecutive elements (fp32 or bf16) as floats.
template <bool kBf16>
__device__ inline void load8(const void *base, size_t i, float out[8]) {
  if (kBf16) {
    const uint4 v = *reinterpret_cast<const uint4 *>(
        reinterpret_cast<const uint16_t *>(base) + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[2 * k] = __uint_as_float(w[k] << 16);
      out[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(
        reinterpret_cast<const float *>(base) + i);
    const float4 b = *reinterpret_cast<const float4 *>(
        reinterpret_cast<const float *>(base) + i + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

// 8 consecutive router-row elements as loaded (bf16: one 16-byte word; fp32:
// two), widened to fp32 only where used.
template <bool kBf16>
struct Raw8 {
  uint4 v[kBf16 ? 1 : 2];
};
__device__ inline uint32_t u4_word(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
template <bool kBf16>
__device__ inline Raw8<kBf16> load_raw8(const void *base, size_t i) {
  Raw8<kBf16> r;
  if (kBf16) {
    r.v[0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + i);
  } else {
    const float *f = reinterpret_cast<const float *>(base) + i;
    r.v[0] = *reinterpret_cast<const uint4 *>(f);
    r.v[kBf16 ? 0 : 1] = *reinterpret_cast<const uint4 *>(f + 4);
  }
  return r;
}
template <bool kBf16>
__device__ inline float raw8_at(const Raw8<kBf16> &r, int k) {
  if (kBf16) {
    const uint32_t w = u4_word(r.v[0], k >> 1);
    return __uint_as_float((k & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  return __uint_as_float(u4_word(r.v[(k >> 2) & (kBf16 ? 0 : 1)], k & 3));
}

// ---------------------------------------------------------------- logits (GEMV)
// grid.x: groups of RW expert rows; grid.y: groups of TT tokens.  The block's 4
// waves split H; a lane issues all loads of a batch of kB 8-column chunks
// (router rows kept as loaded, x as fp32) before using any, and the wave
// partials meet in LDS in a fixed order.  kB = 3 covers a quarter of H = 6144
// in one batch: one memory round trip.
//
// With xp set (fp32 x), the TT blocks past the expert groups of each grid row
// write the staged hi/lo rows of its tokens for the decode batch GEMM instead
// (stage_rows.h), in the same launch.
template <int RW, int TT, bool kXbf, bool kWbf>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void *__restrict__ x, int T, int H, const void *__restrict__ wr,
    int E, const float *__restrict__ bias, float *__restrict__ logits,
    uint16_t *__restrict__ xp, float *__restrict__ xs, int HP) {
  constexpr int kB = 3;
  __shared__ float part[4][RW][TT];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int e0 = blockIdx.x * RW;
  const int t0 = blockIdx.y * TT;
  if (!kXbf && e0 >= E) {
    const int t = t0 + (e0 - ((E + RW - 1) / RW) * RW) / RW;
    if (xp && t < T)
      stage_row(reinterpret_cast<const float *>(x) + size_t(t) * H, H, HP,
                xp + size_t(t) * HP, xp + (size_t(T) + t) * HP, xs + t, &part[0][0][0]);
    return;
  }
  const int Hq = ((H / 4 + 7) / 8) * 8;
  const int cb = wave * Hq, ce = min(H, cb + Hq);
  float acc[RW][TT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = 0.0f;
  for (int c0 = cb; c0 < ce; c0 += kB * kWave * 8) {
    // every load of the batch is issued before any is used: chunks past the
    // slice read its first columns (zeroed below, before their use), rows
    // past E and tokens past T re-read the last ones (never stored)
    Raw8<kWbf> wv[kB][RW];
    float xv[kB][TT][8];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int c = c0 + (b * kWave + lane) * 8;
      const int cl = c < ce ? c : cb;
#pragma unroll
      for (int r = 0; r < RW; ++r)
        wv[b][r] = load_raw8<kWbf>(wr, size_t(min(e0 + r, E - 1)) * H + cl);
#pragma unroll
      for (int t = 0; t < TT; ++t) load8<kXbf>(x, size_t(min(t0 + t, T - 1)) * H + cl, xv[b][t]);
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (c0 + (b * kWave + lane) * 8 >= ce) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
          for (int k = 0; k < (kWbf ? 1 : 2); ++k) wv[b][r].v[k] = uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int k = 0; k < 8; ++k) xv[b][t][k] = 0.0f;
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[r][t] = fmaf(raw8_at(wv[b][r], k), xv[b][t][k], acc[r][t]);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float v = wave_sum(acc[r][t]);
      if (lane == 0) part[wave][r][t] = v;
    }
  __syncthreads();
  if (int(threadIdx.x) < RW * TT) {
    const int r = threadIdx.x / TT, t = threadIdx.x % TT;
    if (e0 + r < E && t0 + t < T)
      logits[size_t(t0 + t) * E + e0 + r] =
          ((part[0][r][t] + part[1][r][t]) + (part[2][r][t] + part[3][r][t])) +
          (bias ? bias[e0 + r] : 0.0f);
  }
}

// ---------------------------------------------------------------- logits (one token)
// grid: E + H/64 blocks of 256 threads.  Block e < E computes the logits of
// expert e for every token (T <= 4): its 4 waves split H, a lane reads 8
// router columns per slot (kNB slots), fp32 FMA, partial sums meet in a fixed
// order.  Block E + g writes group g of x as digit planes (see ffn_narrow.hip),
// in parallel with the logit blocks: it finds the token's max |x| itself,
// token t by wave t (lanes 0..15, four elements each).  Every load of a round
// is issued before any is used (slots past the end read a valid address and
// are ignored at the use), so a round costs one memory round trip.
constexpr int kNB = 4;   // 8-column router slots per lane and round
constexpr int kXR = 8;   // float4 loads of x per thread and round (max scan)

template <bool kWbf>
__global__ __launch_bounds__(256) void router_narrow_kernel(
    const float *__restrict__ x, int T, int H, const void *__restrict__ wr, int E,
    const float *__restrict__ bias, float *__restrict__ logits, NarrowBufs nb) {
  __shared__ float sdot[4][4], smax[4][4];
  __shared__ int sbad[4][4];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (int(blockIdx.x) >= E) {
    // blocks E .. E + H/64 - 1: the x digit planes of group blockIdx.x - E, in
    // parallel with the logit blocks (each finds the token maxima itself)
    const int g = int(blockIdx.x) - E;
    const int el = 4 * lane, pos = aorder_pos(el);
    const bool writer = wave < T && lane < 16;
    float4 gv = {0.0f, 0.0f, 0.0f, 0.0f};
    if (writer) gv = *reinterpret_cast<const float4 *>(x + size_t(wave) * H + 64 * g + el);
    for (int t = 0; t < T; ++t) {
      float m = 0.0f;
      int bd = 0;
      for (int c0 = 4 * int(threadIdx.x); c0 < H; c0 += 4 * int(blockDim.x) * kXR) {
        float4 xv[kXR];
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
          const int c = c0 + 4 * int(blockDim.x) * j;
          xv[j] = *reinterpret_cast<const float4 *>(x + size_t(t) * H + (c < H ? c : 0));
        }
        // slots past the end re-read the row's first elements: the max and
        // the non-finite flag are unchanged by them
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
          m = fmaxf(fmaxf(m, fmaxf(fabsf(xv[j].x), fabsf(xv[j].y))),
                    fmaxf(fabsf(xv[j].z), fabsf(xv[j].w)));
          bd |= !__builtin_isfinite(xv[j].x) | !__builtin_isfinite(xv[j].y) |
                !__builtin_isfinite(xv[j].z) | !__builtin_isfinite(xv[j].w);
        }
      }
      m = wave_max(m);
      bd = __any(bd);
      if (lane == 0) {
        smax[wave][t] = m;
        sbad[wave][t] = bd;
      }
    }
    __syncthreads();
    if (writer) {
      const int t = wave;
      const float m = fmaxf(fmaxf(smax[0][t], smax[1][t]), fmaxf(smax[2][t], smax[3][t]));
      const bool bd = sbad[0][t] | sbad[1][t] | sbad[2][t] | sbad[3][t];
      const int ex = digit_exponent(m);
      if (g == 0 && lane == 0) nb.xsc[t] = bd ? __builtin_nanf("") : ldexpf(1.0f, -ex);
      const int GH = H / 64;
      const float va[4] = {gv.x, gv.y, gv.z, gv.w};
      int d[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) digits4(va[i], ex, d[i]);
      const size_t gbase = (size_t(t) * GH + g) * 4;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<uint32_t *>(nb.xdig + (gbase + p) * 64 + pos) = pack_plane(d, p);
        const int sum = row16_sum_i(d[0][p] + d[1][p] + d[2][p] + d[3][p]);
        if (lane == 0) nb.xcorr[gbase + p] = -8 * sum;
      }
    }
    return;
  }
  const int e = blockIdx.x;
  const int Hq = H / 4;
  const int cb = wave * Hq, ce = cb + Hq;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = cb + 8 * lane; c0 < ce; c0 += 8 * kWave * kNB) {
    Raw8<kWbf> wv[kNB];
    int cc[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int c = c0 + 8 * kWave * b;
      cc[b] = c < ce ? c : cb;
      wv[b] = load_raw8<kWbf>(wr, size_t(e) * H + cc[b]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= T) break;
      float4 xv[kNB][2];
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const float *xp = x + size_t(t) * H + cc[b];
        xv[b][0] = *reinterpret_cast<const float4 *>(xp);
        xv[b][1] = *reinterpret_cast<const float4 *>(xp + 4);
      }
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const float xa[8] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                             xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w};
        float a = acc[t];
#pragma unroll
        for (int k = 0; k < 8; ++k) a = fmaf(raw8_at(wv[b], k), xa[k], a);
        acc[t] = c0 + 8 * kWave * b < ce ? a : acc[t];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float d = wave_sum(acc[t]);
    if (lane == 0) sdot[wave][t] = d;
  }
  __syncthreads();
  if (int(threadIdx.x) < T) {
    const int t = threadIdx.x;
    logits[size_t(t) * E + e] =
        ((sdot[0][t] + sdot[1][t]) + (sdot[2][t] + sdot[3][t])) + (bias ? bias[e] : 0.0f);
  }
}

// ---------------------------------------------------------------- logits (MFMA)
typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Block: 4 waves, tile 64 tokens x 64 experts; wave w owns tokens
// 16*w..16*w+15 and all 64 experts (4 MFMA column fragments).  grid.z splits
// K: block z takes the 32-column k-steps z, z + S, z + 2S, .. (S = grid.z) and,
// for S > 1, writes its partial sums to part[z][t][e] (router_sum_parts adds
// them in a fixed order); for S == 1 it writes the logits.  Loads of four
// k-steps are issued before their MFMAs.
// v_mfma_f32_16x16x32_bf16 operand layout: lane l holds row (l % 16) and
// k = 8*(l / 16) .. +7 of its 16x32 operand; the result lane l holds rows
// 4*(l/16)+i, column l % 16.
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, int T, int H,
    const uint16_t *__restrict__ wr, int E, const float *__restrict__ bias,
    float *__restrict__ out) {
  constexpr int kU = 4;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.x * 64 + wave * 16;
  const int n0 = blockIdx.y * 64;
  const int S = gridDim.z, z = blockIdx.z;
  const int row = lane % 16, kq = (lane / 16) * 8;
  const int mrow = min(m0 + row, T - 1);  // clamp the ragged tail (not stored)
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t *xa = x + size_t(mrow) * H + kq;
  const uint16_t *wb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wb[j] = wr + size_t(min(n0 + 16 * j + row, E - 1)) * H + kq;
  const int nk = H / 32;  // k-steps
  for (int k0 = z; k0 < nk; k0 += kU * S) {
    bf16x8 a[kU], b[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int k = k0 + u * S;
      const int kc = k < nk ? 32 * k : 0;  // past the end: any valid column, not used
      a[u] = *reinterpret_cast<const bf16x8 *>(xa + kc);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[u][j] = *reinterpret_cast<const bf16x8 *>(wb[j] + kc);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + u * S < nk) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][j], acc[j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + (lane / 16) * 4 + i;
      if (m < T && n < E) {
        if (S > 1) out[(size_t(z) * T + m) * E + n] = acc[j][i];
        else out[size_t(m) * E + n] = acc[j][i] + (bias ? bias[n] : 0.0f);
      }
    }
  }
}

// The same logits through LDS (H % 64 == 0): a block computes a 128 x 64 tile
// (tokens x experts) over the k-stages z, z + S, ... of 64 columns.  Each stage
// is read from global memory once per block, as whole 128-byte row segments
// (16 bytes per thread and load), two stages ahead of its use, and written to
// an LDS buffer while the other buffer feeds the matrix cores; wave w takes tokens 32w .. 32w + 31 of
// the tile against all 64 experts (8 accumulator tiles of 16 x 16).  Rows are
// padded to 72 elements, so the 16 rows of an operand read land in distinct
// banks.  Output as router_mfma_kernel (partials when S > 1).
__global__ __launch_bounds__(256) void router_mfma_lds(
    const uint16_t *__restrict__ x, int T, int H,
    const uint16_t *__restrict__ wr, int E, const float *__restrict__ bias,
    float *__restrict__ out) {
  constexpr int BM = 128, BN = 64, BK = 64, LD = BK + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN * LD];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int S = gridDim.z, z = blockIdx.z;
  const int nks = H / BK;
  // loader: A stage = 128 rows x 8 pieces of 16 bytes (4 per thread), B stage
  // = 64 rows x 8 pieces (2 per thread); rows past T or E re-read the last one.
  // Two register sets: the stages one and two ahead are in flight together.
  // one 16-byte piece of a stage: A pieces q < 4 (128 rows x 8), B pieces q >= 4
  // (64 rows x 8); rows past T or E re-read the last one
  auto piece_src = [&](int ks, int q) __attribute__((always_inline)) {
    const int id = tid + 256 * (q & 3), r = id >> 3, c = id & 7;
    return q < 4 ? x + size_t(min(m0 + r, T - 1)) * H + ks * BK + 8 * c
                 : wr + size_t(min(n0 + r, E - 1)) * H + ks * BK + 8 * c;
  };
  auto piece_dst = [&](int buf, int q) __attribute__((always_inline)) {
    const int id = tid + 256 * (q & 3), r = id >> 3, c = id & 7;
    return q < 4 ? &sa[buf][r * LD + 8 * c] : &sb[buf][r * LD + 8 * c];
  };
#define COLI_RMLDS_LOAD(ks, P)                                                 \
  {                                                                            \
    const int ks_ = (ks);                                                      \
    P##0 = *reinterpret_cast<const uint4 *>(piece_src(ks_, 0));                \
    P##1 = *reinterpret_cast<const uint4 *>(piece_src(ks_, 1));                \
    P##2 = *reinterpret_cast<const uint4 *>(piece_src(ks_, 2));                \
    P##3 = *reinterpret_cast<const uint4 *>(piece_src(ks_, 3));                \
    P##4 = *reinterpret_cast<const uint4 *>(piece_src(ks_, 4));                \
    P##5 = *reinterpret_cast<const uint4 *>(piece_src(ks_, 5));                \
  }
#define COLI_RMLDS_STORE(P, buf)                                               \
  {                                                                            \
    *reinterpret_cast<uint4 *>(piece_dst(buf, 0)) = P##0;                      \
    *reinterpret_cast<uint4 *>(piece_dst(buf, 1)) = P##1;                      \
    *reinterpret_cast<uint4 *>(piece_dst(buf, 2)) = P##2;                      \
    *reinterpret_cast<uint4 *>(piece_dst(buf, 3)) = P##3;                      \
    *reinterpret_cast<uint4 *>(piece_dst(buf, 4)) = P##4;                      \
    *reinterpret_cast<uint4 *>(piece_dst(buf, 5)) = P##5;                      \
  }
  f32x4 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int row = lane % 16, kq = (lane / 16) * 8;
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *reinterpret_cast<const bf16x8 *>(&sa[buf][(32 * wave + 16 * mi + row) * LD + 32 * kk + kq]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        b[ni] = *reinterpret_cast<const bf16x8 *>(&sb[buf][(16 * ni + row) * LD + 32 * kk + kq]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  };
  // stage ks is in LDS buffer (its index along the block's stages) & 1; the
  // register sets alternate the same way, two stages ahead
  uint4 u0, u1, u2, u3, u4, u5, v0, v1, v2, v3, v4, v5;  // register sets u, v
  // the block's stages z + j S, j < nmy (nmy >= 1: z < S <= nks); loads past
  // the last stage re-read it (valid addresses, never stored)
  const int nmy = (nks - z + S - 1) / S;
  auto stg = [&](int j) { return min(z + j * S, nks - 1); };
  COLI_RMLDS_LOAD(stg(0), u)
  COLI_RMLDS_LOAD(stg(1), v)
  COLI_RMLDS_STORE(u, 0)
  __syncthreads();
  for (int j = 0; j < nmy; j += 2) {
    // stage j in buffer 0, set v holds stage j + 1, set u takes stage j + 2
    COLI_RMLDS_LOAD(stg(j + 2), u)
    compute(0);
    if (j + 1 < nmy) COLI_RMLDS_STORE(v, 1)
    __syncthreads();
    if (j + 1 < nmy) {  // block-uniform
      COLI_RMLDS_LOAD(stg(j + 3), v)
      compute(1);
      if (j + 2 < nmy) COLI_RMLDS_STORE(u, 0)
      __syncthreads();
    }
  }
#undef COLI_RMLDS_LOAD
#undef COLI_RMLDS_STORE
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = n0 + 16 * ni + row;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * wave + 16 * mi + (lane / 16) * 4 + i;
        if (m < T && n < E) {
          if (S > 1) out[(size_t(z) * T + m) * E + n] = acc[mi][ni][i];
          else out[size_t(m) * E + n] = acc[mi][ni][i] + (bias ? bias[n] : 0.0f);
        }
      }
    }
}

// logits[t][e] = sum over z (in order) of part[z][t][e], plus bias[e]
__global__ __launch_bounds__(256) void router_sum_parts(const float *__restrict__ part, int S,
                                                        int T, int E,
                                                        const float *__restrict__ bias,
                                                        float *__restrict__ logits) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(T) * E) return;
  float v = part[i];
  for (int z = 1; z < S; ++z) v += part[int64_t(z) * T * E + i];
  logits[i] = v + (bias ? bias[i % E] : 0.0f);
}

// ---------------------------------------------------------------- logits (any H)
__device__ inline float load_any(const void *base, int bf16, size_t i) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(base)[i])
              : reinterpret_cast<const float *>(base)[i];
}

// grid (ceil(E / 4), T): wave w of block b computes the logit of expert 4b + w
// for token blockIdx.y (lanes stride H, element loads, fixed-order wave sum).
__global__ __launch_bounds__(256) void router_logits_any(const void *__restrict__ x, int x_bf16,
                                                         int T, int H, const void *__restrict__ wr,
                                                         int w_bf16, int E,
                                                         const float *__restrict__ bias,
                                                         float *__restrict__ logits) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int e = int(blockIdx.x) * 4 + wave, t = blockIdx.y;
  if (e >= E) return;
  float acc = 0.0f;
  for (int h = lane; h < H; h += kWave)
    acc = fmaf(load_any(wr, w_bf16, size_t(e) * H + h), load_any(x, x_bf16, size_t(t) * H + h),
               acc);
  acc = wave_sum(acc);
  if (lane == 0) logits[size_t(t) * E + e] = acc + (bias ? bias[e] : 0.0f);
}

// One block per token: the E logits (any H) go to LDS, then wave 0 selects the
// top-K from there; no logits array in memory.  logit_bias is added to the
// logits (softmax scoring); sc.bias is the sigmoid scoring's selection bias.
__global__ __launch_bounds__(256) void router_topk_fused(const void *__restrict__ x, int x_bf16,
                                                         int H, const void *__restrict__ wr,
                                                         int w_bf16, int E, int K,
                                                         const float *__restrict__ logit_bias,
                                                         Scoring sc, int32_t *__restrict__ idx,
                                                         float *__restrict__ gates) {
  __shared__ float lg[COLI_MAX_EXPERTS];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int t = blockIdx.x;
  for (int e = wave; e < E; e += 4) {
    float acc = 0.0f;
    for (int h = lane; h < H; h += kWave)
      acc = fmaf(load_any(wr, w_bf16, size_t(e) * H + h), load_any(x, x_bf16, size_t(t) * H + h),
                 acc);
    acc = wave_sum(acc);
    if (lane == 0) lg[e] = acc + (logit_bias ? logit_bias[e] : 0.0f);
  }
  __syncthreads();
  if (wave == 0) wave_topk(lg, E, K, lane, idx + size_t(t) * K, gates + size_t(t) * K, sc);
}

// grid: ceil(T/4) blocks of 4 waves; one wave per token.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   int T, int E, int K,
                                                   int32_t *__restrict__ idx,
                                                   float *__restrict__ gates, Scoring sc) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  wave_topk(logits + size_t(t) * E, E, K, lane, idx + size_t(t) * K, gates + size_t(t) * K, sc);
}

// ---------------------------------------------------------------- permute
// The permute walks the T*K (token, slot) pairs p = t*K + slot in chunks of 256
// pairs: per chunk, bm[e] is a 256-bit set (four 64-bit words) with bit
// (p - p0) set if pair p chose expert e, and a pair's rank inside its
// expert's segment is the expert's base plus the pairs of the chunk before it
// (popcounts).  Counting pairs, not tokens, keeps the placement stable and
// complete when a row names the same expert twice.
constexpr int kChunkW = 4;             // 64-bit words per expert and chunk
constexpr int kChunk = 64 * kChunkW;   // pairs per bitmap chunk

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024).
__device__ int block_exclusive_scan(int v, int *wave_tot, int *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = wave_tot[w];
      wave_tot[w] = run;
      run += c;
    }
    *total = run;
  }
  __syncthreads();
  const int res = wave_tot[wave] + inc - v;
  __syncthreads();
  return res;
}

typedef unsigned long long ChunkBits[kChunkW];

// Bitmaps of the pair chunk starting at p0: bm[e] bit (p - p0) set if pair p
// (p < P = T*K) chose e.
__device__ void build_bitmap(const int32_t *__restrict__ idx, int P, int E, int p0,
                             ChunkBits *bm) {
  for (int i = threadIdx.x; i < E * kChunkW; i += blockDim.x) bm[i / kChunkW][i % kChunkW] = 0ull;
  __syncthreads();
  const int pend = min(P, p0 + kChunk);
  for (int p = p0 + int(threadIdx.x); p < pend; p += blockDim.x) {
    const int e = idx[p];
    const int l = p - p0;
    if (e >= 0 && e < E) atomicOr(&bm[e][l >> 6], 1ull << (l & 63));
  }
  __syncthreads();
}

// pairs of the chunk before local position l that chose e
__device__ inline int rank_in_chunk(const ChunkBits &b, int l) {
  int r = 0;
#pragma unroll
  for (int w = 0; w < kChunkW; ++w) {
    if (w < (l >> 6)) r += __popcll(b[w]);
    else if (w == (l >> 6)) r += __popcll(b[w] & ((1ull << (l & 63)) - 1ull));
  }
  return r;
}
__device__ inline int chunk_count(const ChunkBits &b) {
  int r = 0;
#pragma unroll
  for (int w = 0; w < kChunkW; ++w) r += __popcll(b[w]);
  return r;
}

// base: the rank of the chunk's first pair of each expert (LDS or global);
// extra: added to it (the expert's offset when base holds chunk-relative values)
__device__ void place_chunk(const int32_t *__restrict__ idx, int P, int E, int p0,
                            const ChunkBits *bm, const int *base, const int32_t *extra,
                            int32_t *__restrict__ perm) {
  const int pend = min(P, p0 + kChunk);
  for (int p = p0 + int(threadIdx.x); p < pend; p += blockDim.x) {
    const int e = idx[p];
    if (e < 0 || e >= E) continue;  // ids outside [0, E) are skipped
    perm[base[e] + (extra ? extra[e] : 0) + rank_in_chunk(bm[e], p - p0)] = p;
  }
}

// Counts, offsets, unique list from per-expert totals held one per thread.
__device__ void finish_counts(const Routing &r, int T, int K, int E, int cnt_e,
                              int *wave_tot, int *total, int *excl_out, int *uidx = nullptr) {
  const int e = threadIdx.x;
  const int v = e < E ? cnt_e : 0;
  const int excl = block_exclusive_scan(v, wave_tot, total);
  if (e < E) {
    r.counts[e] = v;
    r.offsets[e] = excl;
    if (r.usage && v > 0) atomicAdd(r.usage + e, (unsigned long long)v);  // the history
  }
  if (e == 0) r.offsets[E] = *total;
  const int flag = (e < E && v > 0) ? 1 : 0;
  const int pos = block_exclusive_scan(flag, wave_tot, total);
  if (flag) r.unique[pos] = e;
  if (uidx && e < E) uidx[e] = flag ? pos : -1;
  if (e == 0) *r.n_unique = *total;
  if (excl_out) *excl_out = excl;
}

// One block of 1024 threads: optional top-K, then the whole permute.
__global__ __launch_bounds__(1024) void topk_permute_small(Routing r, int T, int E, int K,
                                                           int do_topk) {
  __shared__ ChunkBits bm[COLI_MAX_EXPERTS];
  __shared__ int cursor[COLI_MAX_EXPERTS];
  __shared__ int cnt[COLI_MAX_EXPERTS];
  __shared__ int wave_tot[16];
  __shared__ int total;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (do_topk)
    for (int t = wave; t < T; t += blockDim.x / kWave)
      wave_topk(r.logits + size_t(t) * E, E, K, lane, r.idx + size_t(t) * K,
                r.gates + size_t(t) * K, r.sc);
  __threadfence_block();
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int P = T * K;
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = r.idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  int excl = 0;
  finish_counts(r, T, K, E, threadIdx.x < E ? cnt[threadIdx.x] : 0, wave_tot, &total, &excl);
  if (threadIdx.x < E) cursor[threadIdx.x] = excl;
  __syncthreads();
  for (int p0 = 0; p0 < P; p0 += kChunk) {
    build_bitmap(r.idx, P, E, p0, bm);
    place_chunk(r.idx, P, E, p0, bm, cursor, nullptr, r.perm);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) cursor[e] += chunk_count(bm[e]);
    __syncthreads();
  }
}

// Decode: one block of 1024 threads does top-K, the permute and the per-unit
// M-chunk prefix.
constexpr int kDecMC = 32;  // tokens per M-chunk of the decode expert kernels

__global__ __launch_bounds__(1024) void route_decode_kernel(Routing r, int T, int E, int K) {
  __shared__ ChunkBits bm[COLI_MAX_EXPERTS];
  __shared__ int cursor[COLI_MAX_EXPERTS];
  __shared__ int cnt[COLI_MAX_EXPERTS];
  __shared__ int uidx[COLI_MAX_EXPERTS];
  __shared__ int wave_tot[16];
  __shared__ int total;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int t = wave; t < T; t += blockDim.x / kWave)
    wave_topk(r.logits + size_t(t) * E, E, K, lane, r.idx + size_t(t) * K,
              r.gates + size_t(t) * K, r.sc);
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int P = T * K;
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = r.idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int ce = threadIdx.x < E ? cnt[threadIdx.x] : 0;
  int excl = 0;
  finish_counts(r, T, K, E, ce, wave_tot, &total, &excl, uidx);
  const int nr = total;
  if (threadIdx.x < E) cursor[threadIdx.x] = excl;
  // M-chunk prefix over units in unique order (ascending expert id)
  const int nch = (threadIdx.x < E && ce > 0) ? (ce + kDecMC - 1) / kDecMC : 0;
  const int cpos = block_exclusive_scan(nch, wave_tot, &total);
  if (threadIdx.x < E && ce > 0) r.chunk[uidx[threadIdx.x]] = cpos;
  if (threadIdx.x == 0) {
    r.chunk[nr] = total;
    r.chunk[nr + 1] = total + (T + kDecMC - 1) / kDecMC;
  }
  __syncthreads();
  for (int p0 = 0; p0 < P; p0 += kChunk) {
    build_bitmap(r.idx, P, E, p0, bm);
    place_chunk(r.idx, P, E, p0, bm, cursor, nullptr, r.perm);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) cursor[e] += chunk_count(bm[e]);
    __syncthreads();
  }
}

// Decode with T <= 64 and T * K <= kSmallPairs: one block, one bitmap chunk.
// The top-K writes the ids to LDS; per-expert token bitmaps give the counts and
// the stable placement (rank = offset + tokens before t with that expert)
// directly, with no read-back of global memory.  The ids of a token come from
// its own top-K, so they are distinct and a token bitmap counts its pairs.
constexpr int kSmallPairs = 2048;

__global__ __launch_bounds__(1024) void route_decode_small(Routing r, int T, int E, int K) {
  __shared__ int32_t sidx[kSmallPairs];
  __shared__ unsigned long long bm[COLI_MAX_EXPERTS];
  __shared__ int cursor[COLI_MAX_EXPERTS];
  __shared__ int uidx[COLI_MAX_EXPERTS];
  __shared__ int wave_tot[16];
  __shared__ int total;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int e = threadIdx.x; e < E; e += blockDim.x) bm[e] = 0ull;
  const int nwv = int(blockDim.x) / kWave;
  if (E > 128 && E <= 256 && T <= 4 * nwv) {
    // the logits of all of the wave's tokens (at most 4) are loaded before the
    // first selection, so the tokens share one load round trip (rows past T
    // re-read row T - 1 and are not selected)
    float lg[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wave + nwv * j;
      topk_load<4>(r.logits + size_t(t < T ? t : T - 1) * E, E, lane, lg[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wave + nwv * j;
      if (t < T)
        topk_select<4>(lg[j], E, K, lane, sidx + t * K, r.gates + size_t(t) * K, r.sc);
    }
  } else {
    for (int t = wave; t < T; t += nwv)
      wave_topk(r.logits + size_t(t) * E, E, K, lane, sidx + t * K, r.gates + size_t(t) * K,
                r.sc);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < T * K; p += blockDim.x) {
    const int e = sidx[p];
    r.idx[p] = e;
    if (e >= 0 && e < E) atomicOr(&bm[e], 1ull << (p / K));
  }
  __syncthreads();
  const int ce = threadIdx.x < E ? __popcll(bm[threadIdx.x]) : 0;
  int excl = 0;
  finish_counts(r, T, K, E, ce, wave_tot, &total, &excl, uidx);
  const int nr = total;
  if (threadIdx.x < E) cursor[threadIdx.x] = excl;
  // M-chunk prefix over units in unique order (ascending expert id)
  const int nch = (threadIdx.x < E && ce > 0) ? (ce + kDecMC - 1) / kDecMC : 0;
  const int cpos = block_exclusive_scan(nch, wave_tot, &total);
  if (threadIdx.x < E && ce > 0) r.chunk[uidx[threadIdx.x]] = cpos;
  if (threadIdx.x == 0) {
    r.chunk[nr] = total;
    r.chunk[nr + 1] = total + (T + kDecMC - 1) / kDecMC;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < T * K; p += blockDim.x) {
    const int e = sidx[p], t = p / K;
    if (e < 0 || e >= E) continue;
    r.perm[cursor[e] + __popcll(bm[e] & ((1ull << t) - 1ull))] = p;
  }
}

// Large T: per-chunk counts -> r.chunk[c*E + e] (chunk c = pairs 256c .. +255).
__global__ __launch_bounds__(256) void permute_count(Routing r, int T, int K, int E) {
  __shared__ ChunkBits bm[COLI_MAX_EXPERTS];
  build_bitmap(r.idx, T * K, E, int(blockIdx.x) * kChunk, bm);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    r.chunk[size_t(blockIdx.x) * E + e] = chunk_count(bm[e]);
}

// One block of 1024: totals per expert, offsets, unique; chunk counts become
// bases relative to the expert's offset (permute_place adds the offset).  The
// chunk column of an expert is read 16 entries at a time (the loads are
// independent; only the running sum is serial).
__global__ __launch_bounds__(1024) void permute_scan(Routing r, int T, int K, int E, int nc) {
  __shared__ int wave_tot[16];
  __shared__ int total;
  constexpr int kB = 16;
  const int e = threadIdx.x;
  int run = 0;
  if (e < E)
    for (int c0 = 0; c0 < nc; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) v[j] = c0 + j < nc ? r.chunk[size_t(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (c0 + j < nc) r.chunk[size_t(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
  int excl = 0;
  finish_counts(r, T, K, E, run, wave_tot, &total, &excl);
}

__global__ __launch_bounds__(256) void permute_place(Routing r, int T, int K, int E) {
  __shared__ ChunkBits bm[COLI_MAX_EXPERTS];
  __shared__ int base[COLI_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += blockDim.x) base[e] = r.chunk[size_t(blockIdx.x) * E + e];
  const int p0 = int(blockIdx.x) * kChunk;
  build_bitmap(r.idx, T * K, E, p0, bm);  // contains the barrier for base[]
  place_chunk(r.idx, T * K, E, p0, bm, base, r.offsets, r.perm);
}

// One block does the whole permute up to this many pairs.
constexpr int kSmallP = 2048;

__global__ __launch_bounds__(256) void copy_union(Routing r, int E, int32_t *__restrict__ unique,
                                                  int32_t *__restrict__ n_unique) {
  const int n = *r.n_unique;
  if (n_unique && threadIdx.x == 0) *n_unique = n;
  if (unique)
    for (int i = threadIdx.x; i < E; i += blockDim.x) unique[i] = i < n ? r.unique[i] : -1;
}

}  // namespace

hipError_t launch_copy_union(const Routing &r, int E, int32_t *unique, int32_t *n_unique,
                             hipStream_t s) {
  copy_union<<<1, 256, 0, s>>>(r, E, unique, n_unique);
  return hipGetLastError();
}

size_t permute_chunk_ints(int T, int K, int E) {
  const int64_t P = int64_t(T) * K;
  return P > kSmallP ? size_t((P + kChunk - 1) / kChunk) * size_t(E) : 0;
}

hipError_t launch_router_logits(const void *x, int x_bf16, int T, int H,
                                const void *wr, int w_bf16, int E,
                                const float *bias, float *logits,
                                hipStream_t s, uint16_t *xp, float *xs, int HP) {
  if (x_bf16) xp = nullptr;  // the staged rows are made from fp32 x only
#define COLI_ROUTER_CASE(RW, TT)                                                  \
  {                                                                               \
    dim3 grid((E + RW - 1) / RW + (xp ? TT : 0), (T + TT - 1) / TT);             \
    if (x_bf16 && w_bf16)                                                         \
      router_logits_kernel<RW, TT, true, true><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits, xp, xs, HP);  \
    else if (x_bf16)                                                              \
      router_logits_kernel<RW, TT, true, false><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits, xp, xs, HP); \
    else if (w_bf16)                                                              \
      router_logits_kernel<RW, TT, false, true><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits, xp, xs, HP); \
    else                                                                          \
      router_logits_kernel<RW, TT, false, false><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits, xp, xs, HP);\
  }
  if (T <= 2) COLI_ROUTER_CASE(4, 2)
  else COLI_ROUTER_CASE(4, 4)
#undef COLI_ROUTER_CASE
  return hipGetLastError();
}

hipError_t launch_router_narrow(const float *x, int T, int H, const void *wr, int w_bf16,
                                int E, const float *bias, float *logits,
                                const NarrowBufs &nb, hipStream_t s, hipEvent_t start,
                                hipEvent_t stop) {
  if (w_bf16)
    hipExtLaunchKernelGGL(router_narrow_kernel<true>, dim3(E + H / 64), dim3(256), 0, s, start, stop, 0, x,
                          T, H, wr, E, bias, logits, nb);
  else
    hipExtLaunchKernelGGL(router_narrow_kernel<false>, dim3(E + H / 64), dim3(256), 0, s, start, stop, 0,
                          x, T, H, wr, E, bias, logits, nb);
  return hipGetLastError();
}

hipError_t launch_router_mfma(const uint16_t *x, int T, int H, const uint16_t *wr, int E,
                              const float *bias, float *logits, float *part, size_t part_bytes,
                              hipStream_t s) {
  if (H % 64 == 0) {
    // tiles of 128 tokens x 64 experts through LDS; K split into S parts so that
    // the grid covers the GPU about twice, as far as the partial-sum scratch
    // allows
    const int64_t tiles = int64_t((T + 127) / 128) * ((E + 63) / 64);
    int S = int(tiles >= 512 ? 1 : (512 + tiles - 1) / tiles);
    if (S > 8) S = 8;
    if (S > H / 64) S = H / 64;
    while (S > 1 && size_t(S) * T * E * 4 > part_bytes) --S;
    dim3 grid((T + 127) / 128, (E + 63) / 64, S);
    router_mfma_lds<<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, S > 1 ? part : logits);
    if (S > 1) {
      const int64_t n = int64_t(T) * E;
      router_sum_parts<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(part, S, T, E, bias, logits);
    }
    return hipGetLastError();
  }
  // K split: enough blocks to cover the GPU several times, as far as the
  // partial-sum scratch allows
  const int64_t tiles = int64_t((T + 63) / 64) * ((E + 63) / 64);
  int S = int(tiles >= 1024 ? 1 : (1024 + tiles - 1) / tiles);
  if (S > 8) S = 8;
  if (S > H / 32) S = H / 32;
  while (S > 1 && size_t(S) * T * E * 4 > part_bytes) --S;
  dim3 grid((T + 63) / 64, (E + 63) / 64, S);
  router_mfma_kernel<<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, S > 1 ? part : logits);
  if (S > 1) {
    const int64_t n = int64_t(T) * E;
    router_sum_parts<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(part, S, T, E, bias, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_any(const void *x, int x_bf16, int T, int H, const void *wr,
                             int w_bf16, int E, const float *bias, float *logits,
                             hipStream_t s) {
  router_logits_any<<<dim3((E + 3) / 4, T), 256, 0, s>>>(x, x_bf16, T, H, wr, w_bf16, E, bias,
                                                         logits);
  return hipGetLastError();
}

hipError_t launch_router_topk_fused(const void *x, int x_bf16, int T, int H, const void *wr,
                                    int w_bf16, int E, int K, const float *logit_bias,
                                    Scoring sc, int32_t *idx, float *gates, hipStream_t s) {
  router_topk_fused<<<dim3(T), 256, 0, s>>>(x, x_bf16, H, wr, w_bf16, E, K, logit_bias, sc, idx,
                                            gates);
  return hipGetLastError();
}

bool router_vec_ok(const void *x, int x_bf16, int H, const void *wr, int w_bf16) {
  // 16-byte loads of both operands at every row start
  const int xr = H * (x_bf16 ? 2 : 4), wrb = H * (w_bf16 ? 2 : 4);
  return H % 8 == 0 && xr % 16 == 0 && wrb % 16 == 0 &&
         (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (reinterpret_cast<uintptr_t>(wr) & 15) == 0;
}

hipError_t launch_route_decode(const Routing &r, int T, int E, int K, hipStream_t s) {
  if (T <= 64 && T * K <= kSmallPairs)
    route_decode_small<<<1, 1024, 0, s>>>(r, T, E, K);
  else
    route_decode_kernel<<<1, 1024, 0, s>>>(r, T, E, K);
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int E, int K, int32_t *idx,
                       float *gates, Scoring sc, hipStream_t s) {
  topk_kernel<<<dim3((T + 3) / 4), 256, 0, s>>>(logits, T, E, K, idx, gates, sc);
  return hipGetLastError();
}

hipError_t launch_topk_permute(const Routing &r, int T, int E, int K,
                               int do_topk, hipStream_t s) {
  if (int64_t(T) * K <= kSmallP) {
    topk_permute_small<<<1, 1024, 0, s>>>(r, T, E, K, do_topk);
    return hipGetLastError();
  }
  if (do_topk)
    topk_kernel<<<dim3((T + 3) / 4), 256, 0, s>>>(r.logits, T, E, K, r.idx, r.gates, r.sc);
  const int nc = int((int64_t(T) * K + kChunk - 1) / kChunk);
  permute_count<<<nc, 256, 0, s>>>(r, T, K, E);
  permute_scan<<<1, 1024, 0, s>>>(r, T, K, E, nc);
  permute_place<<<nc, 256, 0, s>>>(r, T, K, E);
  return hipGetLastError();
}

}  // namespace coli

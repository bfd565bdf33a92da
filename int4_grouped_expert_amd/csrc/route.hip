// route.hip -- router logits, top-K with renormalised gates, batch-union
// permute.
//
// Route step: page "Colibri 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
// section 十一 (the router selects the top-k experts per token); gates are the
// normalised values applied by the layer (page "colibri 路由遥测全解析",
// section 分离计数与追踪); NaN guard (same page, section 测试与 CI 保障).
// Batch union: page "Colibri 深度解析", section 四.
//
// Kernels
//   router_logits_kernel  GEMV-shaped logits for small T (decode): one wave
//                         per (RW expert rows, TT tokens), 16-byte loads of
//                         the router rows, fp32 FMA, butterfly reduction.
//   router_mfma_kernel    logits for large T (prefill): bf16 x bf16 -> fp32
//                         on v_mfma_f32_16x16x32_bf16, operands loaded straight
//                         from global memory (both operands are K-contiguous).
//   topk_kernel           one wave per token: K rounds of wave argmax.
//   topk_permute_small    one block: top-K for all tokens, then the permute
//                         (decode: one launch for the whole route stage).
//   permute_count/scan/place  the permute for large T in three launches:
//                         per-chunk (64 tokens) expert bitmaps, a scan over
//                         chunks, then stable placement by bitmap popcount.
#include "kernels.h"

namespace coli {
namespace {

constexpr int kWave = 64;

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
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

// ---------------------------------------------------------------- logits (GEMV)
// grid.x: groups of 4*RW expert rows; grid.y: groups of TT tokens.
template <int RW, int TT, bool kXbf, bool kWbf>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void *__restrict__ x, int T, int H, const void *__restrict__ wr,
    int E, const float *__restrict__ bias, float *__restrict__ logits) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int e0 = (blockIdx.x * 4 + wave) * RW;
  const int t0 = blockIdx.y * TT;
  if (e0 >= E) return;
  float acc[RW][TT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = 0.0f;

  for (int c = lane * 8; c < H; c += kWave * 8) {
    float wv[RW][8];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (e0 + r < E) load8<kWbf>(wr, size_t(e0 + r) * H + c, wv[r]);
      else
#pragma unroll
        for (int k = 0; k < 8; ++k) wv[r][k] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t0 + t >= T) break;
      float xv[8];
      load8<kXbf>(x, size_t(t0 + t) * H + c, xv);
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[r][t] = fmaf(wv[r][k], xv[k], acc[r][t]);
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float v = wave_sum(acc[r][t]);
      if (lane == 0 && e0 + r < E && t0 + t < T)
        logits[size_t(t0 + t) * E + e0 + r] = v + (bias ? bias[e0 + r] : 0.0f);
    }
}

// ---------------------------------------------------------------- logits (MFMA)
typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Block: 4 waves, tile 64 tokens x 64 experts; wave w owns tokens
// 16*w..16*w+15 and all 64 experts (4 MFMA column fragments).
// v_mfma_f32_16x16x32_bf16 operand layout: lane l holds row (l % 16) and
// k = 8*(l / 16) .. +7 of its 16x32 operand; the result lane l holds rows
// 4*(l/16)+i, column l % 16.
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, int T, int H,
    const uint16_t *__restrict__ wr, int E, const float *__restrict__ bias,
    float *__restrict__ logits) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.x * 64 + wave * 16;
  const int n0 = blockIdx.y * 64;
  const int row = lane % 16, kq = (lane / 16) * 8;
  const int mrow = min(m0 + row, T - 1);  // clamp the ragged tail (not stored)
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t *xa = x + size_t(mrow) * H + kq;
  const uint16_t *wb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wb[j] = wr + size_t(min(n0 + 16 * j + row, E - 1)) * H + kq;
  for (int k = 0; k < H; k += 32) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xa + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b = *reinterpret_cast<const bf16x8 *>(wb[j] + k);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + (lane / 16) * 4 + i;
      if (m < T && n < E) logits[size_t(m) * E + n] = acc[j][i] + (bias ? bias[n] : 0.0f);
    }
  }
}

// ---------------------------------------------------------------- top-K
constexpr int kMaxPerLane = COLI_MAX_PER_LANE;

// Wave-wide top-K of one token.  Writes idx/gates in ascending id order.
__device__ void wave_topk(const float *__restrict__ lrow, int E, int K, int lane,
                          int32_t *__restrict__ idx_out,
                          float *__restrict__ gate_out) {
  float v[kMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + kWave * j;
    v[j] = e < E ? lrow[e] : 0.0f;
  }
  for (int round = 0; round < K; ++round) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !((taken >> j) & 1u) && !__builtin_isnan(v[j]) &&
          (bi < 0 || v[j] > bv)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      const bool take = oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi));
      bv = take ? ov : bv;
      bi = take ? oi : bi;
    }
    if (bi < 0) {
      // No valid candidate: id `round` if free, else the lowest free id.
      int free_lo = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + kWave * j;
        if (e < E && !((taken >> j) & 1u)) { free_lo = min(free_lo, e); }
      }
      int own_free = 0;
      if (round < E && (round % kWave) == lane) own_free = !((taken >> (round / kWave)) & 1u);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        free_lo = min(free_lo, __shfl_xor(free_lo, m, kWave));
        own_free |= __shfl_xor(own_free, m, kWave);
      }
      bi = own_free ? round : free_lo;
    }
    if ((bi % kWave) == lane) taken |= 1u << (bi / kWave);
  }
  // selected max and normaliser (butterfly: identical on every lane)
  float m = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j)
    if ((taken >> j) & 1u) m = fmaxf(m, v[j]);
  m = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j)
    if ((taken >> j) & 1u) z += expf(v[j] - m);
  z = wave_sum(z);
  int before = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const uint64_t bal = __ballot((taken >> j) & 1u);
    if ((taken >> j) & 1u) {
      const int rank = before + __popcll(bal & ((1ull << lane) - 1ull));
      idx_out[rank] = lane + kWave * j;
      gate_out[rank] = expf(v[j] - m) / z;
    }
    before += __popcll(bal);
  }
}

// grid: ceil(T/4) blocks of 4 waves; one wave per token.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   int T, int E, int K,
                                                   int32_t *__restrict__ idx,
                                                   float *__restrict__ gates) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  wave_topk(logits + size_t(t) * E, E, K, lane, idx + size_t(t) * K, gates + size_t(t) * K);
}

// ---------------------------------------------------------------- permute
constexpr int kChunk = 64;  // tokens per bitmap chunk (one bit per token)

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

// Bitmap of one 64-token chunk: bm[e] bit (t - t0) set if token t chose e.
__device__ void build_bitmap(const int32_t *__restrict__ idx, int T, int K, int E,
                             int t0, unsigned long long *bm) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) bm[e] = 0ull;
  __syncthreads();
  const int tend = min(T, t0 + kChunk);
  const int npairs = (tend - t0) * K;
  for (int q = threadIdx.x; q < npairs; q += blockDim.x) {
    const int p = t0 * K + q;
    const int t = p / K;
    const int e = idx[p];
    if (e >= 0 && e < E) atomicOr(&bm[e], 1ull << (t - t0));
  }
  __syncthreads();
}

__device__ void place_chunk(const int32_t *__restrict__ idx, int T, int K, int E, int t0,
                            const unsigned long long *bm, const int *base,
                            int32_t *__restrict__ perm) {
  const int tend = min(T, t0 + kChunk);
  const int npairs = (tend - t0) * K;
  for (int q = threadIdx.x; q < npairs; q += blockDim.x) {
    const int p = t0 * K + q;
    const int t = p / K;
    const int e = idx[p];
    if (e < 0 || e >= E) continue;  // ids outside [0, E) are skipped
    const int rank = base[e] + __popcll(bm[e] & ((1ull << (t - t0)) - 1ull));
    perm[rank] = p;
  }
}

// Counts, offsets, unique list from per-expert totals held one per thread.
__device__ void finish_counts(const Routing &r, int T, int K, int E, int cnt_e,
                              int *wave_tot, int *total, int *excl_out) {
  const int e = threadIdx.x;
  const int v = e < E ? cnt_e : 0;
  const int excl = block_exclusive_scan(v, wave_tot, total);
  if (e < E) {
    r.counts[e] = v;
    r.offsets[e] = excl;
  }
  if (e == 0) r.offsets[E] = *total;
  const int flag = (e < E && v > 0) ? 1 : 0;
  const int pos = block_exclusive_scan(flag, wave_tot, total);
  if (flag) r.unique[pos] = e;
  if (e == 0) *r.n_unique = *total;
  if (excl_out) *excl_out = excl;
}

// One block of 1024 threads: optional top-K, then the whole permute.
__global__ __launch_bounds__(1024) void topk_permute_small(Routing r, int T, int E, int K,
                                                           int do_topk) {
  __shared__ unsigned long long bm[COLI_MAX_EXPERTS];
  __shared__ int cursor[COLI_MAX_EXPERTS];
  __shared__ int cnt[COLI_MAX_EXPERTS];
  __shared__ int wave_tot[16];
  __shared__ int total;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (do_topk)
    for (int t = wave; t < T; t += blockDim.x / kWave)
      wave_topk(r.logits + size_t(t) * E, E, K, lane, r.idx + size_t(t) * K,
                r.gates + size_t(t) * K);
  __threadfence_block();
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < T * K; p += blockDim.x) {
    const int e = r.idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  int excl = 0;
  finish_counts(r, T, K, E, threadIdx.x < E ? cnt[threadIdx.x] : 0, wave_tot, &total, &excl);
  if (threadIdx.x < E) cursor[threadIdx.x] = excl;
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += kChunk) {
    build_bitmap(r.idx, T, K, E, t0, bm);
    place_chunk(r.idx, T, K, E, t0, bm, cursor, r.perm);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) cursor[e] += __popcll(bm[e]);
    __syncthreads();
  }
}

// Large T: per-chunk counts -> r.chunk[c*E + e].
__global__ __launch_bounds__(256) void permute_count(Routing r, int T, int K, int E) {
  __shared__ unsigned long long bm[COLI_MAX_EXPERTS];
  const int t0 = blockIdx.x * kChunk;
  build_bitmap(r.idx, T, K, E, t0, bm);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    r.chunk[size_t(blockIdx.x) * E + e] = __popcll(bm[e]);
}

// One block of 1024: totals per expert, offsets, unique; chunk counts become
// absolute bases.
__global__ __launch_bounds__(1024) void permute_scan(Routing r, int T, int K, int E, int nc) {
  __shared__ int wave_tot[16];
  __shared__ int total;
  const int e = threadIdx.x;
  int run = 0;
  if (e < E)
    for (int c = 0; c < nc; ++c) {
      const int v = r.chunk[size_t(c) * E + e];
      r.chunk[size_t(c) * E + e] = run;
      run += v;
    }
  int excl = 0;
  finish_counts(r, T, K, E, run, wave_tot, &total, &excl);
  if (e < E)
    for (int c = 0; c < nc; ++c) r.chunk[size_t(c) * E + e] += excl;
}

__global__ __launch_bounds__(256) void permute_place(Routing r, int T, int K, int E) {
  __shared__ unsigned long long bm[COLI_MAX_EXPERTS];
  __shared__ int base[COLI_MAX_EXPERTS];
  const int t0 = blockIdx.x * kChunk;
  for (int e = threadIdx.x; e < E; e += blockDim.x) base[e] = r.chunk[size_t(blockIdx.x) * E + e];
  build_bitmap(r.idx, T, K, E, t0, bm);  // contains the barrier for base[]
  place_chunk(r.idx, T, K, E, t0, bm, base, r.perm);
}

constexpr int kSmallT = 2 * kChunk;

}  // namespace

size_t permute_chunk_ints(int T, int E) {
  return T > kSmallT ? size_t((T + kChunk - 1) / kChunk) * size_t(E) : 0;
}

hipError_t launch_router_logits(const void *x, int x_bf16, int T, int H,
                                const void *wr, int w_bf16, int E,
                                const float *bias, float *logits,
                                hipStream_t s) {
#define COLI_ROUTER_CASE(RW, TT)                                                  \
  {                                                                               \
    dim3 grid((E + 4 * RW - 1) / (4 * RW), (T + TT - 1) / TT);                   \
    if (x_bf16 && w_bf16)                                                         \
      router_logits_kernel<RW, TT, true, true><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits);  \
    else if (x_bf16)                                                              \
      router_logits_kernel<RW, TT, true, false><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits); \
    else if (w_bf16)                                                              \
      router_logits_kernel<RW, TT, false, true><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits); \
    else                                                                          \
      router_logits_kernel<RW, TT, false, false><<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits);\
  }
  if (T <= 2) COLI_ROUTER_CASE(1, 2)
  else COLI_ROUTER_CASE(4, 4)
#undef COLI_ROUTER_CASE
  return hipGetLastError();
}

hipError_t launch_router_topk_mfma(const uint16_t *x, int T, int H,
                                   const uint16_t *wr, int E,
                                   const float *bias, int K, float *logits,
                                   int32_t *idx, float *gates, hipStream_t s) {
  dim3 grid((T + 63) / 64, (E + 63) / 64);
  router_mfma_kernel<<<grid, 256, 0, s>>>(x, T, H, wr, E, bias, logits);
  topk_kernel<<<dim3((T + 3) / 4), 256, 0, s>>>(logits, T, E, K, idx, gates);
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int E, int K, int32_t *idx,
                       float *gates, hipStream_t s) {
  topk_kernel<<<dim3((T + 3) / 4), 256, 0, s>>>(logits, T, E, K, idx, gates);
  return hipGetLastError();
}

hipError_t launch_topk_permute(const Routing &r, int T, int E, int K,
                               int do_topk, hipStream_t s) {
  if (T <= kSmallT) {
    topk_permute_small<<<1, 1024, 0, s>>>(r, T, E, K, do_topk);
    return hipGetLastError();
  }
  if (do_topk)
    topk_kernel<<<dim3((T + 3) / 4), 256, 0, s>>>(r.logits, T, E, K, r.idx, r.gates);
  const int nc = (T + kChunk - 1) / kChunk;
  permute_count<<<nc, 256, 0, s>>>(r, T, K, E);
  permute_scan<<<1, 1024, 0, s>>>(r, T, K, E, nc);
  permute_place<<<nc, 256, 0, s>>>(r, T, K, E);
  return hipGetLastError();
}

}  // namespace coli

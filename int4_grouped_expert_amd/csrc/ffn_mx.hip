// ffn_mx.hip -- the experts of a decode layer stored in MXFP4 or
// fp8-e4m3-b128, for one or two tokens, on the gfx950 scaled matrix cores.
//
// Method: the expert FFN of page "Colibrì 深度解析" (sections 四 and 十一):
// h = w_t * SiLU(x Wg^T) * (x Wu^T) per (unit, token), w_t the token's gate
// weight for the unit (0 when it did not pick it, 1 for the shared expert);
// the weights in the MXFP4 element format of section 十 (OCP Microscaling
// v1.0: blocks of 32 E2M1 codes with one E8M0 power-of-two scale) or as E4M3
// codes with one f32 scale per 128 x 128 tile (OCP FP8).
//
// Arithmetic.  v_mfma_scale_f32_16x16x128_f8f6f4 multiplies an E4M3 A operand
// by an E2M1 (or E4M3) B operand and applies one E8M0 scale per 32 k on each
// side, so MXFP4 weight blocks enter exactly as stored, codes and scales; E4M3
// codes enter with the neutral scale and each 128-k product is multiplied by
// its tile's f32 scale in fp32.  The
// activations enter as four E4M3 planes per 32-element block: with e the
// block's exponent (its largest |x| times 2^-e lies in [64, 128)),
// x 2^-e = p0 + p1 / 16 + p2 / 256 + p3 / 4096, each p the round-to-nearest-
// even E4M3 value of 16 times what the planes before it left (the first: of
// x 2^-e itself); plane j carries the A scale 2^(e - 4j).  Every plane value
// stays below 128 in magnitude (no E4M3 overflow), and what the four planes
// leave is below 2^-19 of the block's largest |x| (2^-29 for elements in the
// E4M3 subnormal range).  A block holding a NaN or an infinity becomes NaN
// codes, so its outputs are NaN; an E8M0 scale of 255 (a weight block that was
// not finite) makes the hardware product NaN, as the format defines.
//
// MFMA layout (gfx950, checked element by element against a host product):
// A lane l holds row l % 16 and, with q = l / 16, k = 16 q .. 16 q + 15 in
// bytes 0..15 and k = 64 + 16 q .. + 15 in bytes 16..31; B lane l holds
// column l % 16, k = 32 q .. 32 q + 31 as 32 nibbles (element 2j in the low
// nibble of byte j, the MXFP4 order); the scale of k-block b of row (column)
// i comes from lane 16 b + i; result lane l holds rows 4 q + i, column l % 16.
// Here B column n = r + 8 h is weight row r of an 8-row group reading bytes
// 64 h .. 64 h + 63 of a 128-byte run of the row (elements 128 h .. + 127 of a
// 256-element chunk): the 8 lanes of a row read the whole run, one 16-byte MX
// block each, and pass that block's own scale.  A row m = 8 h + 4 t + j is
// plane j of token t over elements 128 h .. of the chunk: result row m,
// column n is meaningful where h(m) = h(n), and the four planes of one
// (token, weight row, h) are the four values one result lane holds.
//
// Kernels
//   mx_gateup   block b takes row group b (8 rows of I) of every unit, the
//               shared expert first (its blob needs no routing, so its loads
//               leave first); the 8 waves split the 256-element chunks of H and
//               keep their planes of x in registers; a register ring of two
//               items; per-item partials meet in LDS and are reduced once, at
//               the end, into h = w_t SiLU(gate) up.
//   mx_down     one token: output-stationary over row groups of H, every
//               unit in turn (the gate weights are in h, so the combine is
//               the accumulation); h's planes in LDS; writes y and flags a
//               non-finite output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "coli.h"
#include "kernels.h"

namespace coli {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMxWaves = 8;
constexpr int kMxMaxCpw = 4;     // 256-element chunks per wave: H <= 8192
constexpr int kMxMaxItems = 40;  // units per call (routed + shared)

struct MxArgs {
  const uint8_t *experts, *shared;
  size_t blob_bytes;
  size_t q_off[2], s_off[2];  // gate and up sections of a blob
  const int32_t *unique, *n_unique, *idx;
  const float *gates;
  const float *x;  // [T][H]
  float *h;        // [units][T][I]
  int T, H, I, K;
};

__device__ inline void step_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// 2^k as a float, k in [-126, 127]
__device__ inline float pow2f(int k) { return __uint_as_float(uint32_t(k + 127) << 23); }

// Four E4M3 planes of 8 values v (already times 2^-e, |v| < 128): plane j's
// 8 codes in out[j] (two dwords, value i in byte i).
__device__ inline void e4m3_planes(float v[8], uint2 out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d], v[4 * d + 1], 0, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d + 2], v[4 * d + 3], c, true);
      w[d] = uint32_t(c);
      if (j < 3) {
        // exact: the residual of a rounding, times 16
        const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
        const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
        v[4 * d] = (v[4 * d] - b01[0]) * 16.0f;
        v[4 * d + 1] = (v[4 * d + 1] - b01[1]) * 16.0f;
        v[4 * d + 2] = (v[4 * d + 2] - b23[0]) * 16.0f;
        v[4 * d + 3] = (v[4 * d + 3] - b23[1]) * 16.0f;
      }
    }
    out[j] = make_uint2(w[0], w[1]);
  }
}

__device__ inline f32x4 mfma_mx(const i32x8 &a, const uint4 &b, const f32x4 &c, int sa, int sb) {
  const i32x8 bb = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
  // A E4M3 (format 0), B E2M1 (format 4)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, sa, 0, sb);
}

// fp8-e4m3-b128 weights: B E4M3 (format 0) with the neutral E8M0 scale; the
// tile's f32 scale is applied to the product afterwards
__device__ inline f32x4 mfma_f8(const i32x8 &a, const uint4 &b0, const uint4 &b1, int sa) {
  const i32x8 bb = {int(b0.x), int(b0.y), int(b0.z), int(b0.w),
                    int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, z, 0, 0, 0, sa, 0, 127);
}

// The weight side of a format, per 256-element chunk of a row: its bytes,
// the 16-byte loads of a lane (B column n = r + 8 h, quarter q; load i at
// byte 64 i further on) and where the first one starts.  MXFP4: one MX block
// (elements 128 h + 32 q ..); E4M3 (B holds k = 16 q .. and 64 + 16 q ..):
// elements 128 h + 16 q .. and 128 h + 64 + 16 q ...
template <int FMT>
struct Wt {
  static constexpr bool kMx = FMT == COLI_FMT_MXFP4;
  static constexpr int kChunkBytes = kMx ? 128 : 256;
  static constexpr int kLoads = kMx ? 1 : 2;
  __device__ static int off(int hh, int q) { return (kMx ? 64 : 128) * hh + 16 * q; }
};

// The exponent e of a 32-element block (its largest |x| times 2^-e in
// [64, 128), kept >= -115 so that the last plane's scale 2^(e - 12) is an
// E8M0 value) and the four E4M3 planes of this lane's 8 elements.  The block
// is held by 4 consecutive lanes (all active).  A block holding a NaN or an
// infinity gets e = 0 and NaN codes.
__device__ inline int block_planes(float v[8], uint2 pl[4]) {
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  mb = max(mb, uint32_t(__shfl_xor(int(mb), 1)));
  mb = max(mb, uint32_t(__shfl_xor(int(mb), 2)));
  if (mb >= 0x7F800000u) {
#pragma unroll
    for (int p = 0; p < 4; ++p) pl[p] = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    return 0;
  }
  const int ef = int(mb >> 23) < 1 ? 1 : int(mb >> 23);
  const int e = ef - 133 < -115 ? -115 : ef - 133;
  const float f = pow2f(-e);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= f;
  e4m3_planes(v, pl);
  return e;
}

// Fold of one item's result: the four planes, then the two halves of the
// chunks (result lanes 16 t + r and 16 t + r + 40 hold h = 0 and h = 1 of
// token t, weight row r).  Valid on lanes 0..7 and 16..23.
__device__ inline float fold_item(const f32x4 &acc, int lane) {
  float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  return v + __shfl(v, (lane + 40) & 63);
}

// E8M0 scales.  The scales of a row's 256-element chunks c0 .. c0 + nc - 1
// are 8 nc consecutive bytes; lane (n = r + 8 h, q) loads dword 2 q + h of
// them (dword 0 past the end), and the scale of chunk c for lane (r, h, q) --
// byte 4 h + q of chunk c, so byte q of dword 2 c + h -- comes from lane
// (n, c) of the same row.
__device__ inline uint32_t scale_dword(const uint8_t *slice, int nc, int hh, int q) {
  const int d = 2 * q + hh;
  return *reinterpret_cast<const uint32_t *>(slice + 4 * (d < 2 * nc ? d : 0));
}
__device__ inline int scale_of(uint32_t dw, int c, int lane, int q) {
  const uint32_t v = uint32_t(__shfl(int(dw), (lane & 15) + 16 * c));
  return int((v >> (8 * q)) & 0xFFu);
}

template <int FMT, int CPW>
struct GuSlot {
  uint4 wg[CPW][Wt<FMT>::kLoads], wu[CPW][Wt<FMT>::kLoads];
  uint32_t sdg, sdu;     // MXFP4: the row slice's scale dwords
  float sfg[CPW], sfu[CPW];  // fp8: the chunks' tile scales
};

// fp8 tile scale of chunk c0 + c, column half h, for rows of tile row rt:
// tiles [rows / 128][K / 128], two per chunk
__device__ inline float tile_scale(const uint8_t *sec, size_t rt, int ktiles, int c, int hh) {
  return reinterpret_cast<const float *>(sec)[rt * ktiles + 2 * c + hh];
}

template <int FMT, int CPW>
__global__ __launch_bounds__(64 * kMxWaves) void mx_gateup(MxArgs a) {
  using W = Wt<FMT>;
  // the prologue's planes of x and the loop's partials share the LDS
  constexpr int kPlaneBytes = kMxWaves * 2 * 4 * CPW * 256;
  constexpr int kRedBytes = kMxMaxItems * kMxWaves * 2 * 2 * 8 * 4;
  __shared__ __align__(16) uint8_t lds[kPlaneBytes > kRedBytes ? kPlaneBytes : kRedBytes];
  __shared__ int sexp[kMxWaves][2][CPW * 8];
  __shared__ const uint8_t *sblob[kMxMaxItems];
  uint8_t(*xpl)[2][4][CPW * 256] = reinterpret_cast<uint8_t(*)[2][4][CPW * 256]>(lds);
  float(*red)[kMxWaves][2][2][8] = reinterpret_cast<float(*)[kMxWaves][2][2][8]>(lds);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, H = a.H, I = a.I;
  const int nch = H / 256;
  const int c0 = wave * CPW;
  const int nchw = c0 < nch ? (nch - c0 < CPW ? nch - c0 : CPW) : 0;
  const int n = lane & 15, q = lane >> 4;
  const int r = n & 7, hh = n >> 3;
  const size_t row = size_t(blockIdx.x) * 8 + r;
  const size_t woff = row * size_t(H / 256) * W::kChunkBytes + size_t(c0) * W::kChunkBytes +
                      W::off(hh, q);
  const size_t soff = row * size_t(H / 32) + size_t(c0) * 8;  // MXFP4 scale slice
  const size_t rt = row >> 7;                                 // fp8 tile row
  const int ktiles = H / 128;

  auto load = [&](GuSlot<FMT, CPW> &sl, const uint8_t *b) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (c < nchw) {
#pragma unroll
        for (int i = 0; i < W::kLoads; ++i) {
          sl.wg[c][i] = *reinterpret_cast<const uint4 *>(b + a.q_off[0] + woff +
                                                         W::kChunkBytes * c + 64 * i);
          sl.wu[c][i] = *reinterpret_cast<const uint4 *>(b + a.q_off[1] + woff +
                                                         W::kChunkBytes * c + 64 * i);
        }
        if constexpr (!W::kMx) {
          sl.sfg[c] = tile_scale(b + a.s_off[0], rt, ktiles, c0 + c, hh);
          sl.sfu[c] = tile_scale(b + a.s_off[1], rt, ktiles, c0 + c, hh);
        }
      }
    if constexpr (W::kMx) {
      if (nchw > 0) {
        sl.sdg = scale_dword(b + a.s_off[0] + soff, nchw, hh, q);
        sl.sdu = scale_dword(b + a.s_off[1] + soff, nchw, hh, q);
      }
    }
  };
  // items: 0 the shared expert (its loads leave first), k >= 1 unit k - 1;
  // a ring of two items in flight
  GuSlot<FMT, CPW> s0, s1;
  load(s0, a.shared);
  const int nu = *a.n_unique;
  const int nitems = nu + 1;
  const uint8_t *blob1 = nu > 0 ? a.experts + size_t(a.unique[0]) * a.blob_bytes : a.shared;
  if (int(threadIdx.x) < nitems)
    sblob[threadIdx.x] = threadIdx.x == 0
                             ? a.shared
                             : a.experts + size_t(a.unique[threadIdx.x - 1]) * a.blob_bytes;

  // planes of x over this wave's chunks: 4 lanes per 32-element block, 8
  // elements per lane, in passes of 16 blocks
  {
    const int nb = nchw * 8;  // 32-blocks per token in the slice
    for (int j = lane; j < 4 * T * nb; j += 64) {
      const int bi = j >> 2, sub = j & 3;
      const int t = bi / nb, blk = bi - t * nb;
      const float4 *src = reinterpret_cast<const float4 *>(a.x + size_t(t) * H + size_t(c0) * 256 +
                                                           blk * 32 + sub * 8);
      const float4 p0 = src[0], p1 = src[1];
      float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      uint2 pl[4];
      const int e = block_planes(v, pl);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<uint2 *>(&xpl[wave][t][p][blk * 32 + sub * 8]) = pl[p];
      if (sub == 0) sexp[wave][t][blk] = e;
    }
  }
  if (nitems > 1) load(s1, blob1);
  lds_barrier();
  // A operands: row m = 8 h + 4 t + j (plane j of token t, elements 128 h ..)
  i32x8 A[CPW];
  int sA[CPW];
  {
    const int ah = n >> 3, at = (n >> 2) & 1, aj = n & 3;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (c < nchw && at < T) {
        const uint8_t *pl = &xpl[wave][at][aj][c * 256 + 128 * ah + 16 * q];
        const uint4 lo = *reinterpret_cast<const uint4 *>(pl);
        const uint4 hi = *reinterpret_cast<const uint4 *>(pl + 64);
        A[c] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w),
                     int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        sA[c] = sexp[wave][at][c * 8 + 4 * ah + q] - 4 * aj + 127;
      } else {
        A[c] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        sA[c] = 127;
      }
    }
  }
  lds_barrier();  // the planes' LDS becomes the partials'

  // item k from slot sl, which then takes item k + 2
  auto run = [&](GuSlot<FMT, CPW> &sl, int k) __attribute__((always_inline)) {
    const bool more = k + 2 < nitems;
    const uint8_t *nb = sblob[more ? k + 2 : k];
    f32x4 accg = {0.0f, 0.0f, 0.0f, 0.0f}, accu = {0.0f, 0.0f, 0.0f, 0.0f};
    // consume the slot (scales first), then refill it
    int scg[CPW], scu[CPW];
    float sfg[CPW], sfu[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if constexpr (W::kMx) {
        scg[c] = scale_of(sl.sdg, c, lane, q);
        scu[c] = scale_of(sl.sdu, c, lane, q);
      } else {
        sfg[c] = sl.sfg[c];
        sfu[c] = sl.sfu[c];
      }
    }
    if constexpr (W::kMx) {
      if (more && nchw > 0) {
        sl.sdg = scale_dword(nb + a.s_off[0] + soff, nchw, hh, q);
        sl.sdu = scale_dword(nb + a.s_off[1] + soff, nchw, hh, q);
      }
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (c < nchw) {
        uint4 bg[W::kLoads], bu[W::kLoads];
#pragma unroll
        for (int i = 0; i < W::kLoads; ++i) {
          bg[i] = sl.wg[c][i];
          bu[i] = sl.wu[c][i];
        }
        if (more) {
#pragma unroll
          for (int i = 0; i < W::kLoads; ++i) {
            sl.wg[c][i] = *reinterpret_cast<const uint4 *>(nb + a.q_off[0] + woff +
                                                           W::kChunkBytes * c + 64 * i);
            sl.wu[c][i] = *reinterpret_cast<const uint4 *>(nb + a.q_off[1] + woff +
                                                           W::kChunkBytes * c + 64 * i);
          }
          if constexpr (!W::kMx) {
            sl.sfg[c] = tile_scale(nb + a.s_off[0], rt, ktiles, c0 + c, hh);
            sl.sfu[c] = tile_scale(nb + a.s_off[1], rt, ktiles, c0 + c, hh);
          }
        }
        step_fence();
        if constexpr (W::kMx) {
          accg = mfma_mx(A[c], bg[0], accg, sA[c], scg[c]);
          accu = mfma_mx(A[c], bu[0], accu, sA[c], scu[c]);
        } else {
          accg += sfg[c] * mfma_f8(A[c], bg[0], bg[1], sA[c]);
          accu += sfu[c] * mfma_f8(A[c], bu[0], bu[1], sA[c]);
        }
      }
    }
    const float vg = fold_item(accg, lane), vu = fold_item(accu, lane);
    if (lane < 24 && (lane & 15) < 8) {
      red[k][wave][0][lane >> 4][lane & 7] = vg;
      red[k][wave][1][lane >> 4][lane & 7] = vu;
    }
  };
  for (int k = 0; k < nitems; k += 2) {
    run(s0, k);
    if (k + 1 < nitems) run(s1, k + 1);
  }
  lds_barrier();
  for (int i = threadIdx.x; i < nitems * T * 8; i += blockDim.x) {
    const int k = i / (T * 8), t = (i >> 3) % T, rr = i & 7;
    float gv = 0.0f, uv = 0.0f;
#pragma unroll
    for (int w = 0; w < kMxWaves; ++w) {
      gv += red[k][w][0][t][rr];
      uv += red[k][w][1][t][rr];
    }
    const int unit = k == 0 ? nu : k - 1;  // h: routed units first, the shared one last
    float wt = 1.0f;
    if (k > 0) {
      const int e = a.unique[k - 1];
      wt = 0.0f;
      for (int s = 0; s < a.K; ++s)
        if (a.idx[t * a.K + s] == e) wt = a.gates[t * a.K + s];
    }
    a.h[(size_t(unit) * T + t) * I + size_t(blockIdx.x) * 8 + rr] = silu(gv) * uv * wt;
  }
}

// ------------------------------------------------------------------ down
// One token.  Output-stationary: block b takes row groups b, b + G, ... (8
// rows of H each, at most kMxDownItems) and, for each, every unit in turn;
// its 8 waves split the 256-element chunks of I.  The gate weights are in h,
// so the combine over units is the accumulation itself, in unit order.  Each
// wave first turns its chunks of every unit's h into E4M3 planes in its own
// LDS area (the h loads of all its passes issued first, then the weight
// blocks of the first steps, which stream in meanwhile); then a ring of up
// to 8 steps.
constexpr int kMxDownItems = 4;
// steps in flight per wave: 8 KB of weight blocks at most
template <int FMT, int CPW>
constexpr int mx_down_depth() {
  return 8 / (CPW * Wt<FMT>::kLoads) > 2 ? 8 / (CPW * Wt<FMT>::kLoads) : 2;
}
constexpr int kMxDownMaxUC = 18;  // units x chunks per wave (the LDS area)
constexpr int kMxDownPasses = kMxDownMaxUC * 32 / 64;

struct MxDownArgs {
  const uint8_t *experts, *shared;
  size_t blob_bytes, q_off, s_off;  // the down section of a blob
  const int32_t *unique, *n_unique;
  const float *h;  // [units][I]
  float *y;        // [H]
  int32_t *status;
  int H, I, umax;  // umax: the units the LDS areas are sized for
};

template <int CPW>
constexpr int mx_down_unit_bytes() { return CPW * (4 * 256 + 8 * 4); }

template <int FMT, int CPW>
__global__ __launch_bounds__(64 * kMxWaves) void mx_down(MxDownArgs a) {
  using W = Wt<FMT>;
  extern __shared__ __align__(16) uint8_t dyn[];  // per wave: planes, then exponents
  __shared__ float red[kMxDownItems][kMxWaves][8];
  __shared__ const uint8_t *sblob[kMxMaxItems];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int nch = I / 256;
  const int c0 = wave * CPW;
  const int nchw = c0 < nch ? (nch - c0 < CPW ? nch - c0 : CPW) : 0;
  const int n = lane & 15, q = lane >> 4;
  const int r = n & 7, hh = n >> 3;
  const int ah = n >> 3, aj = n & 3;
  const bool arow = ((n >> 2) & 1) == 0;  // A rows of token 0
  const int groups = H / 8;
  int nj = 0;
  for (int g = blockIdx.x; g < groups && nj < kMxDownItems; g += gridDim.x) ++nj;
  const int nu = *a.n_unique;
  const int units = nu + 1;  // unit u < nu: routed, u == nu: the shared expert
  if (int(threadIdx.x) < units)
    sblob[threadIdx.x] = int(threadIdx.x) < nu
                             ? a.experts + size_t(a.unique[threadIdx.x]) * a.blob_bytes
                             : a.shared;
  uint8_t *apl = dyn + size_t(wave) * a.umax * mx_down_unit_bytes<CPW>();
  int *aex = reinterpret_cast<int *>(apl + size_t(a.umax) * CPW * 1024);
  lds_barrier();
  const int total = nj * units;

  // the ring: kMxDownDepth steps in flight
  constexpr int kMxDownDepth = mx_down_depth<FMT, CPW>();
  uint4 rw[kMxDownDepth][CPW][W::kLoads];
  uint32_t rsd[kMxDownDepth];     // MXFP4: the row slice's scale dword
  float rsf[kMxDownDepth][CPW];   // fp8: the chunks' tile scales
  const int ktiles = I / 128;
  auto load = [&](int k, int s) __attribute__((always_inline)) {
    const int j = s / units, u = s - j * units;
    const size_t row = (size_t(blockIdx.x) + size_t(j) * gridDim.x) * 8 + r;
    const uint8_t *b = sblob[u];
    const uint8_t *wp = b + a.q_off + row * size_t(I / 256) * W::kChunkBytes +
                        size_t(c0) * W::kChunkBytes + W::off(hh, q);
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (c < nchw) {
#pragma unroll
        for (int i = 0; i < W::kLoads; ++i)
          rw[k][c][i] = *reinterpret_cast<const uint4 *>(wp + W::kChunkBytes * c + 64 * i);
        if constexpr (!W::kMx) rsf[k][c] = tile_scale(b + a.s_off, row >> 7, ktiles, c0 + c, hh);
      }
    if constexpr (W::kMx) {
      if (nchw > 0)
        rsd[k] = scale_dword(b + a.s_off + row * size_t(I / 32) + size_t(c0) * 8, nchw, hh, q);
    }
  };
  // planes of h over this wave's chunks of every unit: 4 lanes per 32-block.
  // The h loads go first, then the first steps' weight blocks, so that the
  // conversion waits for h alone and runs while the weights stream in.
  {
    const int tasks = units * nchw * 32;
    float4 hv[kMxDownPasses][2];
#pragma unroll
    for (int i = 0; i < kMxDownPasses; ++i) {
      const int j = lane + 64 * i;
      if (j < tasks) {
        const int sub = j & 3, blk = (j >> 2) & 7, uc = j >> 5;
        const int u = uc / nchw, c = uc - u * nchw;
        const float4 *src = reinterpret_cast<const float4 *>(
            a.h + size_t(u) * I + size_t(c0 + c) * 256 + blk * 32 + sub * 8);
        hv[i][0] = src[0];
        hv[i][1] = src[1];
      }
    }
#pragma unroll
    for (int i = 0; i < kMxDownDepth; ++i)
      if (i < total) load(i, i);
#pragma unroll
    for (int i = 0; i < kMxDownPasses; ++i) {
      const int j = lane + 64 * i;
      if (j < tasks) {
        const int sub = j & 3, blk = (j >> 2) & 7, uc = j >> 5;
        const int u = uc / nchw, c = uc - u * nchw;
        float v[8] = {hv[i][0].x, hv[i][0].y, hv[i][0].z, hv[i][0].w,
                      hv[i][1].x, hv[i][1].y, hv[i][1].z, hv[i][1].w};
        uint2 pl[4];
        const int e = block_planes(v, pl);
#pragma unroll
        for (int p = 0; p < 4; ++p)
          *reinterpret_cast<uint2 *>(apl + ((u * CPW + c) * 4 + p) * 256 + blk * 32 + sub * 8) =
              pl[p];
        if (sub == 0) aex[(u * CPW + c) * 8 + blk] = e;
      }
    }
  }
  lds_barrier();

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // step s from slot k, which then takes step s + kMxDownDepth
  auto run = [&](int k, int s) __attribute__((always_inline)) {
    const int j = s / units, u = s - j * units;
    int sw[CPW];
    float sf[CPW];
    uint4 w[CPW][W::kLoads];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if constexpr (W::kMx)
        sw[c] = scale_of(rsd[k], c, lane, q);
      else
        sf[c] = rsf[k][c];
#pragma unroll
      for (int i = 0; i < W::kLoads; ++i) w[c][i] = rw[k][c][i];
    }
    if (s + kMxDownDepth < total) load(k, s + kMxDownDepth);
    step_fence();
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (c < nchw) {
        const uint8_t *pp = apl + ((u * CPW + c) * 4 + aj) * 256 + 128 * ah + 16 * q;
        const uint4 lo = *reinterpret_cast<const uint4 *>(pp);
        const uint4 hi = *reinterpret_cast<const uint4 *>(pp + 64);
        const int ea = aex[(u * CPW + c) * 8 + 4 * ah + q];
        const i32x8 av = arow ? i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x),
                                      int(hi.y), int(hi.z), int(hi.w)}
                              : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        // each block product summed in fp32 here, not in the matrix core's
        // accumulator (which keeps about 2^-15 of its largest term)
        const int sa = arow ? ea - 4 * aj + 127 : 127;
        if constexpr (W::kMx) {
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          acc += mfma_mx(av, w[c][0], z, sa, sw[c]);
        } else {
          acc += sf[c] * mfma_f8(av, w[c][0], w[c][1], sa);
        }
      }
    if (u == units - 1) {
      const float v = fold_item(acc, lane);
      if (lane < 8) red[j][wave][lane] = v;
      acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  for (int s = 0; s < total; s += kMxDownDepth) {
#pragma unroll
    for (int i = 0; i < kMxDownDepth; ++i)
      if (s + i < total) run(i, s + i);
  }
  lds_barrier();
  for (int i = threadIdx.x; i < nj * 8; i += blockDim.x) {
    const int j = i >> 3, rr = i & 7;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kMxWaves; ++w) v += red[j][w][rr];
    a.y[(size_t(blockIdx.x) + size_t(j) * gridDim.x) * 8 + rr] = v;
    if (a.status && !__builtin_isfinite(v)) atomicOr(a.status, COLI_STATUS_NONFINITE);
  }
}

}  // namespace

static bool mx_fmt(int fmt) { return fmt == COLI_FMT_MXFP4 || fmt == COLI_FMT_FP8_E4M3_B128; }

bool mx_gateup_ok(const FmtLayer &L, const float *x, int T) {
  const int units = (L.E < T * L.K ? L.E : T * L.K) + 1;
  return mx_fmt(L.fmt) && T >= 1 && T <= 2 && L.H % 256 == 0 &&
         L.H <= 256 * kMxWaves * kMxMaxCpw && L.I % 8 == 0 && units <= kMxMaxItems &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0 && L.q_off[0] % 16 == 0 &&
         L.q_off[1] % 16 == 0 && L.s_off[0] % 4 == 0 && L.s_off[1] % 4 == 0 &&
         L.blob_bytes % 16 == 0;
}

bool mx_down_ok(const FmtLayer &L, int T) {
  const int units = (L.E < L.K ? L.E : L.K) + 1;
  const int cpw = (L.I / 256 + kMxWaves - 1) / kMxWaves;
  return mx_fmt(L.fmt) && T == 1 && L.I % 256 == 0 && cpw <= kMxMaxCpw &&
         units * cpw <= kMxDownMaxUC && L.H % 8 == 0 && L.H / 8 <= 256 * kMxDownItems &&
         L.q_off[2] % 16 == 0 && L.s_off[2] % 4 == 0 && L.blob_bytes % 16 == 0;
}

template <int FMT>
static void launch_gateup_f(const MxArgs &a, int cpw, dim3 grid, dim3 block, hipStream_t s) {
  switch (cpw) {
    case 1: mx_gateup<FMT, 1><<<grid, block, 0, s>>>(a); break;
    case 2: mx_gateup<FMT, 2><<<grid, block, 0, s>>>(a); break;
    case 3: mx_gateup<FMT, 3><<<grid, block, 0, s>>>(a); break;
    default: mx_gateup<FMT, 4><<<grid, block, 0, s>>>(a); break;
  }
}

hipError_t launch_mx_gateup(const FmtLayer &L, const Routing &r, const float *x, int T, float *h,
                            hipStream_t s) {
  MxArgs a;
  a.experts = L.experts;
  a.shared = L.shared;
  a.blob_bytes = L.blob_bytes;
  a.q_off[0] = L.q_off[0];
  a.q_off[1] = L.q_off[1];
  a.s_off[0] = L.s_off[0];
  a.s_off[1] = L.s_off[1];
  a.unique = r.unique;
  a.n_unique = r.n_unique;
  a.idx = r.idx;
  a.gates = r.gates;
  a.x = x;
  a.h = h;
  a.T = T;
  a.H = L.H;
  a.I = L.I;
  a.K = L.K;
  const dim3 grid(unsigned(L.I / 8)), block(64 * kMxWaves);
  const int cpw = (L.H / 256 + kMxWaves - 1) / kMxWaves;
  if (L.fmt == COLI_FMT_MXFP4)
    launch_gateup_f<COLI_FMT_MXFP4>(a, cpw, grid, block, s);
  else
    launch_gateup_f<COLI_FMT_FP8_E4M3_B128>(a, cpw, grid, block, s);
  return hipGetLastError();
}

template <int FMT, int CPW>
static hipError_t launch_down_t(const MxDownArgs &d, int G, hipStream_t s) {
  static std::atomic<uint64_t> done{0};  // devices whose LDS attribute is set (bit per device)
  const size_t lds = size_t(kMxWaves) * d.umax * mx_down_unit_bytes<CPW>();
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (!bit || !(done.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mx_down<FMT, CPW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(size_t(kMxWaves) * kMxDownMaxUC / CPW * mx_down_unit_bytes<CPW>()));
    if (e != hipSuccess) return e;
    done.fetch_or(bit);
  }
  mx_down<FMT, CPW><<<dim3(unsigned(G)), dim3(64 * kMxWaves), lds, s>>>(d);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_down_f(const MxDownArgs &d, int cpw, int G, hipStream_t s) {
  switch (cpw) {
    case 1: return launch_down_t<FMT, 1>(d, G, s);
    case 2: return launch_down_t<FMT, 2>(d, G, s);
    case 3: return launch_down_t<FMT, 3>(d, G, s);
    default: return launch_down_t<FMT, 4>(d, G, s);
  }
}

hipError_t launch_mx_down(const FmtLayer &L, const Routing &r, const float *h, float *y,
                          int32_t *status, hipStream_t s) {
  MxDownArgs d;
  d.experts = L.experts;
  d.shared = L.shared;
  d.blob_bytes = L.blob_bytes;
  d.q_off = L.q_off[2];
  d.s_off = L.s_off[2];
  d.unique = r.unique;
  d.n_unique = r.n_unique;
  d.h = h;
  d.y = y;
  d.status = status;
  d.H = L.H;
  d.I = L.I;
  d.umax = (L.E < L.K ? L.E : L.K) + 1;
  const int groups = L.H / 8;  // at most 256 * kMxDownItems (mx_down_ok)
  const int G = groups < 256 ? groups : 256;
  const int cpw = (L.I / 256 + kMxWaves - 1) / kMxWaves;
  return L.fmt == COLI_FMT_MXFP4 ? launch_down_f<COLI_FMT_MXFP4>(d, cpw, G, s)
                                 : launch_down_f<COLI_FMT_FP8_E4M3_B128>(d, cpw, G, s);
}

}  // namespace coli

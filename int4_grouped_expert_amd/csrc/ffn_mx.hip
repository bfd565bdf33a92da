// ffn_mx.hip -- the gate/up stage of a decode layer whose experts are stored
// in MXFP4, for one or two tokens, on the gfx950 scaled matrix cores.
//
// Method: the expert FFN of page "Colibrì 深度解析" (sections 四 and 十一):
// h = w_t * SiLU(x Wg^T) * (x Wu^T) per (unit, token), w_t the token's gate
// weight for the unit (0 when it did not pick it, 1 for the shared expert);
// the weights in the MXFP4 element format of section 十 (OCP Microscaling
// v1.0: blocks of 32 E2M1 codes with one E8M0 power-of-two scale).
//
// Arithmetic.  v_mfma_scale_f32_16x16x128_f8f6f4 multiplies an E4M3 A operand
// by an E2M1 B operand and applies one E8M0 scale per 32 k on each side, so
// the weight blocks enter exactly as stored, codes and scales.  The
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
// Kernel mx_gateup: block b takes row group b (8 rows of I) of every unit, the
// shared expert first (its blob needs no routing, so its loads leave first);
// the 8 waves split the 256-element chunks of H and keep their planes of x in
// registers; a register ring one item deep; per-item partials meet in LDS and
// are reduced once, at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

template <int CPW>
__global__ __launch_bounds__(64 * kMxWaves) void mx_gateup(MxArgs a) {
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
  const size_t woff = row * size_t(H / 2) + size_t(c0) * 128 + 64 * hh + 16 * q;
  const size_t soff = row * size_t(H / 32) + size_t(c0) * 8 + 4 * hh + q;

  // the shared expert's gate/up blocks first
  uint4 wg[CPW], wu[CPW];
  uint32_t sg[CPW], su[CPW];
  {
    const uint8_t *b = a.shared;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (c < nchw) {
        wg[c] = *reinterpret_cast<const uint4 *>(b + a.q_off[0] + woff + 128 * c);
        wu[c] = *reinterpret_cast<const uint4 *>(b + a.q_off[1] + woff + 128 * c);
        sg[c] = b[a.s_off[0] + soff + 8 * c];
        su[c] = b[a.s_off[1] + soff + 8 * c];
      }
  }
  const int nu = *a.n_unique;
  const int nitems = nu + 1;  // item 0: the shared expert; item k: unit k - 1
  if (int(threadIdx.x) < nitems)
    sblob[threadIdx.x] = threadIdx.x == 0
                             ? a.shared
                             : a.experts + size_t(a.unique[threadIdx.x - 1]) * a.blob_bytes;

  // planes of x over this wave's chunks: 4 lanes per 32-element block, 8
  // elements per lane, blocks (token, block) in passes of 16
  {
    const int nb = nchw * 8;  // 32-blocks per token in the slice
    for (int j = lane; j < 4 * T * nb; j += 64) {
      const int bi = j >> 2, sub = j & 3;
      const int t = bi / nb, blk = bi - t * nb;
      const float4 *src = reinterpret_cast<const float4 *>(a.x + size_t(t) * H + size_t(c0) * 256 +
                                                           blk * 32 + sub * 8);
      const float4 p0 = src[0], p1 = src[1];
      float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      uint32_t mb = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
      mb = max(mb, uint32_t(__shfl_xor(int(mb), 1)));
      mb = max(mb, uint32_t(__shfl_xor(int(mb), 2)));
      // e: the block's largest |x| times 2^-e in [64, 128); kept >= -115 so
      // that the last plane's scale 2^(e - 12) is an E8M0 value
      const int ef = int(mb >> 23) < 1 ? 1 : int(mb >> 23);
      int e = ef - 133;
      e = e < -115 ? -115 : e;
      uint2 pl[4];
      if (mb >= 0x7F800000u) {
        e = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) pl[p] = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      } else {
        const float f = pow2f(-e);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= f;
        e4m3_planes(v, pl);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<uint2 *>(&xpl[wave][t][p][blk * 32 + sub * 8]) = pl[p];
      if (sub == 0) sexp[wave][t][blk] = e;
    }
  }
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

  for (int k = 0; k < nitems; ++k) {
    const bool more = k + 1 < nitems;
    const uint8_t *nb = sblob[more ? k + 1 : k];
    f32x4 accg = {0.0f, 0.0f, 0.0f, 0.0f}, accu = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (c < nchw) {
        // consume the slot, then refill it with the next item's block
        const uint4 bg = wg[c], bu = wu[c];
        const int scg = int(sg[c]), scu = int(su[c]);
        if (more) {
          wg[c] = *reinterpret_cast<const uint4 *>(nb + a.q_off[0] + woff + 128 * c);
          wu[c] = *reinterpret_cast<const uint4 *>(nb + a.q_off[1] + woff + 128 * c);
          sg[c] = nb[a.s_off[0] + soff + 8 * c];
          su[c] = nb[a.s_off[1] + soff + 8 * c];
        }
        step_fence();
        accg = mfma_mx(A[c], bg, accg, sA[c], scg);
        accu = mfma_mx(A[c], bu, accu, sA[c], scu);
      }
    }
    // the four planes, then the two halves of the 256-element chunks
    float vg = (accg[0] + accg[1]) + (accg[2] + accg[3]);
    float vu = (accu[0] + accu[1]) + (accu[2] + accu[3]);
    vg += __shfl(vg, (lane + 40) & 63);
    vu += __shfl(vu, (lane + 40) & 63);
    if (lane < 24 && (lane & 15) < 8) {
      red[k][wave][0][lane >> 4][lane & 7] = vg;
      red[k][wave][1][lane >> 4][lane & 7] = vu;
    }
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

}  // namespace

bool mx_gateup_ok(const FmtLayer &L, const float *x, int T) {
  const int units = (L.E < T * L.K ? L.E : T * L.K) + 1;
  return L.fmt == COLI_FMT_MXFP4 && T >= 1 && T <= 2 && L.H % 256 == 0 &&
         L.H <= 256 * kMxWaves * kMxMaxCpw && L.I % 8 == 0 && L.I / 8 <= 65535 &&
         units <= kMxMaxItems && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
         L.q_off[0] % 16 == 0 && L.q_off[1] % 16 == 0 && L.blob_bytes % 16 == 0;
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
  switch (cpw) {
    case 1: mx_gateup<1><<<grid, block, 0, s>>>(a); break;
    case 2: mx_gateup<2><<<grid, block, 0, s>>>(a); break;
    case 3: mx_gateup<3><<<grid, block, 0, s>>>(a); break;
    default: mx_gateup<4><<<grid, block, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace coli

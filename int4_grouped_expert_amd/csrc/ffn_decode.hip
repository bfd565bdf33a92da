// ffn_decode.hip -- the routed + shared expert FFN for small T (decode):
// int4-g64 planar weights streamed from HBM into fp16 matrix-core products
// with fp32-accurate activations.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 -- the expert FFN consumes the planar bytes as they are
// (byte k of a 64-group: element k low nibble, element k+32 high nibble,
// u = q + 8; weight = s * (u - 8)).  Batch union (page "Colibrì 深度解析",
// section 四): each unique expert of the batch is read once and applied to all
// of its tokens.
//
// Arithmetic.  An activation a is held as a split pair (hi + lo) * 2^e with
// hi, lo fp16 (about 22 significant bits; e a power-of-two scale per token
// row for x, per 32-column half-group for h), weights as the exact fp16
// integers u - 8.  Every product hi*(u-8), lo*(u-8) is exact in the fp32
// accumulator of v_mfma_f32_16x16x32_f16, so a 32-element step of a group
// sums exactly-rounded fp32 terms; the fp32 group scale s (and the activation
// scale) are applied per group (gate/up) or per step (down) in fp32.  The
// result is as accurate as an fp32 dot product, while the matrix cores do
// the multiply-adds and the K reduction, leaving the VALU to the nibble
// unpack (2 weights per 32-bit op).
//
// MFMA step layout (16x16x32 f16: lane l holds row l%16 and k = 8*(l/16)..+7
// of each operand; the result lane l holds rows 4*(l/16)+i, column l%16).
// For group g the B lane (row n, q = l/16) loads bytes 8q..8q+7 of the group
// (8 bytes): its low nibbles are step 0 (elements 8q + perm8[i]), its high
// nibbles step 1 (elements 32 + 8q + perm8[i]), perm8 = {0,2,1,3,4,6,5,7}
// being the order the fp16 pairs fall out of the unpack.  Activations are
// stored with perm8 applied inside every 8-element run, so each A slot is one
// contiguous 16-byte load.
//
// Kernels
//   gateup_decode  item = (unit, 32 output rows, <= 16*NMF tokens); 4 waves
//                  split the K groups; partial sums meet in LDS; the epilogue
//                  writes h' = gate_weight * SiLU(gate) * up in the split form
//                  with a scale per (row, 32 columns).
//   down_decode    item = (16 output rows, <= 16*NMF tokens), output-
//                  stationary: 8 waves split the K groups, each streams every
//                  unit of the batch (routed experts, then the shared one) and
//                  accumulates y directly -- the gates already sit in h', so
//                  the combine is the accumulation itself, in a fixed order
//                  (no atomics).
// Both keep the weights of several groups in flight per wave (register ring)
// and fetch the next step's activations while the current one multiplies.
#include "kernels.h"

namespace coli {
namespace {

constexpr int kWave = 64;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// fp16 (u - 8) for the 16 nibbles of a lane's 8 group bytes (d0 = bytes 0..3,
// d1 = bytes 4..7): step 0 = low nibbles, step 1 = high nibbles.
// (d >> sh) & 0x000F000F | 0x64006400 = fp16 pair {1024 + u_a, 1024 + u_b};
// adding -1032 gives u - 8 exactly.
__device__ inline f16x8 unpack_step(uint32_t d0, uint32_t d1, int step) {
  const int sh = step * 4;
  const uint32_t M = 0x000F000Fu, X = 0x64006400u;
  const uint32_t p0 = ((d0 >> sh) & M) | X;
  const uint32_t p1 = ((d0 >> (sh + 8)) & M) | X;
  const uint32_t p2 = ((d1 >> sh) & M) | X;
  const uint32_t p3 = ((d1 >> (sh + 8)) & M) | X;
  const f16x2 off = {_Float16(-1032.0f), _Float16(-1032.0f)};
  const f16x2 a = __builtin_bit_cast(f16x2, p0) + off;
  const f16x2 b = __builtin_bit_cast(f16x2, p1) + off;
  const f16x2 c = __builtin_bit_cast(f16x2, p2) + off;
  const f16x2 d = __builtin_bit_cast(f16x2, p3) + off;
  f16x8 o;
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
  o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
  return o;
}

__device__ inline f32x4 mfma(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline int perm8_pos(int o) {
  const int r = o & 7;
  const int pr = (r == 1) ? 2 : (r == 2) ? 1 : (r == 5) ? 6 : (r == 6) ? 5 : r;
  return (o & ~7) | pr;
}

// Max over the 16 lanes of a DPP row (all 16 lanes get it): quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ inline float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// A unit is a unique routed expert of the batch (u < n_unique) or the shared
// expert (u == n_unique).
struct Unit {
  const uint8_t *blob;
  int jb, je;
  bool shared;
};
__device__ inline Unit unit_of(const LayerDev &L, const Routing &r, int u, int nr, int T) {
  Unit U;
  if (u < nr) {
    const int e = r.unique[u];
    U.blob = L.experts + size_t(e) * L.lay.bytes;
    U.jb = r.offsets[e];
    U.je = r.offsets[e + 1];
    U.shared = false;
  } else {
    U.blob = L.shared;
    U.jb = 0;
    U.je = T;
    U.shared = true;
  }
  return U;
}

// ------------------------------------------------------------------ gate/up
// grid: persistent over items; block: 4 waves (K split).  Everything a group
// step reads from global memory -- weights and activation fragments -- sits in
// a ring of kD + 1 register slots filled kD steps ahead.  (Vector-memory
// counters retire in issue order, so a load needed soon must not be issued
// after loads needed late; one ring keeps every load kD steps ahead of use.)
// The fp32 group scales of the item are staged once in LDS, coalesced.
constexpr int kGW = 4;
constexpr int kSW = 32;  // groups of scales staged per window

template <int NMF>
struct GUSlot {
  uint2 w[4];
  f16x8 ah[NMF][2], al[NMF][2];
};

template <int NMF, int kD>
__global__ __launch_bounds__(kGW * kWave) void gateup_decode(
    const uint16_t *__restrict__ xh, const uint16_t *__restrict__ xl,
    const float *__restrict__ xsc, int T, LayerDev L, Routing r,
    uint16_t *__restrict__ hh, uint16_t *__restrict__ hl, float *__restrict__ hsc) {
  __shared__ f32x4 red[kGW][NMF][4][kWave];
  __shared__ float ssc[kGW][4 * 16][kSW + 1];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = L.H, I = L.I, K = L.K;
  const int GH = int(L.lay.GH);
  const int n_nt = I / 32;
  const int nr = *r.n_unique;
  const int n_items = r.chunk[nr + 1] * n_nt;
  const int n16 = lane % 16, q = lane / 16;
  const int g0 = (GH * wave) / kGW, g1 = (GH * (wave + 1)) / kGW;
  const int ng = g1 - g0;
  constexpr int MC = 16 * NMF;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int c = item / n_nt, nt = item % n_nt;
    int lo = 0, hi = nr;  // last unit u with chunk[u] <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (r.chunk[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const Unit U = unit_of(L, r, lo, nr, T);
    const int jb = U.jb + (c - r.chunk[lo]) * MC;
    const int je = min(U.je, jb + MC);
    const int nmf = (je - jb + 15) / 16;

    // A rows of this lane.  Rows past the chunk read token 0: an MFMA result
    // row depends only on its own A row, and those rows are never stored.
    // (Every ring load is unconditional and nothing inspects loaded data
    // before it is used, so the in-order load counters never force an early
    // wait.)
    int64_t arow[NMF];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) {
      const int j = jb + mf * 16 + n16;
      arow[mf] = (j < je) ? int64_t(U.shared ? j : r.perm[j] / K) * H : 0;
    }
    const uint8_t *bq[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int row = nt * 32 + 16 * (f & 1) + n16;
      bq[f] = U.blob + (f < 2 ? L.lay.gq : L.lay.uq) + size_t(row) * GH * 32 + 8 * q;
    }
    // this wave's scales, kSW groups at a time: lane l stages row l % 16 of
    // fragment l / 16 (one contiguous run of the row's scales)
    __syncthreads();  // previous item's readers of red are done
    const float *srow;
    {
      const int f = lane / 16, row = nt * 32 + 16 * (f & 1) + n16;
      srow = reinterpret_cast<const float *>(U.blob + (f < 2 ? L.lay.gs : L.lay.us)) +
             size_t(row) * GH + g0;
    }
    // all of a window's loads are issued before the first LDS store
    const bool vec = ((GH | g0) & 3) == 0;
    auto stage = [&](int w0) {
      const int n = min(kSW, ng - w0);
      if (vec && n == kSW) {
        float4 v[kSW / 4];
#pragma unroll
        for (int k = 0; k < kSW / 4; ++k) v[k] = reinterpret_cast<const float4 *>(srow + w0)[k];
#pragma unroll
        for (int k = 0; k < kSW / 4; ++k) {
          ssc[wave][lane][4 * k] = v[k].x;
          ssc[wave][lane][4 * k + 1] = v[k].y;
          ssc[wave][lane][4 * k + 2] = v[k].z;
          ssc[wave][lane][4 * k + 3] = v[k].w;
        }
      } else {
        float v[kSW];
#pragma unroll
        for (int g = 0; g < kSW; ++g) v[g] = g < n ? srow[w0 + g] : 0.0f;
#pragma unroll
        for (int g = 0; g < kSW; ++g) ssc[wave][lane][g] = v[g];
      }
    };
    stage(0);
    f32x4 acc[NMF][4];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mf][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    GUSlot<NMF> ring[kD + 1];
    // step si reads group g0 + min(si, ng - 1); steps past ng get scale 0
    auto load = [&](GUSlot<NMF> &sl, int si) {
      const int g = g0 + min(si, ng - 1);
#pragma unroll
      for (int f = 0; f < 4; ++f) sl.w[f] = *reinterpret_cast<const uint2 *>(bq[f] + size_t(g) * 32);
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int64_t off = arow[mf] + int64_t(g) * 64 + 32 * st + 8 * q;
          sl.ah[mf][st] = *reinterpret_cast<const f16x8 *>(xh + off);
          sl.al[mf][st] = *reinterpret_cast<const f16x8 *>(xl + off);
        }
    };
    // A wave with no K groups (H < 64 * kGW) skips the ring: its clamped
    // group index would point before the row.
    const int nsteps = ng > 0 ? (ng + kD) / (kD + 1) * (kD + 1) : 0;
    if (ng > 0) {
#pragma unroll
      for (int p = 0; p < kD; ++p) load(ring[p], p);
    }
    for (int sb = 0; sb < nsteps; sb += kD + 1) {
#pragma unroll
      for (int p = 0; p <= kD; ++p) {
        const int si = sb + p;
        load(ring[(p + kD) % (kD + 1)], si + kD);
        if (si % kSW == 0 && si > 0 && si < ng) stage(si);
        const GUSlot<NMF> &sl = ring[p];
        float sc[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) sc[f] = si < ng ? ssc[wave][f * 16 + n16][si % kSW] : 0.0f;
        f16x8 b0[4], b1[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          b0[f] = unpack_step(sl.w[f].x, sl.w[f].y, 0);
          b1[f] = unpack_step(sl.w[f].x, sl.w[f].y, 1);
        }
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
          if (NMF == 1 || mf < nmf) {
            // four independent chains, interleaved
            f32x4 P[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) P[f] = mfma(sl.ah[mf][0], b0[f], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int f = 0; f < 4; ++f) P[f] = mfma(sl.al[mf][0], b0[f], P[f]);
#pragma unroll
            for (int f = 0; f < 4; ++f) P[f] = mfma(sl.ah[mf][1], b1[f], P[f]);
#pragma unroll
            for (int f = 0; f < 4; ++f) P[f] = mfma(sl.al[mf][1], b1[f], P[f]);
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mf][f][i] = fmaf(P[f][i], sc[f], acc[mf][f][i]);
          }
        }
      }
    }
    // K-split partials meet in LDS; wave mf finishes M fragment mf
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
      for (int f = 0; f < 4; ++f) red[wave][mf][f][lane] = acc[mf][f];
    __syncthreads();
    if (wave < nmf) {
      const int mf = wave;
      float hv[2][4];
      float mx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        f32x4 g4 = red[0][mf][pr][lane], u4 = red[0][mf][pr + 2][lane];
#pragma unroll
        for (int w = 1; w < kGW; ++w) {
          g4 += red[w][mf][pr][lane];
          u4 += red[w][mf][pr + 2][lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = jb + mf * 16 + 4 * q + i;
          float v = 0.0f;
          if (j < je) {
            const int t = U.shared ? j : r.perm[j] / K;
            const float xs = xsc[t];
            const float gw = U.shared ? 1.0f : r.gates[r.perm[j]];
            v = gw * silu(g4[i] * xs) * (u4[i] * xs);
          }
          hv[pr][i] = v;
          mx[i] = fmaxf(mx[i], fabsf(v));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m = row16_max(mx[i]);
        const int j = jb + mf * 16 + 4 * q + i;
        if (j >= je) continue;
        // scale 2^e with m * 2^-e in [2^14, 2^15): hi, lo both fp16-normal
        int ex = 0;
        (void)frexpf(m, &ex);
        const int e = m > 0.0f ? max(ex - 15, -140) : 0;
        const int64_t hrow = U.shared ? int64_t(T) * K + j : j;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float a = ldexpf(hv[pr][i], -e);
          const _Float16 h16 = _Float16(a);
          const _Float16 l16 = _Float16(a - float(h16));
          const int o = nt * 32 + 16 * pr + n16;
          hh[hrow * I + perm8_pos(o)] = __builtin_bit_cast(uint16_t, h16);
          hl[hrow * I + perm8_pos(o)] = __builtin_bit_cast(uint16_t, l16);
        }
        if (n16 == 0) hsc[hrow * (I / 32) + nt] = ldexpf(1.0f, e);
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Output-stationary: item = (16 output rows, M-chunk of 16*NMF tokens); kDW
// waves split the K groups; each wave streams (unit, group) steps over every
// unit of the batch.  The ring holds, kD steps ahead, a step's weights and
// group scale, its activation fragments and the activation scales of its
// result rows.  Unit data (blob, h row of each chunk token) is staged in LDS
// in batches of kUB units.
constexpr int kDW = 8;
constexpr int kUB = 64;

template <int NMF>
struct DSlot {
  uint2 w;
  float s;
  f16x8 ah[NMF][2], al[NMF][2];
  float cs[NMF][2][4];  // activation scales of the result rows
  float on[NMF][4];     // 1 if the result row's token is routed to the unit
};

template <int NMF, int kD>
__global__ __launch_bounds__(kDW * kWave) void down_decode(
    const uint16_t *__restrict__ hh, const uint16_t *__restrict__ hl,
    const float *__restrict__ hsc, int T, LayerDev L, Routing r,
    const int32_t *__restrict__ slotmap, float *__restrict__ y) {
  __shared__ f32x4 red[kDW][NMF][kWave];
  __shared__ const uint8_t *ublob[kUB];
  __shared__ int rmap[kUB][16 * NMF];
  constexpr int MC = 16 * NMF;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = L.H, I = L.I, K = L.K;
  const int GI = int(L.lay.GI);
  const int n_nt = H / 16;
  const int n_mc = (T + MC - 1) / MC;
  const int n_items = n_nt * n_mc;
  const int nr = *r.n_unique;
  const int nunits = nr + 1;
  const int n16 = lane % 16, q = lane / 16;
  const int g0 = (GI * wave) / kDW, g1 = (GI * (wave + 1)) / kDW;
  const int ng = g1 - g0;
  const int HS = I / 32;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int mc = item / n_nt, nt = item % n_nt;
    const int t0 = mc * MC;
    const int nmf = (min(T, t0 + MC) - t0 + 15) / 16;
    const int row = nt * 16 + n16;
    f32x4 acc[NMF];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) acc[mf] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ub = 0; ub < nunits; ub += kUB) {
      const int nb = min(kUB, nunits - ub);
      __syncthreads();
      for (int i = threadIdx.x; i < nb * MC; i += blockDim.x) {
        const int ul = i / MC, m = i % MC;
        const int u = ub + ul, t = t0 + m;
        int j = -1;
        if (t < T) j = (u == nr) ? T * K + t : slotmap[size_t(u) * T + t];
        rmap[ul][m] = j;
        if (m == 0)
          ublob[ul] = (u == nr) ? L.shared : L.experts + size_t(r.unique[u]) * L.lay.bytes;
      }
      __syncthreads();
      const int S = nb * ng;
      DSlot<NMF> ring[kD + 1];
      // step s reads (unit, group) of min(s, S - 1); steps past S get scale 0
      auto load = [&](DSlot<NMF> &sl, int s) {
        const int sc_ = min(s, S - 1);
        const int ul = sc_ / ng, g = g0 + sc_ % ng;
        const uint8_t *blob = ublob[ul];
        sl.w = *reinterpret_cast<const uint2 *>(blob + L.lay.dq + (size_t(row) * GI + g) * 32 + 8 * q);
        sl.s = reinterpret_cast<const float *>(blob + L.lay.ds)[size_t(row) * GI + g];
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
          const int j = rmap[ul][mf * 16 + n16];
          // rows of tokens not routed here read h row 0 (finite) and are
          // multiplied by on = 0 below
          const int64_t jrow = j >= 0 ? int64_t(j) * I : 0;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int64_t off = jrow + int64_t(g) * 64 + 32 * st + 8 * q;
            sl.ah[mf][st] = *reinterpret_cast<const f16x8 *>(hh + off);
            sl.al[mf][st] = *reinterpret_cast<const f16x8 *>(hl + off);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jc = rmap[ul][mf * 16 + 4 * q + i];
            const size_t jcr = jc >= 0 ? size_t(jc) : 0;
            sl.on[mf][i] = (jc >= 0 && s < S) ? 1.0f : 0.0f;
#pragma unroll
            for (int st = 0; st < 2; ++st) sl.cs[mf][st][i] = hsc[jcr * HS + 2 * g + st];
          }
        }
      };
      // A wave with no K groups (I < 64 * kDW) skips the ring (S == 0).
      const int nsteps = S > 0 ? (S + kD) / (kD + 1) * (kD + 1) : 0;
      if (S > 0) {
#pragma unroll
        for (int p = 0; p < kD; ++p) load(ring[p], p);
      }
      for (int sb = 0; sb < nsteps; sb += kD + 1) {
#pragma unroll
        for (int p = 0; p <= kD; ++p) {
          const int si = sb + p;
          load(ring[(p + kD) % (kD + 1)], si + kD);
          const DSlot<NMF> &sl = ring[p];
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const f16x8 b = unpack_step(sl.w.x, sl.w.y, st);
#pragma unroll
            for (int mf = 0; mf < NMF; ++mf) {
              if (mf < nmf) {
                f32x4 P = mfma(sl.ah[mf][st], b, f32x4{0.f, 0.f, 0.f, 0.f});
                P = mfma(sl.al[mf][st], b, P);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[mf][i] = fmaf(P[i], sl.s * sl.cs[mf][st][i] * sl.on[mf][i], acc[mf][i]);
              }
            }
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) red[wave][mf][lane] = acc[mf];
    __syncthreads();
    if (wave < nmf) {
      const int mf = wave;
      f32x4 sum = red[0][mf][lane];
#pragma unroll
      for (int w = 1; w < kDW; ++w) sum += red[w][mf][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mf * 16 + 4 * q + i;
        if (t < T) y[int64_t(t) * H + row] = sum[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_ffn_decode(const LayerDev &L, const DecodeBufs &b, int T,
                             const Routing &r, float *y, hipStream_t s, hipEvent_t *ev) {
  // Every unit's token count is at most T, so T <= 16 needs one M fragment;
  // the route kernel's chunk prefix (chunks of 32 tokens) then counts one
  // chunk per unit, which equals the 16-token chunking.
  const bool one = T <= 16;
  const int mc = one ? 16 : 32;
  const int max_units = (T * L.K < L.E ? T * L.K : L.E) + 1;
  const int64_t max_chunks = int64_t(T) * L.K / mc + max_units + (T + mc - 1) / mc;
  const int64_t items = max_chunks * (L.I / 32);
  const int cap = 4096;
  const unsigned gblocks = unsigned(items < cap ? items : cap);
  if (ev) (void)hipEventRecord(ev[0], s);
  if (one)
    gateup_decode<1, 4><<<gblocks, kGW * kWave, 0, s>>>(b.xh, b.xl, b.xsc, T, L, r, b.hh, b.hl,
                                                       b.hsc);
  else
    gateup_decode<2, 2><<<gblocks, kGW * kWave, 0, s>>>(b.xh, b.xl, b.xsc, T, L, r, b.hh, b.hl,
                                                       b.hsc);
  if (ev) (void)hipEventRecord(ev[1], s);
  const int64_t ditems = int64_t(L.H / 16) * ((T + mc - 1) / mc);
  const unsigned dblocks = unsigned(ditems < cap ? ditems : cap);
  if (ev) (void)hipEventRecord(ev[2], s);
  if (one)
    down_decode<1, 4><<<dblocks, kDW * kWave, 0, s>>>(b.hh, b.hl, b.hsc, T, L, r, b.slotmap, y);
  else
    down_decode<2, 2><<<dblocks, kDW * kWave, 0, s>>>(b.hh, b.hl, b.hsc, T, L, r, b.slotmap, y);
  if (ev) (void)hipEventRecord(ev[3], s);
  return hipGetLastError();
}

}  // namespace coli

// ffn_decode.hip -- the routed + shared expert FFN for small T (decode):
// int4-g64 planar weights streamed from HBM into fp16 matrix-core products
// with fp32-accurate activations.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 -- the expert FFN consumes the planar bytes as they are
// (byte k of a 64-group: element k low nibble, element k+32 high nibble,
// u = q + 8; weight = s * (u - 8)).  Batch union (page "Colibri 深度解析",
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
//   gateup_decode  item = (unit, 32 output rows, <= 32 tokens); 4 waves split
//                  the K groups; partial sums meet in LDS; the epilogue writes
//                  h' = gate_weight * SiLU(gate) * up in the split form with a
//                  scale per (row, 32 columns).
//   down_decode    item = (32 output rows, <= 32 tokens), output-stationary:
//                  8 waves split the K groups, each streams every unit of the
//                  batch (routed experts, then the shared one) and accumulates
//                  y directly -- the gates already sit in h', so the combine
//                  is the accumulation itself, in a fixed order (no atomics).
#include "kernels.h"

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kMC = 32;    // tokens per M-chunk (2 MFMA row fragments)

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
// grid: persistent over items; block: 4 waves (K split).
constexpr int kGW = 4;
constexpr int kPF = 2;  // groups of weights prefetched ahead of the one in use

__global__ __launch_bounds__(kGW * kWave) void gateup_decode(
    const uint16_t *__restrict__ xh, const uint16_t *__restrict__ xl,
    const float *__restrict__ xsc, int T, LayerDev L, Routing r,
    uint16_t *__restrict__ hh, uint16_t *__restrict__ hl, float *__restrict__ hsc) {
  __shared__ f32x4 red[kGW][2][4][kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = L.H, I = L.I, K = L.K;
  const int GH = int(L.lay.GH);
  const int n_nt = I / 32;
  const int nr = *r.n_unique;
  const int n_items = r.chunk[nr + 1] * n_nt;
  const int n16 = lane % 16, q = lane / 16;
  // this wave's K groups
  const int g0 = (GH * wave) / kGW, g1 = (GH * (wave + 1)) / kGW;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int c = item / n_nt, nt = item % n_nt;
    int lo = 0, hi = nr;  // last unit u with chunk[u] <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (r.chunk[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const Unit U = unit_of(L, r, lo, nr, T);
    const int jb = U.jb + (c - r.chunk[lo]) * kMC;
    const int je = min(U.je, jb + kMC);
    const int nmf = (je - jb + 15) / 16;

    // A rows of this lane: token row of j = jb + mf*16 + n16
    int64_t arow[2];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf) {
      const int j = jb + mf * 16 + n16;
      arow[mf] = (j < je) ? int64_t(U.shared ? j : r.perm[j] / K) * H : -1;
    }
    // B rows: frags 0,1 gate rows nt*32 + {0..15, 16..31}, frags 2,3 up rows
    const uint8_t *bq[4];
    const float *bs[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int row = nt * 32 + 16 * (f & 1) + n16;
      bq[f] = U.blob + (f < 2 ? L.lay.gq : L.lay.uq) + size_t(row) * GH * 32 + 8 * q;
      bs[f] = reinterpret_cast<const float *>(U.blob + (f < 2 ? L.lay.gs : L.lay.us)) +
              size_t(row) * GH;
    }

    f32x4 acc[2][4];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mf][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // weight prefetch ring of kPF + 1 groups
    uint2 wq[kPF + 1][4];
    float ws[kPF + 1][4];
#pragma unroll
    for (int p = 0; p < kPF; ++p) {
      const int g = g0 + p;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (g < g1) {
          wq[p][f] = *reinterpret_cast<const uint2 *>(bq[f] + size_t(g) * 32);
          ws[p][f] = bs[f][g];
        }
      }
    }
    for (int gb = g0; gb < g1; gb += kPF + 1) {
#pragma unroll
      for (int p = 0; p <= kPF; ++p) {
        const int g = gb + p;
        if (g >= g1) break;
        // issue the load kPF groups ahead into the slot freed last step
        const int gn = g + kPF;
        const int sn = (p + kPF) % (kPF + 1);
        if (gn < g1) {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            wq[sn][f] = *reinterpret_cast<const uint2 *>(bq[f] + size_t(gn) * 32);
            ws[sn][f] = bs[f][gn];
          }
        }
        // activations of this group: 2 steps x (hi, lo) per M fragment
        f16x8 ah[2][2], al[2][2];
#pragma unroll
        for (int mf = 0; mf < 2; ++mf)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            if (mf < nmf && arow[mf] >= 0) {
              const int64_t off = arow[mf] + int64_t(g) * 64 + 32 * st + 8 * q;
              ah[mf][st] = *reinterpret_cast<const f16x8 *>(xh + off);
              al[mf][st] = *reinterpret_cast<const f16x8 *>(xl + off);
            } else {
              ah[mf][st] = f16x8{};
              al[mf][st] = f16x8{};
            }
          }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const f16x8 b0 = unpack_step(wq[p][f].x, wq[p][f].y, 0);
          const f16x8 b1 = unpack_step(wq[p][f].x, wq[p][f].y, 1);
#pragma unroll
          for (int mf = 0; mf < 2; ++mf) {
            if (mf < nmf) {
              f32x4 P = mfma(ah[mf][0], b0, f32x4{0.f, 0.f, 0.f, 0.f});
              P = mfma(al[mf][0], b0, P);
              P = mfma(ah[mf][1], b1, P);
              P = mfma(al[mf][1], b1, P);
              const float s = ws[p][f];
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mf][f][i] = fmaf(P[i], s, acc[mf][f][i]);
            }
          }
        }
      }
    }
    // K-split partials meet in LDS; wave mf finishes M fragment mf
    __syncthreads();
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
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
constexpr int kDW = 8;  // waves per down block (K split)

__global__ __launch_bounds__(kDW * kWave) void down_decode(
    const uint16_t *__restrict__ hh, const uint16_t *__restrict__ hl,
    const float *__restrict__ hsc, int T, LayerDev L, Routing r,
    const int32_t *__restrict__ slotmap, float *__restrict__ y) {
  __shared__ f32x4 red[kDW][2][2][kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = L.H, I = L.I, K = L.K;
  const int GI = int(L.lay.GI);
  const int n_nt = H / 32;
  const int n_mc = (T + kMC - 1) / kMC;
  const int n_items = n_nt * n_mc;
  const int nr = *r.n_unique;
  const int n16 = lane % 16, q = lane / 16;
  const int g0 = (GI * wave) / kDW, g1 = (GI * (wave + 1)) / kDW;
  const int HS = I / 32;  // h scales per row

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int mc = item / n_nt, nt = item % n_nt;
    const int t0 = mc * kMC;
    const int nmf = (min(T, t0 + kMC) - t0 + 15) / 16;
    f32x4 acc[2][2];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[mf][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int u = 0; u <= nr; ++u) {
      const bool shared = u == nr;
      const uint8_t *blob = shared ? L.shared : L.experts + size_t(r.unique[u]) * L.lay.bytes;
      // h rows of this unit for the A lanes (row n16 of each M fragment) and for
      // the C lanes (rows 4q + i); -1 where the token is not routed here
      int64_t arow[2];
      int crow[2][4];
#pragma unroll
      for (int mf = 0; mf < 2; ++mf) {
        const int t = t0 + mf * 16 + n16;
        int j = -1;
        if (t < T) j = shared ? T * K + t : slotmap[size_t(u) * T + t];
        arow[mf] = j >= 0 ? int64_t(j) * I : -1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tc = t0 + mf * 16 + 4 * q + i;
          int jc = -1;
          if (tc < T) jc = shared ? T * K + tc : slotmap[size_t(u) * T + tc];
          crow[mf][i] = jc;
        }
      }
      const uint8_t *bq[2];
      const float *bs[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int row = nt * 32 + 16 * f + n16;
        bq[f] = blob + L.lay.dq + size_t(row) * GI * 32 + 8 * q;
        bs[f] = reinterpret_cast<const float *>(blob + L.lay.ds) + size_t(row) * GI;
      }
      for (int g = g0; g < g1; ++g) {
        uint2 wq[2];
        float ws[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          wq[f] = *reinterpret_cast<const uint2 *>(bq[f] + size_t(g) * 32);
          ws[f] = bs[f][g];
        }
        f16x8 ah[2][2], al[2][2];
        float cs[2][2][4];
#pragma unroll
        for (int mf = 0; mf < 2; ++mf)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            if (mf < nmf && arow[mf] >= 0) {
              const int64_t off = arow[mf] + int64_t(g) * 64 + 32 * st + 8 * q;
              ah[mf][st] = *reinterpret_cast<const f16x8 *>(hh + off);
              al[mf][st] = *reinterpret_cast<const f16x8 *>(hl + off);
            } else {
              ah[mf][st] = f16x8{};
              al[mf][st] = f16x8{};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              cs[mf][st][i] = (mf < nmf && crow[mf][i] >= 0)
                                  ? hsc[size_t(crow[mf][i]) * HS + 2 * g + st]
                                  : 0.0f;
          }
#pragma unroll
        for (int f = 0; f < 2; ++f) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const f16x8 b = unpack_step(wq[f].x, wq[f].y, st);
#pragma unroll
            for (int mf = 0; mf < 2; ++mf) {
              if (mf < nmf) {
                f32x4 P = mfma(ah[mf][st], b, f32x4{0.f, 0.f, 0.f, 0.f});
                P = mfma(al[mf][st], b, P);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[mf][f][i] = fmaf(P[i], ws[f] * cs[mf][st][i], acc[mf][f][i]);
              }
            }
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < 2; ++f) red[wave][mf][f][lane] = acc[mf][f];
    __syncthreads();
    // waves 0..3 finish (mf, f) = (wave / 2, wave % 2)
    if (wave < 4 && wave / 2 < nmf) {
      const int mf = wave / 2, f = wave % 2;
      f32x4 s = red[0][mf][f][lane];
#pragma unroll
      for (int w = 1; w < kDW; ++w) s += red[w][mf][f][lane];
      const int o = nt * 32 + 16 * f + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mf * 16 + 4 * q + i;
        if (t < T) y[int64_t(t) * H + o] = s[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_ffn_decode(const LayerDev &L, const DecodeBufs &b, int T,
                             const Routing &r, float *y, hipStream_t s, hipEvent_t *ev) {
  // gate/up items: sum over units of ceil(n/32) chunks, times I/32 row tiles
  const int max_units = (T * L.K < L.E ? T * L.K : L.E) + 1;
  const int64_t max_chunks = int64_t(T) * L.K / kMC + max_units + (T + kMC - 1) / kMC;
  const int64_t items = max_chunks * (L.I / 32);
  const int cap = 4096;
  gateup_decode<<<unsigned(items < cap ? items : cap), kGW * kWave, 0, s>>>(
      b.xh, b.xl, b.xsc, T, L, r, b.hh, b.hl, b.hsc);
  if (ev) (void)hipEventRecord(ev[0], s);
  const int64_t ditems = int64_t(L.H / 32) * ((T + kMC - 1) / kMC);
  down_decode<<<unsigned(ditems < cap ? ditems : cap), kDW * kWave, 0, s>>>(
      b.hh, b.hl, b.hsc, T, L, r, b.slotmap, y);
  if (ev) (void)hipEventRecord(ev[1], s);
  return hipGetLastError();
}

}  // namespace coli

// ffn_decode.hip -- the routed + shared expert FFN for small T (decode):
// bandwidth-bound grouped int4-g64 GEMVs on the planar bytes.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 -- the expert FFN consumes the converter's planar bytes as
// they are (byte k of a 64-group: element k low nibble, element k+32 high
// nibble, stored as u = q + 8; weight = s * (u - 8)).  Batch union (page
// "Colibri 深度解析", section 四): every unique expert of the batch is read once
// and applied to all of its tokens.
//
// Per lane, one 16-byte load covers half a group: bytes 16*half..16*half+15
// of group g hold elements 16*half+k (low nibbles) and 32+16*half+k (high).
// The dot over those 32 weights uses the offset identity
//   sum_k s (u_k - 8) x_k = s (sum_k u_k x_k - 8 sum_k x_k)
// with sum_k x_k computed once per token slice, so the inner loop is half a
// conversion instruction (two nibbles per v_cvt_pk_f32_fp8) and one FMA per
// weight, plus the nibble masking (3 ops per 8 weights).
//
//   gateup_decode_kernel  work item = (unique expert or the shared one,
//                         4 output rows); a block has one wave per
//                         2048-column chunk of the input; each wave streams
//                         the 8 weight rows (4 gate + 4 up) of its chunk,
//                         partial sums meet in LDS, and the block writes
//                         h = SiLU(gate) * up.  Persistent grid: blocks loop
//                         over the items, whose count is read on the device.
//   down_decode_kernel    8 output rows per block, 4 waves; wave w takes the
//                         units (unique experts, then the shared one) w, w+4,
//                         ...; each token's contribution is multiplied by its
//                         gate and accumulated in a fixed order (deterministic,
//                         no atomics), then the 4 waves' sums are added in
//                         wave order.
#include "kernels.h"

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kRB = 4;   // gate/up output rows per work item
constexpr int kRD = 8;   // down output rows per block
constexpr int kDW = 4;   // waves per down block

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Nibble to float through the fp8 converter: a byte holding u in [0, 15]
// read as fp8 e4m3 is u * 2^-9 exactly (u < 8: subnormal u/8 * 2^-6; u >= 8:
// exponent 1, 2^-6 * (1 + (u-8)/8)), so v_cvt_pk_f32_fp8 turns two masked
// bytes into two floats in one instruction.  kNibUnit is that 2^-9; the
// callers fold its inverse into the group scale (a power of two: exact).
constexpr float kNibUnit = 1.0f / 512.0f;

// The lane's 32 nibbles as floats u * kNibUnit: [0,16) the low nibbles of
// bytes 0..15, [16,32) the high nibbles of the same bytes.
__device__ inline void unpack32(const uint4 w, float uf[32]) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = d[i] & 0x0F0F0F0Fu;
    const uint32_t hi = (d[i] >> 4) & 0x0F0F0F0Fu;
    const f32x2 l01 = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), false);
    const f32x2 l23 = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), true);
    const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), false);
    const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), true);
    uf[4 * i] = l01[0]; uf[4 * i + 1] = l01[1]; uf[4 * i + 2] = l23[0]; uf[4 * i + 3] = l23[1];
    uf[16 + 4 * i] = h01[0]; uf[16 + 4 * i + 1] = h01[1];
    uf[16 + 4 * i + 2] = h23[0]; uf[16 + 4 * i + 3] = h23[1];
  }
}

// Load the lane's 32-element activation slice matching unpack32 and its sum.
__device__ inline float load_slice(const float *__restrict__ row, int64_t g, int half,
                                   bool valid, float xs[32]) {
  float sum = 0.0f;
  if (valid) {
    const float4 *p0 = reinterpret_cast<const float4 *>(row + g * 64 + 16 * half);
    const float4 *p1 = reinterpret_cast<const float4 *>(row + g * 64 + 32 + 16 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = p0[i], b = p1[i];
      xs[4 * i] = a.x; xs[4 * i + 1] = a.y; xs[4 * i + 2] = a.z; xs[4 * i + 3] = a.w;
      xs[16 + 4 * i] = b.x; xs[16 + 4 * i + 1] = b.y;
      xs[16 + 4 * i + 2] = b.z; xs[16 + 4 * i + 3] = b.w;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += xs[i];
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) xs[i] = 0.0f;
  }
  return sum;
}

__device__ inline float dot32(const float uf[32], const float xs[32]) {
  float a = 0.0f, b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a = fmaf(uf[i], xs[i], a);
    b = fmaf(uf[16 + i], xs[16 + i], b);
  }
  return a + b;
}

// A unit is a unique expert of the batch (u < n_unique) or the shared expert.
struct Unit {
  const uint8_t *blob;
  int jb, je;
  bool shared;
};
__device__ inline Unit unit_of(const LayerDev &L, const Routing &r, int u, int nu, int T) {
  Unit U;
  if (u < nu - 1) {
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
template <int NT>
__global__ __launch_bounds__(256) void gateup_decode_kernel(
    const float *__restrict__ x, int T, LayerDev L, Routing r, float *__restrict__ h) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int H = L.H, I = L.I, K = L.K;
  const int64_t GH = L.lay.GH;
  const int nch = int((GH + 31) / 32);
  const int n_rb = (I + kRB - 1) / kRB;
  const int nu = *r.n_unique + 1;
  const int n_items = nu * n_rb;
  const int half = lane & 1;
  __shared__ float red[4][2][kRB][NT];

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int u = item / n_rb, o0 = (item % n_rb) * kRB;
    const Unit U = unit_of(L, r, u, nu, T);
    const uint8_t *wq[2] = {U.blob + L.lay.gq, U.blob + L.lay.uq};
    const float *ws[2] = {reinterpret_cast<const float *>(U.blob + L.lay.gs),
                          reinterpret_cast<const float *>(U.blob + L.lay.us)};
    for (int j0 = U.jb; j0 < U.je; j0 += NT) {
      float acc[2][kRB][NT];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[m][rr][tt] = 0.0f;

      for (int c = wave; c < nch; c += nw) {
        const int64_t g = int64_t(c) * 32 + lane / 2;
        const bool gv = g < GH;
        // weights first: 8 independent 16-byte loads in flight
        uint4 wv[2][kRB];
        float sv[2][kRB];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int rr = 0; rr < kRB; ++rr) {
            const int o = o0 + rr;
            if (gv && o < I) {
              wv[m][rr] = *reinterpret_cast<const uint4 *>(wq[m] + (int64_t(o) * GH + g) * 32 +
                                                           16 * half);
              sv[m][rr] = ws[m][int64_t(o) * GH + g];
            } else {
              wv[m][rr] = uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
              sv[m][rr] = 0.0f;
            }
          }
        float xs[NT][32], xsum[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const int j = j0 + tt;
          const bool tv = j < U.je;
          const int t = tv ? (U.shared ? j : r.perm[j] / K) : 0;
          xsum[tt] = load_slice(x + int64_t(t) * H, g, half, gv && tv, xs[tt]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int rr = 0; rr < kRB; ++rr) {
            // one row's 32 floats live at a time (see down_decode_kernel)
            uint4 wt = wv[m][rr];
            asm volatile("" : "+v"(wt.x), "+v"(wt.y), "+v"(wt.z), "+v"(wt.w));
            float uf[32];
            unpack32(wt, uf);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
              acc[m][rr][tt] = fmaf(sv[m][rr] * (1.0f / kNibUnit),
                                    dot32(uf, xs[tt]) - (8.0f * kNibUnit) * xsum[tt],
                                    acc[m][rr][tt]);
          }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const float v = wave_sum(acc[m][rr][tt]);
            if (lane == 0) red[wave][m][rr][tt] = v;
          }
      __syncthreads();
      if (threadIdx.x < kRB * NT) {
        const int rr = threadIdx.x / NT, tt = threadIdx.x % NT;
        const int j = j0 + tt, o = o0 + rr;
        if (j < U.je && o < I) {
          float gsum = 0.0f, usum = 0.0f;
          for (int w = 0; w < nw; ++w) {
            gsum += red[w][0][rr][tt];
            usum += red[w][1][rr][tt];
          }
          const int64_t hrow = U.shared ? int64_t(T) * K + j : j;
          h[hrow * I + o] = silu(gsum) * usum;
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down
template <bool kOne>
__global__ __launch_bounds__(kDW * kWave) void down_decode_kernel(
    const float *__restrict__ h, int T, LayerDev L, Routing r, float *__restrict__ y) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int H = L.H, I = L.I, K = L.K;
  const int64_t GI = L.lay.GI;
  const int nch = int((GI + 31) / 32);
  const int r0 = blockIdx.x * kRD;
  const int nu = *r.n_unique + 1;
  const int half = lane & 1;
  __shared__ float yacc[kDW][kRD][kOne ? 1 : COLI_MAX_DECODE_T];
  float lacc[kRD];
#pragma unroll
  for (int rr = 0; rr < kRD; ++rr) lacc[rr] = 0.0f;
  if (!kOne)
    for (int t = lane; t < T; t += kWave)
#pragma unroll
      for (int rr = 0; rr < kRD; ++rr) yacc[wave][rr][t] = 0.0f;

  for (int u = wave; u < nu; u += kDW) {
    const Unit U = unit_of(L, r, u, nu, T);
    const uint8_t *wq = U.blob + L.lay.dq;
    const float *ws = reinterpret_cast<const float *>(U.blob + L.lay.ds);
    for (int c = 0; c < nch; ++c) {
      const int64_t g = int64_t(c) * 32 + lane / 2;
      const bool gv = g < GI;
      uint4 wv[kRD];
      float sv[kRD];
#pragma unroll
      for (int rr = 0; rr < kRD; ++rr) {
        const int o = r0 + rr;
        if (gv && o < H) {
          wv[rr] = *reinterpret_cast<const uint4 *>(wq + (int64_t(o) * GI + g) * 32 + 16 * half);
          sv[rr] = ws[int64_t(o) * GI + g];
        } else {
          wv[rr] = uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
          sv[rr] = 0.0f;
        }
      }
      for (int j = U.jb; j < U.je; ++j) {
        int t;
        float gate;
        int64_t hrow;
        if (U.shared) {
          t = j;
          gate = 1.0f;
          hrow = int64_t(T) * K + j;
        } else {
          const int p = r.perm[j];
          t = p / K;
          gate = r.gates[p];
          hrow = j;
        }
        float hs[32];
        const float hsum = load_slice(h + hrow * I, g, half, gv, hs);
#pragma unroll
        for (int rr = 0; rr < kRD; ++rr) {
          // keep the unpack inside the token loop: hoisting it would hold
          // 32 floats per row live across the loop
          uint4 wt = wv[rr];
          asm volatile("" : "+v"(wt.x), "+v"(wt.y), "+v"(wt.z), "+v"(wt.w));
          float uf[32];
          unpack32(wt, uf);
          const float part =
              sv[rr] * (1.0f / kNibUnit) * (dot32(uf, hs) - (8.0f * kNibUnit) * hsum);
          if (kOne) {
            lacc[rr] = fmaf(gate, part, lacc[rr]);
          } else {
            const float v = wave_sum(part);
            if (lane == 0) yacc[wave][rr][t] += gate * v;
          }
        }
      }
    }
  }
  if (kOne) {
#pragma unroll
    for (int rr = 0; rr < kRD; ++rr) {
      const float v = wave_sum(lacc[rr]);
      if (lane == 0) yacc[wave][rr][0] = v;
    }
  }
  __syncthreads();
  const int tmax = kOne ? 1 : T;
  for (int q = threadIdx.x; q < kRD * tmax; q += blockDim.x) {
    const int rr = q / tmax, t = q % tmax;
    const int o = r0 + rr;
    if (o < H) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kDW; ++w) v += yacc[w][rr][t];
      y[int64_t(t) * H + o] = v;
    }
  }
}

}  // namespace

hipError_t launch_ffn_decode(const LayerDev &L, const float *x, int T,
                             const Routing &r, float *h, float *y,
                             hipStream_t s, hipEvent_t *ev) {
  const int nch = int((L.lay.GH + 31) / 32);
  const int nw = nch < 4 ? nch : 4;
  const int n_rb = (L.I + kRB - 1) / kRB;
  // Upper bound of work items: every unit present.  Blocks beyond the live
  // item count return at once; the loop inside covers any excess.
  const int max_units = (T * L.K < L.E ? T * L.K : L.E) + 1;
  int64_t items = int64_t(max_units) * n_rb;
  const int cap = 8192;
  const unsigned blocks = unsigned(items < cap ? items : cap);
  if (T == 1)
    gateup_decode_kernel<1><<<blocks, nw * kWave, 0, s>>>(x, T, L, r, h);
  else
    gateup_decode_kernel<2><<<blocks, nw * kWave, 0, s>>>(x, T, L, r, h);
  if (ev) (void)hipEventRecord(ev[0], s);
  const unsigned dblocks = unsigned((L.H + kRD - 1) / kRD);
  if (T == 1)
    down_decode_kernel<true><<<dblocks, kDW * kWave, 0, s>>>(h, T, L, r, y);
  else
    down_decode_kernel<false><<<dblocks, kDW * kWave, 0, s>>>(h, T, L, r, y);
  if (ev) (void)hipEventRecord(ev[1], s);
  return hipGetLastError();
}

}  // namespace coli

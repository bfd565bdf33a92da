// ffn_prefill.hip -- the routed + shared expert FFN for large T (prefill):
// int4-g64 grouped GEMMs on the fp16 matrix cores.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 (planar int4-g64 bytes consumed as they are; weight =
// s * (u - 8)); batch union, page "Colibrì 深度解析", section 四 (each unique
// expert is read once per batch and applied to all of its tokens).
//
// Work item = (unit, M-chunk of <= 128 of the unit's tokens, N-tile of 256
// weight rows).  A unit is a unique routed expert of the batch or the shared
// expert.  One block of 4 waves (one per SIMD) per CU walks its items; wave w
// owns 64 weight rows (4 column fragments of 16) and all M fragments of the
// chunk, on v_mfma_f32_16x16x32_f16.
//
// Weight stream.  A super-step covers 256 k = 4 groups = 128 contiguous bytes
// of every weight row.  Per fragment two 16-byte loads per lane cover rows
// 0-7 and 8-15 of the fragment, 8 lanes per row, so each load instruction
// reads 8 whole 128-byte lines (instructions that touch 16 half lines run at
// less than half the HBM rate).  Two DPP half-row moves then give lane
// (q, n) = (lane/16, lane%16) the 16-byte parts 2q and 2q+1 of row n: the two
// halves of group 4*ss + q.  Scales: lane (q, n) loads groups 16i + 4q..+3 of
// row n as one float4 per 4 super-steps; a 4x4 transpose over the lane rows
// (v_permlane32_swap, v_permlane16_swap) hands it the scale of group
// 4*ss + q for each of those super-steps.
//
// Dequant without the -8: for a 32-bit word d of nibbles, (d & 0x000F000F) |
// 0x64006400 is the fp16 pair {1024 + u, 1024 + u'} and (d & 0x00F000F0) |
// 0x54005400 is {64 + u, 64 + u'}; one v_pk_fma_f16 with the pair (s, s) and
// the exact constant -1024 s (or -64 s) gives s*u rounded once.  The -8 of
// the code is folded into a correction GEMM: out -= 8 * sum_g s[n][g] *
// S[m][g], S = per-group sums of the fp16 activations, held as fp16 hi + lo
// pairs, run on the same MFMAs as extra k steps (one per 16 groups).
//
// K order.  Word s (0..3) of half t (0, 1) of a group holds elements
// o + {0, 2, 32, 34, 1, 3, 33, 35} with o = 16t + 4s, in that order after
// the extraction above.  The activations are stored (fp16) in the matching
// order, so an MFMA A operand is one contiguous 16-byte run: inside each
// 256-k block, position 128t + 32q + 8s + i holds element 16t + 4s + sigma[i]
// of group 4*block + q, sigma = {0, 2, 32, 34, 1, 3, 33, 35}.  Rows are
// padded to whole 256-k blocks; the padding holds zeros.
//
// Numerics: fp16 operands, fp32 accumulation.  Activations must lie in fp16
// range and scales below 64 (|w| < 448).
//
// Kernels: pf_prep (x bf16 -> fp16 staged copy + group sums), pf_hpad (zero
// the padding of the h rows), prefill_tiles (M-chunk prefix over units),
// pf_gemm<true> (h = SiLU(gate) * up, fp16, staged order, + its group sums),
// pf_gemm<false> (gate-scaled per-slot outputs, fp16), combine (y = sum of a
// token's slots + its shared output, bf16).
#include "kernels.h"

#include <hip/hip_fp16.h>

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                      // one per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kMC = 128;                       // tokens per M-chunk
constexpr int kCorrOff = 512;                  // correction operand inside a staged row
constexpr int kPitch = 512 + 64 + 16;          // LDS bytes per staged row
constexpr int kStage = kMC * kPitch;
constexpr int kLdsRowIdx = 2 * kStage;            // int[kMC]  A / S row of each chunk row
constexpr int kLdsOutRow = kLdsRowIdx + kMC * 4;  // int[kMC]  output row
constexpr int kLdsGate = kLdsOutRow + kMC * 4;    // float[kMC] gate (down)
constexpr int kLdsRed = kLdsGate + kMC * 4;       // float[kWaves][kMC] (gate/up)
constexpr int kLdsBytes = kLdsRed + kWaves * kMC * 4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack_f16x2(_Float16 a, _Float16 b) {
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Position of element e (0..63) of group g in a staged activation row.
__device__ inline int act_pos(int g, int e) {
  const int t = (e >> 4) & 1, s = (e >> 2) & 3;
  const int i = ((e & 1) << 2) | (((e >> 5) & 1) << 1) | ((e >> 1) & 1);
  return (g >> 2) * 256 + t * 128 + (g & 3) * 32 + s * 8 + i;
}

// hi + lo fp16 pair of a float (hi = fp16(v), lo = fp16(v - hi)).
__device__ inline uint32_t split_f16(float v) {
  const _Float16 hi = _Float16(v);
  const _Float16 lo = _Float16(v - float(hi));
  return pack_f16x2(hi, lo);
}

// ------------------------------------------------------------------ prep
// x bf16 [T, H] -> xp fp16 [T, HP] in the staged order, zero padding, and
// sx [T, CSX]: the hi/lo fp16 pair of each group's sum of the fp16 values.
// Thread = (token, group slot g < HP/64, 8-position run c); the 8 threads of
// a group are consecutive lanes.
__global__ __launch_bounds__(256) void pf_prep(const uint16_t *__restrict__ x, int T, int H,
                                               int HP, int CSX, uint16_t *__restrict__ xp,
                                               uint16_t *__restrict__ sx) {
  const int G = H / 64, GP = HP / 64;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int c = int(i & 7);
  const int64_t tg = i >> 3;
  if (tg >= int64_t(T) * GP) return;  // whole groups of 8 lanes leave together
  const int t = int(tg / GP), g = int(tg % GP);
  const int tt = c >> 2, s = c & 3, o = 16 * tt + 4 * s;
  uint4 out = uint4{0u, 0u, 0u, 0u};
  float sum = 0.0f;
  if (g < G) {
    const uint16_t *src = x + int64_t(t) * H + 64 * g + o;
    const uint2 lo = *reinterpret_cast<const uint2 *>(src);
    const uint2 hi = *reinterpret_cast<const uint2 *>(src + 32);
    // b = elements o + {0, 1, 2, 3, 32, 33, 34, 35}
    const uint16_t b[8] = {uint16_t(lo.x), uint16_t(lo.x >> 16), uint16_t(lo.y),
                           uint16_t(lo.y >> 16), uint16_t(hi.x), uint16_t(hi.x >> 16),
                           uint16_t(hi.y), uint16_t(hi.y >> 16)};
    // staged order o + {0, 2, 32, 34, 1, 3, 33, 35}
    const int ord[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    _Float16 h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      h[k] = _Float16(__uint_as_float(uint32_t(b[ord[k]]) << 16));
      sum += float(h[k]);
    }
    out = uint4{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3]), pack_f16x2(h[4], h[5]),
                pack_f16x2(h[6], h[7])};
  }
  sum += __shfl_xor(sum, 1, 8);
  sum += __shfl_xor(sum, 2, 8);
  sum += __shfl_xor(sum, 4, 8);
  *reinterpret_cast<uint4 *>(xp + int64_t(t) * HP + (g >> 2) * 256 + tt * 128 + (g & 3) * 32 +
                             s * 8) = out;
  if (c == 0 && g < G)
    *reinterpret_cast<uint32_t *>(sx + int64_t(t) * CSX + 2 * g) = split_f16(sum);
}

// Zero the padding groups (G..GP-1, all in the last 256-k block) of every h row.
__global__ __launch_bounds__(256) void pf_hpad(uint16_t *__restrict__ h, int64_t rows, int G,
                                               int IP) {
  const int GP = IP / 64, per_row = (GP - G) * 8;  // 8 runs of 16 B per group
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t row = i / per_row;
  const int k = int(i % per_row), g = G + k / 8, c = k % 8;
  *reinterpret_cast<uint4 *>(h + row * IP + (g >> 2) * 256 + (c >> 2) * 128 + (g & 3) * 32 +
                             (c & 3) * 8) = uint4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ tiles
// chunk[u] = number of M-chunks of units < u; chunk[nu] = total.  Unit u <
// n_unique is routed expert unique[u]; unit n_unique is the shared expert.
__global__ __launch_bounds__(1024) void prefill_tiles(Routing r, int T) {
  __shared__ int wave_tot[16];
  const int u = threadIdx.x;
  const int nu = *r.n_unique + 1;
  int c = 0;
  for (int base = 0; base < nu; base += 1024) {
    const int uu = base + u;
    int n = 0;
    if (uu < nu) n = (uu < nu - 1) ? r.counts[r.unique[uu]] : T;
    const int v = (n + kMC - 1) / kMC;
    const int lane = u % kWave, wave = u / kWave;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    int all = 0;
    for (int w = 0; w < 16; ++w) all += wave_tot[w];
    if (uu < nu) r.chunk[uu] = c + before + inc - v;
    __syncthreads();
    c += all;
  }
  if (u == 0) r.chunk[nu] = c;
}

// Item decode shared by the two GEMMs.
struct Item {
  int unit, mchunk, ntile;
  bool shared;
  const uint8_t *blob;
  int jb, je;  // token rows of the chunk: j in [jb, je)
};
__device__ inline void decode_item(const LayerDev &L, const Routing &r, int T, int item, int n_nt,
                                   Item &it) {
  const int nu = *r.n_unique + 1;
  const int c = item / n_nt;
  it.ntile = item % n_nt;
  int lo = 0, hi = nu - 1;  // last u with chunk[u] <= c
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (r.chunk[mid] <= c) lo = mid; else hi = mid - 1;
  }
  it.unit = lo;
  it.mchunk = c - r.chunk[lo];
  it.shared = lo == nu - 1;
  int jb0, je0;
  if (!it.shared) {
    const int e = r.unique[lo];
    it.blob = L.experts + size_t(e) * L.lay.bytes;
    jb0 = r.offsets[e];
    je0 = r.offsets[e + 1];
  } else {
    it.blob = L.shared;
    jb0 = 0;
    je0 = T;
  }
  it.jb = jb0 + it.mchunk * kMC;
  it.je = min(je0, it.jb + kMC);
}

struct PfArgs {
  const uint16_t *A;  // staged activations, row stride AP (elements)
  const uint16_t *S;  // group-sum pairs, row stride CS
  uint16_t *out;      // gate/up: h (row stride OP); down: slot (row stride OP = H)
  uint16_t *sout;     // gate/up: sh (row stride SOP)
  int AP, CS, OP, SOP;
  uint32_t a_bytes, s_bytes;  // sizes of A and S (< 2^31)
};

// m1 = 0x000F000F, m2 = 0x00F000F0 held in VGPRs: gfx9 VOP3 takes no literal
// and one scalar operand, so this keeps each extraction one v_and_or_b32.
__device__ inline f16x8 dequant(uint32_t d, uint32_t m1, uint32_t m2, f16x2 s2, f16x2 c10,
                                f16x2 c6) {
  const uint32_t d8 = d >> 8;
  const f16x2 p0 = __builtin_bit_cast(f16x2, (d & m1) | 0x64006400u);
  const f16x2 p1 = __builtin_bit_cast(f16x2, (d & m2) | 0x54005400u);
  const f16x2 p2 = __builtin_bit_cast(f16x2, (d8 & m1) | 0x64006400u);
  const f16x2 p3 = __builtin_bit_cast(f16x2, (d8 & m2) | 0x54005400u);
  const f16x2 r0 = __builtin_elementwise_fma(p0, s2, c10);
  const f16x2 r1 = __builtin_elementwise_fma(p1, s2, c6);
  const f16x2 r2 = __builtin_elementwise_fma(p2, s2, c10);
  const f16x2 r3 = __builtin_elementwise_fma(p3, s2, c6);
  return f16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

__device__ inline uint32_t word_of(const uint4 &v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// sum over the 16 lanes of each lane row; the total lands in lane 15 of the row
__device__ inline float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
  return v;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// Buffer resource over [p, p + bytes): raw buffer loads at offsets >= bytes
// return zeros, so masked lanes take the offset kOff and no branch.
constexpr uint32_t kOff = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, int(bytes), 0x00020000);
}
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return uint4{uint32_t(v[0]), uint32_t(v[1]), uint32_t(v[2]), uint32_t(v[3])};
}
__device__ inline float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, uint32_t(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0)));
}

// One work item.  NMF = number of 16-row M fragments the chunk needs.  The
// chunk's row tables are in LDS (see pf_gemm).
template <bool kGateUp, int NMF>
__device__ __attribute__((always_inline)) inline void run_item(const LayerDev &L, const PfArgs &pa,
                                                               const Item &it, uint8_t *lds) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int q = lane >> 4, n16 = lane & 15;
  const int *rowidx_s = reinterpret_cast<const int *>(lds + kLdsRowIdx);
  const int G = int(kGateUp ? L.lay.GH : L.lay.GI);
  const int nss = (G + 3) >> 2;
  const uint32_t rowB = uint32_t(G) * 32u;
  const int nrows = it.je - it.jb;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(it.blob, uint32_t(L.lay.bytes));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(pa.A, pa.a_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(pa.S, pa.s_bytes);

  // weight rows of this wave (all valid or all past the matrix: 64 | rows)
  int wrow0;
  bool wvalid;
  if (kGateUp) {
    wrow0 = it.ntile * 128 + 32 * wave;
    wvalid = wrow0 < L.I;
  } else {
    wrow0 = it.ntile * 256 + 64 * wave;
    wvalid = wrow0 < L.H;
  }
  uint32_t xoff[4], soff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int row;
    uint32_t qsec, ssec;
    if (kGateUp) {
      row = wrow0 + 16 * (j & 1);
      qsec = uint32_t(j < 2 ? L.lay.gq : L.lay.uq);
      ssec = uint32_t(j < 2 ? L.lay.gs : L.lay.us);
    } else {
      row = wrow0 + 16 * j;
      qsec = uint32_t(L.lay.dq);
      ssec = uint32_t(L.lay.ds);
    }
    // load lane (a, b) = (q, n16): row b % 8 (+8 for the second load), part 2a + b/8.
    // In the last super-step lanes past G read the next bytes of the blob (a q
    // section is always followed by another section); their scale is 0.
    xoff[j] = qsec + uint32_t(row + (n16 & 7)) * rowB + 16u * uint32_t(2 * q + (n16 >> 3));
    soff[j] = ssec + uint32_t(row + n16) * uint32_t(G) * 4u + 16u * uint32_t(q);
  }

  // activation staging: run c16 of rows mrow + 16p; correction run c4 of rows crow + 64p
  const int c16 = threadIdx.x & 15, mrow = threadIdx.x >> 4;
  const int c4 = threadIdx.x & 3, crow = threadIdx.x >> 2;
  uint32_t aoff[8], coff[2];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int ri = rowidx_s[mrow + 16 * p];
    aoff[p] = ri >= 0 ? (uint32_t(ri) * uint32_t(pa.AP) + 8u * uint32_t(c16)) * 2u : kOff;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ri = rowidx_s[crow + 64 * p];
    coff[p] = ri >= 0 ? (uint32_t(ri) * uint32_t(pa.CS) + 8u * uint32_t(c4)) * 2u : kOff;
  }

  auto load_a = [&](int ss, int hh, uint4(&v)[8]) {
#pragma unroll
    for (int p = 0; p < 8; ++p) v[p] = bload16(ra, aoff[p], uint32_t(512 * ss + 256 * hh));
  };
  auto store_a = [&](int buf, int hh, const uint4(&v)[8]) {
    uint8_t *base = lds + buf * kStage + 256 * hh + 16 * c16;
#pragma unroll
    for (int p = 0; p < 8; ++p) *reinterpret_cast<uint4 *>(base + (mrow + 16 * p) * kPitch) = v[p];
  };
  // correction operand of block i: entries 32i + 8 c4 .. +7 = groups 16i + 4 c4 + d (hi, lo)
  auto load_c = [&](int i, uint4(&v)[2]) {
    const int g0 = 16 * i + 4 * c4;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint4 w = bload16(rs, coff[p], uint32_t(64 * i));
      if (g0 + 0 >= G) w.x = 0u;
      if (g0 + 1 >= G) w.y = 0u;
      if (g0 + 2 >= G) w.z = 0u;
      if (g0 + 3 >= G) w.w = 0u;
      v[p] = w;
    }
  };
  auto store_c = [&](int buf, const uint4(&v)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<uint4 *>(lds + buf * kStage + (crow + 64 * p) * kPitch + kCorrOff +
                                 16 * c4) = v[p];
  };
  auto load_b = [&](int ss, uint4(&x)[4], uint4(&y)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = bload16(rw, xoff[j], 128u * uint32_t(ss));
      y[j] = bload16(rw, xoff[j], 128u * uint32_t(ss) + 8u * rowB);
    }
  };
  // scales of groups 16i + 4q + c (c = 0..3) of the lane's row; 0 past G
  auto load_f = [&](int i, f32x4(&f)[4]) {
    const int g0 = 16 * i + 4 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = soff[j] + 64u * uint32_t(i);
      f32x4 v;
      if ((G & 3) == 0) {
        const uint4 w = bload16(rw, g0 < G ? o : kOff, 0);
        v = f32x4{__builtin_bit_cast(float, w.x), __builtin_bit_cast(float, w.y),
                  __builtin_bit_cast(float, w.z), __builtin_bit_cast(float, w.w)};
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = bload4f(rw, g0 + c < G ? o + 4u * c : kOff);
      }
      f[j] = v;
    }
  };

  f32x4 acc[NMF][4];
#pragma unroll
  for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mf][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: scales of block 0, weights and staged activations of super-step 0
  // (zero-initialised: waves past the matrix never load them)
  f32x4 F[4] = {};
  uint4 bxr[4] = {}, byr[4] = {};
  if (wvalid) {
    load_f(0, F);
    load_b(0, bxr, byr);
  }
  {
    uint4 v[8], cv[2];
    load_a(0, 0, v);
    load_c(0, cv);
    store_a(0, 0, v);
    store_c(0, cv);
    load_a(0, 1, v);
    store_a(0, 1, v);
  }
  __syncthreads();

  float Ft[4][4] = {};
  for (int ss = 0; ss < nss; ++ss) {
    const int buf = ss & 1;
    const bool more = ss + 1 < nss;
    const uint8_t *stage = lds + buf * kStage;
    uint4 av[8];
    if (more) load_a(ss + 1, 0, av);
    if (wvalid) {
      // this super-step's weights into MFMA lane order; refill the raw slot
      uint4 bx[4], by[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t xs[4] = {bxr[j].x, bxr[j].y, bxr[j].z, bxr[j].w};
        const uint32_t ys[4] = {byr[j].x, byr[j].y, byr[j].z, byr[j].w};
        uint32_t xo[4], yo[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // lanes 8..15 of each row take the other load's lanes 0..7, and back
          xo[d] = uint32_t(__builtin_amdgcn_update_dpp(int(xs[d]), int(ys[d]), 0x118, 0xF, 0xC, false));
          yo[d] = uint32_t(__builtin_amdgcn_update_dpp(int(ys[d]), int(xs[d]), 0x108, 0xF, 0x3, false));
        }
        bx[j] = uint4{xo[0], xo[1], xo[2], xo[3]};
        by[j] = uint4{yo[0], yo[1], yo[2], yo[3]};
      }
      if (more) load_b(ss + 1, bxr, byr);
      if ((ss & 3) == 0) {
        // correction GEMM of block i = ss / 4: acc += S (hi, lo) x (-8 s, -8 s)
        f16x8 bc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const _Float16 h0 = _Float16(F[j][0]) * _Float16(-8.0f);
          const _Float16 h1 = _Float16(F[j][1]) * _Float16(-8.0f);
          const _Float16 h2 = _Float16(F[j][2]) * _Float16(-8.0f);
          const _Float16 h3 = _Float16(F[j][3]) * _Float16(-8.0f);
          bc[j] = f16x8{h0, h0, h1, h1, h2, h2, h3, h3};
        }
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
          const f16x8 a = *reinterpret_cast<const f16x8 *>(stage + (mf * 16 + n16) * kPitch +
                                                           kCorrOff + 16 * q);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[mf][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bc[j], acc[mf][j], 0, 0, 0);
        }
        // 4x4 transpose over the lane rows: Ft[j][c] = scale of group 16i + 4c + q
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // elements read by value first: this compiler's SROA folds a bit_cast
          // of an ext_vector element lvalue to element 0
          const uint32_t r0 = __float_as_uint(float(F[j][0]));
          const uint32_t r1 = __float_as_uint(float(F[j][1]));
          const uint32_t r2 = __float_as_uint(float(F[j][2]));
          const uint32_t r3 = __float_as_uint(float(F[j][3]));
          const auto p02 = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
          const auto p13 = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
          const auto p01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
          const auto p23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
          Ft[j][0] = __builtin_bit_cast(float, uint32_t(p01[0]));
          Ft[j][1] = __builtin_bit_cast(float, uint32_t(p01[1]));
          Ft[j][2] = __builtin_bit_cast(float, uint32_t(p23[0]));
          Ft[j][3] = __builtin_bit_cast(float, uint32_t(p23[1]));
        }
        if (ss + 4 < nss) load_f((ss >> 2) + 1, F);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Ft[j][0] = Ft[j][1];
          Ft[j][1] = Ft[j][2];
          Ft[j][2] = Ft[j][3];
        }
      }
      f16x2 s2[4], c10[4], c6[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 h = _Float16(Ft[j][0]);
        s2[j] = f16x2{h, h};
        c10[j] = s2[j] * f16x2{_Float16(-1024.0f), _Float16(-1024.0f)};
        c6[j] = s2[j] * f16x2{_Float16(-64.0f), _Float16(-64.0f)};
      }
      // 8 MFMA steps k = 4t + s; the weights of step k + 1 are dequantised and
      // its A fragments read while the MFMAs of step k run
      uint32_t m1, m2;
      asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m1));
      asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(m2));
      const uint8_t *abase = stage + n16 * kPitch + 64 * q;
      f16x8 a[NMF], b[4];
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
        a[mf] = *reinterpret_cast<const f16x8 *>(abase + mf * 16 * kPitch);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = dequant(bx[j].x, m1, m2, s2[j], c10[j], c6[j]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t1 = (k + 1) >> 2, s1 = (k + 1) & 3;
        f16x8 bn[4];
        if (k < 7) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bn[j] = dequant(word_of(t1 ? by[j] : bx[j], s1), m1, m2, s2[j], c10[j], c6[j]);
        }
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[mf][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mf], b[j], acc[mf][j], 0, 0, 0);
          // refill the fragment for step k + 1 as soon as step k is done with it
          if (k < 7)
            a[mf] = *reinterpret_cast<const f16x8 *>(abase + mf * 16 * kPitch + 256 * t1 + 16 * s1);
        }
        if (k == 3 && more) {
          store_a(buf ^ 1, 0, av);
          load_a(ss + 1, 1, av);
        }
        if (k < 7) {
#pragma unroll
          for (int j = 0; j < 4; ++j) b[j] = bn[j];
        }
      }
      if (more) {
        store_a(buf ^ 1, 1, av);
        if (((ss + 1) & 3) == 0) {
          uint4 cv[2];
          load_c((ss + 1) >> 2, cv);
          store_c(buf ^ 1, cv);
        }
      }
    } else if (more) {
      // rows past the matrix: staging only
      store_a(buf ^ 1, 0, av);
      load_a(ss + 1, 1, av);
      store_a(buf ^ 1, 1, av);
      if (((ss + 1) & 3) == 0) {
        uint4 cv[2];
        load_c((ss + 1) >> 2, cv);
        store_c(buf ^ 1, cv);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds rows m = 16 mf + 4 q + i of column n16 of each fragment
  const int *outrow_s = reinterpret_cast<const int *>(lds + kLdsOutRow);
  if (kGateUp) {
    float *red_s = reinterpret_cast<float *>(lds + kLdsRed);
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mf * 16 + 4 * q + i;
        float part = 0.0f;
        if (wvalid && m < nrows) {
          const int64_t hrow = outrow_s[m];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int f = wrow0 + 16 * jj + n16;
            const _Float16 hv = _Float16(silu(acc[mf][jj][i]) * acc[mf][jj + 2][i]);
            pa.out[hrow * pa.OP + act_pos(f >> 6, f & 63)] = __builtin_bit_cast(uint16_t, hv);
            part += float(hv);
          }
        }
        part = row16_sum(part);
        if (n16 == 15) red_s[wave * kMC + m] = part;
      }
    }
    __syncthreads();
    // group sums of h: waves 2g' and 2g'+1 hold the halves of group 2 ntile + g'
    const int m = threadIdx.x & (kMC - 1), gsel = threadIdx.x >> 7;
    const int g = it.ntile * 2 + gsel;
    if (m < nrows && m < NMF * 16 && 64 * g < L.I) {
      const float sum = red_s[(2 * gsel) * kMC + m] + red_s[(2 * gsel + 1) * kMC + m];
      *reinterpret_cast<uint32_t *>(pa.sout + int64_t(outrow_s[m]) * pa.SOP + 2 * g) =
          split_f16(sum);
    }
  } else {
    const float *gate_s = reinterpret_cast<const float *>(lds + kLdsGate);
    if (wvalid) {
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mf * 16 + 4 * q + i;
          if (m >= nrows) continue;
          const int64_t srow = outrow_s[m];
          const float gate = gate_s[m];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = wrow0 + 16 * j + n16;
            pa.out[srow * pa.OP + n] = __builtin_bit_cast(uint16_t, _Float16(gate * acc[mf][j][i]));
          }
        }
      }
    }
  }
}

// Persistent grouped GEMM: blocks walk (chunk, N-tile) items.  With a grid
// that is a multiple of 8 the items are split into 8 contiguous ranges, one
// per XCD (the hardware deals consecutive blocks round-robin over the 8 XCDs),
// so the N-tiles of one chunk, which share its activations, meet in one L2.
template <bool kGateUp>
__global__ __launch_bounds__(kThreads, 1) void pf_gemm(LayerDev L, Routing r, int T, PfArgs pa) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int *rowidx_s = reinterpret_cast<int *>(lds + kLdsRowIdx);
  int *outrow_s = reinterpret_cast<int *>(lds + kLdsOutRow);
  float *gate_s = reinterpret_cast<float *>(lds + kLdsGate);
  const int K = L.K;
  const int n_nt = kGateUp ? (L.I + 127) / 128 : (L.H + 255) / 256;
  const int nu = *r.n_unique + 1;
  const int n_items = r.chunk[nu] * n_nt;
  int it0, it1, step;
  if ((gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7, nb = gridDim.x >> 3;
    it0 = int(int64_t(n_items) * xcd / 8) + int(blockIdx.x >> 3);
    it1 = int(int64_t(n_items) * (xcd + 1) / 8);
    step = nb;
  } else {
    it0 = blockIdx.x;
    it1 = n_items;
    step = gridDim.x;
  }
  for (int item = it0; item < it1; item += step) {
    Item it;
    decode_item(L, r, T, item, n_nt, it);
    // the item is the same for every lane: keep it in scalar registers
    {
      const uint64_t bp = reinterpret_cast<uint64_t>(it.blob);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(bp));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(bp >> 32));
      it.blob = reinterpret_cast<const uint8_t *>((uint64_t(hi) << 32) | lo);
      it.ntile = __builtin_amdgcn_readfirstlane(it.ntile);
      it.jb = __builtin_amdgcn_readfirstlane(it.jb);
      it.je = __builtin_amdgcn_readfirstlane(it.je);
      it.shared = __builtin_amdgcn_readfirstlane(int(it.shared)) != 0;
    }
    __syncthreads();  // the previous item is done with the row tables
    if (threadIdx.x < kMC) {
      const int j = it.jb + threadIdx.x;
      int ri = -1, orow = 0;
      float gate = 0.0f;
      if (j < it.je) {
        if (kGateUp) {
          ri = it.shared ? j : r.perm[j] / K;
          orow = it.shared ? T * K + j : j;
        } else {
          ri = it.shared ? T * K + j : j;
          if (it.shared) {
            orow = T * K + j;
            gate = 1.0f;
          } else {
            const int p = r.perm[j];
            orow = p;
            gate = r.gates[p];
          }
        }
      }
      rowidx_s[threadIdx.x] = ri;
      outrow_s[threadIdx.x] = orow;
      gate_s[threadIdx.x] = gate;
    }
    __syncthreads();
    const int nmf = (it.je - it.jb + 15) / 16;
    switch (nmf) {
      case 1: run_item<kGateUp, 1>(L, pa, it, lds); break;
      case 2: run_item<kGateUp, 2>(L, pa, it, lds); break;
      case 3: run_item<kGateUp, 3>(L, pa, it, lds); break;
      case 4: run_item<kGateUp, 4>(L, pa, it, lds); break;
      case 5: run_item<kGateUp, 5>(L, pa, it, lds); break;
      case 6: run_item<kGateUp, 6>(L, pa, it, lds); break;
      case 7: run_item<kGateUp, 7>(L, pa, it, lds); break;
      default: run_item<kGateUp, 8>(L, pa, it, lds); break;
    }
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + ((u >> 16) & 1u) + 0x7FFFu) >> 16);
}

// y[t] = sum_k slot[t*K + k] + slot[T*K + t]   (fp16 slots, fp32 sum, bf16 y;
// 8 columns per thread)
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ slot, int T,
                                                      int H, int K, uint16_t *__restrict__ y) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = H / 8;
  if (i >= int64_t(T) * per_row) return;
  const int t = int(i / per_row), c = int(i % per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k <= K; ++k) {
    const int64_t row = k < K ? int64_t(t) * K + k : int64_t(T) * K + t;
    const uint4 v = *reinterpret_cast<const uint4 *>(slot + row * H + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16x2 hv = __builtin_bit_cast(f16x2, w[q]);
      acc[2 * q] += float(hv[0]);
      acc[2 * q + 1] += float(hv[1]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = uint32_t(f32_to_bf16_rne(acc[2 * q])) |
           (uint32_t(f32_to_bf16_rne(acc[2 * q + 1])) << 16);
  *reinterpret_cast<uint4 *>(y + int64_t(t) * H + c) = uint4{o[0], o[1], o[2], o[3]};
}

int cus_of_device() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  return n;
}

template <bool kGateUp>
hipError_t launch_gemm(const LayerDev &L, const Routing &r, int T, const PfArgs &pa,
                       int64_t max_items, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&pf_gemm<kGateUp>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  const int64_t cus = cus_of_device();
  const int64_t grid = max_items < cus ? max_items : cus;
  pf_gemm<kGateUp><<<dim3(unsigned(grid)), dim3(kThreads), kLdsBytes, s>>>(L, r, T, pa);
  return hipGetLastError();
}

}  // namespace

PrefillLayout prefill_layout(int H, int I) {
  PrefillLayout p;
  const int64_t GH = groups_of(H), GI = groups_of(I);
  p.HP = int(256 * ((GH + 3) / 4));
  p.IP = int(256 * ((GI + 3) / 4));
  p.CSX = int(32 * ((GH + 15) / 16));
  p.CSI = int(32 * ((GI + 15) / 16));
  return p;
}

hipError_t launch_ffn_prefill(const LayerDev &L, const uint16_t *x, int T, const Routing &r,
                              const PrefillBufs &b, uint16_t *y, hipStream_t s, hipEvent_t *ev) {
  const PrefillLayout pl = prefill_layout(L.H, L.I);
  const int64_t TK = int64_t(T) * L.K;
  // buffer-resource offsets are 32-bit with the top bit reserved for masking
  if (int64_t(T) * pl.HP * 2 >= (int64_t(1) << 31) || (TK + T) * pl.IP * 2 >= (int64_t(1) << 31) ||
      L.lay.bytes >= (size_t(1) << 31))
    return hipErrorInvalidValue;
  if (ev) (void)hipEventRecord(ev[0], s);
  {
    const int64_t n = int64_t(T) * (pl.HP / 64) * 8;
    pf_prep<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(x, T, L.H, pl.HP, pl.CSX, b.xp, b.sx);
  }
  if (L.I % 256) {
    const int64_t n = (TK + T) * ((pl.IP - L.I) / 64) * 8;
    pf_hpad<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(b.h, TK + T, L.I / 64, pl.IP);
  }
  prefill_tiles<<<1, 1024, 0, s>>>(r, T);
  if (ev) (void)hipEventRecord(ev[1], s);
  const int max_units = int((TK < L.E ? TK : L.E) + 1);
  // sum over units of ceil(n_u / kMC) <= TK / kMC + routed units + shared chunks
  const int64_t max_chunks = TK / kMC + max_units + (T + kMC - 1) / kMC;
  hipError_t e;
  if (ev) (void)hipEventRecord(ev[2], s);
  {
    PfArgs pa{b.xp, b.sx, b.h, b.sh, pl.HP, pl.CSX, pl.IP, pl.CSI,
              uint32_t(int64_t(T) * pl.HP * 2), uint32_t(int64_t(T) * pl.CSX * 2)};
    e = launch_gemm<true>(L, r, T, pa, max_chunks * ((L.I + 127) / 128), s);
    if (e != hipSuccess) return e;
  }
  if (ev) (void)hipEventRecord(ev[3], s);
  if (ev) (void)hipEventRecord(ev[4], s);
  {
    PfArgs pa{b.h, b.sh, b.slot, nullptr, pl.IP, pl.CSI, L.H, 0,
              uint32_t((TK + T) * pl.IP * 2), uint32_t((TK + T) * pl.CSI * 2)};
    e = launch_gemm<false>(L, r, T, pa, max_chunks * ((L.H + 255) / 256), s);
    if (e != hipSuccess) return e;
  }
  if (ev) (void)hipEventRecord(ev[5], s);
  const int64_t nthr = int64_t(T) * (L.H / 8);
  if (ev) (void)hipEventRecord(ev[6], s);
  combine_kernel<<<dim3(unsigned((nthr + 255) / 256)), 256, 0, s>>>(b.slot, T, L.H, L.K, y);
  if (ev) (void)hipEventRecord(ev[7], s);
  return hipGetLastError();
}

}  // namespace coli

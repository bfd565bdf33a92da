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
// expert.  One block of 8 waves (two per SIMD) per CU walks its items; each
// wave owns one 32-row weight fragment (gate or up rows of the same 32
// features; or 32 down rows) and all 32-row M fragments of the chunk, on
// v_mfma_f32_32x32x16_f16 (on gfx950 the 16x16x32 form needs far more
// independent accumulators per wave to approach the matrix-core rate).  The
// two waves on a SIMD share the block's activation stage, so one wave's
// dequant and exchange VALU work runs beside the other's MFMAs.
//
// Weight stream.  A super-step covers 256 k = 4 groups = 128 contiguous bytes
// of every weight row.  Per 32-row fragment four 16-byte loads per lane, load a
// covering rows 8a..8a+7 with 8 lanes per row (each load instruction reads 8
// whole 128-byte lines); lane (h, n) = (lane/32, lane%32) of load a takes row
// 8a + n%8, part 4h + n/8.  A 4x4 exchange between the load index and lane
// bits 3-4 (DPP half-row moves, then v_permlane16_swap) leaves part 4h + d of
// row n in register d: lane (h, n) holds groups 2h, 2h+1 of the super-step.
// Scales: lane (h, n) loads groups 16i + 8h .. +7 of row n as two float4 per 4
// super-steps; v_permlane32_swap between lane halves regroups them so that the
// lane holds groups 4c + 2h, 4c + 2h + 1 for each super-step c of the block.
// Depth: with up to 3 M fragments the weights of super-step ss + 2 are issued
// at the end of super-step ss, after its last DMA, and stay in flight across
// the barrier (vmcnt(8) and a fence-free s_barrier); with 4 fragments the
// registers allow one super-step, issued one load per MFMA step.
//
// Dequant without the -8: for a 32-bit word d of nibbles, (d & 0x000F000F) |
// 0x64006400 is the fp16 pair {1024 + u, 1024 + u'} and (d & 0x00F000F0) |
// 0x54005400 is {64 + u, 64 + u'}; one v_pk_fma_f16 with the pair (s, s) and
// the exact constant -1024 s (or -64 s) gives s*u rounded once.  The -8 of
// the code is folded into a correction GEMM: out -= 8 * sum_g s[n][g] *
// S[m][g], S = per-group sums of the fp16 activations, held as fp16 hi + lo
// pairs, run on the same MFMAs as extra k steps (two per 16 groups).
//
// K order.  Word w (0..3) of half t (0, 1) of a group holds elements
// o + {0, 2, 32, 34, 1, 3, 33, 35} with o = 16t + 4w, in that order after the
// extraction above; it feeds MFMA k-step 8 (g & 1) + 4t + w of its super-step,
// k-half (g & 3) / 2.  The activations are stored (fp16) with every 64-group
// contiguous in the matching order: position 8(4t + w) + i of group g holds
// element 16t + 4w + sigma[i], sigma = {0, 2, 32, 34, 1, 3, 33, 35}, so an MFMA
// A operand is one 16-byte run.  Rows are padded to whole 4-group blocks; the
// padding holds zeros.
//
// Numerics: fp16 operands, fp32 accumulation.  Each token's activations are
// scaled by a power of two 2^-e (the row's largest |x| then lies in [2, 4))
// before the fp16 conversion, and its h by 2^-2e, so rows of any magnitude
// keep fp16 precision; the combine multiplies y back by 2^2e.  Group scales
// must stay below 64 (|w| < 448) for the -1024 s constant; an fp16 operand
// that would overflow (h or a slot output) raises COLI_STATUS_RANGE.
//
// Kernels: pf_prep (x bf16 -> fp16 staged copy + group sums), pf_pads (zero
// the padding of the h and h-sum rows), prefill_tiles (M-chunk prefix over units),
// pf_gemm<true> (h = SiLU(gate) * up, fp16, staged order, + its group sums),
// pf_gemm<false> (gate-scaled per-slot outputs, fp16), combine (y = sum of a
// token's slots + its shared output, bf16).
#include "gemm_stream.h"
#include "kernels.h"
#include "wave.h"

#include <hip/hip_fp16.h>

namespace coli {
namespace {

constexpr int kMC = 128;                       // tokens per M-chunk
constexpr int kStageB = kMC * kRowB;           // one activation stage
constexpr int kCorrB = kMC * 64;               // one correction-operand stage

// hi + lo fp16 pair of a float (hi = fp16(v), lo = fp16(v - hi)).
__device__ inline uint32_t split_f16(float v) {
  const _Float16 hi = _Float16(v);
  const _Float16 lo = _Float16(v - float(hi));
  return pack_f16x2(hi, lo);
}

// ------------------------------------------------------------------ prep
// One block per token: x bf16 [T, H] (any H, any alignment) -> xp fp16 [T, HP]
// in the staged order with zero padding, scaled by 2^-e (e chosen from the
// row's largest |x| so that it lies in [2, 4)), and sx [T, CSX]: the hi/lo
// fp16 pair of each group's sum of the scaled fp16 values.  xe[t] = e.  A
// non-finite x raises COLI_STATUS_NONFINITE; a scaled value beyond the fp16
// range cannot occur (the row's largest is below 4).
// Thread = (group g, 8-position run c) slots of the row, strided by 256.
__global__ __launch_bounds__(256) void pf_prep(const uint16_t *__restrict__ x, int T, int H,
                                               int HP, int CSX, uint16_t *__restrict__ xp,
                                               uint16_t *__restrict__ sx, int *__restrict__ xe,
                                               int32_t *status) {
  __shared__ float red[4];
  __shared__ int rbad[4];
  const int t = blockIdx.x;
  const int G = (H + 63) / 64, GP = HP / 64;
  const uint16_t *row = x + int64_t(t) * H;
  // the row's largest |x| (bit patterns: NaN > Inf > every finite value)
  uint32_t mb = 0;
  for (int i = threadIdx.x; i < H; i += 256) mb = max(mb, uint32_t(row[i]) & 0x7FFFu);
  const uint32_t wm = wave_max_u32(mb);
  if (threadIdx.x % 64 == 0) {
    red[threadIdx.x / 64] = __uint_as_float(wm << 16);
    rbad[threadIdx.x / 64] = wm >= 0x7F80u;
  }
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool bad = rbad[0] | rbad[1] | rbad[2] | rbad[3];
  int e = 0;
  if (m > 0.0f && !bad) {
    int ex = 0;
    (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
    e = ex - 2;            // m * 2^-e in [2, 4)
  }
  if (threadIdx.x == 0) {
    xe[t] = e;
    if (bad) raise_status(status, COLI_STATUS_NONFINITE);
  }
  const bool fast = (H % 64) == 0 && (reinterpret_cast<uintptr_t>(row) & 7) == 0;
  const int ord[8] = {0, 2, 4, 6, 1, 3, 5, 7};  // staged order o + {0, 2, 32, 34, 1, 3, 33, 35}
  for (int i = threadIdx.x; i < GP * 8; i += 256) {
    const int g = i >> 3, c = i & 7;
    const int o = 16 * (c >> 2) + 4 * (c & 3);
    uint4 out = uint4{0u, 0u, 0u, 0u};
    float sum = 0.0f;
    if (g < G) {
      // b = elements o + {0, 1, 2, 3, 32, 33, 34, 35} of the group
      uint16_t b[8];
      const int base = 64 * g + o;
      if (fast) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(row + base);
        const uint2 hi = *reinterpret_cast<const uint2 *>(row + base + 32);
        b[0] = uint16_t(lo.x); b[1] = uint16_t(lo.x >> 16); b[2] = uint16_t(lo.y);
        b[3] = uint16_t(lo.y >> 16); b[4] = uint16_t(hi.x); b[5] = uint16_t(hi.x >> 16);
        b[6] = uint16_t(hi.y); b[7] = uint16_t(hi.y >> 16);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          b[k] = base + k < H ? row[base + k] : uint16_t(0);
          b[4 + k] = base + 32 + k < H ? row[base + 32 + k] : uint16_t(0);
        }
      }
      _Float16 h[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        h[k] = _Float16(ldexpf(__uint_as_float(uint32_t(b[ord[k]]) << 16), -e));
        sum += float(h[k]);
      }
      out = uint4{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3]), pack_f16x2(h[4], h[5]),
                  pack_f16x2(h[6], h[7])};
    }
    // the 8 runs of a group are 8 consecutive lanes
    sum += __shfl_xor(sum, 1, 8);
    sum += __shfl_xor(sum, 2, 8);
    sum += __shfl_xor(sum, 4, 8);
    *reinterpret_cast<uint4 *>(xp + int64_t(t) * HP + 64 * g + 8 * c) = out;
    if (c == 0 && g < G)
      *reinterpret_cast<uint32_t *>(sx + int64_t(t) * CSX + 2 * g) = split_f16(sum);
  }
  // the row's padding entries (groups G .. CSX/2 - 1) are zeros
  for (int k = 2 * G + 2 * int(threadIdx.x); k < CSX; k += 512)
    *reinterpret_cast<uint32_t *>(sx + int64_t(t) * CSX + k) = 0u;
}

// Zero the padding of every h row (groups G..IP/64-1, all in the last 256-k
// block) and of every h group-sum row (entries 2G..CSI-1).  One thread per row.
__global__ __launch_bounds__(256) void pf_pads(uint16_t *__restrict__ h, uint16_t *__restrict__ sh,
                                               int64_t rows, int G, int IP, int CSI) {
  const int64_t row = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (row >= rows) return;
  for (int k = 64 * G; k < IP; k += 8)
    *reinterpret_cast<uint4 *>(h + row * IP + k) = uint4{0u, 0u, 0u, 0u};
  for (int e = 2 * G; e < CSI; e += 2) *reinterpret_cast<uint32_t *>(sh + row * CSI + e) = 0u;
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

struct PfArgs {
  const uint16_t *A;  // staged activations, row stride AP (elements)
  const uint16_t *S;  // group-sum pairs, row stride CS
  uint16_t *out;      // gate/up: h (row stride OP); down: slot (row stride OP = H rounded
                      // up to 8)
  uint16_t *sout;     // gate/up: sh (row stride SOP)
  int AP, CS, OP, SOP;
  uint32_t a_bytes, s_bytes;  // sizes of A and S (< 2^31)
  const int *xe;              // per-token activation exponents (gate/up)
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

// sum over the 16 lanes of each lane row; the total lands in lane 15 of the row
__device__ inline float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
  return v;
}

// LDS of the GEMM kernels.  Two activation stages and two correction stages
// as separate arrays: the stage being read and the stage being filled by DMA
// are then distinct objects to the compiler, which keeps it from waiting for
// the DMA before every read of the other stage.  Staged rows are XOR-swizzled
// in 16-byte chunks (chunk c of row r sits at c ^ (r & 15), correction chunk c
// at c ^ ((r >> 2) & 3)) so that the 16 rows an MFMA operand reads hit 16
// different bank groups; each DMA instruction fills 1 KB of consecutive LDS.
__shared__ __attribute__((aligned(16))) uint8_t g_st0[kStageB];
__shared__ __attribute__((aligned(16))) uint8_t g_st1[kStageB];
__shared__ __attribute__((aligned(16))) uint8_t g_sc0[kCorrB];
__shared__ __attribute__((aligned(16))) uint8_t g_sc1[kCorrB];
__shared__ int g_rowidx[kMC];   // A / S row of each chunk row (-1: padding)
__shared__ int g_outrow[kMC];   // output row
__shared__ float g_gate[kMC];   // gate (down)
__shared__ int g_xe[kMC];       // the token's activation exponent (gate/up)

// Waves of a prefill GEMM block: two per SIMD.  The two waves on one SIMD
// (w and w + 4) share the block's activation stage and split the N rows: wave
// (simd, half) owns one 32-row weight fragment, so that one wave's dequant and
// exchange VALU work runs beside the other wave's MFMAs.
constexpr int kPW = 8;
constexpr int kPThreads = kPW * kWave;
constexpr int kRowsPW = kMC / kPW;      // staged rows each wave's DMA fills (16)
constexpr int kDmaPW = kRowsPW / 2;     // DMA instructions per wave per stage (8)

// One work item.  NMF = number of 32-row M fragments the chunk needs (1..4).
template <bool kGateUp, int NMF>
__device__ __attribute__((always_inline)) inline void run_item(const LayerDev &L, const PfArgs &pa,
                                                               const Item &it, float poison) {
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int sw = wave & 3, half = wave >> 2;  // SIMD slot, fragment of the pair
  const int h = lane >> 5, n = lane & 31;
  const int G = int(kGateUp ? L.lay.GH : L.lay.GI);
  const int nss = (G + 3) >> 2;
  const uint32_t rowB = uint32_t(G) * 32u;
  const int nrows = it.je - it.jb;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(pa.A, pa.a_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(pa.S, pa.s_bytes);
  // empty resource: every access reads zeros (loads of the last super-step)
  const __amdgpu_buffer_rsrc_t rnull = make_rsrc(pa.A, 0);

  // this wave's 32 weight rows: gate/up: features wrow0 .. +31 of the N-tile's
  // 128, gate (half 0) or up (half 1); down: rows wrow0 .. +31 of the 256
  int wrow0;
  bool wvalid;
  uint32_t qsec, ssec;
  if (kGateUp) {
    wrow0 = it.ntile * 128 + 32 * sw;
    wvalid = wrow0 < L.I;
    qsec = uint32_t(half == 0 ? L.lay.gq : L.lay.uq);
    ssec = uint32_t(half == 0 ? L.lay.gs : L.lay.us);
  } else {
    wrow0 = it.ntile * 256 + 64 * sw + 32 * half;
    wvalid = wrow0 < L.H;
    qsec = uint32_t(L.lay.dq);
    ssec = uint32_t(L.lay.ds);
  }
  // a wave past the matrix runs the same instruction stream on an empty weight
  // resource (zeros) and stores nothing: no wave-dependent branch in the loop
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(it.blob, wvalid ? uint32_t(L.lay.bytes) : 0u);
  // load a (0..3) of lane (h, n): row 8a + n%8, part 4h + n/8.  In the last
  // super-step lanes past G read the next bytes of the blob (a q section is
  // always followed by another section); their scale is 0.
  const uint32_t xoff = qsec + uint32_t(wrow0 + (n & 7)) * rowB + 16u * uint32_t(4 * h + (n >> 3));
  // scales of lane (h, n): row n, groups 16i + 8h ..
  const uint32_t soff = ssec + uint32_t(wrow0 + n) * uint32_t(G) * 4u + 32u * uint32_t(h);

  // DMA roles: instruction i of this wave fills staged rows 16w + 2i, 16w + 2i + 1
  // (lane: row + lane/32, LDS chunk lane%32); the correction instruction fills
  // rows 16w .. 16w + 15 (lane: row + lane/4, LDS chunk lane%4)
  uint32_t aoff[kDmaPW], coff;
#pragma unroll
  for (int i = 0; i < kDmaPW; ++i) {
    const int r = kRowsPW * wave + 2 * i + (lane >> 5);
    const int ri = g_rowidx[r];
    const uint32_t chunk = uint32_t((lane & 31) ^ (r & 15));
    aoff[i] = ri >= 0 ? uint32_t(ri) * uint32_t(pa.AP) * 2u + 16u * chunk : kOff;
  }
  {
    const int r = kRowsPW * wave + (lane >> 2);
    const int ri = g_rowidx[r];
    const uint32_t chunk = uint32_t((lane & 3) ^ ((r >> 2) & 3));
    coff = ri >= 0 ? uint32_t(ri) * uint32_t(pa.CS) * 2u + 16u * chunk : kOff;
  }
  auto dma_a = [&](int ss, uint8_t *st) {
#pragma unroll
    for (int i = 0; i < kDmaPW; ++i)
      dma16(ra, st + (kRowsPW * wave + 2 * i) * kRowB, aoff[i], uint32_t(512 * ss));
  };
  // correction operand of block i: entries 32i .. 32i + 31 (groups 16i .. 16i + 15,
  // hi and lo); entries past the groups are zeros in memory
  auto dma_c = [&](int i, uint8_t *sc) {
    dma16(rs, sc + (kRowsPW * wave) * 64, coff, uint32_t(64 * i));
  };
  auto load_b = [&](int ss, uint4(&R)[4]) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
      R[a4] = bload16(rw, xoff, 128u * uint32_t(ss) + 8u * uint32_t(a4) * rowB);
  };
  // scales of groups 16i + 8h + c (c = 0..7) of the lane's row; 0 past G
  auto load_f = [&](int i, float (&F)[8]) {
    const int g0 = 16 * i + 8 * h;
#pragma unroll
    for (int f4 = 0; f4 < 2; ++f4) {
      const int gq = g0 + 4 * f4;
      const uint32_t o = soff + 64u * uint32_t(i) + 16u * uint32_t(f4);
      if ((G & 3) == 0) {
        const uint4 w = bload16(rw, gq < G ? o : kOff, 0);
        F[4 * f4 + 0] = __uint_as_float(w.x);
        F[4 * f4 + 1] = __uint_as_float(w.y);
        F[4 * f4 + 2] = __uint_as_float(w.z);
        F[4 * f4 + 3] = __uint_as_float(w.w);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) F[4 * f4 + c] = bload4f(rw, gq + c < G ? o + 4u * c : kOff);
      }
    }
  };

  f32x16 acc[NMF];
#pragma unroll
  for (int mf = 0; mf < NMF; ++mf) acc[mf] = f32x16{};

  // prologue: stage 0 (activations, correction block 0), scales of block 0, weights of
  // super-steps 0 and 1 (two super-steps of weight loads in flight: the exchange of
  // super-step ss then waits for loads issued two super-steps earlier)
  float F[8] = {};
  uint4 Rb[2][4] = {};
  dma_a(0, g_st0);
  dma_c(0, g_sc0);
  load_f(0, F);
  load_b(0, Rb[0]);
  if (nss > 1) load_b(1, Rb[1]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
  __syncthreads();

  uint32_t m1, m2;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m1));
  asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(m2));
  // per-lane parts of the swizzled addresses: A row n (+32 mf), correction row n
  const uint32_t abase = uint32_t(n * kRowB + 256 * h);
  const uint32_t aswz = uint32_t(n & 15);
  const uint32_t cbase = uint32_t(n * 64);
  const uint32_t cswz = uint32_t((n >> 2) & 3);

  // U[0..7]: the block's scales in super-step order (pairs e = 0, 1 of
  // super-step c at 2c, 2c + 1), rotated by two per super-step
  float U[8] = {};
  // one super-step: compute from (st, sc) while the DMA fills (stn, scn)
  auto super_step = [&](int ss, int par, const uint8_t *st, const uint8_t *sc, uint8_t *stn,
                        uint8_t *scn) {
    const bool more = ss + 1 < nss;
    uint4(&R)[4] = Rb[par];
    if (more && ((ss + 1) & 3) == 0) dma_c((ss + 1) >> 2, scn);
    {
      // this super-step's weights into MFMA lane order: register d of lane (h, n)
      // = part 4h + d of row n (exchange of the load index with lane bits 3, 4)
      uint4 D[4];
      exchange_rows(R, D);
      if ((ss & 3) == 0) {
        // correction GEMM of block i = ss / 4: acc += S (hi, lo) x (-8 s, -8 s);
        // k-step kc, k-half h covers groups 16i + 8h + 4kc .. +3
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const _Float16 h0 = _Float16(F[4 * kc + 0]) * _Float16(-8.0f);
          const _Float16 h1 = _Float16(F[4 * kc + 1]) * _Float16(-8.0f);
          const _Float16 h2 = _Float16(F[4 * kc + 2]) * _Float16(-8.0f);
          const _Float16 h3 = _Float16(F[4 * kc + 3]) * _Float16(-8.0f);
          const f16x8 bc = f16x8{h0, h0, h1, h1, h2, h2, h3, h3};
#pragma unroll
          for (int mf = 0; mf < NMF; ++mf) {
            const f16x8 a = *reinterpret_cast<const f16x8 *>(
                sc + cbase + mf * 32 * 64 + 16 * ((uint32_t(2 * h + kc)) ^ cswz));
            acc[mf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bc, acc[mf], 0, 0, 0);
          }
        }
        // regroup between lane halves: lane h then holds groups 4c + 2h, 4c + 2h + 1
        float T[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) T[c] = F[c];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const auto p0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[c]), __float_as_uint(T[2 + c]), false, false);
          const auto p1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[4 + c]), __float_as_uint(T[6 + c]), false, false);
          T[c] = __uint_as_float(uint32_t(p0[0]));
          T[2 + c] = __uint_as_float(uint32_t(p0[1]));
          T[4 + c] = __uint_as_float(uint32_t(p1[0]));
          T[6 + c] = __uint_as_float(uint32_t(p1[1]));
        }
        // super-step order: c = 0: T0 T1, c = 1: T4 T5, c = 2: T2 T3, c = 3: T6 T7
        U[0] = T[0]; U[1] = T[1]; U[2] = T[4]; U[3] = T[5];
        U[4] = T[2]; U[5] = T[3]; U[6] = T[6]; U[7] = T[7];
        if (ss + 4 < nss) load_f((ss >> 2) + 1, F);
      } else {
#pragma unroll
        for (int c = 0; c < 6; ++c) U[c] = U[c + 2];
      }
      // dequant constants per group half e of the super-step
      f16x2 s2[2], c10[2], c6[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const _Float16 hs = _Float16(U[e]);
        s2[e] = f16x2{hs, hs};
        c10[e] = s2[e] * f16x2{_Float16(-1024.0f), _Float16(-1024.0f)};
        c6[e] = s2[e] * f16x2{_Float16(-64.0f), _Float16(-64.0f)};
      }
      // 16 MFMA k-steps; the weights of step k + 1 are dequantised and its A
      // fragments read while the MFMAs of step k run (pinned with scheduling
      // group barriers: left alone, the scheduler sinks each A read next to its
      // first use and the LDS latency stalls every MFMA group).  The next
      // stage's activations go out by DMA one instruction every other step: issued
      // in one burst after the barrier they would stall every wave on the address
      // unit.
      f16x8 a[NMF], b;
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
        a[mf] = *reinterpret_cast<const f16x8 *>(st + abase + mf * 32 * kRowB + 16 * (0 ^ aswz));
      b = dequant(D[0].x, m1, m2, s2[0], c10[0], c6[0]);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int k1 = k + 1;
        __builtin_amdgcn_sched_barrier(0);
        f16x8 an[NMF], bn;
        if (k < 15) {
#pragma unroll
          for (int mf = 0; mf < NMF; ++mf)
            an[mf] = *reinterpret_cast<const f16x8 *>(st + abase + mf * 32 * kRowB +
                                                      16 * (uint32_t(k1) ^ aswz));
          bn = dequant(word_of(D[k1 >> 2], k1 & 3), m1, m2, s2[k1 >> 3], c10[k1 >> 3],
                       c6[k1 >> 3]);
        }
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf)
          acc[mf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mf], b, acc[mf], 0, 0, 0);
        // (no branch: a branch here would split the step's scheduling region; in
        // the last super-step the instruction reads out of range and writes zeros
        // into the unused stage, landed before the epilogue by the closing wait)
        if ((k & 1) == 0)
          dma16(ra, stn + (kRowsPW * wave + k) * kRowB, more ? aoff[k >> 1] : kOff,
                uint32_t(512 * (ss + 1)));
        if (k < 15) {
          if ((k & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (DMA)
          __builtin_amdgcn_sched_group_barrier(0x100, NMF, 0);  // DS reads
#pragma unroll
          for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 10 / NMF + 1, 0);  // VALU
          }
#pragma unroll
          for (int mf = 0; mf < NMF; ++mf) a[mf] = an[mf];
          b = bn;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the weights of super-step ss + 2 go out after this super-step's last DMA
    // (empty resource past the end: the count stays 4), so the wait below can
    // leave exactly them in flight across the barrier
    {
      const __amdgpu_buffer_rsrc_t rwn2 = ss + 2 < nss ? rw : rnull;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        R[a4] = bload16(rwn2, xoff, 128u * uint32_t(ss + 2) + 8u * uint32_t(a4) * rowB);
      __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0): next stage landed
    }
    // a plain barrier: __syncthreads() would also wait for the loads left in
    // flight (its workgroup release waits for every memory operation);
    // the memory clobber keeps the compiler from moving LDS accesses across
    asm volatile("s_barrier" ::: "memory");
  };
  // pairs of super-steps with no branch inside the loop body (the compiler's
  // load-counter bookkeeping then carries across the back edge), odd tail after
  int ss = 0;
  for (; ss + 1 < nss; ss += 2) {
    super_step(ss, 0, g_st0, g_sc0, g_st1, g_sc1);
    super_step(ss + 1, 1, g_st1, g_sc1, g_st0, g_sc0);
  }
  if (ss < nss) super_step(ss, 0, g_st0, g_sc0, g_st1, g_sc1);
  // the weights issued for super-steps past the end (empty resource) may still
  // count as outstanding: nothing below reads them
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // epilogue through LDS tiles (the stages are free: the last super-step ended
  // with a barrier), then 16-byte stores.  tid is made opaque so that the
  // item-invariant addresses below are not hoisted to the kernel start (where
  // they would be spilled and reloaded from scratch, once per stored row).
  // acc[mf][4j + i] is row 32 mf + 8j + 4h + i, column n of the wave's fragment.
  int tid = int(threadIdx.x);
  asm volatile("" : "+v"(tid));
  const int eh = (tid & 63) >> 5, en = tid & 31;
  bool range = false;  // an fp16 operand out of range: COLI_STATUS_RANGE
  if (kGateUp) {
    // gate (half 0) -> fp32 tile [128 rows][128 features] in stage 0; the up wave
    // of the same SIMD slot then forms h in the staged order (2 groups, 256 B per
    // row) in stage 1.  The row's activations were scaled by 2^-e: gate = 2^e
    // acc_g, up = 2^e acc_u, and h is stored scaled by 2^-2e: SiLU(2^e acc_g) *
    // acc_u * 2^-e.  Features past I (a ragged last group, or a wave past the
    // matrix) are zeros.
    float *gtile = reinterpret_cast<float *>(g_st0);
    uint8_t *htile = g_st1;
    const int fl = 32 * sw + en;  // feature within the N-tile
    if (half == 0 && wvalid) {
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 32 * mf + 8 * (v >> 2) + 4 * eh + (v & 3);
          gtile[m * 128 + fl] = acc[mf][v];
        }
    }
    __syncthreads();
    if (half == 1) {
      const int tpos = 2 * (64 * (fl >> 6) + grp_pos(fl & 63));
      const bool fvalid = wrow0 + en < L.I;
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 32 * mf + 8 * (v >> 2) + 4 * eh + (v & 3);
          const int fe = g_xe[m];
          float hf = 0.0f;
          if (fvalid) {
            hf = silu(ldexpf(gtile[m * 128 + fl], fe)) * ldexpf(acc[mf][v], -fe);
            range |= !(fabsf(hf) <= 65504.0f);
            hf *= poison;
          }
          *reinterpret_cast<_Float16 *>(htile + m * 256 + tpos) = _Float16(hf);
        }
    }
    __syncthreads();
    const int g0 = it.ntile * 2;
    {
      const int c = tid & 15;
      if (64 * (g0 + (c >> 3)) < L.I) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int m = (tid >> 4) + 32 * p;
          if (m < nrows) {
            const uint4 v = *reinterpret_cast<const uint4 *>(htile + m * 256 + 16 * c);
            *reinterpret_cast<uint4 *>(pa.out + int64_t(g_outrow[m]) * pa.OP + 64 * g0 + 8 * c) = v;
          }
        }
      }
    }
    // group sums of h: thread (m, gsel) adds the 64 fp16 values of its group
    if (tid < 2 * kMC) {
      const int m = tid & (kMC - 1), gsel = tid >> 7;
      if (m < nrows && 64 * (g0 + gsel) < L.I) {
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint4 v = *reinterpret_cast<const uint4 *>(htile + m * 256 + gsel * 128 + 16 * c);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const f16x2 hv = __builtin_bit_cast(f16x2, w[d]);
            sum += float(hv[0]) + float(hv[1]);
          }
        }
        *reinterpret_cast<uint32_t *>(pa.sout + int64_t(g_outrow[m]) * pa.SOP + 2 * (g0 + gsel)) =
            split_f16(sum);
      }
    }
  } else {
    // tile row m: the N-tile's 256 gate-scaled outputs (still scaled by the
    // token's 2^-2e; the combine undoes it); outputs past H are zeros
    uint8_t *tile = g_st0;
    if (wvalid) {
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 32 * mf + 8 * (v >> 2) + 4 * eh + (v & 3);
          float o = g_gate[m] * acc[mf][v];
          o = wrow0 + en < L.H ? o : 0.0f;
          range |= fabsf(o) > 65504.0f;  // (NaN h of a poisoned expert is not a range fault)
          *reinterpret_cast<_Float16 *>(tile + m * 512 + 2 * (64 * sw + 32 * half + en)) =
              _Float16(o);
        }
    }
    __syncthreads();
    const int c = tid & 31;
    const int n0 = it.ntile * 256 + 8 * c;
    if (n0 < L.H) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int m = (tid >> 5) + 16 * p;
        if (m < nrows) {
          const uint4 v = *reinterpret_cast<const uint4 *>(tile + m * 512 + 16 * c);
          *reinterpret_cast<uint4 *>(pa.out + int64_t(g_outrow[m]) * pa.OP + n0) = v;
        }
      }
    }
  }
  if (__any(range) && (threadIdx.x % kWave) == 0) raise_status(L.status, COLI_STATUS_RANGE);
}

// Persistent grouped GEMM: blocks walk (chunk, N-tile) items.  With a grid
// that is a multiple of 8 the items are split into 8 contiguous ranges, one
// per XCD (the hardware deals consecutive blocks round-robin over the 8 XCDs),
// so the N-tiles of one chunk, which share its activations, meet in one L2.
template <bool kGateUp>
__global__ __launch_bounds__(kPThreads, 1) void pf_gemm(LayerDev L, Routing r, int T, PfArgs pa) {
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
    decode_item(L, r, T, item, n_nt, it, kMC, r.chunk, *r.n_unique + 1);
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
      g_rowidx[threadIdx.x] = ri;
      g_outrow[threadIdx.x] = orow;
      g_gate[threadIdx.x] = gate;
      g_xe[threadIdx.x] = (kGateUp && ri >= 0) ? pa.xe[ri] : 0;
    }
    __syncthreads();
    const int nmf = (it.je - it.jb + 31) / 32;
    // a routed expert without a slot: its h (and so its outputs) become NaN
    const bool missing = __builtin_amdgcn_readfirstlane(int(it.missing)) != 0;
    if (missing && kGateUp && threadIdx.x == 0) raise_status(L.status, COLI_STATUS_NOT_RESIDENT);
    const float poison = missing ? __builtin_nanf("") : 1.0f;
    switch (nmf) {
      case 1: run_item<kGateUp, 1>(L, pa, it, poison); break;
      case 2: run_item<kGateUp, 2>(L, pa, it, poison); break;
      case 3: run_item<kGateUp, 3>(L, pa, it, poison); break;
      default: run_item<kGateUp, 4>(L, pa, it, poison); break;
    }
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + ((u >> 16) & 1u) + 0x7FFFu) >> 16);
}

// y[t] = 2^(2 e_t) (sum_k slot[t*K + k] + slot[T*K + t])   (fp16 slots of
// stride SP, a multiple of 8; fp32 sum; bf16 y of any H; 8 columns per
// thread).  A non-finite y raises COLI_STATUS_NONFINITE.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ slot, int T,
                                                      int H, int SP, int K,
                                                      const int *__restrict__ xe,
                                                      uint16_t *__restrict__ y, int32_t *status) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = SP / 8;
  bool bad = false;
  if (i < int64_t(T) * per_row) {
    const int t = int(i / per_row), c = int(i % per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k <= K; ++k) {
      const int64_t row = k < K ? int64_t(t) * K + k : int64_t(T) * K + t;
      const uint4 v = *reinterpret_cast<const uint4 *>(slot + row * SP + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x2 hv = __builtin_bit_cast(f16x2, w[q]);
        acc[2 * q] += float(hv[0]);
        acc[2 * q + 1] += float(hv[1]);
      }
    }
    const int e2 = 2 * xe[t];
    uint16_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float v = ldexpf(acc[q], e2);
      bad |= (c + q < H) && !__builtin_isfinite(v);
      o[q] = f32_to_bf16_rne(v);
    }
    uint16_t *yr = y + int64_t(t) * H;
    if ((H & 7) == 0) {
      *reinterpret_cast<uint4 *>(yr + c) =
          uint4{uint32_t(o[0]) | (uint32_t(o[1]) << 16), uint32_t(o[2]) | (uint32_t(o[3]) << 16),
                uint32_t(o[4]) | (uint32_t(o[5]) << 16), uint32_t(o[6]) | (uint32_t(o[7]) << 16)};
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (c + q < H) yr[c + q] = o[q];
    }
  }
  if (__any(bad) && (threadIdx.x % 64) == 0) raise_status(status, COLI_STATUS_NONFINITE);
}

template <bool kGateUp>
hipError_t launch_gemm(const LayerDev &L, const Routing &r, int T, const PfArgs &pa,
                       int64_t max_items, hipStream_t s) {
  const int64_t cus = cus_of_device();
  const int64_t grid = max_items < cus ? max_items : cus;
  pf_gemm<kGateUp><<<dim3(unsigned(grid)), dim3(kPThreads), 0, s>>>(L, r, T, pa);
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
  const int SP = prefill_slot_stride(L.H);
  const int GI = int(groups_of(L.I));
  if (ev) (void)hipEventRecord(ev[0], s);
  pf_prep<<<dim3(unsigned(T)), 256, 0, s>>>(x, T, L.H, pl.HP, pl.CSX, b.xp, b.sx, b.xe, L.status);
  if (pl.IP > 64 * GI || pl.CSI > 2 * GI) {
    const int64_t rows = TK + T;
    pf_pads<<<dim3(unsigned((rows + 255) / 256)), 256, 0, s>>>(b.h, b.sh, rows, GI, pl.IP, pl.CSI);
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
              uint32_t(int64_t(T) * pl.HP * 2), uint32_t(int64_t(T) * pl.CSX * 2), b.xe};
    e = launch_gemm<true>(L, r, T, pa, max_chunks * ((L.I + 127) / 128), s);
    if (e != hipSuccess) return e;
  }
  if (ev) (void)hipEventRecord(ev[3], s);
  if (ev) (void)hipEventRecord(ev[4], s);
  {
    PfArgs pa{b.h, b.sh, b.slot, nullptr, pl.IP, pl.CSI, SP, 0,
              uint32_t((TK + T) * pl.IP * 2), uint32_t((TK + T) * pl.CSI * 2), b.xe};
    e = launch_gemm<false>(L, r, T, pa, max_chunks * ((L.H + 255) / 256), s);
    if (e != hipSuccess) return e;
  }
  if (ev) (void)hipEventRecord(ev[5], s);
  const int64_t nthr = int64_t(T) * (SP / 8);
  if (ev) (void)hipEventRecord(ev[6], s);
  combine_kernel<<<dim3(unsigned((nthr + 255) / 256)), 256, 0, s>>>(b.slot, T, L.H, SP, L.K, b.xe,
                                                                    y, L.status);
  if (ev) (void)hipEventRecord(ev[7], s);
  return hipGetLastError();
}

bool prefill_offsets_ok(int H, int I, int K, int T, size_t blob_bytes) {
  const PrefillLayout pl = prefill_layout(H, I);
  const int64_t R = int64_t(T) * K + T;
  const int64_t lim = int64_t(1) << 31;  // buffer offsets: 32 bits, top bit masks
  return int64_t(T) * pl.HP * 2 < lim && R * pl.IP * 2 < lim &&
         int64_t(T) * pl.CSX * 2 < lim && R * pl.CSI * 2 < lim && int64_t(blob_bytes) < lim;
}

int prefill_slot_stride(int H) { return (H + 7) & ~7; }

}  // namespace coli

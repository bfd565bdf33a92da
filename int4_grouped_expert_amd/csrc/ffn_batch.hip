// ffn_batch.hip -- the routed + shared expert FFN for a decode batch
// (1 < T <= 256): int4-g64 grouped GEMMs on the fp16 matrix cores at
// fp32-class accuracy.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 (planar int4-g64 bytes consumed as they are; weight =
// s * (u - 8)); SiLU(gate) * up, down, gate-weighted sum plus the shared
// expert (page "Colibrì 深度解析", sections 四 and 十一); batch union (same
// page, section 四: each unique expert of the batch is read once).
//
// The weight stream is the prefill GEMMs' (gemm_stream.h): a super-step covers
// 4 groups = 128 contiguous bytes of every weight row, loaded as whole 128-byte
// lines and exchanged into MFMA lane order.
//
// Arithmetic.  Activations are split into fp16 hi + lo rows, (hi + lo) * 2^e
// with one power-of-two scale per row (max |row| * 2^-e in [2^14, 2^15)), so
// that both parts are fp16 normals for every element within 2^-10 of the
// row maximum.  Weights enter as the exact fp16 integers u - 8 ((d & 0x000F000F)
// | 0x64006400 = {1024 + u, ..}, (d & 0x00F000F0) | 0x54005400 = {64 + u, ..},
// then one v_pk_add_f16 of -1032 or -72), so every product is exact in
// the fp32 accumulator.  Each MFMA k-step covers one group: the weight loads
// take part 2 (n / 8) + h instead (same whole-line loads, same exchange), which
// leaves half h of group d of the super-step in register d of lane (h, n), and
// the staged activations (the prefill's staged order, gemm_stream.h) are read
// in group order.  A group's four k-steps
// accumulate hi and lo products into a fresh fp32 tile, which is scaled by the
// fp32 group scale into the output accumulator: the format's arithmetic
// s * sum((u - 8) x) with fp32 scale and fp32 sums.
//
// Work item = (unit, M-chunk of <= 32 of the unit's tokens, N-tile); a chunk's
// 32 hi rows are staged in rows 0..31, its lo rows in rows 32..63.
//   gate/up: h = SiLU(gate) * up in fp32, written per slot row (hf [rows][I]);
//   split_rows turns hf into the staged hi/lo rows of the down step;
//   down: gate * (Wd h) in fp32 per slot row; combine_f32 sums a token's slots.
#include "gemm_stream.h"
#include "kernels.h"
#include "stage_rows.h"

#include <hip/hip_fp16.h>

namespace coli {
namespace {

constexpr int kDMC = 32;            // tokens per M-chunk (the decode route's chunking)
constexpr int kDRows = 2 * kDMC;    // staged rows: the chunk's hi rows, then its lo rows
constexpr int kDStageB = kDRows * kRowB;

// LDS: two activation stages as separate arrays (the stage being read and the
// stage the DMA fills are distinct objects to the compiler), XOR-swizzled in
// 16-byte chunks (chunk c of row r at c ^ (r & 15)); the chunk's row tables.
__shared__ __attribute__((aligned(16))) uint8_t g_st0[kDStageB];
__shared__ __attribute__((aligned(16))) uint8_t g_st1[kDStageB];
__shared__ int g_rowidx[kDRows];  // A row of each staged row (-1: padding)
__shared__ int g_outrow[kDMC];    // output row of each chunk token
__shared__ float g_gate[kDMC];    // gate (down)

// src fp32 [rows][W] -> dst fp16 [2 rows][WP] in the staged order: row r's hi
// part at row r, its lo part at row rows + r, zero padding; sc[r] = 2^e.  One
// block per row.  W % 64 == 0, WP % 256 == 0.
__global__ __launch_bounds__(256) void split_rows(const float *__restrict__ src, int rows, int W,
                                                  int WP, uint16_t *__restrict__ dst,
                                                  float *__restrict__ sc) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  stage_row(src + int64_t(r) * W, W, WP, dst + int64_t(r) * WP, dst + (int64_t(rows) + r) * WP,
            sc + r, red);
}

struct DecArgs {
  const uint16_t *A;   // staged hi/lo rows, row stride AP (elements)
  const float *rsc;    // power-of-two scale of each activation row
  float *out;          // gate/up: hf (row stride OP = I); down: slot (OP = H)
  int AP, OP;
  int lo_rows;         // offset of the lo rows (rows of A / 2)
  uint32_t a_bytes;
};

__shared__ float g_rsc[kDMC];  // scale of each chunk token's activation row
// the batch's chunk prefix (r.chunk[0 .. units + 1]), read once per block: the
// item decode's binary search then costs no memory round trips
__shared__ int g_chunk[COLI_MAX_EXPERTS + 2];

// u - 8 as fp16 for the 8 nibbles of word d, in the staged k order
__device__ inline f16x8 unpack_u8(uint32_t d, uint32_t m1, uint32_t m2) {
  const uint32_t d8 = d >> 8;
  const f16x2 p0 = __builtin_bit_cast(f16x2, (d & m1) | 0x64006400u);
  const f16x2 p1 = __builtin_bit_cast(f16x2, (d & m2) | 0x54005400u);
  const f16x2 p2 = __builtin_bit_cast(f16x2, (d8 & m1) | 0x64006400u);
  const f16x2 p3 = __builtin_bit_cast(f16x2, (d8 & m2) | 0x54005400u);
  const f16x2 c10 = f16x2{_Float16(-1032.0f), _Float16(-1032.0f)};
  const f16x2 c6 = f16x2{_Float16(-72.0f), _Float16(-72.0f)};
  const f16x2 r0 = p0 + c10, r1 = p1 + c6, r2 = p2 + c10, r3 = p3 + c6;
  return f16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// kHalf: a chunk of at most 16 tokens, staged as one 32-row fragment (hi
// rows 0..15, lo rows 16..31), so that each k-step takes one MFMA per weight
// fragment instead of two; the hi and lo result rows are added at the end.
// The item's blob finish tag is loaded with its first weights (its latency
// hides behind theirs); a blob without the tag, or an expert without a slot,
// poisons the item's outputs (NaN) and raises the status flag.
template <bool kGateUp, bool kHalf>
__device__ __attribute__((always_inline)) inline void run_item_dec(const LayerDev &L,
                                                                   const DecArgs &da,
                                                                   const Item &it, bool missing) {
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int h = lane >> 5, n = lane & 31;
  const int G = int(kGateUp ? L.lay.GH : L.lay.GI);
  const int nss = (G + 3) >> 2;
  const uint32_t rowB = uint32_t(G) * 32u;
  const int nrows = it.je - it.jb;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(it.blob, uint32_t(L.lay.bytes));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(da.A, da.a_bytes);
  const __amdgpu_buffer_rsrc_t rnull = make_rsrc(da.A, 0);

  int wrow0;
  bool wvalid;
  if (kGateUp) {
    wrow0 = it.ntile * 128 + 32 * wave;
    wvalid = wrow0 < L.I;
  } else {
    wrow0 = it.ntile * 256 + 64 * wave;
    wvalid = wrow0 < L.H;
  }
  uint32_t xoff[2], soff[2];
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) {
    int row;
    uint32_t qsec, ssec;
    if (kGateUp) {
      row = wrow0;
      qsec = uint32_t(jn == 0 ? L.lay.gq : L.lay.uq);
      ssec = uint32_t(jn == 0 ? L.lay.gsT : L.lay.usT);
    } else {
      row = wrow0 + 32 * jn;
      qsec = uint32_t(L.lay.dq);
      ssec = uint32_t(L.lay.dsT);
    }
    // load a of lane (h, n): row 8a + n%8, part 2 (n / 8) + h (past G in the
    // last super-step: the next bytes of the blob, scale 0)
    xoff[jn] = qsec + uint32_t(row + (n & 7)) * rowB + 16u * uint32_t(2 * (n >> 3) + h);
    // scales of row n, group-major: group g at soff + g * rows * 4 (both lane
    // halves; one load covers 32 consecutive rows, a single cache line)
    soff[jn] = ssec + uint32_t(row + n) * 4u;
  }
  // DMA roles: instruction i of this wave fills staged rows 16w + 2i, +1
  // (lane: row + lane/32, LDS chunk lane%32)
  constexpr int kNdma = kHalf ? 4 : 8;        // DMA instructions per wave per stage
  constexpr int kRowsW = 2 * kNdma;           // staged rows per wave
  uint32_t aoff[kNdma];
#pragma unroll
  for (int i = 0; i < kNdma; ++i) {
    const int r = kRowsW * wave + 2 * i + (lane >> 5);
    const int ri = g_rowidx[r];
    const uint32_t chunk = uint32_t((lane & 31) ^ (r & 15));
    aoff[i] = ri >= 0 ? uint32_t(ri) * uint32_t(da.AP) * 2u + 16u * chunk : kOff;
  }
  auto dma_a = [&](int ss, uint8_t *st) {
#pragma unroll
    for (int i = 0; i < kNdma; ++i)
      dma16(ra, st + (kRowsW * wave + 2 * i) * kRowB, aoff[i], uint32_t(512 * ss));
  };
  auto load_b = [&](int ss, uint4(&R)[2][4]) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        R[jn][a4] = bload16(rw, xoff[jn], 128u * uint32_t(ss) + 8u * uint32_t(a4) * rowB);
  };
  // scales of groups 4 ss .. 4 ss + 3 from the group-major sections: lane half
  // h loads groups 2h and 2h + 1 (two 4-byte loads per fragment, each one cache
  // line for the half; groups past the row end read zeros through the empty
  // offset), and spread() passes each half's pair to the other
  const uint32_t srow4 = uint32_t(kGateUp ? L.I : L.H) * 4u;
  auto load_s = [&](int ss, float (&Fr)[2][2]) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int g = 4 * ss + 2 * h + c;
        Fr[jn][c] = bload4f(rw, g < G ? soff[jn] + uint32_t(g) * srow4 : kOff);
      }
  };
  auto spread = [&](const float (&Fr)[2][2], float (&F)[2][4]) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float mine = Fr[jn][c], theirs = __shfl_xor(mine, 32, kWave);
        F[jn][c] = h ? theirs : mine;
        F[jn][2 + c] = h ? mine : theirs;
      }
  };

  f32x16 acc[2];
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) acc[jn] = f32x16{};
  float F[2][4] = {}, Fr[2][2] = {}, Frn[2][2] = {};
  uint4 R[2][4] = {};
  dma_a(0, g_st0);
  const uint4 tg = *reinterpret_cast<const uint4 *>(it.blob + L.lay.tag);
  if (wvalid) {
    load_s(0, Fr);
    load_b(0, R);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  spread(Fr, F);
  const bool untagged =
      tg.x != L.tag.x || tg.y != L.tag.y || tg.z != L.tag.z || tg.w != L.tag.w;
  if (threadIdx.x == 0) {
    if (untagged && !missing) raise_status(L.status, COLI_STATUS_UNFINISHED);
    if (missing) raise_status(L.status, COLI_STATUS_NOT_RESIDENT);
  }
  const float poison = (untagged || missing) ? __builtin_nanf("") : 1.0f;

  uint32_t m1, m2;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m1));
  asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(m2));
  // A row n (hi) and 32 + n (lo); chunk q of a row sits at q ^ (row & 15)
  const uint32_t abase = uint32_t(n * kRowB);
  const uint32_t aswz = uint32_t(n & 15);

  auto super_step = [&](int ss, const uint8_t *st, uint8_t *stn) {
    const bool more = ss + 1 < nss;
    if (wvalid) {
      uint4 D[2][4];
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) exchange_rows(R[jn], D[jn]);
      const __amdgpu_buffer_rsrc_t rwn = more ? rw : rnull;
      if (more) load_s(ss + 1, Frn);
      // k-step k = 4 d + w: group d of the super-step, word w; lane half h
      // reads chunk 8 d + 4 h + w of its hi and lo rows
      f16x8 ahi, alo = {};
      {
        const uint32_t q = uint32_t(4 * h) ^ aswz;
        ahi = *reinterpret_cast<const f16x8 *>(st + abase + 16 * q);
        if (!kHalf) alo = *reinterpret_cast<const f16x8 *>(st + abase + 32 * kRowB + 16 * q);
      }
      f32x16 C[2];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int d = k >> 2, w = k & 3;
        __builtin_amdgcn_sched_barrier(0);
        f16x8 ahn, aln = {};
        if (k < 15) {
          const int k1 = k + 1;
          const uint32_t q = uint32_t(8 * (k1 >> 2) + 4 * h + (k1 & 3)) ^ aswz;
          ahn = *reinterpret_cast<const f16x8 *>(st + abase + 16 * q);
          if (!kHalf) aln = *reinterpret_cast<const f16x8 *>(st + abase + 32 * kRowB + 16 * q);
        }
        f16x8 b[2];
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
          b[jn] = unpack_u8(word_of(D[jn][d], w), m1, m2);
          if (w == 0) C[jn] = f32x16{};
        }
        // two accumulator chains, interleaved: hi products, then lo
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          C[jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, b[jn], C[jn], 0, 0, 0);
        if (!kHalf) {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn)
            C[jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, b[jn], C[jn], 0, 0, 0);
        }
        if (w == 3) {
          // the group's tile, scaled by its fp32 scale
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const float sg = F[jn][d];
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[jn][v] = fmaf(C[jn][v], sg, acc[jn][v]);
          }
        }
        if ((k & (16 / kNdma - 1)) == 0)
          dma16(ra, stn + (kRowsW * wave + 2 * (k / (16 / kNdma))) * kRowB,
                more ? aoff[k / (16 / kNdma)] : kOff, uint32_t(512 * (ss + 1)));
        if (k < 8)
          R[k >> 2][k & 3] = bload16(rwn, xoff[k >> 2], 128u * uint32_t(ss + 1) + 8u * uint32_t(k & 3) * rowB);
        if (k < 15) {
          ahi = ahn;
          if (!kHalf) alo = aln;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      spread(Frn, F);
    } else if (more) {
      dma_a(ss + 1, stn);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next stage and weights landed
    __syncthreads();
  };
  for (int ss = 0; ss < nss; ss += 2) {
    super_step(ss, g_st0, g_st1);
    if (ss + 1 < nss) super_step(ss + 1, g_st1, g_st0);
  }

  // epilogue: acc[jn][4j + i] is staged row 8j + 4h + i, column n of fragment
  // jn: chunk token 8j + 4h + i, or (kHalf) token m's hi row for v < 8 and its
  // lo row at v + 8, added here
  if (kHalf) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[jn][v] += acc[jn][v + 8];
  }
  if (wvalid) {
    // rows past the matrix (a ragged last tile) are not stored
    const int nrow = kGateUp ? L.I : L.H;
#pragma unroll
    for (int v = 0; v < (kHalf ? 8 : 16); ++v) {
      const int m = 8 * (v >> 2) + 4 * h + (v & 3);
      if (m < nrows) {
        const float rs = g_rsc[m] * poison;
        if (kGateUp) {
          const float gv = acc[0][v] * rs, uv = acc[1][v] * rs;
          if (wrow0 + n < nrow) da.out[int64_t(g_outrow[m]) * da.OP + wrow0 + n] = silu(gv) * uv;
        } else {
          const float gs = rs * g_gate[m];
#pragma unroll
          for (int jn = 0; jn < 2; ++jn)
            if (wrow0 + 32 * jn + n < nrow)
              da.out[int64_t(g_outrow[m]) * da.OP + wrow0 + 32 * jn + n] = acc[jn][v] * gs;
        }
      }
    }
  }
}

// Persistent over (chunk, N-tile) items of 32-token chunks, two blocks per CU
// (66 KB of LDS each; the second block's waves fill the MFMA and memory gaps of
// the first), XCD-contiguous item ranges as in pf_gemm.  Row tables: staged row r < 32
// is chunk token r's hi row, 32 + r its lo row.
template <bool kGateUp>
__global__ __launch_bounds__(kThreads, 2) void dec_gemm(LayerDev L, Routing r, int T, DecArgs da) {
  const int K = L.K;
  const int n_nt = kGateUp ? (L.I + 127) / 128 : (L.H + 255) / 256;
  const int nu = *r.n_unique + 1;
  for (int i = threadIdx.x; i <= nu; i += kThreads) g_chunk[i] = r.chunk[i];
  __syncthreads();
  const int n_items = g_chunk[nu] * n_nt;
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
    decode_item(L, r, T, item, n_nt, it, kDMC, g_chunk, nu);
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
    // staged rows: chunks of up to 16 tokens take hi rows 0..15 and lo rows
    // 16..31, larger ones hi rows 0..31 and lo rows 32..63
    const bool small = it.je - it.jb <= kDMC / 2;
    const int per = small ? kDMC / 2 : kDMC;
    if (threadIdx.x < 2 * kDMC) {
      const int tok = threadIdx.x % per, half = threadIdx.x / per;
      const int j = it.jb + tok;
      int ri = -1;
      if (j < it.je && half < 2) {
        int arow, orow;
        float gate = 1.0f;
        if (kGateUp) {
          arow = it.shared ? j : r.perm[j] / K;  // token
          orow = it.shared ? T * K + j : j;      // slot row
        } else {
          arow = it.shared ? T * K + j : j;      // slot row
          if (it.shared) {
            orow = T * K + j;
          } else {
            const int p = r.perm[j];
            orow = p;
            gate = r.gates[p];
          }
        }
        ri = half < 2 ? arow + half * da.lo_rows : -1;
        if (half == 0) {
          g_outrow[tok] = orow;
          g_gate[tok] = gate;
          g_rsc[tok] = da.rsc[arow];
        }
      }
      g_rowidx[threadIdx.x] = ri;
    }
    __syncthreads();
    // a blob without the finish tag has no valid scale copies: its outputs
    // become NaN and the status flag says why (checked inside, with the item's
    // first loads)
    const bool missing = __builtin_amdgcn_readfirstlane(int(it.missing)) != 0;
    if (small)
      run_item_dec<kGateUp, true>(L, da, it, missing);
    else
      run_item_dec<kGateUp, false>(L, da, it, missing);
  }
}

// y[t] = sum_k slot[t*K + k] + slot[T*K + t], fp32, fixed order (4 columns
// per thread; rows of any length: the slot rows have stride SP, a multiple of
// 4; y rows stride H).  A non-finite y raises COLI_STATUS_NONFINITE.
__global__ __launch_bounds__(256) void combine_f32(const float *__restrict__ slot, int T, int H,
                                                   int SP, int K, float *__restrict__ y,
                                                   int32_t *status) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = SP / 4;
  bool bad = false;
  if (i < int64_t(T) * per_row) {
    const int t = int(i / per_row), c = int(i % per_row) * 4;
    float4 acc = *reinterpret_cast<const float4 *>(slot + (int64_t(t) * K) * SP + c);
    for (int k = 1; k < K; ++k) {
      const float4 v = *reinterpret_cast<const float4 *>(slot + (int64_t(t) * K + k) * SP + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const float4 v = *reinterpret_cast<const float4 *>(slot + (int64_t(T) * K + t) * SP + c);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    const float a[4] = {acc.x, acc.y, acc.z, acc.w};
    float *yr = y + int64_t(t) * H;
    if (c + 4 <= H && (H & 3) == 0) {
      *reinterpret_cast<float4 *>(yr + c) = acc;
      bad = !(__builtin_isfinite(a[0]) && __builtin_isfinite(a[1]) && __builtin_isfinite(a[2]) &&
              __builtin_isfinite(a[3]));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < H) {
          yr[c + k] = a[k];
          bad |= !__builtin_isfinite(a[k]);
        }
    }
  }
  if (__any(bad) && (threadIdx.x % 64) == 0) raise_status(status, COLI_STATUS_NONFINITE);
}

template <bool kGateUp>
hipError_t launch_dec_gemm(const LayerDev &L, const Routing &r, int T, const DecArgs &da,
                           int64_t max_items, hipStream_t s) {
  const int64_t cus = cus_of_device();
  const int64_t grid = max_items < 2 * cus ? max_items : 2 * cus;
  dec_gemm<kGateUp><<<dim3(unsigned(grid)), dim3(kThreads), 0, s>>>(L, r, T, da);
  return hipGetLastError();
}


}  // namespace

hipError_t launch_ffn_batch(const LayerDev &L, const float *x, int T, const Routing &r,
                            const BatchBufs &b, float *y, hipStream_t s, hipEvent_t *ev,
                            bool x_staged) {
  const PrefillLayout pl = prefill_layout(L.H, L.I);
  const int64_t TK = int64_t(T) * L.K, R = TK + T;
  const int SP = batch_slot_stride(L.H);
  const int max_units = int((TK < L.E ? TK : L.E) + 1);
  // sum over units of ceil(n_u / 32) <= TK / 32 + routed units + shared chunks
  const int64_t max_chunks = TK / kDMC + max_units + (T + kDMC - 1) / kDMC;
  if (ev) (void)hipEventRecord(ev[0], s);
  if (!x_staged) split_rows<<<dim3(unsigned(T)), 256, 0, s>>>(x, T, L.H, pl.HP, b.xp, b.xs);
  hipError_t e;
  {
    DecArgs da{b.xp, b.xs, b.hf, pl.HP, L.I, T, uint32_t(int64_t(2) * T * pl.HP * 2)};
    e = launch_dec_gemm<true>(L, r, T, da, max_chunks * ((L.I + 127) / 128), s);
    if (e != hipSuccess) return e;
  }
  if (ev) (void)hipEventRecord(ev[1], s);
  if (ev) (void)hipEventRecord(ev[2], s);
  split_rows<<<dim3(unsigned(R)), 256, 0, s>>>(b.hf, int(R), L.I, pl.IP, b.h16, b.hs);
  {
    DecArgs da{b.h16, b.hs, b.slot, pl.IP, SP, int(R), uint32_t(2 * R * pl.IP * 2)};
    e = launch_dec_gemm<false>(L, r, T, da, max_chunks * ((L.H + 255) / 256), s);
    if (e != hipSuccess) return e;
  }
  const int64_t nthr = int64_t(T) * (SP / 4);
  combine_f32<<<dim3(unsigned((nthr + 255) / 256)), 256, 0, s>>>(b.slot, T, L.H, SP, L.K, y,
                                                                 L.status);
  if (ev) (void)hipEventRecord(ev[3], s);
  return hipGetLastError();
}

bool batch_offsets_ok(int H, int I, int K, int T, size_t blob_bytes) {
  const PrefillLayout pl = prefill_layout(H, I);
  const int64_t R = int64_t(T) * K + T;
  const int64_t lim = int64_t(1) << 31;  // buffer offsets: 32 bits, top bit masks
  return int64_t(2) * T * pl.HP * 2 < lim && 2 * R * pl.IP * 2 < lim &&
         int64_t(blob_bytes) < lim;
}

int batch_slot_stride(int H) { return (H + 3) & ~3; }

}  // namespace coli

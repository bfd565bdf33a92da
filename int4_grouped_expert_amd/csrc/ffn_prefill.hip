// ffn_prefill.hip -- the routed + shared expert FFN for large T (prefill):
// int4-g64 dequant-to-fp16 grouped GEMMs on the matrix cores.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 (planar int4-g64 bytes consumed as they are; weight =
// s * (u - 8)); batch union, page "Colibrì 深度解析", section 四 (each unique
// expert is read once per batch and applied to all of its tokens).
//
// Work item = (unit, M-chunk of <= 64 of the unit's tokens, N-tile of output
// rows).  A unit is a unique routed expert of the batch or the shared expert.
// A block has 4 waves; each wave owns 4 MFMA column fragments (16 weight rows
// each) and all M fragments of the chunk, on v_mfma_f32_16x16x32_f16.
//
// K permutation.  A lane's 16-byte weight load covers bytes 16*(q&1)..+15 of
// group 2*kb + (q>>1) of its row (q = lane/16, kb = 128-column block), i.e.
// 32 nibbles.  MFMA step s (0..3) of the block takes 8 of them: s=0 low
// nibbles of bytes 0..7, s=1 low of 8..15, s=2 high of 0..7, s=3 high of
// 8..15.  Element offset within the 128 block: 64*(q>>1) + 16*(q&1) +
// {0, 8, 32, 40}[s] + perm8[i], perm8 = {0,2,1,3,4,6,5,7} (the order in
// which the fp16 pairs fall out of the nibble extraction below).  Because the
// contraction runs over all k, any permutation shared by both operands gives
// the same product; the activations are stored in global memory as fp16 with
// perm8 applied inside every 8-element run, so each (s, q) slot of the A
// operand is one contiguous 16-byte run and LDS staging is a plain copy.
//
// Dequant (2 weights per 32-bit lane op): (d & 0x000F000F) | 0x64006400 is
// the fp16 pair {1024 + u_a, 1024 + u_b}; v_pk_add_f16 with -1032 gives u - 8
// exactly; v_pk_mul_f16 by the fp16 scale gives the weight (one rounding).
//
// Kernels: prefill_prep (x bf16 -> fp16 in the perm8 layout), prefill_tiles
// (M-chunk prefix over units), gateup_prefill (h = SiLU(gate)*up, fp16,
// perm8 layout), down_prefill (gate-scaled per-slot outputs, fp16),
// combine (y = sum of a token's slots + its shared output, bf16).
#include "kernels.h"

#include <hip/hip_fp16.h>

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kMC = 64;             // tokens per M-chunk
constexpr int kMF = kMC / 16;       // M fragments per chunk
constexpr int kKB = 128;            // columns per K block
constexpr int kRowB = kKB * 2 + 16; // LDS bytes per staged row (padded)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack_f16x2(_Float16 a, _Float16 b) {
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Reorder 8 fp16 values held as 4 pairs [01][23][45][67] into perm8 order
// [02][13][46][57]; perm8 is an involution (swap 1<->2 and 5<->6).
__device__ inline uint4 perm8_pairs(uint4 v) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // lo(x), lo(y)
  o.y = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // hi(x), hi(y)
  o.z = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
  o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
  return o;
}

// ------------------------------------------------------------------ prep
// x bf16 [T, H] -> xp fp16 [T, H], perm8 inside each 8-run.
__global__ __launch_bounds__(256) void prefill_prep(const uint16_t *__restrict__ x,
                                                    int64_t n8,
                                                    uint16_t *__restrict__ xp) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4 *>(x)[i];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = __uint_as_float(w[k] << 16);
    const float b = __uint_as_float(w[k] & 0xFFFF0000u);
    h[k] = pack_f16x2(_Float16(a), _Float16(b));
  }
  reinterpret_cast<uint4 *>(xp)[i] = perm8_pairs(uint4{h[0], h[1], h[2], h[3]});
}

// ------------------------------------------------------------------ tiles
// tiles[u] = number of M-chunks of units < u; tiles[nu] = total.  Unit u <
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
    // block exclusive scan of v
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
__device__ inline bool decode_item(const LayerDev &L, const Routing &r, int T, int item,
                                   int n_nt, Item &it) {
  const int nu = *r.n_unique + 1;
  const int total = r.chunk[nu] * n_nt;
  if (item >= total) return false;
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
  return true;
}

// XCD-aware order: the hardware deals consecutive blocks round-robin over 8
// XCDs; give each XCD a contiguous range of items so that the N-tiles of one
// (unit, M-chunk) -- which share the A tile -- meet in one L2.
__device__ inline int xcd_remap(int i, int n) {
  const int n8 = n & ~7;
  if (i >= n8) return i;
  return (i & 7) * (n8 >> 3) + (i >> 3);
}

// Stage one 128-column block of up to 64 A rows into LDS.
// Thread t copies 16-byte runs c = t % 16 of rows m = t/16 + 16*pass.
struct AStage {
  uint4 v[4];
};
__device__ inline void a_load(const uint16_t *__restrict__ A, int64_t lda, int Kdim,
                              const int64_t *rowoff, int kb, AStage &st) {
  const int c = threadIdx.x % 16;
  const int k = kb * kKB + c * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t ro = rowoff[p];
    if (ro >= 0 && k < Kdim)
      st.v[p] = *reinterpret_cast<const uint4 *>(A + ro + k);
    else
      st.v[p] = uint4{0u, 0u, 0u, 0u};
  }
}
__device__ inline void a_store(uint8_t *lds, const AStage &st) {
  const int c = threadIdx.x % 16;
  const int q = (c >> 3) * 2 + ((c & 3) >> 1);
  const int s = ((c & 7) >> 2) * 2 + (c & 1);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int m = threadIdx.x / 16 + 16 * p;
    *reinterpret_cast<uint4 *>(lds + m * kRowB + (s * 4 + q) * 16) = st.v[p];
  }
}

// B fragment source: 16 weight rows of one matrix.
struct BFrag {
  const uint8_t *q;  // packed row base for this lane's row
  const float *s;    // scale row base for this lane's row
  bool valid;        // row inside the matrix
};
struct BRaw {
  uint4 w;
  float s;
};
__device__ inline BRaw b_load(const BFrag &f, int kb, int64_t G) {
  const int lane = threadIdx.x % kWave;
  const int q = lane / 16;
  const int64_t g = int64_t(kb) * 2 + (q >> 1);
  BRaw r;
  if (f.valid && g < G) {
    r.w = *reinterpret_cast<const uint4 *>(f.q + g * 32 + 16 * (q & 1));
    r.s = f.s[g];
  } else {
    r.w = uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
    r.s = 0.0f;
  }
  return r;
}

// fp16 weights of MFMA step s from the 16 raw bytes (see the header comment).
__device__ inline f16x8 b_dequant(const BRaw &r, int s) {
  const uint32_t d[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
  const uint32_t da = d[(s & 1) * 2], db = d[(s & 1) * 2 + 1];
  const int sh = (s >> 1) * 4;  // 0 for low nibbles, 4 for high nibbles
  const uint32_t M = 0x000F000Fu, X = 0x64006400u;
  uint32_t p[4];
  p[0] = ((da >> sh) & M) | X;
  p[1] = ((da >> (sh + 8)) & M) | X;
  p[2] = ((db >> sh) & M) | X;
  p[3] = ((db >> (sh + 8)) & M) | X;
  const _Float16 sc = _Float16(r.s);
  const f16x2 off = {_Float16(-1032.0f), _Float16(-1032.0f)};
  const f16x2 scv = {sc, sc};
  f16x8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 v = __builtin_bit_cast(f16x2, p[i]);
    v = (v + off) * scv;
    out[2 * i] = v[0];
    out[2 * i + 1] = v[1];
  }
  return out;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// position of column o in the perm8 layout
__device__ inline int perm8_pos(int o) {
  const int r = o & 7;
  const int pr = (r == 1) ? 2 : (r == 2) ? 1 : (r == 5) ? 6 : (r == 6) ? 5 : r;
  return (o & ~7) | pr;
}

// ------------------------------------------------------------------ GEMMs
// kGateUp: A = xp [T, H] (token rows gathered through perm), B = gate/up
// [I, H], N-tile = 128 output rows (per wave 32: gate rows in fragments 0-1,
// up rows in 2-3), epilogue h = SiLU(gate) * up -> hp (fp16, perm8 layout).
// !kGateUp: A = hp [T*K + T, I], B = down [H, I], N-tile = 256 output rows
// (per wave 64), epilogue gate * out -> slot_out (fp16).
template <bool kGateUp>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(
    LayerDev L, Routing r, int T, const uint16_t *__restrict__ A,
    uint16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kMC * kRowB];
  __shared__ int64_t rowoff_s[kMC];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int K = L.K;
  const int Kdim = kGateUp ? L.H : L.I;
  const int Nrows = kGateUp ? L.I : L.H;
  const int64_t G = kGateUp ? L.lay.GH : L.lay.GI;
  const int ntile_rows = kGateUp ? 128 : 256;
  const int n_nt = (Nrows + ntile_rows - 1) / ntile_rows;
  const int nkb = (Kdim + kKB - 1) / kKB;
  const int nu = *r.n_unique + 1;
  const int n_items = r.chunk[nu] * n_nt;

  for (int it0 = blockIdx.x; it0 < n_items; it0 += gridDim.x) {
    Item it;
    decode_item(L, r, T, xcd_remap(it0, n_items), n_nt, it);
    const int nrows = it.je - it.jb;
    const int nmf = (nrows + 15) / 16;
    // A row offsets (element units) for the chunk's rows; -1 = padding row
    __syncthreads();
    if (threadIdx.x < kMC) {
      const int j = it.jb + threadIdx.x;
      int64_t ro = -1;
      if (j < it.je) {
        int64_t row;
        if (kGateUp) row = it.shared ? j : r.perm[j] / K;
        else row = it.shared ? int64_t(T) * K + j : j;
        ro = row * Kdim;
      }
      rowoff_s[threadIdx.x] = ro;
    }
    __syncthreads();
    int64_t rowoff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) rowoff[p] = rowoff_s[threadIdx.x / 16 + 16 * p];

    // B fragments of this wave
    BFrag bf[4];
    const int n16 = lane % 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row;
      const uint8_t *qbase;
      const float *sbase;
      if (kGateUp) {
        row = it.ntile * 128 + wave * 32 + 16 * (j & 1) + n16;
        qbase = it.blob + (j < 2 ? L.lay.gq : L.lay.uq);
        sbase = reinterpret_cast<const float *>(it.blob + (j < 2 ? L.lay.gs : L.lay.us));
      } else {
        row = it.ntile * 256 + wave * 64 + 16 * j + n16;
        qbase = it.blob + L.lay.dq;
        sbase = reinterpret_cast<const float *>(it.blob + L.lay.ds);
      }
      bf[j].valid = row < Nrows;
      const int rr = bf[j].valid ? row : 0;
      bf[j].q = qbase + int64_t(rr) * G * 32;
      bf[j].s = sbase + int64_t(rr) * G;
    }

    f32x4 acc[kMF][4];
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mf][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    AStage ast;
    a_load(A, Kdim, Kdim, rowoff, 0, ast);
    BRaw braw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) braw[j] = b_load(bf[j], 0, G);

    for (int kb = 0; kb < nkb; ++kb) {
      uint8_t *buf = lds[kb & 1];
      a_store(buf, ast);
      __syncthreads();
      if (kb + 1 < nkb) a_load(A, Kdim, Kdim, rowoff, kb + 1, ast);
      BRaw bnext[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bnext[j] = (kb + 1 < nkb) ? b_load(bf[j], kb + 1, G) : braw[j];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = b_dequant(braw[j], s);
#pragma unroll
        for (int mf = 0; mf < kMF; ++mf) {
          if (mf < nmf) {
            const f16x8 a = *reinterpret_cast<const f16x8 *>(
                buf + (mf * 16 + lane % 16) * kRowB + (s * 4 + lane / 16) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mf][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[mf][j], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) braw[j] = bnext[j];
    }

    // epilogue: lane holds rows m = 16*mf + 4*(lane/16) + i, column n16
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf) {
      if (mf >= nmf) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mf * 16 + 4 * (lane / 16) + i;
        const int j = it.jb + m;
        if (j >= it.je) continue;
        if (kGateUp) {
          const int64_t hrow = it.shared ? int64_t(T) * K + j : j;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int o = it.ntile * 128 + wave * 32 + 16 * jj + n16;
            if (o < Nrows) {
              const float hv = silu(acc[mf][jj][i]) * acc[mf][jj + 2][i];
              out[hrow * Nrows + perm8_pos(o)] = __builtin_bit_cast(uint16_t, _Float16(hv));
            }
          }
        } else {
          int64_t srow;
          float gate;
          if (it.shared) {
            srow = int64_t(T) * K + j;
            gate = 1.0f;
          } else {
            const int p = r.perm[j];
            srow = p;
            gate = r.gates[p];
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int o = it.ntile * 256 + wave * 64 + 16 * jj + n16;
            if (o < Nrows)
              out[srow * Nrows + o] =
                  __builtin_bit_cast(uint16_t, _Float16(gate * acc[mf][jj][i]));
          }
        }
      }
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
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ slot,
                                                      int T, int H, int K,
                                                      uint16_t *__restrict__ y) {
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
    o[q] = uint32_t(f32_to_bf16_rne(acc[2 * q])) | (uint32_t(f32_to_bf16_rne(acc[2 * q + 1])) << 16);
  *reinterpret_cast<uint4 *>(y + int64_t(t) * H + c) = uint4{o[0], o[1], o[2], o[3]};
}

}  // namespace

hipError_t launch_ffn_prefill(const LayerDev &L, const uint16_t *x, int T,
                              const Routing &r, uint16_t *h,
                              uint16_t *slot_out, uint16_t *y, hipStream_t s,
                              hipEvent_t *ev) {
  // xp (the fp16 perm8 copy of x) lives in slot_out's space: slot_out is
  // first written by the down GEMM, after the gate/up GEMM has consumed xp.
  uint16_t *xp = slot_out;
  const int64_t n8 = int64_t(T) * L.H / 8;
  if (ev) (void)hipEventRecord(ev[0], s);
  prefill_prep<<<dim3(unsigned((n8 + 255) / 256)), 256, 0, s>>>(x, n8, xp);
  prefill_tiles<<<1, 1024, 0, s>>>(r, T);
  if (ev) (void)hipEventRecord(ev[1], s);
  const int max_units = (T * L.K < L.E ? T * L.K : L.E) + 1;
  // upper bound of M-chunks: every routed pair alone in its chunk is not
  // possible; sum ceil(n/64) <= T*K/64 + routed units, plus the shared chunks
  const int64_t max_chunks = int64_t(T) * L.K / kMC + max_units + (T + kMC - 1) / kMC;
  const int cap = 2048;
  if (ev) (void)hipEventRecord(ev[2], s);
  {
    const int64_t items = max_chunks * ((L.I + 127) / 128);
    grouped_gemm_kernel<true><<<unsigned(items < cap ? items : cap), 256, 0, s>>>(L, r, T, xp, h);
  }
  if (ev) (void)hipEventRecord(ev[3], s);
  if (ev) (void)hipEventRecord(ev[4], s);
  {
    const int64_t items = max_chunks * ((L.H + 255) / 256);
    grouped_gemm_kernel<false><<<unsigned(items < cap ? items : cap), 256, 0, s>>>(L, r, T, h,
                                                                                  slot_out);
  }
  if (ev) (void)hipEventRecord(ev[5], s);
  const int64_t nthr = int64_t(T) * (L.H / 8);
  if (ev) (void)hipEventRecord(ev[6], s);
  combine_kernel<<<dim3(unsigned((nthr + 255) / 256)), 256, 0, s>>>(slot_out, T, L.H, L.K, y);
  if (ev) (void)hipEventRecord(ev[7], s);
  return hipGetLastError();
}

}  // namespace coli

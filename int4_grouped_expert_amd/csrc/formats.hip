// formats.hip -- the sibling weight formats of the registry: byte arithmetic,
// inference of a tensor's format from its byte counts, quantisers, and a
// dequantising matrix-vector product for decode (y[t] = W^ x[t], T <= 8).
//
// Registry and inference: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 (0 f32, 1 int8-row, 2 int4-row, 3 int2-row, 4 int4-grouped,
// 5 int3-g64, 6 E8/IQ3, 7 MXFP4, 8 fp8-e4m3-b128; the format follows from the
// weight bytes, the scale bytes and [O, I] alone).  Raw f32 has no scale array
// (page "Colibrì 深度解析", section 十五).  int3 with a per-group scale is 3.5 bits
// per weight (same page, section 八); the quantised matrix kernels from int4 to
// MXFP4: section 十.  MXFP4 follows the OCP Microscaling (MX) v1.0 specification
// (32 E2M1 elements, one E8M0 scale, the shared exponent floor(log2 amax) - 2,
// elements rounded to nearest even and saturated at 6); E4M3 the OCP FP8
// specification (bias 7, largest finite 448).
//
// Layouts (the formats' names fix no byte order; these are this library's):
//   int3-g64: a group of 64 codes u = q + 4 is 24 bytes, three little-endian
//             64-bit bit planes (bit j of plane p = bit p of u[j]); f32 scale
//             per group, s = amax / 3, q = clip(rint(w / s), -4, 3).
//   MXFP4:    a block of 32 is 16 bytes, element 2j in the low nibble of byte j;
//             nibble = sign << 3 | E2M1 code; one E8M0 byte per block.
//   fp8-b128: E4M3 codes row-major [O, I]; one f32 scale per 128 x 128 tile,
//             s = amax / 448.
// Non-finite inputs: the group / block / tile gets the NaN scale (E8M0 255) and
// neutral codes, and the status flag bit 1 is raised.
//
// The matrix-vector product streams each row's bytes once with 16-byte (8-byte
// for int3) loads, one chunk ahead; x sits in LDS; a wave works on four or
// eight rows at a time so that each x value read from LDS serves them all; the
// per-chunk (= per scale) sums are scaled once; every lane reduces in a fixed
// order, so results are deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "coli.h"
#include "wave.h"

namespace coli {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxT = 8;
constexpr int kXFloats = 24576;  // T * padded I: 96 KiB of LDS

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool fmt_sizes(int fmt, int64_t O, int64_t I, uint64_t *w, uint64_t *s) {
  const int64_t G = cdiv(I, 64);
  switch (fmt) {
    case COLI_FMT_F32: *w = uint64_t(4 * O * I); *s = 0; return true;
    case COLI_FMT_INT8_ROW: *w = uint64_t(O * I); *s = uint64_t(4 * O); return true;
    case COLI_FMT_INT4_ROW: *w = uint64_t(O * cdiv(I, 2)); *s = uint64_t(4 * O); return true;
    case COLI_FMT_INT2_ROW: *w = uint64_t(O * cdiv(I, 4)); *s = uint64_t(4 * O); return true;
    case COLI_FMT_INT4_G64: *w = uint64_t(32 * O * G); *s = uint64_t(4 * O * G); return true;
    case COLI_FMT_INT3_G64: *w = uint64_t(24 * O * G); *s = uint64_t(4 * O * G); return true;
    case COLI_FMT_MXFP4: *w = uint64_t(16 * O * cdiv(I, 32)); *s = uint64_t(O * cdiv(I, 32));
      return true;
    case COLI_FMT_FP8_E4M3_B128: *w = uint64_t(O * I);
      *s = uint64_t(4 * cdiv(O, 128) * cdiv(I, 128)); return true;
    default: return false;  // E8/IQ3 and unknown ordinals
  }
}

bool dims_ok(int64_t O, int64_t I) {
  return O >= 1 && O <= COLI_FMT_MAX_ROWS && I >= 1 && I <= COLI_MAX_DIM;
}

// ------------------------------------------------------------------ quantisers

// int3-g64: one wave per group; lane j holds element j.  The bit planes are
// the ballots of each code bit.
__global__ __launch_bounds__(256) void quant_int3(const float *__restrict__ w, int64_t O, int I,
                                                  int G, uint8_t *__restrict__ packed,
                                                  float *__restrict__ scales,
                                                  int32_t *__restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (grp >= O * G) return;  // whole waves
  const int64_t o = grp / G;
  const int g = int(grp - o * G);
  const int col = g * 64 + lane;
  const float v = col < I ? w[o * I + col] : 0.0f;
  const bool bad = __ballot(!__builtin_isfinite(v)) != 0;
  const float amax = wave_max(fabsf(v));
  const float s = bad ? __builtin_nanf("") : amax / 3.0f;
  int u = 4;
  if (!bad && s != 0.0f) u = int(fminf(fmaxf(rintf(v / s), -4.0f), 3.0f)) + 4;
  const uint64_t p0 = __ballot(u & 1), p1 = __ballot(u & 2), p2 = __ballot(u & 4);
  uint64_t *dst = reinterpret_cast<uint64_t *>(packed + grp * 24);
  if (lane == 0) dst[0] = p0;
  if (lane == 1) dst[1] = p1;
  if (lane == 2) dst[2] = p2;
  if (lane == 3) scales[grp] = s;
  if (lane == 4 && bad && status) atomicOr(status, 1);
}

// E2M1 magnitude code of a (|v| / X, >= 0), round to nearest even, saturating.
__device__ inline uint32_t e2m1_code(float a) {
  return uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) +
         uint32_t(a >= 1.75f) + uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
}

// MXFP4: one half-wave per block of 32; lane i holds element i.
__global__ __launch_bounds__(256) void quant_mxfp4(const float *__restrict__ w, int64_t O, int I,
                                                   int NB, uint8_t *__restrict__ packed,
                                                   uint8_t *__restrict__ scales,
                                                   int32_t *__restrict__ status) {
  const int lane = threadIdx.x & 63, li = lane & 31;
  const int64_t blk = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool live = blk < O * NB;
  const int64_t o = live ? blk / NB : 0;
  const int b = live ? int(blk - o * NB) : 0;
  const int col = b * 32 + li;
  const float v = (live && col < I) ? w[o * I + col] : 0.0f;
  int bad = !__builtin_isfinite(v);
  float amax = fabsf(v);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) {  // within the half-wave
    bad |= __shfl_xor(bad, m, 64);
    amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  }
  uint32_t E = 0, nib = 0;
  if (bad) {
    E = 255;
  } else if (amax != 0.0f) {
    const int ef = int((__float_as_uint(amax) >> 23) & 255u);
    const int fl = ef ? ef - 127 : -127;  // floor(log2 amax), subnormals clamp below
    const int shared = fl - 2 < -127 ? -127 : fl - 2;
    E = uint32_t(shared + 127);
    const float inv = __uint_as_float(uint32_t(127 - shared) << 23);  // 2^-shared, normal
    const float r = v * inv;  // exact: a power-of-two scaling
    nib = (__float_as_uint(v) >> 31) << 3 | e2m1_code(fminf(fabsf(r), 6.0f));
  }
  // eight nibbles per 32-bit word: lanes 8m .. 8m+7 -> word m of the block
  uint32_t word = nib << (4 * (li & 7));
#pragma unroll
  for (int m = 1; m <= 4; m <<= 1) word |= __shfl_xor(word, m, 64);
  if (live && (li & 7) == 0)
    reinterpret_cast<uint32_t *>(packed + blk * 16)[li >> 3] = word;
  if (live && li == 0) {
    scales[blk] = uint8_t(E);
    if (bad && status) atomicOr(status, 1);
  }
}

// fp8-b128, pass 1: one block per 128 x 128 tile -> its scale.
__global__ __launch_bounds__(256) void fp8_tile_scales(const float *__restrict__ w, int64_t O,
                                                       int I, int TI, float *__restrict__ scales,
                                                       int32_t *__restrict__ status) {
  const int64_t ta = blockIdx.x / TI;
  const int tb = int(blockIdx.x - ta * TI);
  const int64_t r0 = ta * 128;
  const int c0 = tb * 128;
  const int nr = int(O - r0 < 128 ? O - r0 : 128), nc = I - c0 < 128 ? I - c0 : 128;
  float amax = 0.0f;
  int bad = 0;
  for (int i = threadIdx.x; i < nr * 128; i += 256) {
    const int r = i >> 7, c = i & 127;
    if (c < nc) {
      const float v = w[(r0 + r) * I + c0 + c];
      bad |= !__builtin_isfinite(v);
      amax = fmaxf(amax, fabsf(v));
    }
  }
  __shared__ float sm[4];
  __shared__ int sb[4];
  amax = wave_max(amax);
  bad = __ballot(bad) != 0;
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wv] = amax;
    sb[wv] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float a = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    const int anybad = sb[0] | sb[1] | sb[2] | sb[3];
    scales[blockIdx.x] = anybad ? __builtin_nanf("") : a / 448.0f;
    if (anybad && status) atomicOr(status, 1);
  }
}

// E4M3 code of a in [0, 448], round to nearest even.
__device__ inline uint32_t e4m3_code(float a) {
  if (a < 0x1p-6f) return uint32_t(rintf(a * 512.0f));  // subnormal steps of 2^-9
  const uint32_t b = __float_as_uint(a);
  return ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
}

// fp8-b128, pass 2: one thread per element.
__global__ __launch_bounds__(256) void fp8_codes(const float *__restrict__ w, int64_t O, int I,
                                                 int TI, const float *__restrict__ scales,
                                                 uint8_t *__restrict__ codes) {
  const int64_t n = O * I;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / I;
    const int c = int(i - r * I);
    const float s = scales[(r >> 7) * TI + (c >> 7)];
    uint32_t code = 0;
    if (s > 0.0f) {  // false for a zero or NaN scale
      const float v = w[i];
      code = (__float_as_uint(v) >> 31) << 7 | e4m3_code(fminf(fabsf(v / s), 448.0f));
    }
    codes[i] = uint8_t(code);
  }
}

// ------------------------------------------------------------------ matvec

template <int FMT>
struct Chunk;  // one lane's unit of a row: bytes, weights, one scale
template <>
struct Chunk<COLI_FMT_FP8_E4M3_B128> {
  static constexpr int kBytes = 16, kW = 16;
};
template <>
struct Chunk<COLI_FMT_MXFP4> {
  static constexpr int kBytes = 16, kW = 32;
};
template <>
struct Chunk<COLI_FMT_INT3_G64> {
  static constexpr int kBytes = 24, kW = 64;
};
template <>
struct Chunk<COLI_FMT_INT4_G64> {
  static constexpr int kBytes = 32, kW = 64;
};

// The chunk's raw bytes (as 32-bit words).
template <int FMT>
struct Raw {
  uint32_t v[Chunk<FMT>::kBytes / 4];
};

template <int FMT>
__device__ inline Raw<FMT> load_chunk(const uint8_t *p) {
  Raw<FMT> r;
  if constexpr (Chunk<FMT>::kBytes % 16 == 0) {
#pragma unroll
    for (int q = 0; q < Chunk<FMT>::kBytes / 16; ++q) {
      const uint4 u = *reinterpret_cast<const uint4 *>(p + 16 * q);
      r.v[4 * q] = u.x;
      r.v[4 * q + 1] = u.y;
      r.v[4 * q + 2] = u.z;
      r.v[4 * q + 3] = u.w;
    }
  } else {  // int3: three 8-byte planes
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const uint2 u = *reinterpret_cast<const uint2 *>(p + 8 * q);
      r.v[2 * q] = u.x;
      r.v[2 * q + 1] = u.y;
    }
  }
  return r;
}

// Byte K of u as a float: one v_cvt_f32_ubyteK (written out, since the
// compiler otherwise folds a preceding mask into a bit-field extract plus a
// conversion).  A plain VALU instruction, no memory access.
template <int K>
__device__ inline float ubyte(uint32_t u) {
  float f;
  if constexpr (K == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(u));
  else if constexpr (K == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(u));
  else if constexpr (K == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(u));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(u));
  return f;
}

// 4 three-bit codes -> one byte each: bits 4m..4m+3 of the three planes.
__device__ inline uint32_t int3_bytes(const uint32_t (&v)[6], int m) {
  const int word = m >> 3, sh = 4 * (m & 7);
  uint32_t out = 0;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const uint32_t nib = (v[2 * p + word] >> sh) & 15u;
    out |= ((nib * 0x00204081u) & 0x01010101u) << p;  // bit k -> byte k
  }
  return out;
}

// Codes of the chunk as floats, piece by piece (4 or 8 weights), in the
// format's own units (E2M1 / E4M3 values, or the unsigned integer codes).
template <int FMT>
struct Piece;
template <>
struct Piece<COLI_FMT_FP8_E4M3_B128> {  // 4 pieces of 4 weights
  static constexpr int kN = 4, kW = 4;
  __device__ static void get(const Raw<COLI_FMT_FP8_E4M3_B128> &r, int q, float (&f)[4]) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(r.v[q], false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(r.v[q], true);
    f[0] = a.x;
    f[1] = a.y;
    f[2] = b.x;
    f[3] = b.y;
  }
  __device__ static int xoff(int q, int k) { return 4 * q + k; }
};
template <>
struct Piece<COLI_FMT_MXFP4> {  // 4 pieces of 8 weights
  static constexpr int kN = 4, kW = 8;
  __device__ static void get(const Raw<COLI_FMT_MXFP4> &r, int q, float (&f)[8]) {
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v[q], 1.0f, 0);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v[q], 1.0f, 1);
    const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v[q], 1.0f, 2);
    const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v[q], 1.0f, 3);
    f[0] = a.x;
    f[1] = a.y;
    f[2] = b.x;
    f[3] = b.y;
    f[4] = c.x;
    f[5] = c.y;
    f[6] = e.x;
    f[7] = e.y;
  }
  __device__ static int xoff(int q, int k) { return 8 * q + k; }
};
template <>
struct Piece<COLI_FMT_INT3_G64> {  // 16 pieces of 4 weights
  static constexpr int kN = 16, kW = 4;
  __device__ static void get(const Raw<COLI_FMT_INT3_G64> &r, int m, float (&f)[4]) {
    const uint32_t u = int3_bytes(r.v, m);
    f[0] = ubyte<0>(u);
    f[1] = ubyte<1>(u);
    f[2] = ubyte<2>(u);
    f[3] = ubyte<3>(u);
  }
  __device__ static int xoff(int m, int k) { return 4 * m + k; }
};
template <>
struct Piece<COLI_FMT_INT4_G64> {  // 8 pieces of 8 weights: 4 low nibbles (k..k+3), 4 high (k+32..)
  static constexpr int kN = 8, kW = 8;
  __device__ static void get(const Raw<COLI_FMT_INT4_G64> &r, int q, float (&f)[8]) {
    const uint32_t lo = r.v[q] & 0x0F0F0F0Fu, hi = (r.v[q] >> 4) & 0x0F0F0F0Fu;
    f[0] = ubyte<0>(lo);
    f[1] = ubyte<1>(lo);
    f[2] = ubyte<2>(lo);
    f[3] = ubyte<3>(lo);
    f[4] = ubyte<0>(hi);
    f[5] = ubyte<1>(hi);
    f[6] = ubyte<2>(hi);
    f[7] = ubyte<3>(hi);
  }
  __device__ static int xoff(int q, int k) { return k < 4 ? 4 * q + k : 32 + 4 * q + (k - 4); }
};

// d[r][t] = sum_k code[r]_k * x[t]_k over one chunk of R rows: each piece of x
// is read from LDS once and serves the R rows.  x is held piece-major in LDS:
// float4 piece p (elements 4p .. 4p+3) of chunk c of token t at
// x4[(t * pieces + p) * chunks + c], so the 64 lanes (64 consecutive chunks)
// read 64 consecutive float4s, free of bank conflicts.  xc = x4 + c; pstride =
// chunks.
template <int FMT, int T, int R>
__device__ inline void chunk_dot_rows(const Raw<FMT> (&raw)[R], const float4 *xc, int pstride,
                                      float (&d)[R][T]) {
  constexpr int kPieces = Chunk<FMT>::kW / 4;
  using P = Piece<FMT>;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < T; ++t) d[r][t] = 0.0f;
#pragma unroll
  for (int q = 0; q < P::kN; ++q) {
    float f[R][P::kW];
#pragma unroll
    for (int r = 0; r < R; ++r) P::get(raw[r], q, f[r]);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float x[P::kW];
#pragma unroll
      for (int k = 0; k < P::kW; k += 4) {
        const float4 v = xc[(t * kPieces + P::xoff(q, k) / 4) * pstride];
        x[k] = v.x;
        x[k + 1] = v.y;
        x[k + 2] = v.z;
        x[k + 3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < P::kW; ++k) d[r][t] = fmaf(f[r][k], x[k], d[r][t]);
    }
  }
}

struct MatvecArgs {
  const uint8_t *packed;
  const void *scales;
  int64_t O;         // rows (gate/up mode: features)
  int I, ldx;        // I: row length; ldx: padded row length of x in LDS (chunks * weights)
  int chunks;        // chunks per row
  int64_t row_bytes;
  int scale_cols;    // fp8: tiles per row of tiles; others: scales per row
  const float *x;
  float *y;
  // grouped modes (one unit per blockIdx.y: the batch's unique experts in
  // ascending id, then the shared expert)
  const uint8_t *experts, *shared;
  size_t blob_bytes;
  size_t q_off[2], s_off[2];  // gate/up mode: gate and up sections; down: [0]
  const int32_t *unique, *n_unique;
  const int32_t *idx;         // [T][K] routed ids and their gates
  const float *gates;
  int K;
  float *h;                   // [units][T][I_ffn]: gate/up output, down input
  float *part;                // [units][T][H]: down output
};

enum { kModePlain = 0, kModeGateUp = 1, kModeDown = 2 };

// The raw scale of chunk c of row o0 + rr: the f32 bits, or the E8M0 byte
// (decoded at use by scale_value, so that the load is not waited for when it
// is issued).  o0 is wave-uniform and a multiple of the rows per step (4 or
// 8), so an fp8 group of rows never straddles a 128-row tile.
template <int FMT>
__device__ inline uint32_t chunk_scale(const void *sbase, int scale_cols, int64_t o0, int rr,
                                       int c) {
  constexpr int CW = Chunk<FMT>::kW;
  if constexpr (FMT == COLI_FMT_FP8_E4M3_B128) {
    const uint32_t *base = reinterpret_cast<const uint32_t *>(sbase) + (o0 >> 7) * scale_cols;
    return base[(c * CW) >> 7];
  } else if constexpr (FMT == COLI_FMT_MXFP4) {
    const uint8_t *base = reinterpret_cast<const uint8_t *>(sbase) + o0 * scale_cols;
    return base[uint32_t(rr * scale_cols + c)];
  } else {
    const uint32_t *base = reinterpret_cast<const uint32_t *>(sbase) + o0 * scale_cols;
    return base[uint32_t(rr * scale_cols + c)];
  }
}

// The scale as a float.  E8M0: 2^(E - 127); E = 0 is 2^-127 (an fp32
// subnormal, bit 22), E = 255 NaN (the exponent field all ones plus bit 22).
template <int FMT>
__device__ inline float scale_value(uint32_t raw) {
  if constexpr (FMT == COLI_FMT_MXFP4) {
    return __uint_as_float((raw << 23) | ((raw == 0u || raw == 255u) ? 0x00400000u : 0u));
  } else {
    return __uint_as_float(raw);
  }
}

// Rows per wave step: eight for fp8 at T <= 2 (16 weights per 16-byte chunk) and
// for MXFP4 at T <= 2 in the layer's stages (measured: 2 % faster there, slower
// for one plain product), else four (the register budget of the wider chunks).
template <int FMT, int T, int MODE>
constexpr int rows_per_step() {
  return (T <= 2 && (FMT == COLI_FMT_FP8_E4M3_B128 ||
                     (FMT == COLI_FMT_MXFP4 && MODE != kModePlain)))
             ? 8
             : 4;
}

// y[t, o] = sum_i W^[o, i] x[t, i].  A wave takes R rows at a time; lane l
// takes the row chunks l, l + 64, ... (kc steps, the same count on every lane;
// lanes past the row's end re-read its last chunk and add nothing).  The
// next step's chunks and scales are loaded before the current step is
// computed.  Per-chunk dot products are scaled by the chunk's scale (and, for
// the offset formats, corrected by the chunk's x sum times the code offset),
// then reduced over the wave.
//
// MODE kModePlain: one matrix (packed, scales), x [T][I] -> y [T][O].
// MODE kModeGateUp: unit blockIdx.y of a layer; a step takes R/2 features of
//   the gate matrix and the same features of the up matrix, x = the tokens
//   [T][H], and writes h[unit][t][f] = SiLU(gate) * up * w_t (w_t: the token's
//   gate weight for this unit, 0 when the token did not route to it, 1 for the
//   shared expert).
// MODE kModeDown: unit blockIdx.y; the down matrix, x = h[unit] [T][I], writes
//   part[unit][t][o].
template <int FMT, int T, int MODE>
__global__ __launch_bounds__(256) void matvec_kernel(MatvecArgs a) {
  constexpr int CW = Chunk<FMT>::kW, CB = Chunk<FMT>::kBytes;
  constexpr int R = rows_per_step<FMT, T, MODE>();
  constexpr int RM = MODE == kModeGateUp ? R / 2 : R;  // rows of one matrix per step
  constexpr bool kOffset = FMT == COLI_FMT_INT3_G64 || FMT == COLI_FMT_INT4_G64;
  constexpr float kOff = FMT == COLI_FMT_INT3_G64 ? 4.0f : 8.0f;
  extern __shared__ float xs[];  // x piece-major [T][pieces][chunks][4], then the chunk sums [T][chunks]
  __shared__ float wtok[T];      // gate/up mode: the tokens' gate weights for the unit
  float *xsum = xs + T * a.ldx;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // the matrices of this block
  const uint8_t *pk[2] = {a.packed, a.packed};
  const void *sb[2] = {a.scales, a.scales};
  const float *xsrc = a.x;
  int unit = 0;
  if constexpr (MODE != kModePlain) {
    unit = int(blockIdx.y);
    const int nu = *a.n_unique;
    if (unit > nu) return;  // whole block, before any barrier
    const int e = unit < nu ? a.unique[unit] : -1;
    const uint8_t *blob = e >= 0 ? a.experts + size_t(e) * a.blob_bytes : a.shared;
    pk[0] = blob + a.q_off[0];
    sb[0] = blob + a.s_off[0];
    pk[1] = blob + a.q_off[1];
    sb[1] = blob + a.s_off[1];
    if constexpr (MODE == kModeGateUp) {
      if (threadIdx.x < T) {
        float w = e < 0 ? 1.0f : 0.0f;
        for (int k = 0; k < a.K; ++k)
          if (e >= 0 && a.idx[threadIdx.x * a.K + k] == e) w = a.gates[threadIdx.x * a.K + k];
        wtok[threadIdx.x] = w;
      }
    } else {
      xsrc = a.h + size_t(unit) * T * a.I;
    }
  }

  const int64_t groups = (a.O + RM - 1) / RM;
  const int64_t gstride = int64_t(gridDim.x) * 4;
  const int kc = (a.chunks + 63) / 64;
  int64_t g = int64_t(blockIdx.x) * 4 + wave;
  int k = 0;

  Raw<FMT> cur[R], nxt[R];
  uint32_t csc[R], nsc[R];
  // Loads of step (gg, kk): a wave-uniform 64-bit base for the group's first
  // row of each matrix, 32-bit offsets for the rows (clamped to the last row:
  // rows past the end are re-read, never stored) and the chunk (clamped to the
  // row's last chunk on lanes past the row's end).
  auto fetch = [&](int64_t gg, int kk, Raw<FMT>(&dst)[R], uint32_t(&sc)[R]) {
    const int64_t o0 = gg * RM;
    const int last = int(a.O - 1 - o0);  // rows of the group that exist: r <= last
    const int c0 = lane + 64 * kk;
    const int c = c0 < a.chunks ? c0 : a.chunks - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m = r / RM;  // 0: gate (or the only matrix), 1: up
      const int ri = r - m * RM;
      const int rr = ri < last ? ri : last;
      const uint8_t *base = pk[m] + o0 * a.row_bytes;
      dst[r] = load_chunk<FMT>(base + uint32_t(rr * int(a.row_bytes) + c * CB));
      sc[r] = chunk_scale<FMT>(sb[m], a.scale_cols, o0, rr, c);
    }
  };
  // the first weights are in flight while x is staged
  if (g < groups) fetch(g, 0, cur, csc);

  // x -> LDS piece-major (see chunk_dot_rows); the zero padding past I
  // completes the last chunk
  constexpr int kPieces = CW / 4;
  float4 *x4 = reinterpret_cast<float4 *>(xs);
  for (int i = threadIdx.x; i < T * kPieces * a.chunks; i += 256) {
    const int c = i % a.chunks, tp = i / a.chunks;
    const int t = tp / kPieces, pc = tp - t * kPieces;
    const int k0 = c * CW + 4 * pc;
    float4 v;
    v.x = k0 < a.I ? xsrc[size_t(t) * a.I + k0] : 0.0f;
    v.y = k0 + 1 < a.I ? xsrc[size_t(t) * a.I + k0 + 1] : 0.0f;
    v.z = k0 + 2 < a.I ? xsrc[size_t(t) * a.I + k0 + 2] : 0.0f;
    v.w = k0 + 3 < a.I ? xsrc[size_t(t) * a.I + k0 + 3] : 0.0f;
    x4[i] = v;
  }
  __syncthreads();
  if constexpr (kOffset) {
    for (int i = threadIdx.x; i < T * a.chunks; i += 256) {
      const int t = i / a.chunks, c = i - t * a.chunks;
      float s = 0.0f;
      for (int pc = 0; pc < kPieces; ++pc) {  // fixed order
        const float4 v = x4[(t * kPieces + pc) * a.chunks + c];
        s += v.x;
        s += v.y;
        s += v.z;
        s += v.w;
      }
      xsum[i] = s;
    }
    __syncthreads();
  }
  if (g >= groups) return;

  float acc[R][T];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[r][t] = 0.0f;
  // One step: load the next step's chunks into (nr, ns), then compute the
  // current one from (cr, cs).  Two buffers alternate, so the next loads stay
  // in flight for a whole step and no register copy waits for them.
  auto step = [&](Raw<FMT>(&cr)[R], uint32_t(&cs)[R], Raw<FMT>(&nr)[R],
                  uint32_t(&ns)[R]) -> bool {
    int64_t g2 = g;
    int k2 = k + 1;
    if (k2 == kc) {
      k2 = 0;
      g2 += gstride;
    }
    const bool more = g2 < groups;
    // past the last step: load the current step again (valid addresses, unused)
    fetch(more ? g2 : g, more ? k2 : k, nr, ns);
    const int c0 = lane + 64 * k;
    const bool valid = c0 < a.chunks;
    const int c = valid ? c0 : a.chunks - 1;
    float d[R][T];
    chunk_dot_rows<FMT, T, R>(cr, x4 + c, a.chunks, d);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float v = d[r][t];
        if constexpr (kOffset) v = fmaf(-kOff, xsum[t * a.chunks + c], v);
        v = scale_value<FMT>(cs[r]) * v;
        acc[r][t] += valid ? v : 0.0f;
      }
    if (k == kc - 1) {
      float tot[R][T];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) {
          tot[r][t] = wave_sum(acc[r][t]);
          acc[r][t] = 0.0f;
        }
      if constexpr (MODE == kModeGateUp) {
        // h = SiLU(gate) * up * w_t for the RM features of the step
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const int64_t f = g * RM + r;
            if (lane == (r * T + t) % 64 && f < a.O) {
              const float gv = tot[r][t], uv = tot[r + RM][t];
              const float hv = gv / (1.0f + expf(-gv)) * uv * wtok[t];
              a.h[(size_t(unit) * T + t) * a.O + f] = hv;
            }
          }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const int64_t o = g * R + r;
            if (lane == (r * T + t) % 64 && o < a.O) {
              if constexpr (MODE == kModeDown)
                a.part[(size_t(unit) * T + t) * a.O + o] = tot[r][t];
              else
                a.y[size_t(t) * a.O + o] = tot[r][t];
            }
          }
      }
    }
    g = g2;
    k = k2;
    return more;
  };
  while (step(cur, csc, nxt, nsc) && step(nxt, nsc, cur, csc)) {
  }
}

// Layer combine: y[t][o] = sum over units, in unit order, of part[unit][t][o]
// (units past the batch's count are skipped).
__global__ __launch_bounds__(256) void fmt_combine(const float *__restrict__ part,
                                                   const int32_t *__restrict__ n_unique, int T,
                                                   int H, float *__restrict__ y,
                                                   int32_t *__restrict__ status) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(T) * H) return;
  const int nu = *n_unique;
  float s = 0.0f;
  for (int u = 0; u <= nu; ++u) s += part[size_t(u) * T * H + i];
  y[i] = s;
  if (status && !__builtin_isfinite(s)) atomicOr(status, COLI_STATUS_NONFINITE);
}

// Blocks per matrix: about 1024 in all (four per CU), so that each block's x
// stage serves many row groups; grouped launches split them over the units.
template <int FMT, int T, int MODE>
int matvec_grid(int64_t O, int units) {
  constexpr int RM = MODE == kModeGateUp ? rows_per_step<FMT, T, MODE>() / 2 : rows_per_step<FMT, T, MODE>();
  const int64_t groups = (O + RM - 1) / RM;
  const int64_t want = cdiv(groups, 4);
  // about 1024 blocks over the units (the layer's stages), 512 for one plain
  // int4-g64 or MXFP4 product (measured: each block then streams twice the rows
  // per x stage, 16 % faster for MXFP4 over [36864, 6144]; the layer stages and
  // the other formats are fastest at 1024)
  constexpr bool kHalfGrid =
      MODE == kModePlain && (FMT == COLI_FMT_MXFP4 || FMT == COLI_FMT_INT4_G64);
  const int64_t cap = cdiv(kHalfGrid ? 512 : 1024, units);
  return int(want < cap ? want : cap);
}

template <int FMT, int MODE, int TT>
void launch_one(const MatvecArgs &a, int units, size_t lds, hipStream_t s) {
  // The x stage may take up to 96 KiB + the chunk sums (6 KiB); the limit leaves
  // room for the kernel's static LDS within the 160 KiB of a CU.  A function's
  // attributes are per device: set once on each device the library launches on
  // (every time past the 64 devices the mask tracks); a failure shows as the
  // launch's error.
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  const bool known = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  const uint64_t bit = known ? (uint64_t(1) << dev) : 0;
  if (!known || !(done.load(std::memory_order_relaxed) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&matvec_kernel<FMT, TT, MODE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024) == hipSuccess)
      done.fetch_or(bit, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((matvec_kernel<FMT, TT, MODE>),
                     dim3(matvec_grid<FMT, TT, MODE>(a.O, units), unsigned(units)), dim3(256), lds, s, a);
}

template <int FMT, int MODE>
hipError_t launch_matvec_t(const MatvecArgs &a, int T, int units, size_t lds, hipStream_t s) {
  switch (T) {
    case 1: launch_one<FMT, MODE, 1>(a, units, lds, s); break;
    case 2: launch_one<FMT, MODE, 2>(a, units, lds, s); break;
    case 3: launch_one<FMT, MODE, 3>(a, units, lds, s); break;
    case 4: launch_one<FMT, MODE, 4>(a, units, lds, s); break;
    default:
      if constexpr (MODE == kModePlain) {
        switch (T) {
          case 5: launch_one<FMT, MODE, 5>(a, units, lds, s); break;
          case 6: launch_one<FMT, MODE, 6>(a, units, lds, s); break;
          case 7: launch_one<FMT, MODE, 7>(a, units, lds, s); break;
          case 8: launch_one<FMT, MODE, 8>(a, units, lds, s); break;
          default: return hipErrorInvalidValue;
        }
        break;
      } else {
        return hipErrorInvalidValue;
      }
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_matvec_fmt(int fmt, const MatvecArgs &a, int T, int units, size_t lds,
                             hipStream_t s) {
  switch (fmt) {
    case COLI_FMT_FP8_E4M3_B128:
      return launch_matvec_t<COLI_FMT_FP8_E4M3_B128, MODE>(a, T, units, lds, s);
    case COLI_FMT_MXFP4: return launch_matvec_t<COLI_FMT_MXFP4, MODE>(a, T, units, lds, s);
    case COLI_FMT_INT3_G64: return launch_matvec_t<COLI_FMT_INT3_G64, MODE>(a, T, units, lds, s);
    default: return launch_matvec_t<COLI_FMT_INT4_G64, MODE>(a, T, units, lds, s);
  }
}

// Row geometry of an [O, I] matrix in fmt: chunk weights, row bytes, scales
// per row (fp8: tiles per row of tiles).
void fmt_geometry(int fmt, int64_t I, int *cw, int64_t *row_bytes, int *scale_cols) {
  switch (fmt) {
    case COLI_FMT_FP8_E4M3_B128:
      *cw = 16;
      *row_bytes = I;
      *scale_cols = int(cdiv(I, 128));
      break;
    case COLI_FMT_MXFP4:
      *cw = 32;
      *row_bytes = 16 * cdiv(I, 32);
      *scale_cols = int(cdiv(I, 32));
      break;
    case COLI_FMT_INT3_G64:
      *cw = 64;
      *row_bytes = 24 * cdiv(I, 64);
      *scale_cols = int(cdiv(I, 64));
      break;
    default:
      *cw = 64;
      *row_bytes = 32 * cdiv(I, 64);
      *scale_cols = int(cdiv(I, 64));
      break;
  }
}

bool aligned_to(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

// ------------------------------------------------------------------ layer

size_t fmt_blob_layout(int fmt, int H, int I, size_t q_off[3], size_t s_off[3]) {
  auto a256 = [](uint64_t n) { return (n + 255) / 256 * 256; };
  uint64_t wq[3], ws[3];
  if (!fmt_sizes(fmt, I, H, &wq[0], &ws[0])) return 0;  // gate [I, H]
  wq[1] = wq[0];
  ws[1] = ws[0];                                       // up [I, H]
  fmt_sizes(fmt, H, I, &wq[2], &ws[2]);                // down [H, I]
  uint64_t o = 0;
  for (int m = 0; m < 3; ++m) {
    q_off[m] = size_t(o);
    o += a256(wq[m]);
  }
  for (int m = 0; m < 3; ++m) {
    s_off[m] = size_t(o);
    o += a256(ws[m] ? ws[m] : 1);
  }
  return size_t(o);
}

bool fmt_layer_supported(int fmt) {
  return fmt == COLI_FMT_INT4_G64 || fmt == COLI_FMT_INT3_G64 || fmt == COLI_FMT_MXFP4 ||
         fmt == COLI_FMT_FP8_E4M3_B128;
}

bool fmt_layer_shape_ok(int fmt, int H, int I, int T) {
  if (T < 1 || T > kFmtLayerMaxT) return false;
  if (fmt == COLI_FMT_FP8_E4M3_B128 && (H % 16 || I % 16)) return false;
  int cw;
  int64_t rb;
  int sc;
  fmt_geometry(fmt, H, &cw, &rb, &sc);
  if (int64_t(T) * cdiv(H, cw) * cw > kXFloats) return false;
  fmt_geometry(fmt, I, &cw, &rb, &sc);
  return int64_t(T) * cdiv(I, cw) * cw <= kXFloats;
}

hipError_t launch_fmt_experts(const FmtLayer &L, const Routing &r, const float *x, int T,
                              float *h, float *part, float *y, int32_t *status, hipStream_t s) {
  const int units = (L.E < T * L.K ? L.E : T * L.K) + 1;  // unique experts + the shared one
  MatvecArgs a = {};
  a.experts = L.experts;
  a.shared = L.shared;
  a.blob_bytes = L.blob_bytes;
  a.unique = r.unique;
  a.n_unique = r.n_unique;
  a.idx = r.idx;
  a.gates = r.gates;
  a.K = L.K;
  a.h = h;
  a.part = part;
  int cw;
  // gate/up: rows are the I features, the row length H, x the tokens
  fmt_geometry(L.fmt, L.H, &cw, &a.row_bytes, &a.scale_cols);
  a.O = L.I;
  a.I = L.H;
  a.x = x;
  a.chunks = int(cdiv(L.H, cw));
  a.ldx = a.chunks * cw;
  a.q_off[0] = L.q_off[0];
  a.q_off[1] = L.q_off[1];
  a.s_off[0] = L.s_off[0];
  a.s_off[1] = L.s_off[1];
  size_t lds = size_t(T) * a.ldx * 4 + size_t(T) * a.chunks * 4;
  // MXFP4 with one or two tokens: the scaled matrix cores
  const bool mxg = mx_gateup_ok(L, x, T);
  hipError_t e = mxg ? launch_mx_gateup(L, r, x, T, h, s)
                     : launch_matvec_fmt<kModeGateUp>(L.fmt, a, T, units, lds, s);
  if (e != hipSuccess) return e;
  if (mxg && mx_down_ok(L, T)) return launch_mx_down(L, r, h, y, status, s);
  // down: rows are the H outputs, the row length I, x = h of the unit
  fmt_geometry(L.fmt, L.I, &cw, &a.row_bytes, &a.scale_cols);
  a.O = L.H;
  a.I = L.I;
  a.x = nullptr;
  a.chunks = int(cdiv(L.I, cw));
  a.ldx = a.chunks * cw;
  a.q_off[0] = a.q_off[1] = L.q_off[2];
  a.s_off[0] = a.s_off[1] = L.s_off[2];
  lds = size_t(T) * a.ldx * 4 + size_t(T) * a.chunks * 4;
  e = launch_matvec_fmt<kModeDown>(L.fmt, a, T, units, lds, s);
  if (e != hipSuccess) return e;
  const int64_t n = int64_t(T) * L.H;
  fmt_combine<<<dim3(unsigned(cdiv(n, 256))), 256, 0, s>>>(part, r.n_unique, T, L.H, y, status);
  return hipGetLastError();
}

}  // namespace coli

using namespace coli;

extern "C" {

int coli_fmt_bytes(int fmt, int64_t O, int64_t I, uint64_t *weight_bytes,
                   uint64_t *scale_bytes) {
  if (!weight_bytes || !scale_bytes) return COLI_EINVAL;
  if (!dims_ok(O, I)) return COLI_ESHAPE;
  uint64_t w, s;
  if (!fmt_sizes(fmt, O, I, &w, &s)) return COLI_EINVAL;
  *weight_bytes = w;
  *scale_bytes = s;
  return COLI_OK;
}

int coli_resolve_fmt(int64_t O, int64_t I, uint64_t weight_bytes, uint64_t scale_bytes,
                     uint32_t *candidates) {
  if (!dims_ok(O, I)) return COLI_ESHAPE;
  uint32_t mask = 0;
  int found = -1;
  for (int f = 0; f <= COLI_FMT_FP8_E4M3_B128; ++f) {
    uint64_t w, s;
    if (fmt_sizes(f, O, I, &w, &s) && w == weight_bytes && s == scale_bytes) {
      mask |= 1u << f;
      found = f;
    }
  }
  if (candidates) *candidates = mask;
  return __builtin_popcount(mask) == 1 ? found : COLI_EFORMAT;
}

int coli_quant_fmt(int fmt, const float *w, int64_t O, int64_t I, void *packed, void *scales,
                   int32_t *status, void *stream) {
  if (!w || !packed || !scales) return COLI_EINVAL;
  if (!dims_ok(O, I)) return COLI_ESHAPE;
  if (!aligned_to(w, 4) || (status && !aligned_to(status, 4))) return COLI_EALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int Ii = int(I);
  switch (fmt) {
    case COLI_FMT_INT4_G64:
      return coli_quant_int4_g64(w, O, I, reinterpret_cast<uint8_t *>(packed),
                                 reinterpret_cast<float *>(scales), status, stream);
    case COLI_FMT_INT3_G64: {
      if (!aligned_to(packed, 8) || !aligned_to(scales, 4)) return COLI_EALIGN;
      const int G = int(cdiv(I, 64));
      const int64_t groups = O * G;
      quant_int3<<<dim3(unsigned(cdiv(groups, 4))), 256, 0, s>>>(
          w, O, Ii, G, reinterpret_cast<uint8_t *>(packed), reinterpret_cast<float *>(scales),
          status);
      break;
    }
    case COLI_FMT_MXFP4: {
      if (!aligned_to(packed, 4)) return COLI_EALIGN;
      const int NB = int(cdiv(I, 32));
      const int64_t blocks = O * NB;
      quant_mxfp4<<<dim3(unsigned(cdiv(blocks, 8))), 256, 0, s>>>(
          w, O, Ii, NB, reinterpret_cast<uint8_t *>(packed), reinterpret_cast<uint8_t *>(scales),
          status);
      break;
    }
    case COLI_FMT_FP8_E4M3_B128: {
      if (!aligned_to(scales, 4)) return COLI_EALIGN;
      const int TI = int(cdiv(I, 128));
      const int64_t tiles = cdiv(O, 128) * TI;
      fp8_tile_scales<<<dim3(unsigned(tiles)), 256, 0, s>>>(
          w, O, Ii, TI, reinterpret_cast<float *>(scales), status);
      const int64_t n = O * I;
      const int64_t gb = cdiv(n, 256);
      fp8_codes<<<dim3(unsigned(gb < 65536 ? gb : 65536)), 256, 0, s>>>(
          w, O, Ii, TI, reinterpret_cast<const float *>(scales),
          reinterpret_cast<uint8_t *>(packed));
      break;
    }
    default:
      return COLI_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

size_t coli_fmt_blob_bytes(int fmt, int H, int I) {
  if (!fmt_layer_supported(fmt) || H < 1 || I < 1 || H > COLI_MAX_DIM || I > COLI_MAX_DIM)
    return 0;
  size_t q[3], sc[3];
  return fmt_blob_layout(fmt, H, I, q, sc);
}

int coli_quant_expert_fmt(int fmt, uint8_t *blob, int H, int I, const float *w_gate,
                          const float *w_up, const float *w_down, int32_t *status, void *stream) {
  if (!blob || !w_gate || !w_up || !w_down) return COLI_EINVAL;
  if (!fmt_layer_supported(fmt)) return COLI_EINVAL;
  if (H < 1 || I < 1 || H > COLI_MAX_DIM || I > COLI_MAX_DIM) return COLI_ESHAPE;
  if (!aligned_to(blob, 256)) return COLI_EALIGN;
  size_t q[3], sc[3];
  fmt_blob_layout(fmt, H, I, q, sc);
  const float *w[3] = {w_gate, w_up, w_down};
  const int64_t rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int m = 0; m < 3; ++m) {
    const int rc = coli_quant_fmt(fmt, w[m], rows[m], cols[m], blob + q[m], blob + sc[m], status,
                                  stream);
    if (rc != COLI_OK) return rc;
  }
  return COLI_OK;
}

int coli_matvec_fmt(int fmt, const void *packed, const void *scales, int64_t O, int64_t I,
                    const float *x, int T, float *y, void *stream) {
  if (!packed || !scales || ((!x || !y) && T > 0)) return COLI_EINVAL;
  if (!dims_ok(O, I) || T < 0 || T > kMaxT) return COLI_ESHAPE;
  if (fmt != COLI_FMT_INT4_G64 && fmt != COLI_FMT_INT3_G64 && fmt != COLI_FMT_MXFP4 &&
      fmt != COLI_FMT_FP8_E4M3_B128)
    return COLI_EINVAL;
  if (fmt == COLI_FMT_FP8_E4M3_B128 && I % 16 != 0) return COLI_ESHAPE;  // 16-byte rows
  if (!aligned_to(x, 4) || !aligned_to(y, 4) || !aligned_to(scales, 4) ||
      !aligned_to(packed, fmt == COLI_FMT_INT3_G64 ? 8 : 16))
    return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  MatvecArgs a = {};
  a.packed = reinterpret_cast<const uint8_t *>(packed);
  a.scales = scales;
  a.O = O;
  a.I = int(I);
  a.x = x;
  a.y = y;
  int cw;
  fmt_geometry(fmt, I, &cw, &a.row_bytes, &a.scale_cols);
  a.chunks = int(cdiv(I, cw));
  a.ldx = a.chunks * cw;
  if (int64_t(T) * a.ldx > kXFloats) return COLI_ESHAPE;
  const size_t lds = size_t(T) * a.ldx * 4 + size_t(T) * a.chunks * 4;
  const hipError_t e = launch_matvec_fmt<kModePlain>(fmt, a, T, 1, lds,
                                                     reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

}  // extern "C"

// stage_rows.h -- one activation row split into the fp16 hi + lo staged rows
// that the decode batch GEMMs read (see ffn_batch.hip): row * 2^-e = hi + lo
// with max |row| * 2^-e in [2^14, 2^15), each 64-group written in the staged
// k order o + {0, 2, 32, 34, 1, 3, 33, 35} (o = 16 (c / 4) + 4 (c % 4) for
// 16-byte chunk c), zero padding up to WP (also for the ragged tail of a row
// whose length is not a multiple of 64).  Used by a whole block of 256
// threads (blockDim.x == 256); red: 4 floats of LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

__device__ inline uint32_t stage_pack_f16x2(_Float16 a, _Float16 b) {
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// The 16-byte run i (group i / 8, chunk i % 8) of a row: elements o .. o+3 and
// o+32 .. o+35, o = 64 (i / 8) + 16 ((i % 8) / 4) + 4 (i % 4), as fp16 hi / lo
// pairs in the staged order.
__device__ inline void stage_run(const float4 &a, const float4 &b, float down, uint4 &hi,
                                 uint4 &lo) {
  const float v[8] = {a.x, a.z, b.x, b.z, a.y, a.w, b.y, b.w};
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float v0 = v[2 * k] * down, v1 = v[2 * k + 1] * down;
    const _Float16 h0 = _Float16(v0), h1 = _Float16(v1);
    ph[k] = stage_pack_f16x2(h0, h1);
    pl[k] = stage_pack_f16x2(_Float16(v0 - float(h0)), _Float16(v1 - float(h1)));
  }
  hi = uint4{ph[0], ph[1], ph[2], ph[3]};
  lo = uint4{pl[0], pl[1], pl[2], pl[3]};
}

__device__ inline int stage_run_offset(int i) {
  return 64 * (i >> 3) + 16 * ((i & 7) >> 2) + 4 * (i & 3);
}

// Max over the block of per-thread maxima; red: 4 floats of LDS.
__device__ inline float stage_block_max(float m, float *red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ inline float stage_absmax4(float m, const float4 &v) {
  return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Scale exponent: max |row| * 2^-e in [2^14, 2^15).
__device__ inline int stage_exponent(float m) {
  int ex = 0;
  (void)frexpf(m, &ex);
  return m > 0.0f ? max(ex - 15, -140) : 0;
}

constexpr int kStageRuns = 4;  // runs per thread held in registers (W <= 8192)

// Any W and row alignment: element loads, elements past W are zeros.
__device__ inline void stage_row_any(const float *__restrict__ row, int W, int WP,
                                     uint16_t *__restrict__ hi_out, uint16_t *__restrict__ lo_out,
                                     float *__restrict__ sc, float *red) {
  const int runs = (WP / 64) * 8;
  float m = 0.0f;
  for (int c = int(threadIdx.x); c < W; c += 256) m = fmaxf(m, fabsf(row[c]));
  m = stage_block_max(m, red);
  const int e = stage_exponent(m);
  const float down = ldexpf(1.0f, -e);
  if (threadIdx.x == 0) *sc = ldexpf(1.0f, e);
  for (int i = threadIdx.x; i < runs; i += 256) {
    const int o = stage_run_offset(i);
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = o + k < W ? row[o + k] : 0.0f;
      v[4 + k] = o + 32 + k < W ? row[o + 32 + k] : 0.0f;
    }
    uint4 hi, lo;
    stage_run(float4{v[0], v[1], v[2], v[3]}, float4{v[4], v[5], v[6], v[7]}, down, hi, lo);
    *reinterpret_cast<uint4 *>(hi_out + 8 * i) = hi;
    *reinterpret_cast<uint4 *>(lo_out + 8 * i) = lo;
  }
}

// row fp32 [W] -> hi [WP], lo [WP] fp16; *sc = 2^e.  WP % 256 == 0.  With
// W % 64 == 0 and a 16-byte aligned row: rows of up to 256 * kStageRuns runs
// are read once, every load issued before the first use (slots past the row
// re-read its first run: the max is unchanged); longer rows take two passes.
// Other rows take stage_row_any.
__device__ inline void stage_row(const float *__restrict__ row, int W, int WP,
                                 uint16_t *__restrict__ hi_out, uint16_t *__restrict__ lo_out,
                                 float *__restrict__ sc, float *red) {
  if (W % 64 != 0 || (reinterpret_cast<uintptr_t>(row) & 15) != 0) {
    stage_row_any(row, W, WP, hi_out, lo_out, sc, red);
    return;
  }
  const int G = W / 64, rv = G * 8, runs = (WP / 64) * 8;
  if (rv <= 256 * kStageRuns) {
    float4 a[kStageRuns], b[kStageRuns];
#pragma unroll
    for (int j = 0; j < kStageRuns; ++j) {
      const int i = int(threadIdx.x) + 256 * j;
      const int o = i < rv ? stage_run_offset(i) : 0;
      a[j] = *reinterpret_cast<const float4 *>(row + o);
      b[j] = *reinterpret_cast<const float4 *>(row + o + 32);
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kStageRuns; ++j) m = stage_absmax4(stage_absmax4(m, a[j]), b[j]);
    m = stage_block_max(m, red);
    const int e = stage_exponent(m);
    const float down = ldexpf(1.0f, -e);
    if (threadIdx.x == 0) *sc = ldexpf(1.0f, e);
    for (int i = threadIdx.x, j = 0; i < runs; i += 256, ++j) {
      uint4 hi = uint4{0u, 0u, 0u, 0u}, lo = hi;
      if (i < rv) {
        // j < kStageRuns here: i < rv <= 256 kStageRuns
#pragma unroll
        for (int jj = 0; jj < kStageRuns; ++jj)
          if (jj == j) stage_run(a[jj], b[jj], down, hi, lo);
      }
      *reinterpret_cast<uint4 *>(hi_out + 8 * i) = hi;
      *reinterpret_cast<uint4 *>(lo_out + 8 * i) = lo;
    }
    return;
  }
  float m = 0.0f;
  for (int c = 4 * int(threadIdx.x); c < W; c += 4 * 256)
    m = stage_absmax4(m, *reinterpret_cast<const float4 *>(row + c));
  m = stage_block_max(m, red);
  const int e = stage_exponent(m);
  const float down = ldexpf(1.0f, -e);
  if (threadIdx.x == 0) *sc = ldexpf(1.0f, e);
  for (int i = threadIdx.x; i < runs; i += 256) {
    uint4 hi = uint4{0u, 0u, 0u, 0u}, lo = hi;
    if (i < rv) {
      const int o = stage_run_offset(i);
      stage_run(*reinterpret_cast<const float4 *>(row + o),
                *reinterpret_cast<const float4 *>(row + o + 32), down, hi, lo);
    }
    *reinterpret_cast<uint4 *>(hi_out + 8 * i) = hi;
    *reinterpret_cast<uint4 *>(lo_out + 8 * i) = lo;
  }
}

}  // namespace coli

// stage_rows.h -- one activation row split into the fp16 hi + lo staged rows
// that the decode batch GEMMs read (see ffn_batch.hip): row * 2^-e = hi + lo
// with max |row| * 2^-e in [2^14, 2^15), each 64-group written in the staged
// k order o + {0, 2, 32, 34, 1, 3, 33, 35} (o = 16 (c / 4) + 4 (c % 4) for
// 16-byte chunk c), zero padding up to WP.  Used by a whole block of 256
// threads (blockDim.x == 256); red: 4 floats of LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

__device__ inline uint32_t stage_pack_f16x2(_Float16 a, _Float16 b) {
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// row fp32 [W] -> hi [WP], lo [WP] fp16; *sc = 2^e.  W % 64 == 0, WP % 256 == 0.
__device__ inline void stage_row(const float *__restrict__ row, int W, int WP,
                                 uint16_t *__restrict__ hi_out, uint16_t *__restrict__ lo_out,
                                 float *__restrict__ sc, float *red) {
  float m = 0.0f;
  for (int c = 4 * int(threadIdx.x); c < W; c += 4 * 256) {
    const float4 v = *reinterpret_cast<const float4 *>(row + c);
    m = fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int ex = 0;
  (void)frexpf(m, &ex);
  const int e = m > 0.0f ? max(ex - 15, -140) : 0;
  const float down = ldexpf(1.0f, -e);
  if (threadIdx.x == 0) *sc = ldexpf(1.0f, e);
  const int G = W / 64, runs = (WP / 64) * 8;
  for (int i = threadIdx.x; i < runs; i += 256) {
    const int g = i >> 3, c = i & 7;
    uint4 hi = uint4{0u, 0u, 0u, 0u}, lo = hi;
    if (g < G) {
      const int o = 64 * g + 16 * (c >> 2) + 4 * (c & 3);
      const float4 a = *reinterpret_cast<const float4 *>(row + o);
      const float4 b = *reinterpret_cast<const float4 *>(row + o + 32);
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
    *reinterpret_cast<uint4 *>(hi_out + 8 * i) = hi;
    *reinterpret_cast<uint4 *>(lo_out + 8 * i) = lo;
  }
}

}  // namespace coli

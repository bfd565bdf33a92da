// quant.hip -- the int4-g64 planar quantiser (HBM-bound streaming kernel).
//
// Format and rule: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 -- groups of 64 along the input dimension, qmax 7,
// q = clip(rint(w/s), -8, 7) stored as unsigned q+8, one fp32 scale per group,
// planar nibbles (byte k: element k low, element k+32 high).
//
// Mapping: a team of 8 lanes owns one 64-group.  Lane j of the team reads
// elements 4j..4j+3 and 32+4j..32+4j+3 (two 16-byte loads), so its four
// output bytes 4j..4j+3 are complete in registers and leave as one 32-bit
// store; a team writes its group's 32 bytes contiguously and a wave covers 8
// groups.  amax and the non-finite flag are reduced over the team with lane
// shuffles.  Bit-exactness: s = amax / 7.0f is an IEEE fp32 divide (this
// translation unit is compiled without fast-math and with fp32 denormals
// preserved), rint is round-half-to-even (v_rndne_f32), and each nibble is
// rint(fl32(w / s)): through a reciprocal product where that provably rounds
// the same way, else through the IEEE divide (near_half below).
#include "kernels.h"

namespace coli {
namespace {

constexpr int kTeam = 8;     // lanes per 64-group
constexpr int kBlock = 256;  // 32 groups per block

__device__ inline float team_max(float v) {
#pragma unroll
  for (int m = 1; m < kTeam; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kTeam));
  return v;
}
__device__ inline int team_or(int v) {
#pragma unroll
  for (int m = 1; m < kTeam; m <<= 1) v |= __shfl_xor(v, m, kTeam);
  return v;
}

__device__ inline uint32_t nibble_of(float quot) {
  const float q = fminf(fmaxf(__builtin_rintf(quot), -8.0f), 7.0f);
  return uint32_t(int(q) + 8);
}

// rint(fl32(w / s)) without a divide for almost every element.  qa = w * rcp(s)
// is within 3 ulp of 8, about 2.4e-6, of the exact quotient when |w / s| <= 8
// and s is a normal number away from the range ends (v_rcp_f32: 1 ulp).  Every
// half-integer up to 8.5 is an fp32 number, so when qa lies farther than 2^-17
// from all of them, the exact quotient and its fp32 rounding lie on the same
// side of each, and the three round to the same integer.  The rest (a guard
// band of about 1.5e-5 per unit of quotient) take the IEEE divide.
__device__ inline bool near_half(float qa) {
  // v_fract_f32 of |qa| (<= 8.5 here) is exactly |qa| - floor(|qa|)
  return fabsf(__builtin_amdgcn_fractf(fabsf(qa)) - 0.5f) < 0x1p-17f;
}

// One team's 64-group (unit = group index over rows * G).  k32: rows * G
// < 2^32, so the group's row and column come from a 32-bit divide (a 64-bit
// one is a long software sequence, a large share of this kernel's ALU work).
template <bool kVec, bool k32>
__device__ __attribute__((always_inline)) inline void quant_group(
    const float *__restrict__ w, int64_t rows, int64_t cols, int64_t G,
    uint8_t *__restrict__ packed, float *__restrict__ scales, int32_t *__restrict__ status,
    int64_t unit, int j) {
  const bool live = unit < rows * G;
  int64_t r = 0, g = 0;
  if (live) {
    if (k32) {
      const uint32_t u = uint32_t(unit), G32 = uint32_t(G), q = u / G32;
      r = q;
      g = u - q * G32;
    } else {
      r = unit / G;
      g = unit % G;
    }
  }
  const float *src = w + r * cols + g * 64;

  float lo[4], hi[4];
  if (kVec && live && g * 64 + 64 <= cols) {
    const float4 a = *reinterpret_cast<const float4 *>(src + 4 * j);
    const float4 b = *reinterpret_cast<const float4 *>(src + 32 + 4 * j);
    lo[0] = a.x; lo[1] = a.y; lo[2] = a.z; lo[3] = a.w;
    hi[0] = b.x; hi[1] = b.y; hi[2] = b.z; hi[3] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t cl = g * 64 + 4 * j + i, ch = cl + 32;
      lo[i] = (live && cl < cols) ? src[4 * j + i] : 0.0f;  // zero pad
      hi[i] = (live && ch < cols) ? src[32 + 4 * j + i] : 0.0f;
    }
  }

  float amax = 0.0f;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax = fmaxf(amax, fmaxf(fabsf(lo[i]), fabsf(hi[i])));
    bad |= !__builtin_isfinite(lo[i]) | !__builtin_isfinite(hi[i]);
  }
  amax = team_max(amax);
  bad = team_or(bad);
  if (!live) return;

  const float s = bad ? __builtin_nanf("") : amax / 7.0f;
  const bool quant = !bad && s != 0.0f;
  const bool fast = s >= 0x1p-125f && s <= 0x1p125f;  // false for NaN
  const float rs = __builtin_amdgcn_rcpf(fast ? s : 1.0f);
  float ql[4], qh[4];
  bool slow = quant && !fast;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ql[i] = lo[i] * rs;
    qh[i] = hi[i] * rs;
    slow |= quant && (near_half(ql[i]) || near_half(qh[i]));
  }
  // wave-uniform branch: the divides run only in waves that need them
  if (__builtin_amdgcn_ballot_w64(slow) != 0 && slow) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ql[i] = lo[i] / s;
      qh[i] = hi[i] / s;
    }
  }
  uint32_t word = 0x88888888u;
  if (quant) {
    word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      word |= (nibble_of(ql[i]) | (nibble_of(qh[i]) << 4)) << (8 * i);
  }
  *reinterpret_cast<uint32_t *>(packed + r * G * 32 + g * 32 + 4 * j) = word;
  if (j == 0) {
    scales[r * G + g] = s;
    if (bad && status) atomicOr(status, 1);
  }
}

template <bool kVec, bool k32>
__global__ __launch_bounds__(kBlock) void quant_int4_g64_kernel(
    const float *__restrict__ w, int64_t rows, int64_t cols, int64_t G,
    uint8_t *__restrict__ packed, float *__restrict__ scales,
    int32_t *__restrict__ status) {
  quant_group<kVec, k32>(w, rows, cols, G, packed, scales, status,
                         (int64_t(blockIdx.x) * kBlock + threadIdx.x) / kTeam,
                         threadIdx.x % kTeam);
}

// Many matrices of one shape in one launch: matrix blockIdx.y, its pointers
// read from the device arrays (the 16-byte loads where that matrix allows).
template <bool k32>
__global__ __launch_bounds__(kBlock) void quant_int4_g64_many(
    const float *const *__restrict__ w, uint8_t *const *__restrict__ packed,
    float *const *__restrict__ scales, int64_t rows, int64_t cols, int64_t G,
    int32_t *__restrict__ status) {
  const float *wm = w[blockIdx.y];
  uint8_t *pm = packed[blockIdx.y];
  float *sm = scales[blockIdx.y];
  const int64_t unit = (int64_t(blockIdx.x) * kBlock + threadIdx.x) / kTeam;
  const int j = threadIdx.x % kTeam;
  if ((cols % 4) == 0 && (reinterpret_cast<uintptr_t>(wm) & 15) == 0)
    quant_group<true, k32>(wm, rows, cols, G, pm, sm, status, unit, j);
  else
    quant_group<false, k32>(wm, rows, cols, G, pm, sm, status, unit, j);
}

// Scales [rows][G] -> [G][rows] through 32 x 33 LDS tiles (coalesced reads
// and writes).  Block (32, 8): tile (blockIdx.x: groups, blockIdx.y: rows).
__global__ __launch_bounds__(256) void scales_group_major(const float *__restrict__ src,
                                                          float *__restrict__ dst,
                                                          int rows, int G) {
  __shared__ float tile[32][33];
  const int g0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x, ty = threadIdx.y;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int r = r0 + ty + i, g = g0 + tx;
    if (r < rows && g < G) tile[ty + i][tx] = src[int64_t(r) * G + g];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int g = g0 + ty + i, r = r0 + tx;
    if (g < G && r < rows) dst[int64_t(g) * rows + r] = tile[tx][ty + i];
  }
}

// Row-major scales [rows][G] -> blocked by 8 rows: dst[b][g][r] = src[8 b + r][g],
// zero in the rows past `rows` of the last block.  One thread per element of dst.
__global__ __launch_bounds__(256) void scales_blocked8(const float *__restrict__ src,
                                                       float *__restrict__ dst, int rows, int G) {
  const int64_t n = int64_t((rows + 7) / 8) * 8 * G;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t b = i / (int64_t(G) * 8), rem = i - b * int64_t(G) * 8;
  const int64_t g = rem / 8, o = 8 * b + rem % 8;
  dst[i] = o < rows ? src[o * G + g] : 0.0f;
}

// The finish tag of a blob (one 16-byte vector store).
__global__ void write_tag(uint4 *dst, uint4 tag) {
  if (threadIdx.x == 0) *dst = tag;
}

}  // namespace

hipError_t launch_quant_int4_g64_many(const float *const *w, uint8_t *const *packed,
                                      float *const *scales, int n, int64_t rows, int64_t cols,
                                      int32_t *status, hipStream_t s) {
  const int64_t G = groups_of(cols);
  const int64_t units = rows * G;
  if (units == 0 || n == 0) return hipSuccess;
  const int64_t per_block = kBlock / kTeam;
  const int64_t blocks = (units + per_block - 1) / per_block;
  if (units < (int64_t(1) << 32))
    quant_int4_g64_many<true><<<dim3(unsigned(blocks), unsigned(n)), kBlock, 0, s>>>(
        w, packed, scales, rows, cols, G, status);
  else
    quant_int4_g64_many<false><<<dim3(unsigned(blocks), unsigned(n)), kBlock, 0, s>>>(
        w, packed, scales, rows, cols, G, status);
  return hipGetLastError();
}

hipError_t launch_expert_finish(uint8_t *blob, const BlobLayout &lay, int H, int I,
                                hipStream_t s) {
  struct {
    size_t src, dst;
    int rows, G;
  } m[3] = {{lay.gs, lay.gsT, I, int(lay.GH)}, {lay.us, lay.usT, I, int(lay.GH)},
            {lay.ds, lay.dsT, H, int(lay.GI)}};
  for (const auto &x : m) {
    const dim3 grid(unsigned((x.G + 31) / 32), unsigned((x.rows + 31) / 32));
    scales_group_major<<<grid, dim3(32, 8), 0, s>>>(reinterpret_cast<const float *>(blob + x.src),
                                                     reinterpret_cast<float *>(blob + x.dst),
                                                     x.rows, x.G);
  }
  const size_t bdst[3] = {lay.gsB, lay.usB, lay.dsB};
  for (int k = 0; k < 3; ++k) {
    const int64_t n = int64_t((m[k].rows + 7) / 8) * 8 * m[k].G;
    scales_blocked8<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(
        reinterpret_cast<const float *>(blob + m[k].src), reinterpret_cast<float *>(blob + bdst[k]),
        m[k].rows, m[k].G);
  }
  // the tag goes last, in stream order after the copies it vouches for
  write_tag<<<1, 64, 0, s>>>(reinterpret_cast<uint4 *>(blob + lay.tag), finish_tag(H, I));
  return hipGetLastError();
}

hipError_t launch_quant_int4_g64(const float *w, int64_t rows, int64_t cols,
                                 uint8_t *packed, float *scales,
                                 int32_t *status, hipStream_t s) {
  const int64_t G = groups_of(cols);
  const int64_t units = rows * G;
  if (units == 0) return hipSuccess;
  const int64_t per_block = kBlock / kTeam;
  const int64_t blocks = (units + per_block - 1) / per_block;
  const bool vec = (cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
  const bool i32 = units < (int64_t(1) << 32);
  const dim3 grid{unsigned(blocks)};
  if (vec && i32)
    quant_int4_g64_kernel<true, true><<<grid, kBlock, 0, s>>>(w, rows, cols, G, packed, scales, status);
  else if (vec)
    quant_int4_g64_kernel<true, false><<<grid, kBlock, 0, s>>>(w, rows, cols, G, packed, scales, status);
  else if (i32)
    quant_int4_g64_kernel<false, true><<<grid, kBlock, 0, s>>>(w, rows, cols, G, packed, scales, status);
  else
    quant_int4_g64_kernel<false, false><<<grid, kBlock, 0, s>>>(w, rows, cols, G, packed, scales, status);
  return hipGetLastError();
}

}  // namespace coli

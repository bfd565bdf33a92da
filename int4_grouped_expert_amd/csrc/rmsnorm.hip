// rmsnorm.hip -- unit-weight RMSNorm between stacked MoE layers:
// y[t] = x[t] / sqrt(mean(x[t]^2) + eps).  One block per token; the sum of
// squares is reduced in fp32 with a fixed tree (deterministic).  Rows of up to
// 8192 elements (H % 4 == 0) are held in registers; others take a strided loop.  The pages
// keep norm weights in F32 (page "从源码开始colibri纯C引擎的编译、权重转换与
// .bin直映射实战", section 权重转换); the unit weight and the absence of a
// residual are readings for a stack of MoE layers without attention.
#include "kernels.h"

namespace coli {
namespace {

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ x,
                                                      float *__restrict__ y, int H,
                                                      float eps) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const float *xr = x + int64_t(t) * H;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < H; c += 256) ss = fmaf(xr[c], xr[c], ss);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float d = sqrtf(tot / float(H) + eps);
  for (int c = threadIdx.x; c < H; c += 256) y[int64_t(t) * H + c] = xr[c] / d;
}

// The same with the row held in registers: every load of the row is issued
// before the first use (one memory round trip), and the output is written from
// the registers.  kV float4 per thread (H % 4 == 0, H <= 1024 kV, 16-byte rows).
// Each thread writes only the elements it read, so x == y is allowed.
template <int kV>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const float *__restrict__ x,
                                                          float *__restrict__ y, int H,
                                                          float eps) {
  __shared__ float part[4];
  const int t = blockIdx.x, n4 = H / 4;
  const float4 *xr = reinterpret_cast<const float4 *>(x + int64_t(t) * H);
  float4 v[kV];
#pragma unroll
  for (int i = 0; i < kV; ++i) {
    const int c = int(threadIdx.x) + 256 * i;
    v[i] = c < n4 ? xr[c] : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kV; ++i)
    ss = fmaf(v[i].w, v[i].w, fmaf(v[i].z, v[i].z, fmaf(v[i].y, v[i].y, fmaf(v[i].x, v[i].x, ss))));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float d = sqrtf(tot / float(H) + eps);
  float4 *yr = reinterpret_cast<float4 *>(y + int64_t(t) * H);
#pragma unroll
  for (int i = 0; i < kV; ++i) {
    const int c = int(threadIdx.x) + 256 * i;
    if (c < n4) yr[c] = float4{v[i].x / d, v[i].y / d, v[i].z / d, v[i].w / d};
  }
}

}  // namespace

hipError_t launch_rmsnorm_f32(const float *x, float *y, int T, int H, float eps,
                              hipStream_t s) {
  const bool vec = H % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  const int n4 = H / 4;
  if (vec && n4 <= 256) rmsnorm_reg_kernel<1><<<T, 256, 0, s>>>(x, y, H, eps);
  else if (vec && n4 <= 512) rmsnorm_reg_kernel<2><<<T, 256, 0, s>>>(x, y, H, eps);
  else if (vec && n4 <= 1024) rmsnorm_reg_kernel<4><<<T, 256, 0, s>>>(x, y, H, eps);
  else if (vec && n4 <= 2048) rmsnorm_reg_kernel<8><<<T, 256, 0, s>>>(x, y, H, eps);
  else rmsnorm_kernel<<<T, 256, 0, s>>>(x, y, H, eps);
  return hipGetLastError();
}

}  // namespace coli

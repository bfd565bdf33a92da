// rmsnorm.hip -- unit-weight RMSNorm between stacked MoE layers:
// y[t] = x[t] / sqrt(mean(x[t]^2) + eps).  One block per token; the sum of
// squares is reduced in fp32 with a fixed tree (deterministic).  The pages
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

}  // namespace

hipError_t launch_rmsnorm_f32(const float *x, float *y, int T, int H, float eps,
                              hipStream_t s) {
  rmsnorm_kernel<<<T, 256, 0, s>>>(x, y, H, eps);
  return hipGetLastError();
}

}  // namespace coli

// lambda re-parameterisation on the device and its gradient ("Differential
// Attention in Large Language Models: How Denoising Subtraction Eliminates
// Attention Noise and Outlier Activations" (llms.blog), "Learnable Lambda
// Re-parameterization", lambda equation):
//   lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init
//   dlq1 = dlambda e1 lk1, dlk1 = dlambda e1 lq1, dlq2 = -dlambda e2 lk2,
//   dlk2 = -dlambda e2 lq2, with e1 = exp(lq1 . lk1), e2 = exp(lq2 . lk2).
// One workgroup; the two dot products are summed per thread in a fixed order
// and then over the workgroup in a fixed tree (deterministic).
#include <math.h>

#include "kernels.h"

namespace da {
namespace {

constexpr int kT = 256;

__device__ __forceinline__ void two_dots(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                                         int dim, float& d1, float& d2) {
  __shared__ float r1[kT], r2[kT];
  float a = 0.f, b = 0.f;
  for (int i = threadIdx.x; i < dim; i += kT) {
    a = fmaf(lq1[i], lk1[i], a);
    b = fmaf(lq2[i], lk2[i], b);
  }
  r1[threadIdx.x] = a;
  r2[threadIdx.x] = b;
  __syncthreads();
  for (int o = kT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      r1[threadIdx.x] += r1[threadIdx.x + o];
      r2[threadIdx.x] += r2[threadIdx.x + o];
    }
    __syncthreads();
  }
  d1 = r1[0];
  d2 = r2[0];
}

__global__ __launch_bounds__(kT) void lambda_reparam_kernel(const float* lq1, const float* lk1, const float* lq2,
                                                            const float* lk2, int dim, float lambda_init, float* out) {
  float d1, d2;
  two_dots(lq1, lk1, lq2, lk2, dim, d1, d2);
  if (threadIdx.x == 0) out[0] = expf(d1) - expf(d2) + lambda_init;
}

__global__ __launch_bounds__(kT) void lambda_reparam_bwd_kernel(const float* lq1, const float* lk1, const float* lq2,
                                                                const float* lk2, int dim, const float* dlambda,
                                                                float* dlq1, float* dlk1, float* dlq2, float* dlk2) {
  float d1, d2;
  two_dots(lq1, lk1, lq2, lk2, dim, d1, d2);
  const float g = dlambda[0], g1 = g * expf(d1), g2 = -g * expf(d2);
  for (int i = threadIdx.x; i < dim; i += kT) {
    dlq1[i] = g1 * lk1[i];
    dlk1[i] = g1 * lq1[i];
    dlq2[i] = g2 * lk2[i];
    dlk2[i] = g2 * lq2[i];
  }
}

}  // namespace

hipError_t launch_lambda_reparam(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int dim,
                                 float lambda_init, float* out, hipStream_t s) {
  hipLaunchKernelGGL(lambda_reparam_kernel, dim3(1), dim3(kT), 0, s, lq1, lk1, lq2, lk2, dim, lambda_init, out);
  return hipGetLastError();
}

hipError_t launch_lambda_reparam_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int dim,
                                     const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                                     hipStream_t s) {
  hipLaunchKernelGGL(lambda_reparam_bwd_kernel, dim3(1), dim3(kT), 0, s, lq1, lk1, lq2, lk2, dim, dlambda, dlq1, dlk1,
                     dlq2, dlk2);
  return hipGetLastError();
}

}  // namespace da

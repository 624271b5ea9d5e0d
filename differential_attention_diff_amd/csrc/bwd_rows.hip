// Backward row passes: the head-norm backward and the per-row statistics the
// score passes need, and the final reduction of dlambda and dw.
//
// The forward is "Differential Attention in Large Language Models: How
// Denoising Subtraction Eliminates Attention Noise and Outlier Activations"
// (llms.blog), "Differential Attention Architecture" (DiffAttn equation) and
// "Headwise Normalization" (head_bar_i equation).  Per row (b, i, h), with
// o1 = A1 V and o2 = A2 V saved by the forward, o = o1 - lambda o2,
// r = sqrt(mean(o^2) + eps), c = 1 - lambda_init and y = c w o / r:
//   do = c w dy / r - o sum_k(c w_k dy_k o_k) / (dv r^3)      (dy without the norm)
//   dlambda = -sum over rows of do . o2
//   dw_k    = sum over rows of dy_k c o_k / r
// and the score passes need D1 = do . o1, D2 = do . o2 (the softmax backward's
// row sums) and the forward's log-sum-exps in log2 units.  o1 and o2 come in
// fp32 (o is their difference, which the norm's backward divides by its
// RMS).  D1 and D2 use do rounded to the storage type, the operand the score
// passes multiply by V.
#include <math.h>

#include "kernels.h"

namespace da {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return (float)p[0];
}

// One wavefront per row, grid-stride over rows; channels lane and lane + 64.
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dv = p.dv;
  const int64_t rows = (int64_t)p.B * p.N * p.Hs;
  const int64_t plane = rows * dv;  // one map of o_maps
  const float cst = 1.0f - p.lam_init;
  float lam_part = 0.f, dw0 = 0.f, dw1 = 0.f;
  const int c0 = lane, c1 = lane + 64;
  const bool v0 = c0 < dv, v1 = c1 < dv;
  float w0 = 1.f, w1 = 1.f;
  if (p.normalize && p.norm_w) {
    if (v0) w0 = p.norm_w[c0];
    if (v1) w1 = p.norm_w[c1];
  }
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < rows; row += (int64_t)gridDim.x * 4) {
    const int h = (int)(row % p.Hs);
    const int64_t t = row / p.Hs;
    const int i = (int)(t % p.N);
    const int b = (int)(t / p.N);
    const T* dy = (const T*)p.dout + b * p.sdo[0] + (int64_t)i * p.sdo[1] + h * p.sdo[2];
    const float* o1 = p.o_maps + row * dv;
    const float* o2 = o1 + plane;
    const float y0 = v0 ? ld(dy + c0) : 0.f, y1 = v1 ? ld(dy + c1) : 0.f;
    const float a0 = v0 ? ld(o1 + c0) : 0.f, a1 = v1 ? ld(o1 + c1) : 0.f;
    const float z0 = v0 ? ld(o2 + c0) : 0.f, z1 = v1 ? ld(o2 + c1) : 0.f;
    const float o0 = __builtin_fmaf(-p.lam, z0, a0), oo1 = __builtin_fmaf(-p.lam, z1, a1);
    float d0 = y0, d1 = y1;
    if (p.normalize) {
      const float r = sqrtf(wave_sum(o0 * o0 + oo1 * oo1) / dv + p.eps);
      const float ir = 1.0f / r;
      const float g0 = cst * w0 * y0, g1 = cst * w1 * y1;
      const float tt = wave_sum(g0 * o0 + g1 * oo1) * ir * ir * ir / dv;
      d0 = g0 * ir - o0 * tt;
      d1 = g1 * ir - oo1 * tt;
      dw0 += y0 * cst * o0 * ir;
      dw1 += y1 * cst * oo1 * ir;
    }
    lam_part -= wave_sum(d0 * z0 + d1 * z1);
    const T r0 = (T)d0, r1 = (T)d1;
    T* dop = (T*)p.dop + row * dv;
    if (v0) dop[c0] = r0;
    if (v1) dop[c1] = r1;
    const float e0 = (float)r0, e1 = (float)r1;
    const float D1 = wave_sum(e0 * a0 + e1 * a1), D2 = wave_sum(e0 * z0 + e1 * z1);
    if (lane == 0) {
      const int64_t li = ((int64_t)b * p.Hs + h) * p.N + i;
      const float l1 = p.lse[li], l2 = p.lse[(int64_t)p.B * p.Hs * p.N + li];
      *(float4*)(p.rowstat + 4 * li) = make_float4(l1 * kLog2e, l2 * kLog2e, D1, D2);
    }
  }
  // workgroup sums into this workgroup's row of `partial`
  __shared__ float red[4][129];
  red[wave][0] = lam_part;  // identical in every lane (wave sums)
  if (v0) red[wave][1 + c0] = dw0;
  if (v1) red[wave][1 + c1] = dw1;
  __syncthreads();
  for (int k = threadIdx.x; k < 1 + dv; k += blockDim.x)
    p.partial[(int64_t)blockIdx.x * (1 + dv) + k] = red[0][k] + red[1][k] + red[2][k] + red[3][k];
}

// One workgroup: sums the per-workgroup partials in a fixed order.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdParams p) {
  const int dv = p.dv;
  for (int k = threadIdx.x; k < 1 + dv; k += blockDim.x) {
    float s = 0.f;
    for (int w = 0; w < p.nprep; ++w) s += p.partial[(int64_t)w * (1 + dv) + k];
    if (k == 0)
      p.dlambda[0] = s;
    else if (p.dnorm_w)
      p.dnorm_w[k - 1] = s;
  }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(BwdParams p) {
  for (int k = threadIdx.x; k < 1 + p.dv; k += blockDim.x) {
    if (k == 0)
      p.dlambda[0] = 0.f;
    else if (p.dnorm_w)
      p.dnorm_w[k - 1] = 0.f;
  }
}

}  // namespace

hipError_t launch_bwd_prep(const BwdParams& p, int dtype, hipStream_t s) {
  if (dtype == DA_BF16)
    hipLaunchKernelGGL(bwd_prep_kernel<__bf16>, dim3(p.nprep), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3(p.nprep), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_zero(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

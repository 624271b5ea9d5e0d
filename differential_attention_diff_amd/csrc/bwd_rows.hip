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

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store8(float* p, const float (&x)[8], float (&r)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = r[e] = x[e];
    b[e] = r[4 + e] = x[4 + e];
  }
  *(f32x4*)p = a;
  *(f32x4*)(p + 4) = b;
}
__device__ __forceinline__ void store8(__bf16* p, const float (&x)[8], float (&r)[8]) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)x[e];
    r[e] = (float)a[e];
  }
  *(bf16x8*)p = a;
}

// sum over the L lanes of a row group (L a power of two, groups aligned)
template <int L>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Each row's dv channels are spread over L = dv / 8 lanes, 8 channels per lane
// (16-byte loads); a wavefront holds 64 / L rows at a time and walks the rows
// grid-stride, with the loads of its next rows (do, both o_maps planes and the
// two log-sum-exps) issued before the current rows are processed.
template <typename T>
struct PrepRow {
  typedef T t8 __attribute__((ext_vector_type(8)));
  t8 y;            // do
  f32x4 a[2], z[2];  // o1, o2
  float l1, l2;    // lse of both maps
};

template <typename T, int DV>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int L = DV / 8, RPW = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % L, c0 = sub * 8;
  const int64_t rows = (int64_t)p.B * p.N * p.Hs;
  const int64_t plane = rows * DV;  // one map of o_maps
  const int64_t lplane = (int64_t)p.B * p.Hs * p.N;  // one map of lse
  const float cst = 1.0f - p.lam_init;
  const float lam = lambda_of(p.lam_dev, p.lam);
  const float sgn = lam > 0.f ? -1.f : 1.f, llam = log2f(fabsf(lam));  // log2 0 = -inf
  double lam_part = 0.0, dw[8] = {};  // sums over many rows: fp64
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = (p.normalize && p.norm_w) ? p.norm_w[c0 + e] : 1.0f;
  // (batch, token, head) of a row (clamped to the last row) and its lse index
  const bool narrow = rows <= (int64_t)UINT32_MAX;  // 32-bit index division suffices
  auto coords = [&](int64_t row, int& b, int& i, int& h) {
    const int64_t rr = row < rows ? row : rows - 1;
    if (narrow) {
      const uint32_t r32 = (uint32_t)rr, t = r32 / (uint32_t)p.Hs;
      h = (int)(r32 - t * (uint32_t)p.Hs);
      b = (int)(t / (uint32_t)p.N);
      i = (int)(t - (uint32_t)b * (uint32_t)p.N);
    } else {
      h = (int)(rr % p.Hs);
      const int64_t t = rr / p.Hs;
      i = (int)(t % p.N);
      b = (int)(t / p.N);
    }
    return rr;
  };
  auto fetch = [&](int64_t row, PrepRow<T>& f) {
    int b, i, h;
    const int64_t rr = coords(row, b, i, h);
    f.y = *(const typename PrepRow<T>::t8*)((const T*)p.dout + b * p.sdo[0] + (int64_t)i * p.sdo[1] +
                                            h * p.sdo[2] + c0);
    const float* o1 = p.o_maps + rr * DV + c0;
    f.a[0] = *(const f32x4*)o1;
    f.a[1] = *(const f32x4*)(o1 + 4);
    f.z[0] = *(const f32x4*)(o1 + plane);
    f.z[1] = *(const f32x4*)(o1 + plane + 4);
    const int64_t li = ((int64_t)b * p.Hs + h) * p.N + i;
    f.l1 = p.lse[li];
    f.l2 = p.lse[lplane + li];
  };
  const int64_t step = (int64_t)gridDim.x * 4 * RPW;
  int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  PrepRow<T> cur;
  if (row0 < rows) fetch(row0 + lane / L, cur);
  for (; row0 < rows; row0 += step) {
    PrepRow<T> nxt;
    if (row0 + step < rows) fetch(row0 + step + lane / L, nxt);
    const int64_t row = row0 + lane / L;
    const bool valid = row < rows;
    int b, i, h;
    const int64_t rr = coords(row, b, i, h);
    float y[8], a[8], z[8], o[8], dd[8], e8[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = cur.a[0][e];
      a[4 + e] = cur.a[1][e];
      z[e] = cur.z[0][e];
      z[4 + e] = cur.z[1][e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)cur.y[e];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!valid) y[e] = a[e] = z[e] = 0.f;
      o[e] = __builtin_fmaf(-lam, z[e], a[e]);
      ss = __builtin_fmaf(o[e], o[e], ss);
      dd[e] = y[e];
    }
    if (p.normalize) {
      const float r = sqrtf(group_sum<L>(ss) / DV + p.eps);
      const float ir = 1.0f / r;
      float g[8], gt = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[e] = cst * w[e] * y[e];
        gt = __builtin_fmaf(g[e], o[e], gt);
      }
      const float tt = group_sum<L>(gt) * ir * ir * ir / DV;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dd[e] = g[e] * ir - o[e] * tt;
        dw[e] += (double)(y[e] * cst * o[e] * ir);
      }
    }
    float lp = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) lp = __builtin_fmaf(dd[e], z[e], lp);
    lam_part -= (double)lp;
    if (valid) store8((T*)p.dop + rr * DV + c0, dd, e8);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!valid) e8[e] = (float)(T)dd[e];
      s1 = __builtin_fmaf(e8[e], a[e], s1);
      s2 = __builtin_fmaf(e8[e], z[e], s2);
    }
    const float D1 = group_sum<L>(s1), D2 = group_sum<L>(s2);
    if (valid && sub == 0) {
      const int64_t li = ((int64_t)b * p.Hs + h) * p.N + i;
      // map 2 folded with lambda: 2^(s - (lse2' - log2|lambda|)) = |lambda| P2 (0 for
      // lambda = 0), and sgn D2 with -lambda = sgn |lambda|
      *(float4*)(p.rowstat + 4 * li) = make_float4(cur.l1 * kLog2e, cur.l2 * kLog2e - llam, D1, sgn * D2);
    }
    cur = nxt;
  }
  // sums over the wavefront's row slots, then over the 4 wavefronts, into this
  // workgroup's row of `partial`
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lam_part += __shfl_xor(lam_part, o, 64);
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int o = L; o < 64; o <<= 1) dw[e] += __shfl_xor(dw[e], o, 64);
  __shared__ double red[4][1 + DV];
  if (lane == 0) red[wave][0] = lam_part;
  if (lane < L)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][1 + c0 + e] = dw[e];
  __syncthreads();
  for (int k = threadIdx.x; k < 1 + DV; k += blockDim.x)
    p.partial[(int64_t)blockIdx.x * (1 + DV) + k] = red[0][k] + red[1][k] + red[2][k] + red[3][k];
}

// One workgroup per column of `partial` (dlambda, then dw channel by channel):
// thread t sums rows t, t + 256, ..., then a fixed-order tree over the threads.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdParams p) {
  const int k = blockIdx.x, dv = p.dv;
  if (k > 0 && !p.dnorm_w) return;  // whole workgroup
  double s = 0.0;
  for (int w = threadIdx.x; w < p.nprep; w += 256) s += p.partial[(int64_t)w * (1 + dv) + k];
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (k == 0)
      p.dlambda[0] = (float)red[0];
    else
      p.dnorm_w[k - 1] = (float)red[0];
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
  if (dtype == DA_BF16) {
    if (p.dv == 128)
      hipLaunchKernelGGL((bwd_prep_kernel<__bf16, 128>), dim3(p.nprep), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<__bf16, 64>), dim3(p.nprep), dim3(256), 0, s, p);
  } else {
    if (p.dv == 128)
      hipLaunchKernelGGL((bwd_prep_kernel<float, 128>), dim3(p.nprep), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<float, 64>), dim3(p.nprep), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3(1 + p.dv), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_zero(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

// fp32 prefill: differential / grouped differential attention with the
// per-head RMS norm, in fp32 throughout (VALU; gfx950 has no xf32 MFMA).
//
// Follows "Differential Attention in Large Language Models: How Denoising
// Subtraction Eliminates Attention Noise and Outlier Activations" (llms.blog),
// "Differential Attention Architecture" (DiffAttn equation) and "Headwise
// Normalization" (head_bar_i equation); head grouping per "Grouped
// Differential Attention" (mlsanity.com), "Abstract".
//
// One wavefront per (sequence, signal head, query row).  Keys are visited in chunks
// of 64 (one per lane); each map keeps a running max and sum (online softmax,
// natural-log units) and an unnormalised output, so the result equals the
// full-row softmax up to rounding.  Output channels c and c+64 belong to lane c.
#include <math.h>

#include "kernels.h"

namespace da {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p) {
  const int h = blockIdx.y;
  // the sequence: batch b, tokens [tok0, tok0 + N); packed sequences live in
  // batch 0 at the offsets cu_seqlens gives, clamped to the token axis
  int b = blockIdx.z, tok0 = 0, N = p.N;
  if (p.cu_seqlens) {
    const int s0 = p.cu_seqlens[b], s1 = p.cu_seqlens[b + 1];
    b = 0;
    tok0 = min(max(s0, 0), p.N);
    N = max(min(min(s1, p.N) - tok0, p.max_seqlen), 0);
  }
  const int i = N - 1 - (int)blockIdx.x;  // longest rows first
  if (i < 0) return;                      // whole block: row past the sequence
  const int lane = threadIdx.x;
  const int64_t t0 = tok0;
  const int n = p.nz[h], kh = p.kv[h];
  const int d = p.d, dv = p.dv;

  __shared__ float q1s[64], q2s[64], p1s[64], p2s[64];
  const float* q1 = (const float*)p.q1 + b * p.sq1[0] + (t0 + i) * p.sq1[1] + h * p.sq1[2];
  const float* q2 = (const float*)p.q2 + b * p.sq2[0] + (t0 + i) * p.sq2[1] + n * p.sq2[2];
  const float* k1 = (const float*)p.k1 + b * p.sk1[0] + t0 * p.sk1[1] + kh * p.sk1[2];
  const float* k2 = (const float*)p.k2 + b * p.sk2[0] + t0 * p.sk2[1] + n * p.sk2[2];
  const float* v = (const float*)p.v + b * p.sv[0] + t0 * p.sv[1] + kh * p.sv[2];
  if (lane < d) {
    q1s[lane] = q1[lane];
    q2s[lane] = q2[lane];
  }
  __syncthreads();

  const int last = p.causal ? i : N - 1;  // last visible key
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  float o1a = 0.f, o1b = 0.f, o2a = 0.f, o2b = 0.f;  // channels lane, lane + 64
  const int ca = lane, cb = lane + 64;

  for (int j0 = 0; j0 <= last; j0 += 64) {
    const int j = j0 + lane;
    float s1 = -INFINITY, s2 = -INFINITY;
    if (j <= last) {
      const float* r1 = k1 + (int64_t)j * p.sk1[1];
      const float* r2 = k2 + (int64_t)j * p.sk2[1];
      float a1 = 0.f, a2 = 0.f;
      for (int t = 0; t < d; ++t) {
        a1 = fmaf(q1s[t], r1[t], a1);
        a2 = fmaf(q2s[t], r2[t], a2);
      }
      s1 = a1 * p.sm_scale;
      s2 = a2 * p.sm_scale;
    }
    const float nm1 = fmaxf(m1, wave_max(s1));
    const float nm2 = fmaxf(m2, wave_max(s2));
    const float al1 = expf(m1 - nm1), al2 = expf(m2 - nm2);  // exp(-inf) = 0 on the first chunk
    const float e1 = (j <= last) ? expf(s1 - nm1) : 0.f;
    const float e2 = (j <= last) ? expf(s2 - nm2) : 0.f;
    l1 = l1 * al1 + wave_sum(e1);
    l2 = l2 * al2 + wave_sum(e2);
    m1 = nm1;
    m2 = nm2;
    p1s[lane] = e1;
    p2s[lane] = e2;
    __syncthreads();
    const int cnt = min(64, last - j0 + 1);
    o1a *= al1;
    o1b *= al1;
    o2a *= al2;
    o2b *= al2;
    const float* vr = v + (int64_t)j0 * p.sv[1];
    for (int t = 0; t < cnt; ++t) {
      const float w1 = p1s[t], w2 = p2s[t];
      if (ca < dv) {
        const float x = vr[ca];
        o1a = fmaf(w1, x, o1a);
        o2a = fmaf(w2, x, o2a);
      }
      if (cb < dv) {
        const float x = vr[cb];
        o1b = fmaf(w1, x, o1b);
        o2b = fmaf(w2, x, o2b);
      }
      vr += p.sv[1];
    }
    __syncthreads();
  }

  // o = O1/l1 - lambda O2/l2.  Both maps go through identical operations, so
  // identical maps with lambda = 1 cancel to exactly zero.
  const float r1 = 1.0f / l1, r2 = 1.0f / l2;
  const float lam = lambda_of(p.lam_dev, p.lam);
  if (p.o_maps) {  // each map's own output, A1 V and A2 V
    float* om1 = p.o_maps + ((((int64_t)b * p.N + tok0 + i) * p.Hs + h) * dv);
    float* om2 = om1 + (int64_t)p.B * p.N * p.Hs * dv;
    if (ca < dv) {
      om1[ca] = __fmul_rn(o1a, r1);
      om2[ca] = __fmul_rn(o2a, r2);
    }
    if (cb < dv) {
      om1[cb] = __fmul_rn(o1b, r1);
      om2[cb] = __fmul_rn(o2b, r2);
    }
  }
  float oa = fmaf(-lam, __fmul_rn(o2a, r2), __fmul_rn(o1a, r1));
  float ob = fmaf(-lam, __fmul_rn(o2b, r2), __fmul_rn(o1b, r1));
  if (ca >= dv) oa = 0.f;
  if (cb >= dv) ob = 0.f;
  float scale = 1.0f;
  if (p.normalize) {
    const float ms = wave_sum(oa * oa + ob * ob) / (float)dv;
    scale = (1.0f - p.lam_init) / sqrtf(ms + p.eps);
  }
  float* out = (float*)p.out + b * p.so[0] + (t0 + i) * p.so[1] + h * p.so[2];
  if (ca < dv) out[ca] = oa * scale * (p.normalize && p.norm_w ? p.norm_w[ca] : 1.0f);
  if (cb < dv) out[cb] = ob * scale * (p.normalize && p.norm_w ? p.norm_w[cb] : 1.0f);
  if (p.lse && lane == 0) {
    const int64_t base = ((int64_t)b * p.Hs + h) * p.N + tok0 + i;
    const int64_t plane = (int64_t)p.B * p.Hs * p.N;
    p.lse[base] = m1 + logf(l1);
    p.lse[plane + base] = m2 + logf(l2);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s) {
  dim3 grid((unsigned)p.max_seqlen, (unsigned)p.Hs, (unsigned)p.nseq);
  hipLaunchKernelGGL(fwd_f32_kernel, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

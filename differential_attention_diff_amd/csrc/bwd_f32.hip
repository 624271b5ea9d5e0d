// fp32 backward score passes (VALU): the exact path, one wavefront per row.
//
// Gradients of "Differential Attention in Large Language Models: How
// Denoising Subtraction Eliminates Attention Noise and Outlier Activations"
// (llms.blog), "Differential Attention Architecture", DiffAttn equation, with
// the noise heads of "Grouped Differential Attention" (mlsanity.com),
// "Abstract".  With the row statistics of the prep pass (lse in log2 units,
// D1, D2) and do, per query i and visible key j of signal head h:
//   p1 = 2^(s1 sc - lse1'), p2 = 2^(s2 sc - lse2'), dp = do_i . v_j
//   ds1 = p1 (dp - D1),  ds2 = -lambda p2 (dp - D2)
// (the statistics hold lse2' - log2|lambda| and sgn D2 with -lambda = sgn |lambda|:
// the code forms |lambda| p2 and ds2 = (|lambda| p2) (sgn dp - sgn D2))
//   dq1_i += ds1 k1_j / sqrt(d)   dk1_j += ds1 q1_i / sqrt(d)   dv_j += (p1 - lambda p2) do_i
//   dq2_i += ds2 k2_j / sqrt(d)   dk2_j += ds2 q2_i / sqrt(d)
// Shared heads are summed inside one wavefront (a noise group's signal heads
// for dq2 and dk2, a key/value head's signal heads for dk1 and dv), so every
// gradient row is written once, without atomics.
#include <math.h>

#include "kernels.h"

namespace da {
namespace {

struct RowStat {
  float l1, l2, d1, d2;
};

__device__ __forceinline__ RowStat row_stat(const BwdParams& p, int b, int h, int i) {
  const float4 v = *(const float4*)(p.rowstat + 4 * (((int64_t)b * p.Hs + h) * p.N + i));
  return {v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ float dot_lds(const float* a, const float* g, int n) {
  float s = 0.f;
  for (int t = 0; t < n; ++t) s = fmaf(a[t], g[t], s);
  return s;
}

// dq1 (per signal head) and dq2 (per noise head): one wavefront per (b, noise
// head, query row); lane c < d owns channel c.
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(BwdParams p) {
  const int i = p.N - 1 - (int)blockIdx.x;  // longest rows first
  const int n = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, d = p.d, dv = p.dv;
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;
  __shared__ float q1s[64], q2s[64], dos[128], ds1s[64], ds2s[64];
  const float* q2 = (const float*)p.q2 + b * p.sq2[0] + (int64_t)i * p.sq2[1] + n * p.sq2[2];
  if (lane < d) q2s[lane] = q2[lane];
  const float* k2 = (const float*)p.k2 + b * p.sk2[0] + n * p.sk2[2];
  const int last = p.causal ? i : p.N - 1;
  float dq2 = 0.f;
  for (int t = 0; t < p.g; ++t) {
    const int h = p.members[n * p.g + t], kh = p.kv[h];
    const float* q1 = (const float*)p.q1 + b * p.sq1[0] + (int64_t)i * p.sq1[1] + h * p.sq1[2];
    const float* dop = (const float*)p.dop + (((int64_t)b * p.N + i) * p.Hs + h) * dv;
    if (lane < d) q1s[lane] = q1[lane];
    for (int c = lane; c < dv; c += 64) dos[c] = dop[c];
    __syncthreads();
    const RowStat rs = row_stat(p, b, h, i);
    const float* k1 = (const float*)p.k1 + b * p.sk1[0] + kh * p.sk1[2];
    const float* v = (const float*)p.v + b * p.sv[0] + kh * p.sv[2];
    float dq1 = 0.f;
    for (int j0 = 0; j0 <= last; j0 += 64) {
      const int j = j0 + lane;
      float ds1 = 0.f, ds2 = 0.f;
      if (j <= last) {
        const float s1 = dot_lds(q1s, k1 + (int64_t)j * p.sk1[1], d);
        const float s2 = dot_lds(q2s, k2 + (int64_t)j * p.sk2[1], d);
        const float dp = dot_lds(dos, v + (int64_t)j * p.sv[1], dv);
        const float p1 = exp2f(fmaf(s1, p.sm_scale_log2, -rs.l1));
        const float p2 = exp2f(fmaf(s2, p.sm_scale_log2, -rs.l2));
        ds1 = p1 * (dp - rs.d1);
        ds2 = p2 * fmaf(sgn, dp, -rs.d2);
      }
      ds1s[lane] = ds1;
      ds2s[lane] = ds2;
      __syncthreads();
      const int cnt = min(64, last - j0 + 1);
      if (lane < d)
        for (int jj = 0; jj < cnt; ++jj) {
          dq1 = fmaf(ds1s[jj], k1[(int64_t)(j0 + jj) * p.sk1[1] + lane], dq1);
          dq2 = fmaf(ds2s[jj], k2[(int64_t)(j0 + jj) * p.sk2[1] + lane], dq2);
        }
      __syncthreads();
    }
    if (lane < d) ((float*)p.gq1)[b * p.sgq1[0] + (int64_t)i * p.sgq1[1] + h * p.sgq1[2] + lane] = dq1 * p.sm_scale;
  }
  if (lane < d) ((float*)p.gq2)[b * p.sgq2[0] + (int64_t)i * p.sgq2[1] + n * p.sgq2[2] + lane] = dq2 * p.sm_scale;
}

// dk2: one wavefront per (b, noise head, key row), summing the group's heads.
__global__ __launch_bounds__(64) void bwd_f32_dk2_kernel(BwdParams p) {
  const int j = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, d = p.d, dv = p.dv;
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;
  __shared__ float k2s[64], vs[128], ds2s[64];
  const float* k2 = (const float*)p.k2 + b * p.sk2[0] + (int64_t)j * p.sk2[1] + n * p.sk2[2];
  if (lane < d) k2s[lane] = k2[lane];
  const float* q2 = (const float*)p.q2 + b * p.sq2[0] + n * p.sq2[2];
  const int first = p.causal ? j : 0;
  float dk2 = 0.f;
  for (int t = 0; t < p.g; ++t) {
    const int h = p.members[n * p.g + t], kh = p.kv[h];
    const float* v = (const float*)p.v + b * p.sv[0] + (int64_t)j * p.sv[1] + kh * p.sv[2];
    for (int c = lane; c < dv; c += 64) vs[c] = v[c];
    __syncthreads();
    for (int i0 = first; i0 < p.N; i0 += 64) {
      const int i = i0 + lane;
      float ds2 = 0.f;
      if (i < p.N) {
        const RowStat rs = row_stat(p, b, h, i);
        const float s2 = dot_lds(k2s, q2 + (int64_t)i * p.sq2[1], d);
        const float dp = dot_lds(vs, (const float*)p.dop + (((int64_t)b * p.N + i) * p.Hs + h) * dv, dv);
        ds2 = exp2f(fmaf(s2, p.sm_scale_log2, -rs.l2)) * fmaf(sgn, dp, -rs.d2);
      }
      ds2s[lane] = ds2;
      __syncthreads();
      const int cnt = min(64, p.N - i0);
      if (lane < d)
        for (int ii = 0; ii < cnt; ++ii) dk2 = fmaf(ds2s[ii], q2[(int64_t)(i0 + ii) * p.sq2[1] + lane], dk2);
      __syncthreads();
    }
  }
  if (lane < d) ((float*)p.gk2)[b * p.sgk2[0] + (int64_t)j * p.sgk2[1] + n * p.sgk2[2] + lane] = dk2 * p.sm_scale;
}

// dk1 and dv: one wavefront per (b, key/value head, key row), summing the
// signal heads that share the key/value head; dv channels lane and lane + 64.
__global__ __launch_bounds__(64) void bwd_f32_dk1dv_kernel(BwdParams p) {
  const int j = blockIdx.x, k = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, d = p.d, dv = p.dv;
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;
  __shared__ float k1s[64], k2s[64], vs[128], ds1s[64], pcs[64];
  const float* k1 = (const float*)p.k1 + b * p.sk1[0] + (int64_t)j * p.sk1[1] + k * p.sk1[2];
  const float* v = (const float*)p.v + b * p.sv[0] + (int64_t)j * p.sv[1] + k * p.sv[2];
  if (lane < d) k1s[lane] = k1[lane];
  for (int c = lane; c < dv; c += 64) vs[c] = v[c];
  const int first = p.causal ? j : 0;
  float dk1 = 0.f, dva = 0.f, dvb = 0.f;
  for (int t = 0; t < p.gk; ++t) {
    const int h = p.kvmembers[k * p.gk + t], n = p.nz[h];
    const float* k2 = (const float*)p.k2 + b * p.sk2[0] + (int64_t)j * p.sk2[1] + n * p.sk2[2];
    __syncthreads();  // the previous head's readers of k2s are done
    if (lane < d) k2s[lane] = k2[lane];
    __syncthreads();
    const float* q1 = (const float*)p.q1 + b * p.sq1[0] + h * p.sq1[2];
    const float* q2 = (const float*)p.q2 + b * p.sq2[0] + n * p.sq2[2];
    const float* dop = (const float*)p.dop + ((int64_t)b * p.N * p.Hs + h) * dv;  // row i at + i Hs dv
    for (int i0 = first; i0 < p.N; i0 += 64) {
      const int i = i0 + lane;
      float ds1 = 0.f, pc = 0.f;
      if (i < p.N) {
        const RowStat rs = row_stat(p, b, h, i);
        const float s1 = dot_lds(k1s, q1 + (int64_t)i * p.sq1[1], d);
        const float s2 = dot_lds(k2s, q2 + (int64_t)i * p.sq2[1], d);
        const float dp = dot_lds(vs, dop + (int64_t)i * p.Hs * dv, dv);
        const float p1 = exp2f(fmaf(s1, p.sm_scale_log2, -rs.l1));
        const float p2 = exp2f(fmaf(s2, p.sm_scale_log2, -rs.l2));
        ds1 = p1 * (dp - rs.d1);
        pc = fmaf(sgn, p2, p1);
      }
      ds1s[lane] = ds1;
      pcs[lane] = pc;
      __syncthreads();
      const int cnt = min(64, p.N - i0);
      for (int ii = 0; ii < cnt; ++ii) {
        const int64_t ir = i0 + ii;
        if (lane < d) dk1 = fmaf(ds1s[ii], q1[ir * p.sq1[1] + lane], dk1);
        const float* dr = dop + ir * p.Hs * dv;
        if (lane < dv) dva = fmaf(pcs[ii], dr[lane], dva);
        if (lane + 64 < dv) dvb = fmaf(pcs[ii], dr[lane + 64], dvb);
      }
      __syncthreads();
    }
  }
  if (lane < d) ((float*)p.gk1)[b * p.sgk1[0] + (int64_t)j * p.sgk1[1] + k * p.sgk1[2] + lane] = dk1 * p.sm_scale;
  float* gv = (float*)p.gv + b * p.sgv[0] + (int64_t)j * p.sgv[1] + k * p.sgv[2];
  if (lane < dv) gv[lane] = dva;
  if (lane + 64 < dv) gv[lane + 64] = dvb;
}

}  // namespace

hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_f32_dq_kernel, dim3(p.N, p.Hn, p.B), dim3(64), 0, s, p);
  hipLaunchKernelGGL(bwd_f32_dk2_kernel, dim3(p.N, p.Hn, p.B), dim3(64), 0, s, p);
  hipLaunchKernelGGL(bwd_f32_dk1dv_kernel, dim3(p.N, p.Hkv, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

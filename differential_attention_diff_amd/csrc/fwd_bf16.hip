// bf16 fused prefill for gfx950: differential attention and Grouped
// Differential Attention, dual online softmax on MFMA, fused head RMS norm.
//
// Computes, per signal head h and query i ("Differential Attention in Large
// Language Models: How Denoising Subtraction Eliminates Attention Noise and
// Outlier Activations" (llms.blog), "Differential Attention Architecture",
// DiffAttn equation; "Headwise Normalization", head_bar_i equation):
//   o = softmax(Q1 K1^T/sqrt(d)) V - lambda softmax(Q2 K2^T/sqrt(d)) V
//   out = (1 - lambda_init) * w * o / sqrt(mean(o^2) + eps)
// with Q2/K2 taken from the noise head of h and K1/V from its key/value head
// ("Grouped Differential Attention" (mlsanity.com), "Abstract": noise heads
// shared GQA-style).
//
// Work decomposition
//   * A workgroup (4 wavefronts) owns 128 queries of one (batch, signal head).
//     Workgroup ids are remapped so that each XCD (ids congruent mod 8) walks
//     a contiguous range of (batch, noise group) items, longest causal
//     q-block first, the signal heads of a noise group back to back -- the
//     group's K2/Q2 and the head's K1/V stay hot in that XCD's L2.
//   * K1, K2 and V tiles of 64 keys are staged through registers into a
//     double-buffered LDS ring (one barrier per tile); both softmax maps and
//     all four wavefronts read them from LDS.
//   * Scores are computed transposed, S^T = K Q^T on v_mfma_f32_32x32x16_bf16,
//     so lane (q, half) holds 16 keys of ONE query row: the row max needs one
//     v_permlane32_swap, the row sum none until the epilogue.
//   * Each map keeps its running max m and sum l in fp32 per row; m is only
//     moved when a new tile's max exceeds it by more than 8 (log2 units), so
//     the O rescale is rare; the stale reference bounds p by 2^8, and the final
//     O/l is unchanged (exact up to rounding).
//   * P (bf16) feeds O^T += V^T P^T straight from registers; V^T fragments
//     come from LDS with ds_read_b64_tr_b16 (4 keys x 16 channels per 16
//     lanes), each fragment loaded once and used by the MFMAs of BOTH maps.
//   * Epilogue: o = O1/l1 - lambda O2/l2, RMS over dv (in-lane + one swap),
//     times (1 - lambda_init) w, round to bf16, store.
#include <math.h>

#include "kernels.h"

namespace da {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kQW = 32;                // queries per wavefront (MFMA N dim)
constexpr int kQB = kWaves * kQW;      // queries per workgroup
constexpr int kKT = 64;                // keys per LDS tile
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleSlack = 8.0f;  // log2 units a stale max may lag

template <int D>
struct Cfg {
  static constexpr int DV = 2 * D;
  static constexpr int KS = D + 8;     // LDS row stride of K tiles (elements): 16 B pad
  static constexpr int VS = DV + 16;   // LDS row stride of the V tile: 32 B pad
  static constexpr int KE = kKT * KS;
  static constexpr int VE = kKT * VS;
  static constexpr int STAGE = 2 * KE + VE;               // bf16 elements per ring slot
  static constexpr int KCH = kKT * D / 8 / kThreads;      // 16-B chunks / thread / K tile
  static constexpr int VCH = kKT * DV / 8 / kThreads;     // 16-B chunks / thread / V tile
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");
};

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                            float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, bf16x8);
}

// One softmax map's update for a 32-key sub-block held as S^T in `s` (lane =
// query row, 16 keys per lane half).  Produces the bf16 P^T operands of the
// two 16-key PV steps and rescales `o` when the reference max moves.
template <int NCB>
__device__ __forceinline__ void online_softmax(f32x16& s, float sc, float& m, float& l, f32x16 (&o)[NCB],
                                               bf16x8& p0, bf16x8& p1) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = half_swap_max(mx) * sc;
  const bool need = mx > m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float mu = need ? mx : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mu);
    m = mu;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
  }
  float pr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sc, -m));
  p0 = to_bf16x8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
  p1 = to_bf16x8(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
  // l accumulates the bf16-rounded weights the PV product uses, so each row of
  // P/l sums to one up to fp32 rounding (v_dot2_f32_bf16 against (1, 1))
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  float sum = 0.f;
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 0, 1), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 2, 3), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 4, 5), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 6, 7), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 0, 1), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 2, 3), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 4, 5), one2, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 6, 7), one2, sum, false);
  l += sum;
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D>;
  constexpr int DV = C::DV, NCB = DV / 32, NKS = D / 16;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work item: XCD-contiguous, (batch, noise group) major, longest q-block first
  const int nq = (p.N + kQB - 1) / kQB;
  const int total = p.B * p.Hs * nq;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  const int logical = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int member = logical % p.g;
  int t = logical / p.g;
  const int qb = nq - 1 - t % nq;
  t /= nq;
  const int n = t % p.Hn;
  const int b = t / p.Hn;
  const int h = p.members[n * p.g + member];
  const int kh = p.kv[h];
  const int q0 = qb * kQB;
  const int qw0 = q0 + wave * kQW;
  const bool wave_live = qw0 < p.N;

  const __bf16* Q1 = (const __bf16*)p.q1 + b * p.sq1[0] + h * p.sq1[2];
  const __bf16* Q2 = (const __bf16*)p.q2 + b * p.sq2[0] + n * p.sq2[2];
  const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + kh * p.sk1[2];
  const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[2];
  const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + kh * p.sv[2];

  // Q fragments: B operand of S^T = K Q^T; lane (q, half) holds Q[q][16s + 8 half + 0..7]
  bf16x8 q1f[NKS], q2f[NKS];
  {
    const int q = qw0 + l32;
    const bool ok = q < p.N;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
      if (ok) {
        a = *(const u32x4*)(Q1 + (int64_t)q * p.sq1[1] + 16 * s + 8 * hh);
        c = *(const u32x4*)(Q2 + (int64_t)q * p.sq2[1] + 16 * s + 8 * hh);
      }
      q1f[s] = __builtin_bit_cast(bf16x8, a);
      q2f[s] = __builtin_bit_cast(bf16x8, c);
    }
  }

  const int q_end = min(q0 + kQB, p.N);
  const int kend = p.causal ? q_end : p.N;
  const int ntiles = (kend + kKT - 1) / kKT;

  f32x16 o1[NCB], o2[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o1[c][r] = 0.f;
      o2[c][r] = 0.f;
    }
  float m1 = -1e30f, m2 = -1e30f, l1 = 0.f, l2 = 0.f;
  const float sc = p.sm_scale_log2;

  // ---- global -> register staging of one tile (rows past N are zero)
  u32x4 rk1[C::KCH], rk2[C::KCH], rv[C::VCH];
  auto gload = [&](int tile) {
    const int key0 = tile * kKT;
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int c = tid + kThreads * u, row = c / (D / 8), col = c % (D / 8), key = key0 + row;
      u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      if (key < p.N) {
        x = *(const u32x4*)(K1 + (int64_t)key * p.sk1[1] + col * 8);
        y = *(const u32x4*)(K2 + (int64_t)key * p.sk2[1] + col * 8);
      }
      rk1[u] = x;
      rk2[u] = y;
    }
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) {
      const int c = tid + kThreads * u, row = c / (DV / 8), col = c % (DV / 8), key = key0 + row;
      u32x4 x = {0, 0, 0, 0};
      if (key < p.N) x = *(const u32x4*)(V + (int64_t)key * p.sv[1] + col * 8);
      rv[u] = x;
    }
  };
  auto sstore = [&](int buf) {
    __bf16* base = smem + buf * C::STAGE;
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int c = tid + kThreads * u, row = c / (D / 8), col = c % (D / 8);
      *(u32x4*)(base + row * C::KS + col * 8) = rk1[u];
      *(u32x4*)(base + C::KE + row * C::KS + col * 8) = rk2[u];
    }
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) {
      const int c = tid + kThreads * u, row = c / (DV / 8), col = c % (DV / 8);
      *(u32x4*)(base + 2 * C::KE + row * C::VS + col * 8) = rv[u];
    }
  };

  // lane's element offset for the ds_read_b64_tr_b16 of V^T fragments: lane j of
  // each 16-lane group reads V[key0 + j/4][c0 + 4 (j%4) .. +3]; the transpose
  // hands lane i the 4 keys of channel c0 + i.
  const int vt_lane = (4 * hh + (lane & 15) / 4) * C::VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  gload(0);
  sstore(0);
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) gload(tile + 1);
    const __bf16* K1s = smem + buf * C::STAGE;
    const __bf16* K2s = K1s + C::KE;
    const __bf16* Vs = K1s + 2 * C::KE;
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb) {
      const int k0 = tile * kKT + kb * 32;
      if (!wave_live || k0 >= kend) continue;
      if (p.causal && k0 > qw0 + kQW - 1) continue;  // sub-block above this wavefront's diagonal
      f32x16 s1, s2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s1[r] = 0.f;
        s2[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 a = *(const bf16x8*)(K1s + (kb * 32 + l32) * C::KS + 16 * s + 8 * hh);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q1f[s], s1, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 a = *(const bf16x8*)(K2s + (kb * 32 + l32) * C::KS + 16 * s + 8 * hh);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q2f[s], s2, 0, 0, 0);
      }
      // S^T[r] of lane (q, half): key k0 + 8 (r/4) + 4 half + r%4, query qw0 + q
      const bool diag = p.causal && (k0 + 31 > qw0);
      const bool tail = !p.causal && (k0 + 32 > p.N);
      if (diag || tail) {
        const int q = qw0 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r / 4) + 4 * hh + (r & 3);
          const bool hide = p.causal ? (key > q) : (key >= p.N);
          if (hide) {
            s1[r] = -INFINITY;
            s2[r] = -INFINITY;
          }
        }
      }
      bf16x8 pa0, pa1, pb0, pb1;
      online_softmax<NCB>(s1, sc, m1, l1, o1, pa0, pa1);
      online_softmax<NCB>(s2, sc, m2, l2, o2, pb0, pb1);
      // O^T += V^T P^T for both maps; V^T fragment (32 channels x 16 keys) loaded once
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const __bf16* vb = Vs + vt_lane + (kb * 32 + ks * 16) * C::VS + cb * 32;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vb);
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + 8 * C::VS));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ks ? pa1 : pa0, o1[cb], 0, 0, 0);
          o2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ks ? pb1 : pb0, o2[cb], 0, 0, 0);
        }
      }
    }
    if (tile + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;

  // ---- epilogue: o = O1/l1 - lambda O2/l2, then the head RMS norm
  l1 = half_swap_sum(l1);
  l2 = half_swap_sum(l2);
  const float i1 = 1.0f / l1, i2 = 1.0f / l2;
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // both maps take identical operations: identical maps with lambda = 1 give exact zeros
      const float x = __builtin_fmaf(-p.lam, __fmul_rn(o2[c][r], i2), __fmul_rn(o1[c][r], i1));
      o1[c][r] = x;
      ss = __builtin_fmaf(x, x, ss);
    }
  float scale = 1.0f;
  if (p.normalize) {
    ss = half_swap_sum(ss);
    scale = (1.0f - p.lam_init) / sqrtf(ss * (1.0f / DV) + p.eps);
  }
  const int q = qw0 + l32;
  if (q < p.N) {
    __bf16* out = (__bf16*)p.out + b * p.so[0] + (int64_t)q * p.so[1] + h * p.so[2];
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ch = c * 32 + 8 * g4 + 4 * hh;  // channels ch..ch+3 live in o1[c][4 g4 .. 4 g4 + 3]
        f32x4 w = {1.f, 1.f, 1.f, 1.f};
        if (p.normalize && p.norm_w) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = p.norm_w[ch + e];
        }
        f32x4 y = {o1[c][4 * g4] * scale * w[0], o1[c][4 * g4 + 1] * scale * w[1],
                   o1[c][4 * g4 + 2] * scale * w[2], o1[c][4 * g4 + 3] * scale * w[3]};
        *(bf16x4*)(out + ch) = __builtin_convertvector(y, bf16x4);
      }
    if (p.lse && hh == 0) {
      const int64_t base = ((int64_t)b * p.Hs + h) * p.N + q;
      const int64_t plane = (int64_t)p.B * p.Hs * p.N;
      constexpr float kLn2 = 0.69314718055994531f;
      p.lse[base] = (m1 + __log2f(l1)) * kLn2;
      p.lse[plane + base] = (m2 + __log2f(l2)) * kLn2;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s) {
  const int64_t nq = (p.N + kQB - 1) / kQB;
  const int64_t total = (int64_t)p.B * p.Hs * nq;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  if (p.d == 64)
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)total), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<32>, dim3((unsigned)total), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

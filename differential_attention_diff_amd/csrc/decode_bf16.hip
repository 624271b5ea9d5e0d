// bf16 split-K decode for differential / grouped differential attention.
//
// One new query per sequence against its caches (the serving step the
// "Hardware Implementations and Serving Considerations" section of
// "Differential Attention in Large Language Models: How Denoising Subtraction
// Eliminates Attention Noise and Outlier Activations" (llms.blog) points at),
// computing that page's DiffAttn equation and head_bar_i norm for every signal
// head, with the noise heads shared GQA-style ("Grouped Differential
// Attention" (mlsanity.com), "Abstract").
//
// Kernel 1 (partial): one workgroup per (chunk of `chunk` cached positions,
// noise group, sequence).  Every cached K2 byte of the group and every K1/V
// byte of the group's distinct key/value heads is read from HBM once, in
// coalesced 16-B rows staged through LDS:
//   pass A  scores of the g signal queries (against K1) and the noise query
//           (against K2) for all chunk positions, kept in LDS (v_dot2 bf16);
//   pass B  exact chunk max m and sum l per query (log2 units), P in place;
//   pass C  unnormalised outputs: one per signal head (map 1) and one per
//           distinct V head (map 2, shared by the group's signal heads).
// Each (m, l, o[dv]) goes to the workspace.
// Kernel 2 (combine): one wavefront per (sequence, signal head) merges the
// chunks of each map (rescale by 2^(m_c - M)), forms O1/L1 - lambda O2/L2 and
// applies the head norm.  Fixed merge order: results are deterministic.
#include <math.h>

#include "kernels.h"

namespace da {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 256;        // threads per partial workgroup
constexpr int kSub = 128;      // cached positions per LDS sub-tile
constexpr int kD = 64;         // d (the kernel is specialised to d = 64, dv = 128)
constexpr int kDV = 128;
constexpr int kKS = kD + 8;    // LDS row stride of K sub-tiles (bf16)
constexpr int kVS = kDV + 8;   // LDS row stride of the V sub-tile (bf16)
constexpr int kMaxQ = 8;       // g + 1 scored queries per group
constexpr int kMaxOut = 8;     // g + u outputs per group
constexpr int kTileBytes = 2 * kSub * kKS * 2;  // >= kSub * kVS * 2 and >= the reduction buffer

static_assert(kSub * kVS * 2 <= kTileBytes, "V sub-tile must fit the tile region");
static_assert(4 * kMaxOut * kDV * 4 <= kTileBytes, "reduction buffer must fit the tile region");

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

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kT) void decode_partial_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
  const int c = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  const int key_lo = c * p.chunk;
  if (key_lo >= L) return;  // whole workgroup exits together (uniform)
  const int nk = min(key_lo + p.chunk, L) - key_lo;
  const int g = p.g, nu = p.nu[n], nq = g + 1;

  // LDS: [tile region][q bf16 (nq x 64)][S fp32 (nq x chunk)][m,l (2 x nq)]
  unsigned char* tile = dsm;
  uint32_t* qs = (uint32_t*)(dsm + kTileBytes);            // nq x 32 bf16 pairs
  float* S = (float*)(dsm + kTileBytes + kMaxQ * kD * 2);  // nq x chunk
  float* ml = S + nq * p.chunk;                            // m[nq], l[nq]

  // queries: 0..g-1 the group's signal heads (map 1), g the noise head (map 2)
  for (int i = tid; i < nq * (kD / 2); i += kT) {
    const int qi = i / (kD / 2), w = i % (kD / 2);
    const uint32_t* src = qi < g ? (const uint32_t*)((const __bf16*)p.q1 + b * p.sq1[0] +
                                                     p.members[n * g + qi] * p.sq1[1])
                                 : (const uint32_t*)((const __bf16*)p.q2 + b * p.sq2[0] + n * p.sq2[1]);
    qs[i] = src[w];
  }

  // ---- pass A: scores into S (log2 units)
  for (int s0 = 0; s0 < nk; s0 += kSub) {
    const int ns = min(kSub, nk - s0);
    for (int u = 0; u < nu; ++u) {
      const int kvh = p.ukv[n * g + u];
      const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + kvh * p.sk1[1] + (int64_t)(key_lo + s0) * p.sk1[2];
      const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[1] + (int64_t)(key_lo + s0) * p.sk2[2];
      const bool with_k2 = (u == 0);
      __syncthreads();  // previous users of the tile region are done
      // stage K1 (and K2) rows [0, ns): 8 chunks of 16 B per row
      u32x4 st[2 * kSub * 8 / kT];
#pragma unroll
      for (int i = 0; i < kSub * 8 / kT; ++i) {
        const int ch = tid + kT * i, row = ch / 8, col = ch % 8;
        u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
        if (row < ns) {
          x = *(const u32x4*)(K1 + (int64_t)row * p.sk1[2] + col * 8);
          if (with_k2) y = *(const u32x4*)(K2 + (int64_t)row * p.sk2[2] + col * 8);
        }
        st[i] = x;
        st[kSub * 8 / kT + i] = y;
      }
#pragma unroll
      for (int i = 0; i < kSub * 8 / kT; ++i) {
        const int ch = tid + kT * i, row = ch / 8, col = ch % 8;
        *(u32x4*)(tile + (row * kKS + col * 8) * 2) = st[i];
        *(u32x4*)(tile + (kSub * kKS + row * kKS + col * 8) * 2) = st[kSub * 8 / kT + i];
      }
      __syncthreads();
      // thread -> (position j, query parity): each scores its queries on map kv u
      const int j = tid % kSub, sel = tid / kSub;
      if (j < ns) {
        const uint32_t* k1row = (const uint32_t*)(tile + j * kKS * 2);
        const uint32_t* k2row = (const uint32_t*)(tile + (kSub * kKS + j * kKS) * 2);
        for (int qi = sel; qi < nq; qi += kT / kSub) {
          const bool noise = qi == g;
          if (noise ? !with_k2 : (p.kv[p.members[n * g + qi]] != kvh)) continue;
          const uint32_t* kr = noise ? k2row : k1row;
          const uint32_t* qr = qs + qi * (kD / 2);
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < kD / 2; w += 4) {
            const u32x4 kk = *(const u32x4*)(kr + w);
            const u32x4 qq = *(const u32x4*)(qr + w);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // copy the lanes to scalars first: this compiler's __builtin_bit_cast of a
              // vector element reads element 0
              const uint32_t kw = kk[e], qw = qq[e];
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw), __builtin_bit_cast(bf16x2, qw),
                                                    acc, false);
            }
          }
          S[qi * p.chunk + s0 + j] = acc * p.sm_scale_log2;
        }
      }
    }
  }
  __syncthreads();

  // ---- pass B: chunk max / sum per query, P in place
  for (int qi = wave; qi < nq; qi += kT / 64) {
    float* row = S + qi * p.chunk;
    float mx = -INFINITY;
    for (int j = lane; j < nk; j += 64) mx = fmaxf(mx, row[j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < nk; j += 64) {
      const float e = __builtin_amdgcn_exp2f(row[j] - mx);
      row[j] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      ml[qi] = mx;
      ml[nq + qi] = sum;
    }
  }

  // ---- pass C: outputs.  thread -> (channel pair cp, position quarter kq)
  const int cp = tid % 64, kq = tid / 64;
  float acc0[kMaxOut], acc1[kMaxOut];
#pragma unroll
  for (int o = 0; o < kMaxOut; ++o) acc0[o] = acc1[o] = 0.f;
  for (int s0 = 0; s0 < nk; s0 += kSub) {
    const int ns = min(kSub, nk - s0);
    for (int u = 0; u < nu; ++u) {
      const int kvh = p.ukv[n * g + u];
      const __bf16* Vg = (const __bf16*)p.v + b * p.sv[0] + kvh * p.sv[1] + (int64_t)(key_lo + s0) * p.sv[2];
      __syncthreads();
      u32x4 st[kSub * 16 / kT];
#pragma unroll
      for (int i = 0; i < kSub * 16 / kT; ++i) {
        const int ch = tid + kT * i, row = ch / 16, col = ch % 16;
        u32x4 x = {0, 0, 0, 0};
        if (row < ns) x = *(const u32x4*)(Vg + (int64_t)row * p.sv[2] + col * 8);
        st[i] = x;
      }
#pragma unroll
      for (int i = 0; i < kSub * 16 / kT; ++i) {
        const int ch = tid + kT * i, row = ch / 16, col = ch % 16;
        *(u32x4*)(tile + (row * kVS + col * 8) * 2) = st[i];
      }
      __syncthreads();
      const int jlo = kq * (kSub / 4), jhi = min(jlo + kSub / 4, ns);
      for (int j = jlo; j < jhi; ++j) {
        const uint32_t vw = *(const uint32_t*)(tile + (j * kVS + 2 * cp) * 2);
        const float v0 = bf_lo(vw), v1 = bf_hi(vw);
#pragma unroll
        for (int o = 0; o < kMaxOut; ++o) {
          // outputs 0..g-1: map 1 of member o (if its kv head is kvh); g+u: map 2 on V head u
          int src = -1;
          if (o < g) {
            if (p.kv[p.members[n * g + o]] == kvh) src = o;
          } else if (o == g + u) {
            src = g;
          }
          if (src >= 0) {
            const float w = S[src * p.chunk + s0 + j];
            acc0[o] = __builtin_fmaf(w, v0, acc0[o]);
            acc1[o] = __builtin_fmaf(w, v1, acc1[o]);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- reduce the four position quarters and write (m, l, o) per output slot
  float* red = (float*)tile;  // [4][kMaxOut][dv]
#pragma unroll
  for (int o = 0; o < kMaxOut; ++o) {
    red[(kq * kMaxOut + o) * kDV + 2 * cp] = acc0[o];
    red[(kq * kMaxOut + o) * kDV + 2 * cp + 1] = acc1[o];
  }
  __syncthreads();
  const int nout = g + nu;
  float* ws = p.ws + (((int64_t)b * p.Hn + n) * p.nchunks + c) * (int64_t)p.slots * (kDV + 2);
  for (int i = tid; i < nout * kDV; i += kT) {
    const int o = i / kDV, ch = i % kDV;
    const float v = red[(0 * kMaxOut + o) * kDV + ch] + red[(1 * kMaxOut + o) * kDV + ch] +
                    red[(2 * kMaxOut + o) * kDV + ch] + red[(3 * kMaxOut + o) * kDV + ch];
    ws[o * (kDV + 2) + 2 + ch] = v;
  }
  if (tid < nout) {
    const int q = tid < g ? tid : g;
    ws[tid * (kDV + 2) + 0] = ml[q];
    ws[tid * (kDV + 2) + 1] = ml[nq + q];
  }
}

// One wavefront per (sequence, signal head); lane owns channels 2 lane, 2 lane + 1.
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  __bf16* out = (__bf16*)p.out + b * p.so[0] + h * p.so[1];
  const int c0 = 2 * lane;
  if (L == 0) {
    bf16x2 z = {(__bf16)0.f, (__bf16)0.f};
    *(bf16x2*)(out + c0) = z;
    return;
  }
  const int n = [&] {
    for (int m = 0; m < p.Hn * p.g; ++m)
      if (p.members[m] == h) return m / p.g;
    return 0;
  }();
  int slot1 = 0;
  for (int j = 0; j < p.g; ++j)
    if (p.members[n * p.g + j] == h) slot1 = j;
  const int slot2 = p.g + p.uidx[h];
  const int nch = (L + p.chunk - 1) / p.chunk;
  const float* base = p.ws + ((int64_t)b * p.Hn + n) * p.nchunks * (int64_t)p.slots * (kDV + 2);
  const int64_t cstride = (int64_t)p.slots * (kDV + 2);
  float M1 = -INFINITY, M2 = -INFINITY;
  for (int c = 0; c < nch; ++c) {
    M1 = fmaxf(M1, base[c * cstride + slot1 * (kDV + 2)]);
    M2 = fmaxf(M2, base[c * cstride + slot2 * (kDV + 2)]);
  }
  float L1 = 0.f, L2 = 0.f, a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float* s1 = base + c * cstride + slot1 * (kDV + 2);
    const float* s2 = base + c * cstride + slot2 * (kDV + 2);
    const float f1 = __builtin_amdgcn_exp2f(s1[0] - M1), f2 = __builtin_amdgcn_exp2f(s2[0] - M2);
    L1 = __builtin_fmaf(s1[1], f1, L1);
    L2 = __builtin_fmaf(s2[1], f2, L2);
    a0 = __builtin_fmaf(s1[2 + c0], f1, a0);
    a1 = __builtin_fmaf(s1[3 + c0], f1, a1);
    b0 = __builtin_fmaf(s2[2 + c0], f2, b0);
    b1 = __builtin_fmaf(s2[3 + c0], f2, b1);
  }
  const float i1 = 1.0f / L1, i2 = 1.0f / L2;
  const float o0 = __builtin_fmaf(-p.lam, __fmul_rn(b0, i2), __fmul_rn(a0, i1));
  const float o1 = __builtin_fmaf(-p.lam, __fmul_rn(b1, i2), __fmul_rn(a1, i1));
  float scale = 1.0f, w0 = 1.0f, w1 = 1.0f;
  if (p.normalize) {
    const float ms = wave_sum(o0 * o0 + o1 * o1) * (1.0f / kDV);
    scale = (1.0f - p.lam_init) / sqrtf(ms + p.eps);
    if (p.norm_w) {
      w0 = p.norm_w[c0];
      w1 = p.norm_w[c0 + 1];
    }
  }
  bf16x2 y = {(__bf16)(o0 * scale * w0), (__bf16)(o1 * scale * w1)};
  *(bf16x2*)(out + c0) = y;
}

}  // namespace

size_t decode_lds_bytes(const DecodeParams& p) {
  return kTileBytes + kMaxQ * kD * 2 + (size_t)(p.g + 1) * p.chunk * 4 + 2 * kMaxQ * 4;
}

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s) {
  (void)dtype;
  if (p.d != kD || p.dv != kDV || p.g + 1 > kMaxQ || p.slots > kMaxOut) return hipErrorInvalidValue;
  if (p.nchunks > 0) {
    const size_t lds = decode_lds_bytes(p);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)decode_partial_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(decode_partial_kernel, dim3(p.nchunks, p.Hn, p.B), dim3(kT), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.Hs, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

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
// The step is bound by HBM bandwidth (about 3 FLOP per cached byte), so the
// kernels are organised around keeping enough bytes in flight:
//
// Kernel 1 (partial): one workgroup per (chunk of cached positions, noise
// group, sequence).  The chunk is walked in sub-chunks of kC = 128 positions
// (256 for e4m3 caches); each of the four wavefronts owns a quarter of every
// sub-chunk and runs its own softmax over it, so the loop has no workgroup
// barrier.  A wavefront's loads of a sub-chunk -- K2 of the noise head, K1 and
// V of the group's key/value head (16 KiB for d = 64) -- are all in flight at
// once, into registers; the next sub-chunk's keys are loaded as soon as the
// scores are taken and its values as soon as P.V is done:
//   scores  S = K Q^T on v_mfma_f32_16x16x32_bf16, 16 cached rows per product
//           with the group's queries as the columns: the g signal queries
//           against K1, the noise query against K2, in log2 units; lane l
//           keeps the scores of query l%16;
//   softmax the 4 lanes of a query column reduce its max and sum by lane
//           swaps; the wavefront's running max m and sum l per query move
//           (its accumulators are rescaled by 2^(m_old - m_new)); the bf16
//           weights go to the wavefront's own LDS rows;
//   P.V     thread (8 rows, 8 channels; rows taken in pairs, one v_dot2 per
//           channel and pair) accumulates one output per signal head
//           (map 1) and one per distinct V head (map 2, shared by the group's
//           signal heads) from its V registers.
// At the end the four wavefronts' partials are put on a common max (rescale by
// 2^(m_w - M)) and summed over the chunk's rows through LDS.
// Each output's (m, l, o[dv]) goes to the workspace.  A group whose signal
// heads use several key/value heads loops over them.
// Kernel 2 (combine): one workgroup per (noise group, sequence) merges the
// chunks of every output slot once (rescale by 2^(m_c - M)), then forms
// O1/L1 - lambda O2/L2 per signal head and applies the head norm.  Fixed merge
// order: results are deterministic.
#include <math.h>

#include <mutex>

#include "kernels.h"

namespace da {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8 cache elements as one register chunk: 16 bytes of bf16 or 8 bytes of fp8
template <bool FP8>
struct Chunk {
  typedef u32x4 T;
};
template <>
struct Chunk<true> {
  typedef u32x2 T;
};

// 8 OCP e4m3 bytes (little-endian: element e is byte e) as 8 bf16 in 4 dwords.
// Every e4m3 value is exact in bf16 (3 mantissa bits, exponents inside bf16's
// range), so the products below are the same as on bf16 caches of those values.
__device__ __forceinline__ u32x4 fp8_to_bf16(u32x2 c) {
  const uint32_t lo = c[0], hi = c[1];
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, e),
               __builtin_bit_cast(uint32_t, f)};
}
__device__ __forceinline__ u32x4 as_bf16(u32x4 c) { return c; }
// a cache chunk, loaded non-temporally: every cache byte is read once per
// call, so keeping it in the caches only evicts what other loads reuse
// (-8% for bf16 caches against plain loads, -2% for e4m3)
template <typename T>
__device__ __forceinline__ T ld_cache(const T* a) {
  return __builtin_nontemporal_load(a);
}
__device__ __forceinline__ u32x4 as_bf16(u32x2 c) { return fp8_to_bf16(c); }

constexpr int kT = 256;       // threads per workgroup
constexpr int kC = 128;       // cached positions per sub-chunk (bf16 caches; e4m3: 2 kC)
constexpr int kD = 64;        // the kernels are specialised to d = 64, dv = 128
constexpr int kDV = 128;
constexpr int kMaxQ = 8;      // g + 1 scored queries per group (largest instantiation)
constexpr int kMaxOut = 8;    // g + u outputs per group (largest instantiation)
static_assert(kC * (kD / 8) / kT == 4 && kC * (kDV / 8) / kT == 8,
              "layout below assumes 128 positions, d = 64, 256 threads");

// Cross-lane steps on DPP (VALU, no LDS round trip): quad_perm xor 1 / xor 2,
// row_half_mirror (lane i <-> 7 - i of each 8) and row_mirror (i <-> 15 - i of
// each 16); a 16-lane result is combined across the four rows with readlane.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

__device__ __forceinline__ float sum8(float x) {  // every lane of each 8-lane group gets the group sum
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  return x + dpp<kRowHalfMirror>(x);
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = sum8(x);
  x += dpp<kRowMirror>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
// x rounded to the nearest bf16 (ties to even), returned as the fp32 of that value
__device__ __forceinline__ float round_bf16(float x) {
  const __bf16 h = (__bf16)x;
  return (float)h;
}

// Channels of two cached rows a, b (8 each) as bf16 pairs: cv[c] = (a[c], b[c]), so a
// v_dot2 against the pair of the rows' weights adds both rows' products at once.
// e4m3: the fp8 bytes are interleaved first and then converted (exact, as above).
__device__ __forceinline__ void pair_rows(u32x4 a, u32x4 b, uint32_t (&cv)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = a[e], y = b[e];
    cv[2 * e] = __builtin_amdgcn_perm(y, x, 0x05040100u);      // low halves
    cv[2 * e + 1] = __builtin_amdgcn_perm(y, x, 0x07060302u);  // high halves
  }
}
__device__ __forceinline__ void pair_rows(u32x2 a, u32x2 b, uint32_t (&cv)[8]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t x = a[e], y = b[e];
    const uint32_t lo = __builtin_amdgcn_perm(y, x, 0x05010400u);  // a.c0 b.c0 a.c1 b.c1
    const uint32_t hi = __builtin_amdgcn_perm(y, x, 0x07030602u);  // a.c2 b.c2 a.c3 b.c3
    cv[4 * e + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    cv[4 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    cv[4 * e + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    cv[4 * e + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  }
}

// MAXO bounds both g + 1 (scored queries) and g + u (outputs); 4 covers 3:1 GDA
// with one key/value head per group, 8 the general case.
// MULTI: some noise group spans several key/value heads (u > 1); the kernel then
// re-loads K1 / V per head inside the sub-chunk.  Without it the loops collapse.
// FP8: the caches hold OCP e4m3 bytes (8-byte chunks of 8 elements, same thread
// layout, twice the positions per sub-chunk), converted to bf16 in registers;
// keys are read as value * k_scale by scaling the scores, values as
// value * v_scale by scaling the partial outputs.
template <int MAXO, bool MULTI, bool FP8>
__global__ __launch_bounds__(kT, 3) void decode_partial_kernel(DecodeParams p) {
  constexpr int kMaxQ = MAXO, kMaxOut = MAXO;
  constexpr uint32_t ES = FP8 ? 1 : 2;  // cache bytes per element
  // positions per sub-chunk: fp8 caches take twice as many, so a sub-chunk keeps the
  // same bytes (and registers) in flight
  constexpr int CP = FP8 ? 2 * kC : kC;
  constexpr int kKC = CP * (kD / 8) / kT;   // K chunks of 8 elements per thread
  constexpr int kVC = CP * (kDV / 8) / kT;  // V chunks of 8 elements per thread
  static_assert(kKC == 2 * (CP / 64) && kD == 64, "K: two 32-dim steps per 16-row group, CP / 64 groups per wave");
  static_assert(kT / 64 == 4 && kVC == CP / 16, "four waves, each with CP/4 rows of every sub-chunk");
  typedef typename Chunk<FP8>::T CK;
  // weights of a wave's rows of the current sub-chunk, per query (each wave its own)
  __shared__ __attribute__((aligned(16))) float SW[kT / 64][kMaxQ][CP / 4];
  __shared__ float MLW[kT / 64][2][kMaxQ];      // each wave's running max and sum per query
  __shared__ u32x4 QS[kMaxQ][kD / 8];           // the group's queries
  __shared__ float red[kT / 16][kMaxOut][kDV];  // partial outputs per 16-lane row group
  const int c = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  const int key_lo = c * p.chunk;
  if (key_lo >= L) return;  // uniform across the workgroup
  const int nk = min(p.chunk, L - key_lo);
  // Head-map entries, read once before any cache load is in flight (the 16-bit tables are
  // read with vector loads, and each such read would otherwise wait for every outstanding
  // load of the chunk) and kept in scalar registers: they are uniform.
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int g = p.g, nu = MULTI ? uni(p.nu[n]) : 1, nq = g + 1, nout = g + nu;
  int mem_h[kMaxQ], mem_kv[kMaxQ], ukv[kMaxOut];
#pragma unroll
  for (int i = 0; i < kMaxQ; ++i) {
    mem_h[i] = i < g ? uni(p.members[n * g + i]) : 0;
    mem_kv[i] = i < g ? uni(p.kv[mem_h[i]]) : -1;
  }
#pragma unroll
  for (int u = 0; u < kMaxOut; ++u) ukv[u] = u < nu ? uni(p.ukv[n * g + u]) : -1;

  // K layout (A operands of v_mfma_f32_16x16x32_bf16): wave w owns CP/4 rows in groups of
  // 16; for group j and 32-dim step s, lane l holds row 16 j + l%16 of the wave's rows,
  // dims 32 s + 8 (l/16) .. +7 (register i = 2 j + s)
  const int krow = wave * (CP / 4) + (lane & 15), kq = lane >> 4;
  // V layout: wave w owns the same CP/4 rows as for K; lane l holds rows l/16 + 4 i of them
  // (i < kVC), channels 8 (l%16) .. +7
  const int vrow = wave * (CP / 4) + (lane >> 4), vcol = lane & 15;

  CK k1r[kKC], k2r[kKC], vr[kVC];
  // Rows [r0, r0 + ns) of the chunk (relative to key_lo).  Loads are branch-free so the
  // compiler can count them and wait for exactly the ones a step needs: a row past ns
  // re-reads row ns - 1 (in bounds); its score is masked and its weight is zero.
  // Addresses: a uniform 64-bit base (scalar registers) plus a 32-bit per-lane byte
  // offset (the host bounds the position stride so chunk offsets fit in 32 bits).
  // Cache rows are read with non-temporal loads (ld_cache).
  // rows [pos, pos + CP) of a cache: one block of a paged cache holds the whole sub-chunk
  auto cache_row0 = [&](const int64_t* st, int head, int pos) -> int64_t {
    if (p.block_table) {
      const int blk = min(max(p.block_table[(int64_t)b * p.max_blocks + pos / p.block_size], 0), p.num_blocks - 1);
      return blk * st[0] + head * st[1] + (int64_t)(pos % p.block_size) * st[2];
    }
    return b * st[0] + head * st[1] + (int64_t)pos * st[2];
  };
  auto load_k = [&](CK(&dst)[kKC], const void* base, const int64_t* st, int head, int r0, int ns) {
    const char* K = (const char*)base + cache_row0(st, head, key_lo + r0) * ES;
    const uint32_t rs = (uint32_t)st[2] * ES;
#pragma unroll
    for (int i = 0; i < kKC; ++i) {
      const uint32_t r = (uint32_t)min(krow + 16 * (i >> 1), ns - 1);
      dst[i] = ld_cache((const CK*)(K + (r * rs + 8u * ES * (uint32_t)(kq + 4 * (i & 1)))));
    }
  };
  auto load_v = [&](int head, int r0, int ns) {
    const char* V = (const char*)p.v + cache_row0(p.sv, head, key_lo + r0) * ES;
    const uint32_t rs = (uint32_t)p.sv[2] * ES;
#pragma unroll
    for (int i = 0; i < kVC; ++i) {
      const uint32_t r = (uint32_t)min(vrow + 4 * i, ns - 1);
      vr[i] = ld_cache((const CK*)(V + (r * rs + 8u * ES * (uint32_t)vcol)));
    }
  };
  // the group's queries in LDS (each thread reads its 8 dims when scoring):
  // qs[qi] for qi < g the signal member qi, qs[g] the noise query
  for (int i = tid; i < (g + 1) * (kD / 8); i += kT) {
    const int qi = i / (kD / 8), col = i % (kD / 8);
    const __bf16* q = qi < g ? (const __bf16*)p.q1 + b * p.sq1[0] + mem_h[qi] * p.sq1[1]
                             : (const __bf16*)p.q2 + b * p.sq2[0] + n * p.sq2[1];
    QS[qi][col] = *(const u32x4*)(q + 8 * col);
  }
  // scores in log2 units; e4m3 keys carry their cache's scale
  const float sc1 = p.sm_scale_log2 * (FP8 ? p.k1_scale : 1.0f), sc2 = p.sm_scale_log2 * (FP8 ? p.k2_scale : 1.0f);
  // S = K Q^T per 16 rows on MFMA: the B operand holds the group's queries as columns
  // (lane l: query l%16, zero past the noise query g), so one product of K1 gives the
  // signal queries' scores and one of K2 the noise query's; lane l receives rows
  // 4 (l/16) .. +3 of column l%16 and keeps those of its own query and map.
  const int qq = lane & 15;
  int qkv = -1;  // key/value head of the signal query in column qq
#pragma unroll
  for (int i = 0; i < kMaxQ; ++i) qkv = qq == i ? mem_kv[i] : qkv;
  bf16x8 qf[2];
  auto score_rows = [&](f32x4(&sv)[kKC / 2], const CK(&kr)[kKC], bool mine, float scale) {
#pragma unroll
    for (int j = 0; j < kKC / 2; ++j) {
      f32x4 c = {};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, as_bf16(kr[2 * j + s])), qf[s], c, 0, 0,
                                                    0);
      sv[j] = mine ? c * scale : sv[j];
    }
  };

  float acc[kMaxOut][8];
#pragma unroll
  for (int o = 0; o < kMaxOut; ++o)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[o][e] = 0.f;
  // this wave's running max and sum for the query in column qq (the same in the 4 lanes
  // qq + 16 k); the max starts finite so that rows all masked give factor 1, weight 0
  float m_run = -1e30f, l_run = 0.f;

  // ---- every load of the first sub-chunk (the group's first key/value head) up front
  const int kv0 = ukv[0];
  int ns = min(CP, nk);
  // issue order K2, K1, then V (the scheduler must not interleave them): the scores then
  // wait only for the keys while the values are still in flight
  load_k(k2r, p.k2, p.sk2, n, 0, ns);
  load_k(k1r, p.k1, p.sk1, kv0, 0, ns);
  __builtin_amdgcn_sched_barrier(0);
  load_v(kv0, 0, ns);
  __builtin_amdgcn_sched_barrier(0);

  // The queries are in LDS after this barrier.  From here on each wave walks its own
  // CP/4 rows of every sub-chunk with its own running softmax: no workgroup barrier until
  // the four waves' partials are merged at the end.
  __syncthreads();
  float(*W)[CP / 4] = SW[wave];
  for (int r0 = 0; r0 < nk; r0 += CP) {
    const int nxt = r0 + CP, ns_next = min(CP, nk - nxt);
    // ---- scores (log2 units): the noise query on K2, each signal query on its K1
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 x = QS[min(qq, g)][4 * s + kq];
      qf[s] = __builtin_bit_cast(bf16x8, qq <= g ? x : u32x4{0u, 0u, 0u, 0u});
    }
    f32x4 sv[kKC / 2];
#pragma unroll
    for (int j = 0; j < kKC / 2; ++j) sv[j] = f32x4{};
    score_rows(sv, k2r, qq == g, sc2);
#pragma unroll
    for (int u = 0; u < (MULTI ? kMaxOut : 1); ++u) {
      if (u < nu) {
        const int kvh = ukv[u];
        if (u > 0) load_k(k1r, p.k1, p.sk1, kvh, r0, ns);
        score_rows(sv, k1r, qq < g && qkv == kvh, sc1);
      }
    }
    if (nxt < nk) {  // K registers are free: prefetch the next sub-chunk's keys
      __builtin_amdgcn_sched_barrier(0);
      load_k(k2r, p.k2, p.sk2, n, nxt, ns_next);
      load_k(k1r, p.k1, p.sk1, kv0, nxt, ns_next);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- this wave's rows into the running softmax of the query in column qq: the lane's
    // rows are rb + 16 j + r; the 4 lanes qq + 16 k hold the query's rows between them
    const int rb = wave * (CP / 4) + 4 * kq;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKC / 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[j][r] = rb + 16 * j + r < ns ? sv[j][r] : -INFINITY;
        mx = fmaxf(mx, sv[j][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the wave's first valid rows
    // weights are rounded to bf16 here: P.V consumes them as bf16 and the running sum
    // accumulates the same rounded values (masked rows: 2^-inf = 0)
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < kKC / 2; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[j][r] = round_bf16(__builtin_amdgcn_exp2f(sv[j][r] - m_new));
        tot += sv[j][r];
      }
      if (qq <= g) *(f32x4*)&W[qq][16 * j + 4 * kq] = sv[j];
    }
    tot += __shfl_xor(tot, 16);
    tot += __shfl_xor(tot, 32);
    l_run = l_run * alpha + tot;
    m_run = m_new;
    // the weights were written by other lanes of this wave: LDS serves a wave's accesses in
    // order, and nothing may be moved across this point
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- P.V: outputs 0..g-1 = map 1 of each member, g + u = map 2 on the group's u-th V head
#pragma unroll
    for (int o = 0; o < kMaxOut; ++o) {
      if (o < nout) {
        const float a = lane_f(alpha, o < g ? o : g);  // lane q holds query q's factor
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[o][e] *= a;
      }
    }
#pragma unroll
    for (int u = 0; u < (MULTI ? kMaxOut : 1); ++u) {
      if (u >= nu) continue;
      const int kvh = ukv[u];
      if (u > 0) load_v(kvh, r0, ns);
      static_assert(kVC % 2 == 0, "rows are taken in pairs");
#pragma unroll
      for (int i = 0; i < kVC; i += 2) {
        const int lr = (lane >> 4) + 4 * i;  // the wave's rows lr and lr + 4
        uint32_t cv[8];
        pair_rows(vr[i], vr[i + 1], cv);
#pragma unroll
        for (int o = 0; o < kMaxOut; ++o) {
          int src = -1;
          if (o < g) {
            if (mem_kv[o] == kvh) src = o;
          } else if (o == g + u) {
            src = g;
          }
          if (src >= 0) {
            // the two rows' bf16 weights (the upper halves of their fp32 values, which are
            // bf16-rounded) as one pair: each v_dot2 adds w_r v_r[c] + w_r' v_r'[c]
            const uint32_t wp =
                __builtin_amdgcn_perm(__float_as_uint(W[src][lr + 4]), __float_as_uint(W[src][lr]), 0x07060302u);
#pragma unroll
            for (int ch = 0; ch < 8; ++ch)
              acc[o][ch] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cv[ch]),
                                                           __builtin_bit_cast(bf16x2, wp), acc[o][ch], false);
          }
        }
        // one row pair's weights live at a time (keeps the kernel's wavefronts per SIMD)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (nxt < nk) {  // V registers are free: prefetch
      __builtin_amdgcn_sched_barrier(0);
      load_v(kv0, nxt, ns_next);
      __builtin_amdgcn_sched_barrier(0);
    }
    ns = ns_next;
    // the next sub-chunk's weights overwrite these only after this wave's reads above
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves (each relative to its own running max), then reduce over the
  // 16 row groups (threads t and t + 16 k hold the same channels) via LDS
  if (lane <= g) {
    MLW[wave][0][lane] = m_run;
    MLW[wave][1][lane] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int o = 0; o < kMaxOut; ++o)
    if (o < nout) {
      const int q = o < g ? o : g;
      const float M = fmaxf(fmaxf(MLW[0][0][q], MLW[1][0][q]), fmaxf(MLW[2][0][q], MLW[3][0][q]));
      const float f = __builtin_amdgcn_exp2f(MLW[wave][0][q] - M);
#pragma unroll
      for (int e = 0; e < 8; ++e) red[tid >> 4][o][8 * vcol + e] = acc[o][e] * f;
    }
  __syncthreads();
  float* ws = p.ws + (((int64_t)b * p.Hn + n) * p.nchunks + c) * (int64_t)p.slots * (kDV + 2);
  for (int i = tid; i < nout * kDV; i += kT) {
    const int o = i / kDV, ch = i % kDV;
    float x = 0.f;
#pragma unroll
    for (int k = 0; k < kT / 16; ++k) x += red[k][o][ch];
    ws[o * (kDV + 2) + 2 + ch] = FP8 ? x * p.v_scale : x;
  }
  if (tid < nout) {
    const int q = tid < g ? tid : g;
    const float M = fmaxf(fmaxf(MLW[0][0][q], MLW[1][0][q]), fmaxf(MLW[2][0][q], MLW[3][0][q]));
    float Lq = 0.f;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) Lq += MLW[w][1][q] * __builtin_amdgcn_exp2f(MLW[w][0][q] - M);
    ws[tid * (kDV + 2) + 0] = M;
    ws[tid * (kDV + 2) + 1] = Lq;
  }
}

// One workgroup per (noise group, sequence): wave w merges output slots w, w+4, ...
// (lane owns channels 2 lane, 2 lane + 1), then each signal head's output is formed.
__global__ __launch_bounds__(kT) void decode_combine_kernel(DecodeParams p) {
  __shared__ float merged[kMaxOut][kDV + 2];  // -, L, O[dv]
  const int n = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = p.g, nout = g + p.nu[n];
  const int L = min(max(p.seq_lens[b], 0), p.Lmax);
  const int nch = (L + p.chunk - 1) / p.chunk;
  const int64_t cstride = (int64_t)p.slots * (kDV + 2);
  const float* base = p.ws + ((int64_t)b * p.Hn + n) * p.nchunks * cstride;
  const int c0 = 2 * lane;
  const float lam = lambda_of(p.lam_dev, p.lam);
  for (int o = wave; o < nout; o += kT / 64) {
    // chunk maxima and sums: lane c holds chunk c (64 chunks per pass), all loads
    // of a pass in flight together
    float M = -INFINITY;
    for (int cb = 0; cb < nch; cb += 64) {
      const int c = cb + lane;
      M = fmaxf(M, c < nch ? base[c * cstride + o * (kDV + 2)] : -INFINITY);
    }
    M = wave_max(M);
    float Ls = 0.f, a0 = 0.f, a1 = 0.f;
    for (int cb = 0; cb < nch; cb += 64) {
      const int c = cb + lane;
      const float* sc = base + min(c, nch - 1) * cstride + o * (kDV + 2);
      const float f = c < nch ? __builtin_amdgcn_exp2f(sc[0] - M) : 0.f;
      Ls += wave_sum(sc[1] * f);
      // channel pair c0, c0 + 1 of every chunk of the pass, weighted by its chunk's
      // factor (broadcast from lane k); 8 chunks' loads in flight at a time.  Slots
      // past the last chunk re-read the last chunk (in bounds) with factor 0.
      const int n_pass = min(64, nch - cb);
      for (int k0 = 0; k0 < n_pass; k0 += 8) {
        float v0[8], v1[8], fk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + u;  // <= 63
          fk[u] = lane_f(f, k);
          const float* sk = base + min(cb + k, nch - 1) * cstride + o * (kDV + 2);
          v0[u] = sk[2 + c0];
          v1[u] = sk[3 + c0];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a0 = __builtin_fmaf(v0[u], fk[u], a0);
          a1 = __builtin_fmaf(v1[u], fk[u], a1);
        }
      }
    }
    merged[o][2 + c0] = a0;
    merged[o][3 + c0] = a1;
    if (lane == 0) merged[o][1] = Ls;
  }
  __syncthreads();
  for (int j = wave; j < g; j += kT / 64) {
    const int h = p.members[n * g + j];
    __bf16* out = (__bf16*)p.out + b * p.so[0] + h * p.so[1];
    if (L == 0) {
      bf16x2 z = {(__bf16)0.f, (__bf16)0.f};
      *(bf16x2*)(out + c0) = z;
      continue;
    }
    const int s2 = g + p.uidx[h];
    const float i1 = 1.0f / merged[j][1], i2 = 1.0f / merged[s2][1];
    // identical operations on both maps: identical maps with lambda = 1 give exact zeros
    const float o0 = __builtin_fmaf(-lam, __fmul_rn(merged[s2][2 + c0], i2), __fmul_rn(merged[j][2 + c0], i1));
    const float o1 = __builtin_fmaf(-lam, __fmul_rn(merged[s2][3 + c0], i2), __fmul_rn(merged[j][3 + c0], i1));
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
}

// Fixed device scratch for the allocation-free decode entry point: the chunk
// partials live here instead of in a caller workspace.  One copy per GPU, held
// until the process ends; every call on a GPU shares it and it keeps the last
// call's contents (the combine reads only the partials the same call wrote, so
// nothing needs clearing).  In host code `scratch` is only the runtime's handle
// of the array: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t decode_scratch(float** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // first call on this device, with it current
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = (float*)addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s) {
  (void)dtype;
  if (p.d != kD || p.dv != kDV || p.g + 1 > kMaxQ || p.slots > kMaxOut || p.chunk % (p.fp8 ? 2 * kC : kC) != 0)
    return hipErrorInvalidValue;
  if (p.nchunks > 0) {
    const dim3 grid(p.nchunks, p.Hn, p.B);
    const bool multi = p.slots > p.g + 1;  // some group uses more than one key/value head
    const bool small = p.g + 1 <= 4 && p.slots <= 4 && !multi;
    if (p.fp8) {
      if (small)
        hipLaunchKernelGGL((decode_partial_kernel<4, false, true>), grid, dim3(kT), 0, s, p);
      else if (!multi)
        hipLaunchKernelGGL((decode_partial_kernel<8, false, true>), grid, dim3(kT), 0, s, p);
      else
        hipLaunchKernelGGL((decode_partial_kernel<8, true, true>), grid, dim3(kT), 0, s, p);
    } else {
      if (small)
        hipLaunchKernelGGL((decode_partial_kernel<4, false, false>), grid, dim3(kT), 0, s, p);
      else if (!multi)
        hipLaunchKernelGGL((decode_partial_kernel<8, false, false>), grid, dim3(kT), 0, s, p);
      else
        hipLaunchKernelGGL((decode_partial_kernel<8, true, false>), grid, dim3(kT), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.Hn, p.B), dim3(kT), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

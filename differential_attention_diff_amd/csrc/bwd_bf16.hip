// bf16 backward score passes for gfx950 (MFMA) at d = 32: dQ1/dQ2
// query-major, then dK1/dK2/dV key-major, both recomputing scores and weights
// from the saved log-sum-exps.  (d = 64 runs the LDS-ring passes of
// bwd_ring_bf16.hip; launch_bwd_bf16 below dispatches.)
//
// Gradients of "Differential Attention in Large Language Models: How
// Denoising Subtraction Eliminates Attention Noise and Outlier Activations"
// (llms.blog), "Differential Attention Architecture", DiffAttn equation, with
// the noise heads of "Grouped Differential Attention" (mlsanity.com),
// "Abstract".  With do and the row statistics of the prep pass (lse1', lse2'
// in log2 units, D1 = do . o1, D2 = do . o2), per query i, visible key j:
//   p1 = 2^(s1 sc - lse1'), p2 = 2^(s2 sc - lse2'), dp = do_i . v_j
//   ds1 = p1 (dp - D1),  ds2 = -lambda p2 (dp - D2)
// The prep pass stores lse2' - log2|lambda| and sgn D2 (-lambda = sgn |lambda|), so
// the kernels form |lambda| p2 directly and ds2 = (|lambda| p2) (sgn dp - sgn D2),
// P1 - lambda P2 = p1 + sgn (|lambda| p2).
//   dQ1 = dS1 K1 / sqrt(d), dK1 = dS1^T Q1 / sqrt(d), dV = (P1 - lambda P2)^T do,
//   dQ2 = dS2 K2 / sqrt(d), dK2 = dS2^T Q2 / sqrt(d)
// One dp = do V^T product serves both maps (both use the head's V).
//
// Both passes: a workgroup of 8 wavefronts owns 128 rows (16 per wavefront) of
// one (batch, noise group) and walks the group's signal heads in turn, so the
// noise head's sums (dQ2, dK2) stay in registers and every gradient row is
// written once; the other operand side is staged through LDS in 64-row tiles,
// double-buffered (the next tile's global loads are in flight during the
// current tile's products; one barrier per tile).  v_mfma_f32_16x16x32_bf16
// throughout (lane l: A row l%16, B column l%16, k 8 (l/16) .. +7; accumulator
// rows 4 (l/16) + r of column l%16): a 16-row wavefront needs about half the
// registers of a 32-row one, so two fit per SIMD.  Operands that must be
// transposed are read with ds_read_b64_tr_b16.  A product's B operand taken
// from other products' accumulators uses their row order as its k order, and
// the A operand read from LDS follows the same order.
//   dQ pass: S^T = K Q^T (lane = query), so the weights of a lane's query are
//     in its own registers and dS^T is the B operand of dQ^T = K^T dS^T.
//   dKV pass: S = Q K^T (lane = key), so dS and P1 - lambda P2 are the B
//     operands of dK^T = Q^T dS and dV^T = do^T (P1 - lambda P2); the per-query
//     statistics are LDS broadcasts.
// In the dKV pass the signal heads of a key/value head must be consecutive in
// the group (checked on the host): dK1/dV accumulate over that run and are
// stored when the key/value head changes.
#include <math.h>

#include <type_traits>

#include "kernels.h"

namespace da {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kRB = 128;              // rows per workgroup
constexpr int kRW = 16;               // rows per wavefront
constexpr int kWaves = kRB / kRW;     // 8
constexpr int kThreads = 64 * kWaves;
constexpr int kTR = 64;               // rows per LDS tile
constexpr int kRowPad = 32;           // LDS tile row padding, bytes

template <int D>
struct BC {
  static constexpr int DV = 2 * D;
  static constexpr int NS = D / 32, NVS = DV / 32;     // 32-wide k steps over d, dv
  static constexpr int NDT = D / 16, NVT = DV / 16;    // 16-row output tiles over d, dv
  static constexpr int KCH = 2 * D / 16, VCH = 2 * DV / 16;  // 16-B chunks per row
  static constexpr int KT = kTR * (2 * D + kRowPad), VT = kTR * (2 * DV + kRowPad);  // tile bytes
  // 16-B tile loads per thread (a tile of fewer chunks than threads leaves the last threads idle)
  static constexpr int KL = (kTR * KCH + kThreads - 1) / kThreads, VL = (kTR * VCH + kThreads - 1) / kThreads;
};

// LDS byte offset of 16-B chunk c of row r in a tile with `ch` chunks per row.
// Rows are padded by 32 B (8 of the 64 four-byte banks), so every operand read
// is one per-lane base plus compile-time offsets.  A transposing read (32
// lanes: 8 consecutive rows x 32 B) then hits 64 distinct banks; a row-wise
// 16-B read (16 lanes, 16 consecutive rows) puts rows r and r + 8 on the same
// banks.  That 2-way conflict costs less than the per-read address arithmetic
// of an XOR swizzle (measured: the backward runs 6% faster this way).
__device__ __forceinline__ int toff(int r, int c, int ch) { return r * (ch * 16 + kRowPad) + (c << 4); }

// Rows [r0, r0 + 64) of a tensor (element row stride rs) into registers, then into
// an LDS tile; rows past `last` re-read row `last`; thread t handles chunks t,
// t + kThreads, ...
template <int CH, int L>
__device__ __forceinline__ void tile_load(u32x4 (&reg)[L], const __bf16* base, int64_t rs, int r0, int last) {
#pragma unroll
  for (int k = 0; k < L; ++k) {
    const int idx = (int)threadIdx.x + kThreads * k, r = idx / CH, c = idx % CH;
    if (kTR * CH % kThreads == 0 || idx < kTR * CH)
      reg[k] = *(const u32x4*)(base + (int64_t)min(r0 + r, last) * rs + c * 8);
  }
}
template <int CH, int L>
__device__ __forceinline__ void tile_store(unsigned char* t, const u32x4 (&reg)[L]) {
#pragma unroll
  for (int k = 0; k < L; ++k) {
    const int idx = (int)threadIdx.x + kThreads * k, r = idx / CH, c = idx % CH;
    if (kTR * CH % kThreads == 0 || idx < kTR * CH) *(u32x4*)(t + toff(r, c, CH)) = reg[k];
  }
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand of a 16 x 32 step read row-wise: lane l holds row rb + l%16, elements
// 32 s + 8 (l/16) .. + 7.
__device__ __forceinline__ bf16x8 rd_rows16(const unsigned char* t, int rb, int s, int ch, int lane) {
  return *(const bf16x8*)(t + toff(rb + (lane & 15), 4 * s + (lane >> 4), ch));
}
// Transposed A operand of a 16 x 32 step: rows rb + {4 (l/16) + 0..3} and rb + 16 + {..}
// (the order of two 16-row accumulator tiles), columns 16 ct + l%16.  Lane i of a 16-lane
// group reads row 4 (l/16) + i/4 at columns 16 ct + 4 (i%4); the transposing read hands
// lane i the 4 rows of column 16 ct + i.
__device__ __forceinline__ bf16x8 rd_tr16(const unsigned char* t, int rb, int ct, int ch, int lane) {
  const int row = rb + 4 * (lane >> 4) + (lane & 15) / 4;
  const int col = ct * 16 + 4 * (lane & 3);
  const int cc = col >> 3, within = (col & 7) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + toff(row, cc, ch) + within));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + toff(row + 16, cc, ch) + within));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Accumulator tiles as a gradient row: lane l of tile ct holds columns
// 16 ct + 4 (l/16) + 0..3 of the row; stored as bf16 after `scale`.
template <int NT>
__device__ __forceinline__ void store_row16(__bf16* row, const f32x4 (&acc)[NT], float scale, int jg) {
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const f32x4 y = acc[ct] * scale;
    *(bf16x4*)(row + 16 * ct + 4 * jg) = __builtin_convertvector(y, bf16x4);
  }
}

__device__ __forceinline__ int xcd_logical(int bid, int total) {
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  return xcd * q8 + min(xcd, r8) + (bid >> 3);
}

// Work item `logical` of ngroups (batch, noise group) pairs x nblk blocks.
// With few pairs per XCD (grouped heads) and few blocks per pair, clusters of
// about one XCD's pairs are walked block-major, longest block first across the
// cluster, so the XCD's workgroups finish together; otherwise each pair's
// blocks are consecutive (its operands stay in L2) and balance the XCD by
// themselves.  blk counts from the first block walked.
__device__ __forceinline__ void bwd_item(int logical, int ngroups, int nblk, int& grp, int& blk) {
  const int cl = (ngroups >= 64 || nblk >= 64) ? 1 : (ngroups + 7) / 8;
  const int per = cl * nblk, c = logical / per, idx = logical % per;
  const int cs = min(cl, ngroups - c * cl);  // the last cluster may be smaller
  blk = idx / cs;
  grp = c * cl + idx % cs;
}

// ---------------------------------------------------------------------------
// dQ pass: workgroup = (b, noise group n, 128 queries)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdParams p) {
  using C = BC<D>;
  constexpr int STAGE = 2 * C::KT + C::VT;
  constexpr int NS = C::NS, NVS = C::NVS, NDT = C::NDT;
  constexpr int KL = C::KL, VL = C::VL;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];
  const int lane = threadIdx.x & 63, l16 = lane & 15, jg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int nq = (p.N + kRB - 1) / kRB;
  int t0, blk;
  bwd_item(xcd_logical(blockIdx.x, (int)gridDim.x), p.B * p.Hn, nq, t0, blk);
  const int qb = nq - 1 - blk;  // longest causal range first
  const int n = t0 % p.Hn, b = t0 / p.Hn;
  const int q0 = qb * kRB, qw = q0 + wave * kRW, q = qw + l16, qc = min(q, p.N - 1);
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;  // -lambda = sgn |lambda|
  const int kend = p.causal ? min(q0 + kRB, p.N) : p.N;
  const int ntile = (kend + kTR - 1) / kTR;
  const int klast = p.causal ? min(qw + kRW - 1, p.N - 1) : p.N - 1;  // last key this wavefront sees
  const int kvis = p.causal ? min(q, p.N - 1) : p.N - 1;                  // last key this lane sees
  const int kfree = p.causal ? min(qw, p.N - 1) : p.N - 1;                // keys every query sees

  const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[2];
  bf16x8 q2f[NS];
  {
    const __bf16* Q2 = (const __bf16*)p.q2 + b * p.sq2[0] + (int64_t)qc * p.sq2[1] + n * p.sq2[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) q2f[s] = *(const bf16x8*)(Q2 + 32 * s + 8 * jg);
  }
  f32x4 dq2[NDT];
#pragma unroll
  for (int ct = 0; ct < NDT; ++ct) dq2[ct] = f32x4{};

  for (int mem = 0; mem < p.g; ++mem) {
    const int h = __builtin_amdgcn_readfirstlane(p.members[n * p.g + mem]);
    const int kh = __builtin_amdgcn_readfirstlane(p.kv[h]);
    const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + kh * p.sk1[2];
    const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + kh * p.sv[2];
    bf16x8 q1f[NS], dof[NVS];
    {
      const __bf16* Q1 = (const __bf16*)p.q1 + b * p.sq1[0] + (int64_t)qc * p.sq1[1] + h * p.sq1[2];
      const __bf16* DO = (const __bf16*)p.dop + (((int64_t)b * p.N + qc) * p.Hs + h) * C::DV;
#pragma unroll
      for (int s = 0; s < NS; ++s) q1f[s] = *(const bf16x8*)(Q1 + 32 * s + 8 * jg);
#pragma unroll
      for (int s = 0; s < NVS; ++s) dof[s] = *(const bf16x8*)(DO + 32 * s + 8 * jg);
    }
    const float4 rs = *(const float4*)(p.rowstat + 4 * (((int64_t)b * p.Hs + h) * p.N + qc));
    f32x4 dq1[NDT];
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) dq1[ct] = f32x4{};

    u32x4 r1[KL], r2[KL], rv[VL];
    tile_load<C::KCH>(r1, K1, p.sk1[1], 0, p.N - 1);
    tile_load<C::KCH>(r2, K2, p.sk2[1], 0, p.N - 1);
    tile_load<C::VCH>(rv, V, p.sv[1], 0, p.N - 1);
    tile_store<C::KCH>(lds, r1);
    tile_store<C::KCH>(lds + C::KT, r2);
    tile_store<C::VCH>(lds + 2 * C::KT, rv);
    __syncthreads();
    for (int tile = 0; tile < ntile; ++tile) {
      if (tile + 1 < ntile) {
        const int r0 = (tile + 1) * kTR;
        tile_load<C::KCH>(r1, K1, p.sk1[1], r0, p.N - 1);
        tile_load<C::KCH>(r2, K2, p.sk2[1], r0, p.N - 1);
        tile_load<C::VCH>(rv, V, p.sv[1], r0, p.N - 1);
      }
      const unsigned char* tk1 = lds + (tile & 1) * STAGE;
      const unsigned char* tk2 = tk1 + C::KT;
      const unsigned char* tv = tk1 + 2 * C::KT;
      // one 32-key block (two 16-key accumulator tiles); MASK only where some key of
      // the block is hidden from some query of the wavefront
      auto block = [&](auto mask, int jb) {
        constexpr bool MASK = decltype(mask)::value;
        const int key0 = tile * kTR + jb * 32;
        f32x4 s1[2], s2[2], dp[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          s1[t] = s2[t] = dp[t] = f32x4{};
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            s1[t] = mfma16(rd_rows16(tk1, jb * 32 + 16 * t, s, C::KCH, lane), q1f[s], s1[t]);
            s2[t] = mfma16(rd_rows16(tk2, jb * 32 + 16 * t, s, C::KCH, lane), q2f[s], s2[t]);
          }
#pragma unroll
          for (int s = 0; s < NVS; ++s) dp[t] = mfma16(rd_rows16(tv, jb * 32 + 16 * t, s, C::VCH, lane), dof[s], dp[t]);
        }
        // k order of the dS^T operand: slots 0-3 = tile 0 rows 4 (l/16) + r, slots 4-7 = tile 1
        bf16x8 b1, b2;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[t][r], p.sm_scale_log2, -rs.x));
            float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[t][r], p.sm_scale_log2, -rs.y));  // |lambda| P2
            if (MASK) {
              const int key = key0 + 16 * t + 4 * jg + r;
              p1 = key <= kvis ? p1 : 0.f;
              p2 = key <= kvis ? p2 : 0.f;
            }
            b1[4 * t + r] = (__bf16)(p1 * (dp[t][r] - rs.z));
            b2[4 * t + r] = (__bf16)(p2 * __builtin_fmaf(sgn, dp[t][r], -rs.w));
          }
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          dq1[ct] = mfma16(rd_tr16(tk1, jb * 32, ct, C::KCH, lane), b1, dq1[ct]);
          dq2[ct] = mfma16(rd_tr16(tk2, jb * 32, ct, C::KCH, lane), b2, dq2[ct]);
        }
      };
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int key0 = tile * kTR + jb * 32;
        if (key0 > klast) continue;  // wavefront-uniform: every key of the block is hidden
        if (key0 + 31 <= kfree)
          block(std::false_type{}, jb);
        else
          block(std::true_type{}, jb);
      }
      if (tile + 1 < ntile) {
        unsigned char* nt = lds + ((tile + 1) & 1) * STAGE;
        tile_store<C::KCH>(nt, r1);
        tile_store<C::KCH>(nt + C::KT, r2);
        tile_store<C::VCH>(nt + 2 * C::KT, rv);
      }
      __syncthreads();
    }
    if (q < p.N)
      store_row16((__bf16*)p.gq1 + b * p.sgq1[0] + (int64_t)q * p.sgq1[1] + h * p.sgq1[2], dq1, p.sm_scale, jg);
  }
  if (q < p.N)
    store_row16((__bf16*)p.gq2 + b * p.sgq2[0] + (int64_t)q * p.sgq2[1] + n * p.sgq2[2], dq2, p.sm_scale, jg);
}

// ---------------------------------------------------------------------------
// dKV pass: workgroup = (b, noise group n, 128 keys)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkv_kernel(BwdParams p) {
  using C = BC<D>;
  constexpr int RS = kTR * 16;  // row statistics of a tile (float4 per query)
  constexpr int STAGE = 2 * C::KT + C::VT + RS;
  constexpr int NS = C::NS, NVS = C::NVS, NDT = C::NDT, NVT = C::NVT;
  constexpr int KL = C::KL, VL = C::VL;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, jg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int nk = (p.N + kRB - 1) / kRB;
  int t0, blk;
  bwd_item(xcd_logical(blockIdx.x, (int)gridDim.x), p.B * p.Hn, nk, t0, blk);
  const int kb = p.causal ? blk : nk - 1 - blk;  // causal: most queries first
  const int n = t0 % p.Hn, b = t0 / p.Hn;
  const int k0 = kb * kRB, kw = k0 + wave * kRW, key = kw + l16, kc = min(key, p.N - 1);
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;  // -lambda = sgn |lambda|
  const int qt0 = p.causal ? k0 / kTR : 0;
  const int ntile = (p.N + kTR - 1) / kTR;
  const int vis_lo = p.causal ? key : 0;                 // first query that sees this lane's key
  const uint32_t vrange = (uint32_t)(p.N - vis_lo);      // visible queries: [vis_lo, N)

  const __bf16* Q2 = (const __bf16*)p.q2 + b * p.sq2[0] + n * p.sq2[2];
  bf16x8 kf2[NS];
  {
    const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + (int64_t)kc * p.sk2[1] + n * p.sk2[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) kf2[s] = *(const bf16x8*)(K2 + 32 * s + 8 * jg);
  }
  f32x4 dk2[NDT], dk1[NDT], dv[NVT];
#pragma unroll
  for (int ct = 0; ct < NDT; ++ct) dk2[ct] = dk1[ct] = f32x4{};
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) dv[vt] = f32x4{};
  bf16x8 kf1[NS], vf[NVS];
  int cur = -1;  // key/value head of the accumulating run

  for (int mem = 0; mem < p.g; ++mem) {
    const int h = __builtin_amdgcn_readfirstlane(p.members[n * p.g + mem]);
    const int kh = __builtin_amdgcn_readfirstlane(p.kv[h]);
    if (kh != cur) {
      if (cur >= 0 && key < p.N) {
        store_row16((__bf16*)p.gk1 + b * p.sgk1[0] + (int64_t)key * p.sgk1[1] + cur * p.sgk1[2], dk1, p.sm_scale, jg);
        store_row16((__bf16*)p.gv + b * p.sgv[0] + (int64_t)key * p.sgv[1] + cur * p.sgv[2], dv, 1.0f, jg);
      }
#pragma unroll
      for (int ct = 0; ct < NDT; ++ct) dk1[ct] = f32x4{};
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) dv[vt] = f32x4{};
      cur = kh;
      const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + (int64_t)kc * p.sk1[1] + kh * p.sk1[2];
      const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + (int64_t)kc * p.sv[1] + kh * p.sv[2];
#pragma unroll
      for (int s = 0; s < NS; ++s) kf1[s] = *(const bf16x8*)(K1 + 32 * s + 8 * jg);
#pragma unroll
      for (int s = 0; s < NVS; ++s) vf[s] = *(const bf16x8*)(V + 32 * s + 8 * jg);
    }
    const __bf16* Q1 = (const __bf16*)p.q1 + b * p.sq1[0] + h * p.sq1[2];
    const __bf16* DO = (const __bf16*)p.dop + ((int64_t)b * p.N * p.Hs + h) * C::DV;  // row i at + i Hs dv
    const float* RSB = p.rowstat + 4 * ((int64_t)b * p.Hs + h) * p.N;
    const int64_t dors = (int64_t)p.Hs * C::DV;

    u32x4 r1[KL], r2[KL], rv[VL], rr;
    auto load_all = [&](int qt) {
      const int r0 = qt * kTR;
      tile_load<C::KCH>(r1, Q1, p.sq1[1], r0, p.N - 1);
      tile_load<C::KCH>(r2, Q2, p.sq2[1], r0, p.N - 1);
      tile_load<C::VCH>(rv, DO, dors, r0, p.N - 1);
      if (tid < kTR) rr = *(const u32x4*)(RSB + 4 * (int64_t)min(r0 + tid, p.N - 1));
    };
    auto store_all = [&](unsigned char* t) {
      tile_store<C::KCH>(t, r1);
      tile_store<C::KCH>(t + C::KT, r2);
      tile_store<C::VCH>(t + 2 * C::KT, rv);
      if (tid < kTR) *(u32x4*)(t + 2 * C::KT + C::VT + 16 * tid) = rr;
    };
    load_all(qt0);
    store_all(lds);
    __syncthreads();
    for (int qt = qt0; qt < ntile; ++qt) {
      if (qt + 1 < ntile) load_all(qt + 1);
      const unsigned char* tq1 = lds + ((qt - qt0) & 1) * STAGE;
      const unsigned char* tq2 = tq1 + C::KT;
      const unsigned char* tdo = tq1 + 2 * C::KT;
      const float* trs = (const float*)(tq1 + 2 * C::KT + C::VT);
      // one 32-query sub-block (two 16-query accumulator tiles), always masked: an
      // unmasked copy next to it does not fit two wavefronts' registers per SIMD
      auto block = [&](auto mask, int sb) {
        constexpr bool MASK = decltype(mask)::value;
        const int qs0 = qt * kTR + sb * 32;
        const int vd0 = qs0 + 4 * jg - vis_lo;
        f32x4 s1[2], s2[2], dp[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          s1[t] = s2[t] = dp[t] = f32x4{};
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            s1[t] = mfma16(rd_rows16(tq1, sb * 32 + 16 * t, s, C::KCH, lane), kf1[s], s1[t]);
            s2[t] = mfma16(rd_rows16(tq2, sb * 32 + 16 * t, s, C::KCH, lane), kf2[s], s2[t]);
          }
#pragma unroll
          for (int s = 0; s < NVS; ++s) dp[t] = mfma16(rd_rows16(tdo, sb * 32 + 16 * t, s, C::VCH, lane), vf[s], dp[t]);
        }
        // the score and dP products are issued before the weights are formed: letting
        // the scheduler interleave the two measured 5% slower
        __builtin_amdgcn_sched_barrier(0);
        // k order of the B operands: slots 0-3 = tile 0 rows 4 (l/16) + r, slots 4-7 = tile 1
        bf16x8 bc, b1, b2;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int qi = sb * 32 + 16 * t + 4 * jg + r;  // query row in the tile
            const float4 st = *(const float4*)(trs + 4 * qi);
            float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[t][r], p.sm_scale_log2, -st.x));
            float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[t][r], p.sm_scale_log2, -st.y));  // |lambda| P2
            if (MASK) {
              // query qs0 + 16 t + 4 jg + r is visible iff it lies in [vis_lo, N): one
              // unsigned compare, no control flow (for keys past N the range wraps, and
              // their sums are never stored)
              const bool vis = (uint32_t)(vd0 + 16 * t + r) < vrange;
              p1 = vis ? p1 : 0.f;
              p2 = vis ? p2 : 0.f;
            }
            bc[4 * t + r] = (__bf16)__builtin_fmaf(sgn, p2, p1);
            b1[4 * t + r] = (__bf16)(p1 * (dp[t][r] - st.z));
            b2[4 * t + r] = (__bf16)(p2 * __builtin_fmaf(sgn, dp[t][r], -st.w));
          }
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) dv[vt] = mfma16(rd_tr16(tdo, sb * 32, vt, C::VCH, lane), bc, dv[vt]);
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          dk1[ct] = mfma16(rd_tr16(tq1, sb * 32, ct, C::KCH, lane), b1, dk1[ct]);
          dk2[ct] = mfma16(rd_tr16(tq2, sb * 32, ct, C::KCH, lane), b2, dk2[ct]);
        }
      };
      // unrolled: the second sub-block's operand addresses are the first's plus constants
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int qs0 = qt * kTR + sb * 32;
        if (qs0 >= p.N || (p.causal && qs0 + 31 < kw)) continue;  // wavefront-uniform: nothing visible
        block(std::true_type{}, sb);
      }
      if (qt + 1 < ntile) store_all(lds + ((qt + 1 - qt0) & 1) * STAGE);
      __syncthreads();
    }
  }
  if (key < p.N) {
    store_row16((__bf16*)p.gk1 + b * p.sgk1[0] + (int64_t)key * p.sgk1[1] + cur * p.sgk1[2], dk1, p.sm_scale, jg);
    store_row16((__bf16*)p.gv + b * p.sgv[0] + (int64_t)key * p.sgv[1] + cur * p.sgv[2], dv, 1.0f, jg);
    store_row16((__bf16*)p.gk2 + b * p.sgk2[0] + (int64_t)key * p.sgk2[1] + n * p.sgk2[2], dk2, p.sm_scale, jg);
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s) {
  const int64_t nblk = (p.N + kRB - 1) / kRB;
  const int64_t grid = (int64_t)p.B * p.Hn * nblk;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (bwd_ring_applies(p)) return launch_bwd_ring_bf16(p, s);
  if (p.d != 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_kernel<32>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(bwd_dkv_kernel<32>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

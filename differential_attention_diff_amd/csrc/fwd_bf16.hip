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
//   * A workgroup (4 wavefronts x 32 queries) owns 128 queries of one (batch,
//     signal head); two workgroups share a CU.  Workgroup ids are remapped so
//     that each XCD (ids congruent mod 8) walks a contiguous range of (batch,
//     noise group) items, longest causal block first, the signal heads of a
//     noise group back to back: the group's K2/Q2 and the head's K1/V stay hot
//     in that XCD's L2.
//   * K1, K2 and V tiles of 64 keys go straight from global memory into a
//     two-slot LDS ring with global_load_lds_dwordx4 (no staging registers);
//     16-byte chunks are XOR-swizzled by row so that neither the MFMA operand
//     reads nor the transposing V reads conflict on LDS banks.  Tile t + 1 is
//     in flight while tile t is computed; one barrier per tile.
//   * Tiles below every wavefront's diagonal run a branch-free loop; only the
//     (at most two) diagonal tiles test which 32-key blocks to skip or mask.
//   * Scores are computed transposed, S^T = K Q^T on v_mfma_f32_32x32x16_bf16:
//     lane (q, half) holds 16 keys of ONE query row, so the row max needs one
//     v_permlane32_swap and the row sum none until the epilogue.
//   * Each map keeps its running max m and sum l in fp32 per row; m moves only
//     when a block's max exceeds it by more than 8 (log2 units), so the O
//     rescale is rare, weights stay <= 2^8, and O/l is unchanged up to
//     rounding.  l accumulates the bf16-rounded weights the P.V product uses.
//   * P^T (bf16) feeds O^T += V^T P^T straight from registers; V^T fragments
//     come from LDS with ds_read_b64_tr_b16 and each feeds the MFMAs of BOTH
//     maps.
//   * Epilogue: o = O1/l1 - lambda O2/l2, RMS over dv (in-lane + one swap),
//     times (1 - lambda_init) w, round to bf16, store; optional LSE.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kQW = 32;                // queries per wavefront (MFMA N dim)
constexpr int kQB = kWaves * kQW;      // queries per workgroup
constexpr int kKT = 64;                // keys per LDS tile
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleSlack = 8.0f;  // log2 units a stale max may lag

template <int D>
struct Cfg {
  static constexpr int DV = 2 * D;
  static constexpr int KROW = D * 2;             // bytes per K row in LDS (no padding; swizzled)
  static constexpr int VROW = DV * 2;            // bytes per V row
  static constexpr int KBYTES = kKT * KROW;      // one K tile
  static constexpr int VBYTES = kKT * VROW;      // the V tile
  static constexpr int STAGE = 2 * KBYTES + VBYTES;
  static constexpr int KCH = KROW / 16;          // 16-B chunks per K row (8 for d = 64)
  static constexpr int VCH = VROW / 16;          // 16-B chunks per V row (16 for dv = 128)
  static constexpr int KSW = (KCH >= 8 ? 8 : KCH) - 1;   // K swizzle mask
  static constexpr int VSH = VCH >= 16 ? 2 : 1;           // V swizzle: chunk ^ ((r mod 4) << VSH)
  static constexpr int KLOADS = KBYTES / 1024 / kWaves;  // 1-KiB DMA loads per wave per K tile
  static constexpr int VLOADS = VBYTES / 1024 / kWaves;
  static_assert(KLOADS >= 1 && VLOADS >= 1, "tile too small for 4 wavefronts");
  static_assert(VCH >= 8, "V swizzle needs 8 chunks per row");
};

// LDS byte offset of 16-B chunk c of row r (XOR swizzle).  K: chunk ^ (r mod
// 8) spreads the rows an MFMA operand read touches over all banks.  V:
// chunk ^ ((r mod 4) << VSH) puts the 4 rows a transposing read touches in
// distinct bank windows (64 B apart for dv = 128, 32 B for dv = 64).
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * Cfg<D>::KROW + ((c ^ (r & Cfg<D>::KSW)) << 4);
}
template <int D>
__device__ __forceinline__ int v_off(int r, int c) {
  return r * Cfg<D>::VROW + ((c ^ ((r & 3) << Cfg<D>::VSH)) << 4);
}

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* a) {
  f32x8 f = {a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]};
  return __builtin_convertvector(f, bf16x8);
}

// One softmax map's update for a 32-key block held as S^T in `s` (lane = query
// row, 16 keys per lane half).  Produces the bf16 P^T operands of the two
// 16-key PV steps and rescales `o` when the reference max moves.
template <int NCB>
__device__ __forceinline__ void online_softmax(const f32x16& s, float sc, float& m, float& l, f32x16 (&o)[NCB],
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
  p0 = to_bf16x8(pr);
  p1 = to_bf16x8(pr + 8);
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

// Per-wavefront state of the forward.
template <int D>
struct Wave {
  static constexpr int DV = 2 * D, NCB = DV / 32, NKS = D / 16;
  f32x16 o1[NCB], o2[NCB];
  bf16x8 q1f[NKS], q2f[NKS];
  float m1, m2, l1, l2;
};

// One 32-key block: rows kr0.. of the tile in LDS slot `stage`, absolute keys
// k0..  MASK: hide keys past the causal diagonal (or past N when not causal).
template <int D, bool MASK>
__device__ __forceinline__ void block32(Wave<D>& w, const unsigned char* stage, int kr0, int k0, int qw0, int l32,
                                        int hh, int vt_lane, const FwdParams& p) {
  using C = Cfg<D>;
  constexpr int NCB = Wave<D>::NCB, NKS = Wave<D>::NKS;
  const unsigned char* K1s = stage;
  const unsigned char* K2s = stage + C::KBYTES;
  const unsigned char* Vs = stage + 2 * C::KBYTES;
  f32x16 s1, s2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s1[r] = 0.f;
    s2[r] = 0.f;
  }
  const int kr = kr0 + l32;  // this lane's key row within the tile (A operand row)
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const bf16x8 a1 = *(const bf16x8*)(K1s + k_off<D>(kr, 2 * s + hh));
    const bf16x8 a2 = *(const bf16x8*)(K2s + k_off<D>(kr, 2 * s + hh));
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, w.q1f[s], s1, 0, 0, 0);
    s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, w.q2f[s], s2, 0, 0, 0);
  }
  if (MASK) {
    // S^T[r] of lane (q, half): key k0 + 8 (r/4) + 4 half + r%4, query qw0 + q
    const int q = qw0 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r / 4) + 4 * hh + (r & 3);
      const bool hide = p.causal ? (key > q) : (key >= p.N);
      s1[r] = hide ? -INFINITY : s1[r];
      s2[r] = hide ? -INFINITY : s2[r];
    }
  }
  bf16x8 pa0, pa1, pb0, pb1;
  const float sc = p.sm_scale_log2;
  online_softmax<NCB>(s1, sc, w.m1, w.l1, w.o1, pa0, pa1);
  online_softmax<NCB>(s2, sc, w.m2, w.l2, w.o2, pb0, pb1);
  // O^T += V^T P^T for both maps; each V^T fragment (32 channels x 16 keys) is read once.
  // Lane j of a 16-lane group reads row (4 half + j/4) at channels c0 + 4 (j%4): the
  // transposing read hands lane i the 4 keys of channel c0 + i.
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row = kr0 + ks * 16 + (vt_lane >> 8);
      const int ch = cb * 32 + (vt_lane & 0xff);
      const int c = ch >> 3, within = (ch & 7) * 2;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vs + v_off<D>(row, c) + within));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vs + v_off<D>(row + 8, c) + within));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      w.o1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ks ? pa1 : pa0, w.o1[cb], 0, 0, 0);
      w.o2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ks ? pb1 : pb0, w.o2[cb], 0, 0, 0);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D>;
  constexpr int DV = C::DV, NCB = DV / 32, NKS = D / 16;
  // the two ring slots are separate objects, so the compiler can tell the DMA into one
  // slot from the reads of the other (and need not wait for the DMA before reading)
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[C::STAGE];

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
  const int h = __builtin_amdgcn_readfirstlane(p.members[n * p.g + member]);
  const int kh = __builtin_amdgcn_readfirstlane(p.kv[h]);
  const int q0 = qb * kQB;
  const int qw0 = q0 + wave * kQW;
  const bool wave_live = qw0 < p.N;

  const __bf16* Q1 = (const __bf16*)p.q1 + b * p.sq1[0] + h * p.sq1[2];
  const __bf16* Q2 = (const __bf16*)p.q2 + b * p.sq2[0] + n * p.sq2[2];
  const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + kh * p.sk1[2];
  const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[2];
  const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + kh * p.sv[2];

  const int q_end = min(q0 + kQB, p.N);
  const int kend = p.causal ? q_end : p.N;
  const int ntiles = (kend + kKT - 1) / kKT;
  // tiles every wavefront sees whole: all keys <= every query of the block (causal),
  // or all keys < N (not causal)
  const int full_tiles = p.causal ? min(ntiles, q0 / kKT) : p.N / kKT;

  // ---- DMA of one tile into a ring slot: each wave issues its share of 1-KiB
  // loads; lane l of a load writes LDS bytes [16 l, 16 l + 16) of that KiB, so the
  // global chunk a lane fetches implements the swizzle.  Rows past N re-read row
  // N - 1 (in bounds); those keys are always masked (causal: beyond every valid
  // query; otherwise: >= N).
  // Addresses: a uniform base per tile (scalar registers) plus a 32-bit per-lane byte
  // offset, recomputed per tile (rows are clamped to N - 1 on the last tile).
  const uint32_t rk1 = (uint32_t)p.sk1[1] * 2u, rk2 = (uint32_t)p.sk2[1] * 2u, rv = (uint32_t)p.sv[1] * 2u;
  auto issue_tile = [&](int tile, unsigned char* base) {
    const int key0 = tile * kKT;
    const int lim = p.N - 1 - key0;  // last valid row of this tile
    const char* k1b = (const char*)(K1 + (int64_t)key0 * p.sk1[1]);
    const char* k2b = (const char*)(K2 + (int64_t)key0 * p.sk2[1]);
    const char* vb = (const char*)(V + (int64_t)key0 * p.sv[1]);
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int j = wave * C::KLOADS + i;                  // 1-KiB block of the K tile
      const int r = j * (1024 / C::KROW) + lane / C::KCH;  // row this lane's 16 B land in
      const uint32_t c16 = (uint32_t)(((lane % C::KCH) ^ (r & C::KSW)) << 4);  // global chunk for that slot
      const uint32_t rr = (uint32_t)min(r, lim);
      __builtin_amdgcn_global_load_lds((const void*)(k1b + (rr * rk1 + c16)), (lds_void*)(base + j * 1024), 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds((const void*)(k2b + (rr * rk2 + c16)),
                                       (lds_void*)(base + C::KBYTES + j * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int j = wave * C::VLOADS + i;
      const int r = j * (1024 / C::VROW) + lane / C::VCH;
      const uint32_t c16 = (uint32_t)(((lane % C::VCH) ^ ((r & 3) << C::VSH)) << 4);
      const uint32_t rr = (uint32_t)min(r, lim);
      __builtin_amdgcn_global_load_lds((const void*)(vb + (rr * rv + c16)),
                                       (lds_void*)(base + 2 * C::KBYTES + j * 1024), 16, 0, 0);
    }
  };

  if (ntiles > 0) issue_tile(0, slot0);

  Wave<D> w;
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      w.o1[c][r] = 0.f;
      w.o2[c][r] = 0.f;
    }
  w.m1 = w.m2 = -1e30f;
  w.l1 = w.l2 = 0.f;
  {
    // Q fragments: B operand of S^T = K Q^T; lane (q, half) holds Q[q][16s + 8 half + 0..7]
    const int q = min(qw0 + l32, p.N - 1);  // rows past N: any valid row (results discarded)
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const u32x4 a = *(const u32x4*)(Q1 + (int64_t)q * p.sq1[1] + 16 * s + 8 * hh);
      const u32x4 c = *(const u32x4*)(Q2 + (int64_t)q * p.sq2[1] + 16 * s + 8 * hh);
      w.q1f[s] = __builtin_bit_cast(bf16x8, a);
      w.q2f[s] = __builtin_bit_cast(bf16x8, c);
    }
  }
  // lane's (row within a 16-key step) << 8 | channel offset within a 32-channel block
  const int vt_lane = ((4 * hh + (lane & 15) / 4) << 8) | (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  // ---- tiles every wavefront sees whole: branch-free; unrolled by two so that each
  // step reads one named slot while the DMA fills the other
  auto full_step = [&](int tile, const unsigned char* cur, unsigned char* nxt) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of the tile (issued a step ago) has landed
    __syncthreads();                // ... every wave's; and the other slot is no longer read
    if (tile + 1 < ntiles) issue_tile(tile + 1, nxt);
    block32<D, false>(w, cur, 0, tile * kKT, qw0, l32, hh, vt_lane, p);
    block32<D, false>(w, cur, 32, tile * kKT + 32, qw0, l32, hh, vt_lane, p);
  };
  int tile = 0;
  for (; tile + 1 < full_tiles; tile += 2) {
    full_step(tile, slot0, slot1);
    full_step(tile + 1, slot1, slot0);
  }
  if (tile < full_tiles) {
    full_step(tile, slot0, slot1);
    ++tile;
  }
  // ---- the diagonal tiles (causal) or the ragged last tile: per 32-key block,
  // skip it (entirely above this wavefront's queries), mask it, or take it whole
  for (; tile < ntiles; ++tile) {
    unsigned char* cur = (tile & 1) ? slot1 : slot0;
    unsigned char* nxt = (tile & 1) ? slot0 : slot1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tile + 1 < ntiles) issue_tile(tile + 1, nxt);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = tile * kKT + kb * 32;
      if (!wave_live || k0 >= kend) continue;
      if (p.causal && k0 > qw0 + kQW - 1) continue;
      const bool mask = p.causal ? (k0 + 31 > qw0) : (k0 + 32 > p.N);
      if (mask)
        block32<D, true>(w, cur, kb * 32, k0, qw0, l32, hh, vt_lane, p);
      else
        block32<D, false>(w, cur, kb * 32, k0, qw0, l32, hh, vt_lane, p);
    }
  }

  if (!wave_live) return;

  // ---- epilogue: o = O1/l1 - lambda O2/l2, then the head RMS norm
  const float l1 = half_swap_sum(w.l1), l2 = half_swap_sum(w.l2);
  const float i1 = 1.0f / l1, i2 = 1.0f / l2;
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // both maps take identical operations: identical maps with lambda = 1 give exact zeros
      const float x = __builtin_fmaf(-p.lam, __fmul_rn(w.o2[c][r], i2), __fmul_rn(w.o1[c][r], i1));
      w.o1[c][r] = x;
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
        f32x4 wv = {1.f, 1.f, 1.f, 1.f};
        if (p.normalize && p.norm_w) {
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[e] = p.norm_w[ch + e];
        }
        f32x4 y = {w.o1[c][4 * g4] * scale * wv[0], w.o1[c][4 * g4 + 1] * scale * wv[1],
                   w.o1[c][4 * g4 + 2] * scale * wv[2], w.o1[c][4 * g4 + 3] * scale * wv[3]};
        *(bf16x4*)(out + ch) = __builtin_convertvector(y, bf16x4);
      }
    if (p.lse && hh == 0) {
      const int64_t base = ((int64_t)b * p.Hs + h) * p.N + q;
      const int64_t plane = (int64_t)p.B * p.Hs * p.N;
      constexpr float kLn2 = 0.69314718055994531f;
      p.lse[base] = (w.m1 + __log2f(l1)) * kLn2;
      p.lse[plane + base] = (w.m2 + __log2f(l2)) * kLn2;
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

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
//   * A workgroup owns 128 queries (4 groups of 32) of one (batch, signal
//     head) and runs 8 wavefronts: one per (query group, softmax map).  The
//     two wavefronts of a query group share a SIMD, each holds only its own
//     map's O (64 registers), so a wavefront fits in 256 registers with room
//     for the pipeline below.  Workgroup ids are remapped so that each XCD (ids
//     congruent mod 8) walks a contiguous range of items ordered (batch, noise
//     group, query block longest causal block first, signal head of the
//     group) when a head has fewer than 64 query blocks -- the longest blocks
//     of every head of the group start first, so the XCD's queue drains
//     evenly -- and (batch, noise group, signal head, query block) otherwise,
//     where a head's many blocks balance the XCD and the ~32 workgroups it
//     runs at once share that head's K1/V and the group's K2 in its 4 MB L2.
//   * K1, K2 and V tiles of 64 keys go straight from global memory into a
//     four-slot LDS ring (global_load_lds_dwordx4, no staging registers); the
//     two tiles after the two being read are in flight.  One barrier per
//     tile.  16-byte chunks are XOR-swizzled by row so that neither the MFMA
//     operand reads nor the transposing V reads conflict on LDS banks.  Each
//     V tile feeds both maps' P.V products.
//   * Scores are computed transposed, S^T = K Q^T on v_mfma_f32_32x32x16_bf16:
//     lane (q, half) holds 16 keys of ONE query row, so a row reduction needs
//     one v_permlane32_swap and the row sum none until the epilogue.
//   * Software pipeline over 32-key blocks j, one iteration per block: the
//     softmax of block j (VALU) is interleaved with the score products of block
//     j + 1 and the P.V products of block j - 1 (MFMA), and with the LDS
//     operand reads for the next iteration.
//   * Each map keeps a reference max m and a sum l in fp32 per row.  A block's
//     weights are formed against m without computing the block max: one FMA,
//     one exp2, half a conversion and half a dot2 per score.  Only when some
//     lane's weights of a block sum past 2^12 (the first block, or a later
//     block whose scores climb well above m) does the wavefront recompute the
//     block's scores, move m to the row's running max, rescale O and l, and
//     form the weights again.  Weights stay <= 2^12 and O/l is unchanged up to
//     rounding.  l accumulates the bf16-rounded weights the P.V product uses.
//   * Blocks on or past a wavefront's causal diagonal (or past N) are masked;
//     every wavefront of a workgroup walks the same blocks.
//   * Epilogue: the map-2 wavefront hands O2/l2 to its partner through LDS;
//     the map-1 wavefront forms o = O1/l1 - lambda O2/l2, the RMS over dv
//     (in-lane + one swap), times (1 - lambda_init) w, rounds to bf16 and
//     stores.  Each wavefront writes its map's LSE when asked.
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
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kGroups = 4;             // query groups per workgroup
constexpr int kWaves = 2 * kGroups;    // one wavefront per (query group, map)
constexpr int kQW = 32;                // queries per wavefront (MFMA N dim)
constexpr int kQB = kGroups * kQW;     // queries per workgroup
constexpr int kKT = 64;                // keys per LDS tile
constexpr int kKB = 32;                // keys per pipeline block
constexpr int kSlots = 4;              // LDS ring slots
constexpr int kThreads = kWaves * 64;
constexpr float kSumLimit = 4096.0f;   // lane weight sum that forces a reference move

template <int D>
struct Cfg {
  static constexpr int DV = 2 * D, NCB = DV / 32, NKS = D / 16;
  static constexpr int KROW = D * 2;             // bytes per K row in LDS (no padding; swizzled)
  static constexpr int VROW = DV * 2;            // bytes per V row
  static constexpr int KBYTES = kKT * KROW;      // one K tile
  static constexpr int VBYTES = kKT * VROW;      // the V tile
  static constexpr int STAGE = 2 * KBYTES + VBYTES;
  static constexpr int KCH = KROW / 16;          // 16-B chunks per K row (8 for d = 64)
  static constexpr int VCH = VROW / 16;          // 16-B chunks per V row (16 for dv = 128)
  static constexpr int KSW = (KCH >= 8 ? 8 : KCH) - 1;   // K swizzle mask
  static constexpr int KSH = KROW >= 128 ? 1 : 2;         // K swizzle term: (r >> KSH) & KSW
  static constexpr int VSH = VCH >= 16 ? 2 : 1;           // V swizzle: chunk ^ ((r mod 4) << VSH)
  static constexpr int KRPL = 1024 / KROW, VRPL = 1024 / VROW;  // rows per KiB
  // tile DMA: waves 0-1 load K1, 2-3 K2, 4-7 V, TLOADS KiB each
  static constexpr int TLOADS = STAGE / 1024 / kWaves;
  static constexpr int QBYTES = kQB * KROW;      // the workgroup's Q1 (or Q2) rows
  static constexpr int QLOADS = 2 * QBYTES / 1024 / kWaves;
  static_assert(TLOADS * 2 * 1024 == KBYTES && TLOADS * 4 * 1024 == VBYTES, "tile split over waves");
  static_assert(QLOADS * 4 * 1024 == QBYTES, "Q split over waves");
  static_assert(VCH >= 8, "V swizzle needs 8 chunks per row");
  // the K swizzle term of row row0 + l (row0 a multiple of KRPL, l < KRPL) is the
  // term of row l, XOR KFLIP when row0 / KRPL is odd
  static constexpr int KFLIP = (KRPL >> KSH) & KSW;
  static_assert(((2 * KRPL) >> KSH) % (KSW + 1) == 0 && (KFLIP == 0 || ((KRPL - 1) >> KSH) < KFLIP),
                "K swizzle term of a 1-KiB load: the lane's term, flipped by the load's parity");
  static_assert(VRPL % 4 == 0, "V swizzle term must depend on the lane only");
  static_assert(KFLIP == 0 || (TLOADS % 2 == 0 && QLOADS % 2 == 0), "a wave's K and Q loads start on an even KiB");
  static_assert(2 * QBYTES <= STAGE, "Q1 and Q2 are staged in one ring slot");
  static_assert(kGroups * kQW * DV * 4 <= 2 * STAGE, "O2 hand-off fits in two ring slots");
};

// A ring slot: NK key tiles (K1 and K2 for the general kernel, one map's keys
// for the shared-value kernels) followed by the V tile.
template <int D, int NK>
struct Lay {
  static constexpr int VOFF = NK * Cfg<D>::KBYTES;
  static constexpr int STAGE = VOFF + Cfg<D>::VBYTES;
};

// LDS byte offset of 16-B chunk c of row r (XOR swizzle).  K (and Q): chunk ^
// ((r >> KSH) mod 8) -- an MFMA operand read takes one chunk of 16 consecutive
// rows per 16 lanes, and with rows of 128 B (two per 256-B bank window) the
// term must differ between the 8 even rows and between the 8 odd ones, so it
// counts pairs of rows (quads for 64-B rows).  V: chunk ^ ((r mod 4) << VSH)
// puts the 4 rows a transposing read touches in distinct bank windows (64 B
// apart for dv = 128, 32 B for dv = 64).
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * Cfg<D>::KROW + ((c ^ ((r >> Cfg<D>::KSH) & Cfg<D>::KSW)) << 4);
}
template <int D>
__device__ __forceinline__ int v_off(int r, int c) {
  return r * Cfg<D>::VROW + ((c ^ ((r & 3) << Cfg<D>::VSH)) << 4);
}

// 16 bytes per lane from gbase + goff straight into LDS: lane l writes LDS bytes
// [lds + 16 l, lds + 16 l + 16).  Issued as inline assembly so the compiler does
// not order the ring's LDS reads behind these loads; completion is awaited
// explicitly (s_waitcnt vmcnt + barrier) before a slot is read.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t goff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(goff), "s"(gbase), "s"(lds)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most `tiles` tiles of T loads each are still in flight
template <int T>
__device__ __forceinline__ void wait_tiles_in_flight(int tiles) {
  if (tiles <= 0)
    wait_vmcnt<0>();
  else if (tiles == 1)
    wait_vmcnt<T>();
  else if (tiles == 2)
    wait_vmcnt<2 * T>();
  else
    wait_vmcnt<3 * T>();
}
__device__ __forceinline__ void wait_lds_and_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// maxima are NaN-propagating (v_maximum3_f32): no operand canonicalisation
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max16(const f32x16& s) {
  const float a = vmax(vmax(s[0], s[1]), s[2]), b = vmax(vmax(s[3], s[4]), s[5]);
  const float c = vmax(vmax(s[6], s[7]), s[8]), d = vmax(vmax(s[9], s[10]), s[11]);
  const float e = vmax(vmax(s[12], s[13]), s[14]);
  return vmax(vmax(vmax(a, b), c), vmax(vmax(d, e), s[15]));
}

// Per-wavefront pipeline state (one softmax map).  Parity-indexed members
// alternate between consecutive blocks (indices are compile-time constants).
template <int D>
struct St {
  static constexpr int NCB = Cfg<D>::NCB, NKS = Cfg<D>::NKS;
  f32x16 o[NCB];            // O^T accumulator
  f32x16 s[2];              // S^T of block j (parity j) and j + 1
  bf16x8 p[2][2];           // P^T operands: keys 0-15, 16-31
  bf16x8 kf[NKS];           // K operands of the next score products
  bf16x8 vf[NCB][2];        // V^T operands of the next P.V products
  bf16x8 qf[NKS];
  float m, l;
};

// Everything a pipeline step needs besides the state.
struct Ctx {
  const unsigned char* ring;
  int koff;     // byte offset of this wavefront's map in a K tile (0 or KBYTES)
  int l32, hh, vt_lane;
  int kmax;     // last key this lane's query sees (causal: its row; else N - 1)
  int jmask;    // first block that needs a mask for this wavefront
  float sc;     // log2(e)/sqrt(d)
};

template <int D, int NK>
__device__ __forceinline__ const unsigned char* slot_of(const Ctx& c, int tile) {
  return c.ring + (tile % kSlots) * Lay<D, NK>::STAGE;
}

// K operands of block jj: A operand of S^T = K Q^T, lane (k, half) holds
// K[k][16 s + 8 half + 0..7].
template <int D, int NK>
__device__ __forceinline__ void read_k(bf16x8 (&kf)[Cfg<D>::NKS], const Ctx& c, int jj) {
  const unsigned char* t = slot_of<D, NK>(c, jj >> 1) + c.koff;
  const int kr = (jj & 1) * kKB + c.l32;
#pragma unroll
  for (int s = 0; s < Cfg<D>::NKS; ++s) kf[s] = *(const bf16x8*)(t + k_off<D>(kr, 2 * s + c.hh));
}

// V^T operands of block jj (32 channels x 16 keys per (cb, ks)): lane j of a
// 16-lane group reads row (4 half + j/4) at channels c0 + 4 (j%4); the
// transposing read hands lane i the 4 keys of channel c0 + i.
template <int D, int NK>
__device__ __forceinline__ void read_v(St<D>& st, const Ctx& c, int jj) {
  using C = Cfg<D>;
  const unsigned char* vs = slot_of<D, NK>(c, jj >> 1) + Lay<D, NK>::VOFF;
  const int r0 = (jj & 1) * kKB + (c.vt_lane >> 8);
#pragma unroll
  for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row = r0 + ks * 16;
      const int ch = cb * 32 + (c.vt_lane & 0xff);
      const int cc = ch >> 3, within = (ch & 7) * 2;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + v_off<D>(row, cc) + within));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + v_off<D>(row + 8, cc) + within));
      st.vf[cb][ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

template <int D>
__device__ __forceinline__ f32x16 score_products(const bf16x8 (&kf)[Cfg<D>::NKS], const bf16x8 (&qf)[Cfg<D>::NKS]) {
  f32x16 a = {};
#pragma unroll
  for (int s = 0; s < Cfg<D>::NKS; ++s) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], a, 0, 0, 0);
  return a;
}

template <int D, int PAR>
__device__ __forceinline__ void pv_products(St<D>& st) {
#pragma unroll
  for (int cb = 0; cb < Cfg<D>::NCB; ++cb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      st.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.vf[cb][ks], st.p[PAR][ks], st.o[cb], 0, 0, 0);
}

// S^T[r] of lane (q, half) is key k0 + 4 half + 8 (r/4) + r%4; keys past the
// lane's last visible key are hidden
__device__ __forceinline__ void mask_scores(f32x16& s, int k0, const Ctx& c) {
  const int lim = c.kmax - k0 - 4 * c.hh;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = (8 * (r / 4) + (r & 3) > lim) ? -INFINITY : s[r];
}

// bf16 weights 2^(s sc - m) of a block as the P^T operands of its two 16-key
// P.V steps; returns the sum of this lane's 16 bf16-rounded weights
// (v_dot2_f32_bf16 against (1, 1)), i.e. exactly what the P.V product uses.
__device__ __forceinline__ float block_weights(const f32x16& s, float sc, float m, bf16x8& p0, bf16x8& p1) {
  float pr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sc, -m));
  const f32x8 lo = {pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]};
  const f32x8 hi = {pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]};
  p0 = __builtin_convertvector(lo, bf16x8);
  p1 = __builtin_convertvector(hi, bf16x8);
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  float t0 = 0.f, t1 = 0.f;
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 0, 1), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 0, 1), one2, t1, false);
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 2, 3), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 2, 3), one2, t1, false);
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 4, 5), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 4, 5), one2, t1, false);
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 6, 7), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 6, 7), one2, t1, false);
  return t0 + t1;
}

// Interleave pattern of a step: each MFMA followed by VALU work and LDS operand
// reads.
template <int D>
__device__ __forceinline__ void step_schedule() {
  constexpr int NKS = Cfg<D>::NKS, NPV = 2 * Cfg<D>::NCB;
#pragma unroll
  for (int i = 0; i < NKS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (scores of block j + 1)
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU (softmax of block j)
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read (K of block j + 2)
  }
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (P.V of block j - 1)
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads (V of block j)
  }
}

// Pipeline iteration for block j (PAR = j mod 2): scores of block j + 1, P.V of
// block j - 1, softmax of block j, LDS reads of K(j + 2) and V(j).  Past the
// last block the score products and K reads work on stale ring data and their
// results are never used; before the first block P(-1) and V(-1) are zero.
template <int D, int NK, int PAR, bool MASK>
__device__ __forceinline__ void step(St<D>& st, const Ctx& c, int j) {
  constexpr int NCB = Cfg<D>::NCB;
  st.s[PAR ^ 1] = score_products<D>(st.kf, st.qf);
  read_k<D, NK>(st.kf, c, j + 2);
  pv_products<D, PAR ^ 1>(st);
  f32x16 sj = st.s[PAR];
  if (MASK) mask_scores(sj, j * kKB, c);
  float sum = block_weights(sj, c.sc, st.m, st.p[PAR][0], st.p[PAR][1]);
  read_v<D, NK>(st, c, j);
  step_schedule<D>();
  // keep the weights in this block (they would otherwise sink past the branch below)
  asm volatile("" ::"v"(st.p[PAR][0]), "v"(st.p[PAR][1]), "v"(sum));
  // rare: some lane's weights sum past the limit or are not finite (the first
  // block, where m = -1e30).  Recompute this block's scores (so they need not stay
  // live), move m to the row's running max, rescale O (which already holds
  // P(j-1) V(j-1)) and l, and form the weights again.
  if (__builtin_amdgcn_ballot_w64(!(sum <= kSumLimit))) {
    asm volatile("" ::: "memory");  // re-read the K operands from LDS
    bf16x8 kj[Cfg<D>::NKS];
    read_k<D, NK>(kj, c, j);
    f32x16 s = score_products<D>(kj, st.qf);
    if (MASK) mask_scores(s, j * kKB, c);
    const float mu = vmax(st.m, half_swap_max(max16(s)) * c.sc);
    const float alpha = __builtin_amdgcn_exp2f(st.m - mu);
    st.m = mu;
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[cb][r] *= alpha;
    sum = block_weights(s, c.sc, st.m, st.p[PAR][0], st.p[PAR][1]);
  }
  st.l += sum;
}

// Epilogue of a map-1 wavefront: o = O1/l1 - lambda O2/l2 from this lane's O1
// accumulators (times inv = 1/l1) and map 2's value o2(cb, r) of the same
// accumulator slot (both maps take identical operations: identical maps with
// lambda = 1 give exact zeros), the head RMS norm over dv (in-lane + one
// swap), times (1 - lambda_init) w, rounded to bf16 and stored to `out` (the
// lane's output row; nullptr: not stored).  Channels ch..ch+3, ch = 32 cb +
// 8 g4 + 4 hh, live in o[cb][4 g4 .. 4 g4 + 3].
template <int D, typename O2>
__device__ __forceinline__ void combine_store(St<D>& st, float inv, O2 o2, const FwdParams& p, __bf16* out, int hh) {
  constexpr int NCB = Cfg<D>::NCB, DV = Cfg<D>::DV;
  const float lam = lambda_of(p.lam_dev, p.lam);
  float ss = 0.f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = __builtin_fmaf(-lam, o2(cb, r), __fmul_rn(st.o[cb][r], inv));
      st.o[cb][r] = x;
      ss = __builtin_fmaf(x, x, ss);
    }
  float scale = 1.0f;
  if (p.normalize) {
    ss = half_swap_sum(ss);
    scale = (1.0f - p.lam_init) / sqrtf(ss * (1.0f / DV) + p.eps);
  }
  if (!out) return;
  // all weights first: a wait for a load between the stores would also wait
  // for every store before it (one counter), serialising them
  f32x4 wv[NCB][4];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) wv[cb][g4] = f32x4{1.f, 1.f, 1.f, 1.f};
  if (p.normalize && p.norm_w) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[cb][g4][e] = p.norm_w[cb * 32 + 8 * g4 + 4 * hh + e];
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int ch = cb * 32 + 8 * g4 + 4 * hh;
      const f32x4 w = wv[cb][g4];
      f32x4 y = {st.o[cb][4 * g4] * scale * w[0], st.o[cb][4 * g4 + 1] * scale * w[1],
                 st.o[cb][4 * g4 + 2] * scale * w[2], st.o[cb][4 * g4 + 3] * scale * w[3]};
      *(bf16x4*)(out + ch) = __builtin_convertvector(y, bf16x4);
    }
}

// The block walk of a wavefront: tile t's sync precedes block 2t; blocks
// before the wavefront's first masked block run unmasked, every wavefront runs
// the same sequence of syncs; then the last block's P.V.  qw0 is the
// wavefront's first query when causal, else -1 (keys past N - 1 are masked).
template <int D, int NK, typename Sync>
__device__ __forceinline__ void walk_blocks(St<D>& st, const Ctx& c, int nb, Sync& tile_sync, int lane, int qw0,
                                            int N) {
  const int jm = min(c.jmask, nb);
  int j = 0;
  for (; j + 1 < jm; j += 2) {
    tile_sync(j >> 1);
    step<D, NK, 0, false>(st, c, j);
    step<D, NK, 1, false>(st, c, j + 1);
  }
  if (j < jm) {  // jm odd: one more unmasked (even) block
    tile_sync(j >> 1);
    step<D, NK, 0, false>(st, c, j);
    ++j;
  }
  // the masked blocks recompute the lane constants from an opaque lane index, so
  // nothing derived for the loop above has to stay live across it
  Ctx cm = c;
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    cm.l32 = ln & 31;
    cm.hh = ln >> 5;
    cm.vt_lane = ((4 * cm.hh + (ln & 15) / 4) << 8) | (16 * ((ln >> 4) & 1) + 4 * (ln & 3));
    cm.kmax = qw0 >= 0 ? qw0 + cm.l32 : N - 1;
  }
  if ((j & 1) && j < nb) {  // first masked block is odd
    step<D, NK, 1, true>(st, cm, j);
    ++j;
  }
  for (; j < nb; j += 2) {
    tile_sync(j >> 1);
    step<D, NK, 0, true>(st, cm, j);
    if (j + 1 < nb) step<D, NK, 1, true>(st, cm, j + 1);
  }
  // drain: P(nb-1) V(nb-1)
  if ((nb - 1) & 1)
    pv_products<D, 1>(st);
  else
    pv_products<D, 0>(st);
}

// One work item of the general kernel: index `logical` of the item order below
// (query block fastest, longest first); `ring` is the workgroup's LDS.
template <int D>
__device__ __forceinline__ void fwd_item(const FwdParams& p, unsigned char* ring, int logical) {
  using C = Cfg<D>;
  constexpr int DV = C::DV, NCB = C::NCB, NKS = C::NKS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave % kGroups, map = wave / kGroups;  // map 0: Q1/K1, map 1: Q2/K2
  const int l32 = lane & 31, hh = lane >> 5;
  const int nq = (p.max_seqlen + kQB - 1) / kQB;
  int qb, member, n, sq;  // sq: sequence
  if (p.cu_seqlens) {
    // packed sequences of unequal lengths: sequence fastest, so the contiguous
    // range each XCD walks holds every sequence's share of the work
    qb = nq - 1 - logical % nq;
    int t = logical / nq;
    sq = t % p.nseq;
    t /= p.nseq;
    member = t % p.g;
    n = t / p.g;
  } else if (nq < 64) {
    // few query blocks per head: the signal heads of a noise group interleaved,
    // longest query block first, so an XCD's workgroups finish together (a
    // head's blocks alone are about one round of the XCD's CUs); the ones
    // running at once share the group's K2
    const int per = p.g * nq, idx = logical % per, grp = logical / per;
    qb = nq - 1 - idx / p.g;
    member = idx % p.g;
    n = grp % p.Hn;
    sq = grp / p.Hn;
  } else {
    // long sequences: a head's blocks are consecutive, longest first (the
    // workgroups running at once share that head's K/V prefix in L2)
    qb = nq - 1 - logical % nq;
    int t = logical / nq;
    member = t % p.g;
    t /= p.g;
    n = t % p.Hn;
    sq = t / p.Hn;
  }
  const int h = __builtin_amdgcn_readfirstlane(p.members[n * p.g + member]);
  const int kh = __builtin_amdgcn_readfirstlane(p.kv[h]);
  const int q0 = qb * kQB;
  const int qw0 = q0 + grp * kQW;

  // the sequence: batch b, tokens [tok0, tok0 + N).  Packed sequences live in
  // batch 0 at the offsets cu_seqlens gives, clamped to the token axis.
  int b = sq, tok0 = 0, N = p.N;
  if (p.cu_seqlens) {
    const int s0 = p.cu_seqlens[sq], s1 = p.cu_seqlens[sq + 1];
    b = 0;
    tok0 = min(max(s0, 0), p.N);
    N = max(min(min(s1, p.N) - tok0, p.max_seqlen), 0);
  }
  if (q0 >= N) return;  // whole workgroup: no query row of this block exists

  const int64_t t0 = tok0;
  const __bf16* Q1 = (const __bf16*)p.q1 + b * p.sq1[0] + t0 * p.sq1[1] + h * p.sq1[2];
  const __bf16* Q2 = (const __bf16*)p.q2 + b * p.sq2[0] + t0 * p.sq2[1] + n * p.sq2[2];
  const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + t0 * p.sk1[1] + kh * p.sk1[2];
  const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + t0 * p.sk2[1] + n * p.sk2[2];
  const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + t0 * p.sv[1] + kh * p.sv[2];

  const int kend = p.causal ? min(q0 + kQB, N) : N;
  const int nb = (kend + kKB - 1) / kKB;      // 32-key blocks every wavefront walks
  const int ntiles = (nb + 1) / 2;

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8*)ring;

  // ---- tile DMA.  Each wave loads TLOADS KiB of one tensor: waves 0-1 K1, 2-3 K2,
  // 4-7 V.  Lane l of a 1-KiB load writes LDS bytes [16 l, 16 l + 16) of that KiB,
  // so the global chunk a lane fetches implements the swizzle; within a KiB the
  // row is row0 + l / (chunks per row) with row0 a multiple of 4 (V) or 8 (K), so
  // the swizzle term and the per-lane source offset depend on the lane only.  On
  // a tile that runs past N, rows past N re-read row N - 1 (in bounds): keys that
  // are always masked (causal: beyond every valid query; otherwise: >= N).
  const bool v_wave = wave >= 4;
  const __bf16* tsrc = v_wave ? V : (wave < 2 ? K1 : K2);
  const int64_t trow = v_wave ? p.sv[1] : (wave < 2 ? p.sk1[1] : p.sk2[1]);  // element stride of a row
  const uint32_t trs = (uint32_t)trow * 2u;                                     // byte stride of a row
  const int rpl = v_wave ? C::VRPL : C::KRPL;
  const int tblk0 = v_wave ? (wave - 4) * C::TLOADS : (wave & 1) * C::TLOADS;  // first KiB of this wave's share
  const uint32_t tdst = (v_wave ? 2 * C::KBYTES : (wave < 2 ? 0 : C::KBYTES)) + tblk0 * 1024;
  const int lrow = v_wave ? lane / C::VCH : lane / C::KCH;
  const uint32_t lchunk = v_wave ? (uint32_t)(((lane % C::VCH) ^ ((lrow & 3) << C::VSH)) << 4)
                                 : (uint32_t)(((lane % C::KCH) ^ ((lrow >> C::KSH) & C::KSW)) << 4);
  // K rows of the odd KiB loads (tblk0 is even) take the flipped term
  const uint32_t lflip = v_wave ? 0u : (uint32_t)(C::KFLIP << 4);
  const uint32_t loff = (uint32_t)lrow * trs + lchunk, loff1 = (uint32_t)lrow * trs + (lchunk ^ lflip);
  auto issue_tile = [&](int tile) {
    const uint32_t dst = ring_lds + (tile % kSlots) * C::STAGE + tdst;
    const int key0 = tile * kKT;  // < N for every tile issued
    if (key0 + kKT <= N) {
      const char* g = (const char*)(tsrc + (int64_t)(key0 + tblk0 * rpl) * trow);
#pragma unroll
      for (int i = 0; i < C::TLOADS; ++i) dma16(g + (uint32_t)(i * rpl) * trs, (i & 1) ? loff1 : loff, dst + i * 1024);
    } else {
      // rows relative to the tile start, clamped to the last valid row N - 1 - key0 >= 0
      const char* g = (const char*)(tsrc + (int64_t)key0 * trow);
      const int lim = N - 1 - key0;
#pragma unroll
      for (int i = 0; i < C::TLOADS; ++i)
        dma16(g, (uint32_t)min((tblk0 + i) * rpl + lrow, lim) * trs + ((i & 1) ? (lchunk ^ lflip) : lchunk),
              dst + i * 1024);
    }
  };
  // before block 2t: blocks 2t and 2t + 1 read tiles t and t + 1.  Wait for this
  // wave's loads of tile t + 1 (later tiles may stay in flight), then for every
  // wave's; after the barrier the slot of tile t - 1 is no longer read and
  // receives tile t + kSlots - 1.
  static_assert(kSlots >= 4 && kSlots <= 6, "ring depth");
  auto tile_sync = [&](int tt) {
    if (tt + 1 >= ntiles) return;
    wait_tiles_in_flight<C::TLOADS>(min(kSlots - 3, ntiles - tt - 2));
    wait_lds_and_barrier();
    if (tt + kSlots - 1 < ntiles) issue_tile(tt + kSlots - 1);
  };

  // ---- prologue: Q1 (waves 0-3) and Q2 (waves 4-7) of the workgroup into the last
  // slot, tiles 0..kSlots-2 into the others
  {
    const bool q2w = wave >= 4;
    const __bf16* qsrc = q2w ? Q2 : Q1;
    const int64_t qrow = q2w ? p.sq2[1] : p.sq1[1];
    const uint32_t qrs = (uint32_t)qrow * 2u;
    const int qblk0 = (wave & 3) * C::QLOADS;
    const int kr_l = lane / C::KCH;
    const uint32_t kc_l = (uint32_t)(((lane % C::KCH) ^ ((kr_l >> C::KSH) & C::KSW)) << 4);
    const uint32_t kc_l1 = kc_l ^ (uint32_t)(C::KFLIP << 4);  // odd KiB loads (qblk0 is even)
    const uint32_t qdst = ring_lds + (kSlots - 1) * C::STAGE + (q2w ? C::QBYTES : 0) + qblk0 * 1024;
    const int lim = N - 1 - q0;  // query rows past N re-read row N - 1 (never stored)
    const char* g = (const char*)(qsrc + (int64_t)q0 * qrow);
#pragma unroll
    for (int i = 0; i < C::QLOADS; ++i)
      dma16(g, (uint32_t)min((qblk0 + i) * C::KRPL + kr_l, lim) * qrs + ((i & 1) ? kc_l1 : kc_l), qdst + i * 1024);
  }
  for (int tt = 0; tt < min(ntiles, kSlots - 1); ++tt) issue_tile(tt);
  wait_tiles_in_flight<C::TLOADS>(min(ntiles, kSlots - 1) - 1);  // the Q rows and tile 0 have landed
  wait_lds_and_barrier();

  Ctx c;
  c.ring = ring;
  c.koff = map * C::KBYTES;
  c.l32 = l32;
  c.hh = hh;
  c.vt_lane = ((4 * hh + (lane & 15) / 4) << 8) | (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  c.kmax = p.causal ? qw0 + l32 : N - 1;
  c.jmask = p.causal ? qw0 / kKB : N / kKB;
  c.sc = p.sm_scale_log2;

  St<D> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.o[cb] = f32x16{};
  st.m = -1e30f;
  st.l = 0.f;
  {
    // Q fragments: B operand of S^T = K Q^T; lane (q, half) holds Q[q][16 s + 8 half + 0..7]
    const unsigned char* qs = ring + (kSlots - 1) * C::STAGE + map * C::QBYTES;
    const int qr = grp * kQW + l32;
#pragma unroll
    for (int s = 0; s < NKS; ++s) st.qf[s] = *(const bf16x8*)(qs + k_off<D>(qr, 2 * s + hh));
  }
  // P(-1) and V(-1) are zero: the first step's P.V adds nothing
  st.p[1][0] = st.p[1][1] = bf16x8{};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.vf[cb][0] = st.vf[cb][1] = bf16x8{};
  read_k<D, 2>(st.kf, c, 0);
  st.s[0] = score_products<D>(st.kf, st.qf);
  read_k<D, 2>(st.kf, c, 1);

  walk_blocks<D, 2>(st, c, nb, tile_sync, lane, p.causal ? qw0 : -1, N);

  // ---- epilogue.  The ring is free once every wave is past its last read (all
  // tile loads were awaited before their tiles were read).
  wait_lds_and_barrier();
  const float lsum = half_swap_sum(st.l);
  const float inv = 1.0f / lsum;
  const int q = qw0 + l32;
  if (p.lse && hh == 0 && q < N) {
    const int64_t base = ((int64_t)b * p.Hs + h) * p.N + tok0 + q;
    constexpr float kLn2 = 0.69314718055994531f;
    p.lse[(int64_t)map * p.B * p.Hs * p.N + base] = (st.m + __log2f(lsum)) * kLn2;
  }
  // hand-off of O2/l2 in the accumulator layout: register r of lane l of query
  // group g at float index ((g NCB + cb) 16 + r) 64 + l
  float* xo = (float*)ring;
  if (map == 1) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[((grp * NCB + cb) * 16 + r) * 64 + lane] = __fmul_rn(st.o[cb][r], inv);
  }
  __syncthreads();
  if (map == 1 || qw0 >= N) return;

  if (p.o_maps && q < N) {  // each map's own output, A1 V and A2 V, in fp32
    float* om1 = p.o_maps + ((((int64_t)b * p.N + tok0 + q) * p.Hs + h) * DV);
    float* om2 = om1 + (int64_t)p.B * p.N * p.Hs * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ch = cb * 32 + 8 * g4 + 4 * hh;
        f32x4 a, z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = __fmul_rn(st.o[cb][4 * g4 + e], inv);
          z[e] = xo[((grp * NCB + cb) * 16 + 4 * g4 + e) * 64 + lane];
        }
        *(f32x4*)(om1 + ch) = a;
        *(f32x4*)(om2 + ch) = z;
      }
  }

  combine_store<D>(st, inv, [&](int cb, int r) { return xo[((grp * NCB + cb) * 16 + r) * 64 + lane]; }, p,
                   q < N ? (__bf16*)p.out + b * p.so[0] + (t0 + q) * p.so[1] + h * p.so[2] : nullptr, hh);
}

// Work items are numbered so that each XCD (workgroup ids congruent mod 8) owns
// a contiguous range of them.  With one workgroup per item the hardware
// dispatcher hands an XCD's items out in that order as its compute units free
// up.  For fixed-length batches with at least two items per compute unit the
// launcher sizes a persistent grid instead (one workgroup per compute unit,
// which the 128 KiB of LDS of a d = 64 workgroup ensures): the workgroups of
// an XCD take its items in a snake over rounds -- round r gives rank r w + w'
// (w workgroups on the XCD; w' = this one's index within it, or w - 1 minus
// it for odd r) -- so pairs of rounds even out the causal lengths, and the
// items running at once are the ones the dispatcher would run.  With one item
// per workgroup the loop runs once.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSlots * C::STAGE];
  const int nq = (p.max_seqlen + kQB - 1) / kQB;
  const int total = p.nseq * p.Hs * nq;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  const int xstart = xcd * q8 + min(xcd, r8), xcount = q8 + (xcd < r8 ? 1 : 0);
  const int nw = ((int)gridDim.x - xcd + 7) >> 3, w = bid >> 3;  // the XCD's workgroups, this one's index
  for (int r = 0;; ++r) {
    const int rank = r * nw + ((r & 1) ? nw - 1 - w : w);
    if (rank >= xcount) break;
    fwd_item<D>(p, ring, xstart + rank);
    __syncthreads();  // every wavefront is past this item's LDS reads before the next item's loads
  }
}

// ---- layers whose signal heads share noise and key/value heads
//
// Signal heads with the same noise head and the same key/value head (a
// "combo": with GQA key/value heads under GDA noise heads, e.g. 16 signal, 4
// noise and 8 key/value heads, each noise group holds two combos of two) have
// the same map 2 output softmax(Q2 K2^T/sqrt(d)) V ("Grouped Differential
// Attention" (mlsanity.com), "Abstract": noise heads shared GQA-style), so A2 V
// is one product per combo, and the combo's members share their K1 and V
// tiles.  Two launches:
//   * the noise kernel (SIG = false): a workgroup owns 256 queries (8 query
//     groups of 32, one wavefront each) of one (batch, combo) and forms
//     A2 V / l2 in fp32.  With no workspace in the prefill's arguments, it
//     parks these rows in the combo's own output rows: channels 0-63 in the
//     bf16 row of its first member, 64-127 in its second's (256 bytes each);
//     it also writes each member's map-2 LSE and A2 V when asked.
//   * the signal kernel (SIG = true): a workgroup owns 256 / gs queries of one
//     (batch, combo of gs heads) and runs one wavefront per (member, query
//     group of 32); every K1 and V tile in LDS serves all members.  Its epilogue reads
//     the parked A2 V rows of its queries into registers, meets the other
//     wavefronts at a barrier (so no parked row is overwritten before every
//     wavefront has read it) and then forms o = A1 V - lambda A2 V, the head
//     norm and the stores, in the same operations as the general kernel.
// The pipeline, the ring (four slots of one K tile and the V tile, filled by
// DMA: each wavefront loads one KiB of K and two of V per tile) and the block
// walk are the general kernel's; only the wavefront-to-work map differs.
constexpr int kSharedRows = 256;  // Q rows staged per workgroup (either kernel)

template <int D, bool SIG>
__global__ __launch_bounds__(kThreads, 1) void fwd_shared_kernel(FwdParams p) {
  using C = Cfg<D>;
  using Lo = Lay<D, 1>;
  constexpr int DV = C::DV, NCB = C::NCB, NKS = C::NKS;
  static_assert(D == 64, "one K KiB and two V KiB per wavefront and tile");
  static_assert(kKT * C::KROW == kWaves * 1024 && kKT * C::VROW == 2 * kWaves * 1024, "tile split over waves");
  constexpr int QREG = kSharedRows * C::KROW;  // staged Q rows
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSlots * Lo::STAGE + QREG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int g = p.gs;                        // heads per combo: 2, 4 or 8 (host-checked)
  const int qpw = SIG ? kSharedRows / g : kSharedRows;  // queries per workgroup
  const int mi = SIG ? wave % g : 0;         // this wavefront's member (signal kernel)
  const int qg = SIG ? wave / g : wave;      // its query group

  // ---- work item: XCD-contiguous ranges, (batch, combo) pairs in turn, each
  // pair's query blocks longest first
  const int N = p.N;
  const int nq = (N + qpw - 1) / qpw;
  const int total = p.B * p.ncombo * nq;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  const int logical = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int qb = nq - 1 - logical % nq;
  const int cmb = (logical / nq) % p.ncombo;
  const int b = logical / nq / p.ncombo;
  const int m0 = __builtin_amdgcn_readfirstlane(p.cmem[cmb * g]);
  const int m1 = __builtin_amdgcn_readfirstlane(p.cmem[cmb * g + 1]);
  const int n = __builtin_amdgcn_readfirstlane(p.nz[m0]);
  const int kh = __builtin_amdgcn_readfirstlane(p.kv[m0]);
  const int q0 = qb * qpw;  // < N
  const int qw0 = q0 + qg * kQW;

  const __bf16* K = SIG ? (const __bf16*)p.k1 + b * p.sk1[0] + kh * p.sk1[2]
                        : (const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[2];
  const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + kh * p.sv[2];
  const int64_t krow = SIG ? p.sk1[1] : p.sk2[1], vrow = p.sv[1];  // element strides of a token
  const uint32_t krs = (uint32_t)krow * 2u, vrs = (uint32_t)vrow * 2u;

  const int kend = p.causal ? min(q0 + qpw, N) : N;
  const int nb = (kend + kKB - 1) / kKB;
  const int ntiles = (nb + 1) / 2;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8*)ring;

  // ---- tile DMA: wave w loads K rows [8 w, 8 w + 8) (one KiB) and V rows
  // [8 w, 8 w + 8) (two KiB) of the 64-key tile.  The lane's global chunk
  // implements the swizzle of k_off / v_off; rows past N re-read row N - 1.
  const int lrk = lane >> 3, lrv = lane >> 4;
  const uint32_t kch = (uint32_t)(((lane & 7) ^ (((8 * wave + lrk) >> 1) & 7)) << 4);
  const uint32_t vch = (uint32_t)(((lane & 15) ^ (lrv << 2)) << 4);
  const uint32_t kl = (uint32_t)(8 * wave + lrk) * krs + kch;
  const uint32_t vl = (uint32_t)(8 * wave + lrv) * vrs + vch;
  auto issue_tile = [&](int tile) {
    const uint32_t dst = ring_lds + (tile % kSlots) * Lo::STAGE;
    const int key0 = tile * kKT;  // < N for every tile issued
    const char* gk = (const char*)(K + (int64_t)key0 * krow);
    const char* gv = (const char*)(V + (int64_t)key0 * vrow);
    if (key0 + kKT <= N) {
      dma16(gk, kl, dst + wave * 1024);
      dma16(gv, vl, dst + Lo::VOFF + 2 * wave * 1024);
      dma16(gv, vl + 4 * vrs, dst + Lo::VOFF + (2 * wave + 1) * 1024);
    } else {
      const int lim = N - 1 - key0;
      dma16(gk, (uint32_t)min(8 * wave + lrk, lim) * krs + kch, dst + wave * 1024);
      dma16(gv, (uint32_t)min(8 * wave + lrv, lim) * vrs + vch, dst + Lo::VOFF + 2 * wave * 1024);
      dma16(gv, (uint32_t)min(8 * wave + 4 + lrv, lim) * vrs + vch, dst + Lo::VOFF + (2 * wave + 1) * 1024);
    }
  };
  constexpr int TL = 3;  // DMA instructions per wave and tile
  auto tile_sync = [&](int tt) {
    if (tt + 1 >= ntiles) return;
    wait_tiles_in_flight<TL>(min(kSlots - 3, ntiles - tt - 2));
    wait_lds_and_barrier();
    if (tt + kSlots - 1 < ntiles) issue_tile(tt + kSlots - 1);
  };

  // ---- prologue: the workgroup's Q rows after the ring (row r: signal kernel
  // member r / qpw at query q0 + r % qpw; noise kernel query q0 + r), wave w
  // loading rows [32 w, 32 w + 32); then tiles 0..kSlots-2
  {
    const int r0 = kQW * wave;
    const int src_m = SIG ? r0 / qpw : 0, qo = SIG ? r0 % qpw : r0;
    const int hq = __builtin_amdgcn_readfirstlane(SIG ? p.cmem[cmb * g + src_m] : n);
    const __bf16* qsrc = SIG ? (const __bf16*)p.q1 + b * p.sq1[0] + hq * p.sq1[2]
                             : (const __bf16*)p.q2 + b * p.sq2[0] + hq * p.sq2[2];
    const int64_t qrow = SIG ? p.sq1[1] : p.sq2[1];
    const uint32_t qrs = (uint32_t)qrow * 2u;
    const int qfirst = min(q0 + qo, N - 1), lim = N - 1 - qfirst;  // rows past N re-read row N - 1
    const char* gq = (const char*)(qsrc + (int64_t)qfirst * qrow);
    const uint32_t qdst = ring_lds + kSlots * Lo::STAGE + r0 * C::KROW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // rows r0 + 8 i + lrk: swizzle term ((8 i + lrk) >> 1) & 7, r0 a multiple of 32
      const uint32_t ch = (uint32_t)(((lane & 7) ^ ((4 * (i & 1)) | (lrk >> 1))) << 4);
      dma16(gq, (uint32_t)min(8 * i + lrk, lim) * qrs + ch, qdst + i * 1024);
    }
  }
  for (int tt = 0; tt < min(ntiles, kSlots - 1); ++tt) issue_tile(tt);
  wait_tiles_in_flight<TL>(min(ntiles, kSlots - 1) - 1);  // the Q rows and tile 0 have landed
  wait_lds_and_barrier();

  Ctx c;
  c.ring = ring;
  c.koff = 0;
  c.l32 = l32;
  c.hh = hh;
  c.vt_lane = ((4 * hh + (lane & 15) / 4) << 8) | (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  c.kmax = p.causal ? qw0 + l32 : N - 1;
  c.jmask = p.causal ? qw0 / kKB : N / kKB;
  c.sc = p.sm_scale_log2;

  St<D> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.o[cb] = f32x16{};
  st.m = -1e30f;
  st.l = 0.f;
  {
    const unsigned char* qs = ring + kSlots * Lo::STAGE;
    const int qr = mi * qpw + qg * kQW + l32;
#pragma unroll
    for (int s = 0; s < NKS; ++s) st.qf[s] = *(const bf16x8*)(qs + k_off<D>(qr, 2 * s + hh));
  }
  st.p[1][0] = st.p[1][1] = bf16x8{};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.vf[cb][0] = st.vf[cb][1] = bf16x8{};
  read_k<D, 1>(st.kf, c, 0);
  st.s[0] = score_products<D>(st.kf, st.qf);
  read_k<D, 1>(st.kf, c, 1);

  walk_blocks<D, 1>(st, c, nb, tile_sync, lane, p.causal ? qw0 : -1, N);

  // ---- epilogue
  const float lsum = half_swap_sum(st.l);
  const float inv = 1.0f / lsum;
  const int q = qw0 + l32;
  constexpr float kLn2 = 0.69314718055994531f;
  const int64_t orow = (int64_t)b * p.so[0] + (int64_t)q * p.so[1];  // + head * so[2]: a bf16 output row
  if (!SIG) {
    if (q < N) {
      const float lse = (st.m + __log2f(lsum)) * kLn2;
      float* par0 = (float*)((__bf16*)p.out + orow + m0 * p.so[2]);  // channels 0-63
      float* par1 = (float*)((__bf16*)p.out + orow + m1 * p.so[2]);  // channels 64-127
      for (int i = 0; i < g; ++i) {
        const int h = p.cmem[cmb * g + i];
        if (p.lse && hh == 0) p.lse[(int64_t)p.B * p.Hs * p.N + ((int64_t)b * p.Hs + h) * p.N + q] = lse;
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int ch = cb * 32 + 8 * g4 + 4 * hh;
          f32x4 z;
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = __fmul_rn(st.o[cb][4 * g4 + e], inv);
          *(f32x4*)(ch < DV / 2 ? par0 + ch : par1 + (ch - DV / 2)) = z;
          if (p.o_maps)
            for (int i = 0; i < g; ++i) {
              const int h = p.cmem[cmb * g + i];
              float* om2 = p.o_maps + (int64_t)p.B * p.N * p.Hs * DV + (((int64_t)b * p.N + q) * p.Hs + h) * DV;
              *(f32x4*)(om2 + ch) = z;
            }
        }
    }
    return;
  }

  const int h = __builtin_amdgcn_readfirstlane(p.cmem[cmb * g + mi]);
  if (p.lse && hh == 0 && q < N)
    p.lse[((int64_t)b * p.Hs + h) * p.N + q] = (st.m + __log2f(lsum)) * kLn2;
  // the parked A2 V / l2 of this lane's query and channels
  f32x4 z[NCB][4];
  if (q < N) {
    const float* par0 = (const float*)((const __bf16*)p.out + orow + m0 * p.so[2]);
    const float* par1 = (const float*)((const __bf16*)p.out + orow + m1 * p.so[2]);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ch = cb * 32 + 8 * g4 + 4 * hh;
        z[cb][g4] = *(const f32x4*)(ch < DV / 2 ? par0 + ch : par1 + (ch - DV / 2));
      }
  }
  // every parked row of the workgroup's queries has been read (the loads have
  // returned) before any wavefront stores an output row
  wait_vmcnt<0>();
  __syncthreads();
  if (q >= N) return;

  if (p.o_maps) {
    float* om1 = p.o_maps + (((int64_t)b * p.N + q) * p.Hs + h) * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = __fmul_rn(st.o[cb][4 * g4 + e], inv);
        *(f32x4*)(om1 + cb * 32 + 8 * g4 + 4 * hh) = a;
      }
  }
  combine_store<D>(st, inv, [&](int cb, int r) { return z[cb][r / 4][r % 4]; }, p,
                   (__bf16*)p.out + orow + h * p.so[2], hh);
}

// Compute units of the current device, queried once per device.
hipError_t compute_units(int* n) {
  constexpr int kMaxDevices = 64;
  static int count[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (count[dev] == 0) {
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    count[dev] = c;
  }
  *n = count[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s) {
  const int64_t nq = (p.max_seqlen + kQB - 1) / kQB;
  const int64_t total = (int64_t)p.nseq * p.Hs * nq;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  // persistent grid for fixed-length batches at d = 64 with at least two items per compute unit
  int64_t grid = total;
  if (p.d == 64 && !p.cu_seqlens) {
    int cus = 0;
    const hipError_t e = compute_units(&cus);
    if (e != hipSuccess) return e;
    if (cus > 0 && total >= 2 * (int64_t)cus) grid = cus;
  }
  if (p.d == 64)
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<32>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

bool shared_kv_plan(FwdParams& p) {
  if (p.d != 64 || p.cu_seqlens) return false;
  // combos in noise-group order (the combos of a noise group share its K2 in L2),
  // members in head order; every combo must hold the same number of heads
  int gs = 0, nc = 0, fill = 0;
  bool used[DA_MAX_HEADS] = {};
  for (int i = 0; i < p.Hn * p.g; ++i) {
    const int h0 = p.members[i];
    if (used[h0]) continue;
    int cnt = 0;
    for (int j = i; j < (i / p.g + 1) * p.g; ++j) {  // the rest of i's noise group
      const int h = p.members[j];
      if (!used[h] && p.kv[h] == p.kv[h0]) {
        used[h] = true;
        p.cmem[fill++] = (int16_t)h;
        ++cnt;
      }
    }
    if (gs == 0) gs = cnt;
    if (cnt != gs) return false;
    ++nc;
  }
  if (!(gs == 2 || gs == 4 || gs == 8)) return false;
  // A2 V is parked in the output rows of each combo's first two members, so the
  // output's (batch, token, head) rows must not overlap: nested row-major strides
  const int64_t dv = p.dv;
  if (p.so[2] < dv || p.so[1] < (int64_t)(p.Hs - 1) * p.so[2] + dv) return false;
  if (p.B > 1 && p.so[0] < (int64_t)(p.N - 1) * p.so[1] + (int64_t)(p.Hs - 1) * p.so[2] + dv) return false;
  p.gs = gs;
  p.ncombo = nc;
  return true;
}

hipError_t launch_fwd_shared_bf16(const FwdParams& p, hipStream_t s) {
  const int64_t pairs = (int64_t)p.B * p.ncombo;
  const int64_t noise = pairs * ((p.N + kSharedRows - 1) / kSharedRows);
  const int qs = kSharedRows / p.gs;
  const int64_t sig = pairs * ((p.N + qs - 1) / qs);
  if (sig > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_shared_kernel<64, false>), dim3((unsigned)noise), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL((fwd_shared_kernel<64, true>), dim3((unsigned)sig), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

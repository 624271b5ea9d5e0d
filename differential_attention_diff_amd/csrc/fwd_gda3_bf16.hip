// bf16 fused prefill for Grouped Differential Attention with three signal heads
// per noise head, each with its own key/value head: one workgroup per (batch,
// noise group, 64-query block), so the noise map -- its scores, its online
// softmax and its K2 tile in LDS -- is formed once per group and its weights
// serve the three signal heads.
//
// Computes, per signal head h and query i ("Differential Attention in Large
// Language Models: How Denoising Subtraction Eliminates Attention Noise and
// Outlier Activations" (llms.blog), "Differential Attention Architecture",
// DiffAttn equation; "Headwise Normalization", head_bar_i equation):
//   o = softmax(Q1 K1^T/sqrt(d)) V - lambda softmax(Q2 K2^T/sqrt(d)) V
//   out = (1 - lambda_init) * w * o / sqrt(mean(o^2) + eps)
// with Q2/K2 of the group's noise head shared by its three signal heads
// ("Grouped Differential Attention" (mlsanity.com), "Abstract": noise heads
// repeated GQA-style).
//
// Work decomposition (d = 64, dv = 128)
//   * Two query groups of 32 queries; per query group four wavefronts: three
//     signal wavefronts (one per member head: its map-1 scores and softmax) and
//     one noise wavefront (the group's map-2 scores and softmax).  Per 32-key
//     block each query group needs 4 x 4 score MFMAs and 6 x 8 P.V MFMAs (A1 V
//     and A2 V for each member); the P.V work is split by V channels so every
//     wavefront issues 16 MFMAs and one softmax per block:
//       signal m: O1_m (all 128 channels) and O2_m channels 0..63, both from
//                 the V fragments of its member (read once);
//       noise:    O2_m channels 64..127 of all three members.
//     The noise wavefront hands its bf16 weights P2 of each block to the
//     signal wavefronts of its query group through LDS (2 KiB per block).
//   * K tiles (K1 of the three members and K2, 16 KiB per 32 keys) and V tiles
//     (V of the three members, 24 KiB) go global -> LDS by DMA
//     (global_load_lds_dwordx4) into separate rings of 4 and 3 slots: at the
//     barrier before block j the K tiles of j+1 and the V tiles of j have
//     landed, and K(j+3), V(j+2) are issued; two tiles of each stay in
//     flight.  16-byte chunks are XOR-swizzled by row (implemented by the
//     global chunk each lane fetches), so neither the MFMA operand reads nor
//     the transposing V reads conflict on LDS banks.
//   * Scores are transposed, S^T = K Q^T on v_mfma_f32_32x32x16_bf16: lane
//     (q, half) holds 16 keys of one query row.
//   * One step per block j: P.V of block j-1, scores of block j+1 and the
//     softmax of block j, with the LDS reads of K(j+1) and V(j).
//   * Each map keeps a reference max m and a sum l per row in fp32; weights
//     are 2^(s sc - m) without a block max.  When some lane's weights of a
//     block sum past 2^12 (the first block, or scores climbing far above m)
//     the wavefront recomputes the block's scores from the K tile (still in
//     its slot), moves m to the running max and rescales its accumulators.
//     A move of the noise map is published with the block's weights (a flag
//     and the factor per query), and the signal wavefronts rescale their
//     share of O2 before adding that block.
//   * Epilogue: the noise wavefront hands O2 channels 64..127 / l2 of each
//     member and 1/l2 through LDS; each signal wavefront forms o = O1/l1 -
//     lambda O2/l2, the RMS norm over 128 channels, times (1 - lambda_init) w,
//     stores bf16 and the LSE (the noise wavefront stores map 2's LSE).
#include <math.h>

#include "fwd_common.h"
#include "kernels.h"

namespace da {
namespace {

using namespace fwdc;

constexpr int kG = 3;                     // signal heads per noise group (distinct V each)
constexpr int kRoles = kG + 1;            // wavefronts per query group: kG signal + 1 noise
constexpr int kQGroups = 2;               // query groups per workgroup
constexpr int kWaves = kQGroups * kRoles;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;                   // queries per wavefront (MFMA N dim)
constexpr int kQB = kQGroups * kQW;       // queries per workgroup
constexpr int kKT = 32;                   // keys per tile and per pipeline block
constexpr int kKSlots = 4, kVSlots = 3;   // ring depths
constexpr float kSumLimit = 4096.0f;      // lane weight sum that forces a reference move

constexpr int D = 64, DV = 128, NCB = DV / 32, NKS = D / 16;
constexpr int KROW = 2 * D, VROW = 2 * DV;            // bytes per row
constexpr int KTILE = kKT * KROW, VTILE = kKT * VROW; // 4 KiB, 8 KiB
constexpr int KSTAGE = (kG + 1) * KTILE;              // K1 of the members, then K2
constexpr int VSTAGE = kG * VTILE;                    // V of the members
constexpr int KLOADS = KSTAGE / 1024 / kWaves;        // 1-KiB DMA loads per wave and K tile
constexpr int VLOADS = VSTAGE / 1024 / kWaves;        // ... and V tile
constexpr int QTILE = kQB * KROW;                     // one tensor's rows of the query block
constexpr int QLOADS = (kG + 1) * QTILE / 1024 / kWaves;
constexpr int KRING = 0;
constexpr int VRING = KRING + kKSlots * KSTAGE;
constexpr int XCH = VRING + kVSlots * VSTAGE;         // P2 hand-off, per (query group, block parity)
constexpr int XALPHA = 2048, XFLAG = 2048 + 128, XSLOT = 2048 + 256;  // weights, factors, flag
constexpr int LDS_BYTES = XCH + kQGroups * 2 * XSLOT;
constexpr int QSTAGE = VRING + VSTAGE;                // Q rows wait in V slots 1-2 before the loop
constexpr int XO_BYTES = kG * 2 * 16 * 64 * 4 + 64 * 4;  // epilogue hand-off per query group (K ring)
static_assert(KLOADS * kWaves * 1024 == KSTAGE && VLOADS * kWaves * 1024 == VSTAGE, "tile split over waves");
static_assert(QLOADS * kWaves * 1024 == (kG + 1) * QTILE, "Q split over waves");
static_assert(KLOADS == 2 && VLOADS == 3 && QLOADS == 4, "load maps below");
static_assert((kG + 1) * QTILE <= (kVSlots - 1) * VSTAGE, "Q staging fits V slots 1 and 2");
static_assert(kQGroups * XO_BYTES <= kKSlots * KSTAGE, "epilogue hand-off fits the K ring");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// LDS byte offset of 16-B chunk c of row r (XOR swizzle).  K and Q rows (128 B):
// chunk ^ ((r >> 1) mod 8) -- an MFMA operand read takes one chunk of 16
// consecutive rows per 16 lanes, two rows per 256-B bank window, so the term
// counts pairs of rows.  V rows (256 B): chunk ^ ((r mod 4) << 2) puts the 4
// rows a transposing read touches 64 B apart.
__device__ __forceinline__ int k_off(int r, int c) { return r * KROW + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int v_off(int r, int c) { return r * VROW + ((c ^ ((r & 3) << 2)) << 4); }

struct Ctx {
  lds_u8* lds;         // the workgroup's LDS array
  int kten;            // K tensor of this wave in a K stage: member m (K1) or kG (K2)
  int l32, hh;
  int kmax;            // last key this lane's query sees (causal: its row; else N - 1)
  int qg;
  float sc;            // log2(e)/sqrt(d)
  uint32_t kl[NKS];    // LDS offset of the lane's K chunk pair s in the first K slot (swizzled)
  uint32_t vl[NCB];    // LDS offset of its V^T read of channel block cb in the first V slot
};

__device__ __forceinline__ lds_u8* xslot(const Ctx& c, int par) {
  return c.lds + XCH + (c.qg * 2 + par) * XSLOT;
}

// Per-lane LDS offsets.  K (A operand of S^T = K Q^T): lane (k, half) reads
// K[k][16 s + 8 half + 0..7], chunk 2 s + half of row k.  V^T (32 channels x 16
// keys per read pair): lane j of a 16-lane group reads row 4 half + j/4 at
// channels c0 + 4 (j%4) of block cb; the transposing read hands lane i the 4
// keys of channel c0 + i.  Rows 8 and 16 further keep row mod 4, hence the
// swizzle term: those reads are the same offsets plus 8 or 16 rows.
__device__ __forceinline__ void lane_offsets(Ctx& c, int lane) {
#pragma unroll
  for (int s = 0; s < NKS; ++s) c.kl[s] = (uint32_t)(KRING + c.kten * KTILE + k_off(c.l32, 2 * s + c.hh));
  const int vt = ((4 * c.hh + (lane & 15) / 4) << 8) | (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  const int r0 = vt >> 8;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int ch = cb * 32 + (vt & 0xff);
    c.vl[cb] = (uint32_t)(VRING + v_off(r0, ch >> 3) + (ch & 7) * 2);
  }
}

__device__ __forceinline__ void read_k(bf16x8 (&kf)[NKS], const Ctx& c, int t) {
  const uint32_t slot = ((uint32_t)t % kKSlots) * KSTAGE;
#pragma unroll
  for (int s = 0; s < NKS; ++s) kf[s] = lds_ld16(c.lds + opaque(c.kl[s] + slot));
}

// V^T operands of channel block cb of member m's V in tile t (keys 0-15, 16-31);
// the ring base is in the opaque part so the remaining constants fit the 16-bit
// offset field
__device__ __forceinline__ void read_v_cb(bf16x8 (&vf)[2], const Ctx& c, int t, int m, int cb) {
  const lds_u8* vs = c.lds + opaque(((uint32_t)t % kVSlots) * VSTAGE + c.vl[cb]) + m * VTILE;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x4 lo = lds_ld_tr8(vs + ks * 16 * VROW);
    const bf16x4 hi = lds_ld_tr8(vs + (ks * 16 + 8) * VROW);
    vf[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

__device__ __forceinline__ f32x16 score_products(const bf16x8 (&kf)[NKS], const bf16x8 (&qf)[NKS]) {
  f32x16 a = {};
#pragma unroll
  for (int s = 0; s < NKS; ++s) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], a, 0, 0, 0);
  return a;
}

__device__ __forceinline__ void pv(f32x16& o, const bf16x8 (&vf)[2], const bf16x8& p0, const bf16x8& p1) {
  o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0], p0, o, 0, 0, 0);
  o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1], p1, o, 0, 0, 0);
}

// The rare reference move of block j: recompute its scores from the K tile,
// move m to the row's running max, return the factor for the accumulators and
// the weights against the new reference.
template <bool MASK>
__device__ __forceinline__ float move_reference(const Ctx& c, const bf16x8 (&qf)[NKS], int j, float& m, bf16x8& p0,
                                                bf16x8& p1, float& sum) {
  asm volatile("" ::: "memory");  // re-read the K operands from LDS
  bf16x8 kj[NKS];
  read_k(kj, c, j);
  f32x16 s = score_products(kj, qf);
  if (MASK) mask_scores(s, c.kmax - j * kKT - 4 * c.hh);
  const float mu = vmax(m, half_swap_max(max16(s)) * c.sc);
  const float alpha = __builtin_amdgcn_exp2f(m - mu);
  m = mu;
  sum = block_weights(s, c.sc, m, p0, p1);
  return alpha;
}

// ---------------------------------------------------------------------------
// signal wavefront: map 1 of member m (all channels) and map 2 channels 0..63
// ---------------------------------------------------------------------------
struct SigSt {
  f32x16 o1[NCB];
  f32x16 o2[2];
  f32x16 s[2];          // S^T of block j (parity j) and j + 1
  bf16x8 p[2][2];       // own weights of block j (parity j) and j - 1
  bf16x8 qf[NKS];
  float m, l;
};

// P.V of block jv for a signal wavefront: map 2 (channel blocks 0, 1) from the
// noise weights in hand-off slot `par`, after the rescale the noise wavefront
// published with them, then map 1 (all channel blocks) from its own weights
// pa/pb.  The published move is tested first, so that the rest of the step --
// these products, the next scores and this block's softmax -- is one
// scheduling region.
__device__ __forceinline__ void sig_pv(SigSt& st, const Ctx& c, int m, int jv, int par, const bf16x8& pa,
                                       const bf16x8& pb) {
  const lds_u8* xs = xslot(c, par);
  const int moved = lds_ldi(xs + XFLAG);
  bf16x8 va[2], vb[2];
  read_v_cb(va, c, jv, m, 0);
  read_v_cb(vb, c, jv, m, 1);
  const lds_u8* xl = xs + (c.l32 * 16 + c.hh * 512);
  const bf16x8 pn0 = lds_ld16(xl), pn1 = lds_ld16(xl + 1024);
  if (__builtin_amdgcn_readfirstlane(moved)) {
    const float a = lds_ldf(xs + XALPHA + 4 * c.l32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      st.o2[0][r] *= a;
      st.o2[1][r] *= a;
    }
  }
  pv(st.o2[0], va, pn0, pn1);
  pv(st.o2[1], vb, pn0, pn1);
  pv(st.o1[0], va, pa, pb);
  pv(st.o1[1], vb, pa, pb);
  read_v_cb(va, c, jv, m, 2);
  read_v_cb(vb, c, jv, m, 3);
  pv(st.o1[2], va, pa, pb);
  pv(st.o1[3], vb, pa, pb);
}

template <int PAR, bool MASK, bool FIRST = false>
__device__ __forceinline__ void sig_step(SigSt& st, const Ctx& c, int m, int j) {
  // P.V of block j - 1 (its V tile is still resident; none before block 0)
  if (!FIRST) sig_pv(st, c, m, j - 1, PAR ^ 1, st.p[PAR ^ 1][0], st.p[PAR ^ 1][1]);
  bf16x8 kf[NKS];
  read_k(kf, c, j + 1);
  // scores of block j + 1
  st.s[PAR ^ 1] = score_products(kf, st.qf);
  // softmax of block j
  f32x16 sj = st.s[PAR];
  if (MASK) mask_scores(sj, c.kmax - j * kKT - 4 * c.hh);
  float sum = block_weights(sj, c.sc, st.m, st.p[PAR][0], st.p[PAR][1]);
  asm volatile("" ::"v"(st.p[PAR][0]), "v"(st.p[PAR][1]), "v"(sum));
  if (__builtin_amdgcn_ballot_w64(!(sum <= kSumLimit))) {
    const float alpha = move_reference<MASK>(c, st.qf, j, st.m, st.p[PAR][0], st.p[PAR][1], sum);
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o1[cb][r] *= alpha;
  }
  st.l += sum;
}

// ---------------------------------------------------------------------------
// noise wavefront: map 2 of the group, channels 64..127 of each member's A2 V
// ---------------------------------------------------------------------------
struct NzSt {
  f32x16 o[kG][2];
  f32x16 s[2];
  bf16x8 p[2][2];
  bf16x8 qf[NKS];
  float m, l;
};

// P.V of block jv for the noise wavefront: channel blocks 2, 3 of every member's V
__device__ __forceinline__ void nz_pv(NzSt& st, const Ctx& c, int jv, const bf16x8& pa, const bf16x8& pb) {
#pragma unroll
  for (int m = 0; m < kG; ++m)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      bf16x8 v[2];
      read_v_cb(v, c, jv, m, 2 + cc);
      pv(st.o[m][cc], v, pa, pb);
    }
}

template <int PAR, bool MASK, bool FIRST = false>
__device__ __forceinline__ void nz_step(NzSt& st, const Ctx& c, int j) {
  bf16x8 kf[NKS];
  read_k(kf, c, j + 1);
  if (!FIRST) nz_pv(st, c, j - 1, st.p[PAR ^ 1][0], st.p[PAR ^ 1][1]);
  st.s[PAR ^ 1] = score_products(kf, st.qf);
  f32x16 sj = st.s[PAR];
  if (MASK) mask_scores(sj, c.kmax - j * kKT - 4 * c.hh);
  float sum = block_weights(sj, c.sc, st.m, st.p[PAR][0], st.p[PAR][1]);
  asm volatile("" ::"v"(st.p[PAR][0]), "v"(st.p[PAR][1]), "v"(sum));
  int moved = 0;
  float alpha = 1.0f;
  if (__builtin_amdgcn_ballot_w64(!(sum <= kSumLimit))) {
    alpha = move_reference<MASK>(c, st.qf, j, st.m, st.p[PAR][0], st.p[PAR][1], sum);
    moved = 1;
    st.l *= alpha;
#pragma unroll
    for (int m = 0; m < kG; ++m)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[m][cc][r] *= alpha;
  }
  st.l += sum;
  // publish block j's weights (and the move) for the signal wavefronts of this
  // query group; they read them after the next barrier
  lds_u8* xs = xslot(c, PAR);
  lds_u8* xl = xs + (c.l32 * 16 + c.hh * 512);
  lds_st16(xl, st.p[PAR][0]);
  lds_st16(xl + 1024, st.p[PAR][1]);
  if (moved && c.hh == 0) lds_stf(xs + XALPHA + 4 * c.l32, alpha);
  if ((c.l32 | c.hh) == 0) lds_sti(xs + XFLAG, moved);
}

__global__ __launch_bounds__(kThreads, 1) void fwd_gda3_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave / kRoles, role = wave % kRoles;  // role kG: the noise wavefront
  const bool noise = role == kG;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work item: XCD-contiguous range, query block fastest (longest first)
  const int N = p.N;
  const int nq = (N + kQB - 1) / kQB;
  const int logical = xcd_logical(blockIdx.x, p.B * p.Hn * nq);
  const int qb = nq - 1 - logical % nq;
  const int n = (logical / nq) % p.Hn, b = logical / nq / p.Hn;
  const int q0 = qb * kQB;
  const int qw0 = q0 + qg * kQW;

  const int kend = p.causal ? min(q0 + kQB, N) : N;
  const int nb = (kend + kKT - 1) / kKT;  // 32-key blocks (= tiles) every wavefront walks
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8*)lds;

  // ---- tile DMA.  K stage: KiB i = 2 wave + t (t < 2) is KiB i % 4 of tensor i / 4
  // (K1 of members 0..2, then K2), rows 8 (i % 4) + lane / 8.  V stage: KiB i =
  // 3 wave + t (t < 3) is KiB i % 8 of member i / 8's V, rows 4 (i % 8) + lane / 16.
  // Lane l of a 1-KiB load writes LDS bytes [16 l, 16 l + 16), so the global
  // chunk it fetches implements the swizzle.  On a tile that runs past N, rows
  // past N re-read row N - 1 (in bounds): keys that are always masked.
  const int kt = wave / 2;  // K tensor this wave loads
  const char* kg;           // rows of the next K tile this wave issues
  int64_t krs;              // element stride of a K row
  if (kt < kG) {
    const int kh = p.kv[p.members[n * kG + kt]];
    kg = (const char*)((const __bf16*)p.k1 + b * p.sk1[0] + kh * p.sk1[2]);
    krs = p.sk1[1];
  } else {
    kg = (const char*)((const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[2]);
    krs = p.sk2[1];
  }
  const uint32_t kbs = (uint32_t)krs * 2u;  // bytes per K row
  const int kkk0 = (wave & 1) * 2;          // first KiB of the wave's K share in its tensor
  // per-lane source offset of load t (rows relative to the tile's first key, at most lim)
  auto k_lane_off = [&](int t, int lim) {
    const int r = (kkk0 + t) * 8 + lane / 8;
    return (uint32_t)min(r, lim) * kbs + (uint32_t)(((lane % 8) ^ ((r >> 1) & 7)) << 4);
  };
  uint32_t koff[KLOADS];
#pragma unroll
  for (int t = 0; t < KLOADS; ++t) koff[t] = k_lane_off(t, kKT);
  const int64_t vrs = p.sv[1];
  const uint32_t vbs = (uint32_t)vrs * 2u;
  const uint32_t vch = (uint32_t)(((lane % 16) ^ ((lane / 16) << 2)) << 4);  // row mod 4 = lane / 16
  const char* vg[VLOADS];   // rows of the next V tile, from the first row of load t
  uint32_t vdst[VLOADS];
  int vkk[VLOADS];
#pragma unroll
  for (int t = 0; t < VLOADS; ++t) {
    const int i = VLOADS * wave + t, m = i / 8;
    vkk[t] = i % 8;
    const int vh = p.kv[p.members[n * kG + m]];
    vg[t] = (const char*)((const __bf16*)p.v + b * p.sv[0] + (4 * vkk[t]) * p.sv[1] + vh * p.sv[2]);
    vdst[t] = (uint32_t)(m * VTILE + vkk[t] * 1024);
  }
  const uint32_t voff = (uint32_t)(lane / 16) * vbs + vch;
  const int nfull = N / kKT;  // tiles with all kKT rows inside the sequence
  // the tiles are issued in order: running source pointers and ring destinations
  int knext = 0, vnext = 0;
  uint32_t kdst = lds_base + KRING + kt * KTILE + kkk0 * 1024;
  uint32_t vdst0 = lds_base + VRING;
  auto issue_k = [&]() {
    if (knext < nfull) {
#pragma unroll
      for (int t = 0; t < KLOADS; ++t) dma16(kg, koff[t], kdst + t * 1024);
    } else {  // rows past N re-read row N - 1 (in bounds): keys that are always masked
      const int lim = N - 1 - knext * kKT;
#pragma unroll
      for (int t = 0; t < KLOADS; ++t) dma16(kg, k_lane_off(t, lim), kdst + t * 1024);
    }
    kg += (size_t)kKT * kbs;
    ++knext;
    kdst = (knext % kKSlots) ? kdst + KSTAGE : kdst - (kKSlots - 1) * KSTAGE;
  };
  auto issue_v = [&]() {
    if (vnext < nfull) {
#pragma unroll
      for (int t = 0; t < VLOADS; ++t) dma16(vg[t], voff, vdst0 + vdst[t]);
    } else {
      const int lim = N - 1 - vnext * kKT;
#pragma unroll
      for (int t = 0; t < VLOADS; ++t)
        dma16(vg[t] - (size_t)(4 * vkk[t]) * vbs, (uint32_t)min(4 * vkk[t] + lane / 16, lim) * vbs + vch,
              vdst0 + vdst[t]);
    }
#pragma unroll
    for (int t = 0; t < VLOADS; ++t) vg[t] += (size_t)kKT * vbs;
    ++vnext;
    vdst0 = (vnext % kVSlots) ? vdst0 + VSTAGE : vdst0 - (kVSlots - 1) * VSTAGE;
  };
  // barrier before block j.  Step j reads K(j+1) (and K(j) on a reference move)
  // and V(j-1); both were issued two barriers earlier (or in the prologue, whose
  // loads were all awaited): the loads issued at the barrier before block j - 1
  // may stay in flight.  After the barrier the slots of K(j-1) and V(j-2) are
  // free and receive K(j+3) and V(j+1).
  auto issued_at = [&](int j) { return (j + 3 < nb ? KLOADS : 0) + (j + 1 < nb ? VLOADS : 0); };
  auto tile_sync = [&](int j) {
    const int keep = j == 0 ? 0 : issued_at(j - 1);
    if (keep >= KLOADS + VLOADS)
      wait_vmcnt<KLOADS + VLOADS>();
    else if (keep >= VLOADS)
      wait_vmcnt<VLOADS>();
    else
      wait_vmcnt<0>();
    wait_lds_and_barrier();
    if (j + 3 < nb) issue_k();  // tile j + 3
    if (j + 1 < nb) issue_v();  // tile j + 1
  };

  // ---- prologue: the query rows (Q1 of the members, Q2) into V slots 1-2 (V(1)
  // is issued at the first block's barrier, after every wave holds its rows),
  // K(0..2) and V(0)
  {
#pragma unroll
    for (int t = 0; t < QLOADS; ++t) {
      const int i = QLOADS * wave + t, m = i / 8, kk = i % 8;
      const __bf16* qsrc;
      int64_t qrs;
      if (m < kG) {
        qsrc = (const __bf16*)p.q1 + b * p.sq1[0] + q0 * p.sq1[1] + p.members[n * kG + m] * p.sq1[2];
        qrs = p.sq1[1];
      } else {
        qsrc = (const __bf16*)p.q2 + b * p.sq2[0] + q0 * p.sq2[1] + n * p.sq2[2];
        qrs = p.sq2[1];
      }
      const int r = kk * 8 + lane / 8;
      const uint32_t ch = (uint32_t)(((lane % 8) ^ ((r >> 1) & 7)) << 4);
      // query rows past N re-read row N - 1 (never stored)
      dma16(qsrc, (uint32_t)min(r, N - 1 - q0) * ((uint32_t)qrs * 2u) + ch,
            lds_base + QSTAGE + m * QTILE + kk * 1024);
    }
  }
  for (int tt = 0; tt < min(nb, 3); ++tt) issue_k();  // tiles 0..2
  issue_v();                                          // tile 0
  wait_vmcnt<0>();
  wait_lds_and_barrier();

  Ctx c;
  c.lds = (lds_u8*)lds;
  c.kten = noise ? kG : role;
  c.l32 = l32;
  c.hh = hh;
  lane_offsets(c, lane);
  c.kmax = p.causal ? qw0 + l32 : N - 1;
  c.qg = qg;
  c.sc = p.sm_scale_log2;
  const int jmask = p.causal ? qw0 / kKT : N / kKT;  // first block that needs a mask
  const int jm = min(jmask, nb);
  const float lam = lambda_of(p.lam_dev, p.lam);
  lds_u8* const xo_base = (lds_u8*)lds + (KRING + qg * XO_BYTES);  // epilogue hand-off of this query group

  // Q fragments: B operand of S^T = K Q^T; lane (q, half) holds Q[q][16 s + 8 half + 0..7]
  auto read_q = [&](bf16x8 (&qf)[NKS]) {
    const lds_u8* qs = (lds_u8*)lds + (QSTAGE + c.kten * QTILE);
    const int qr = qg * kQW + l32;
#pragma unroll
    for (int s = 0; s < NKS; ++s) qf[s] = lds_ld16(qs + k_off(qr, 2 * s + hh));
  };

  if (!noise) {
    // ======================= signal wavefront =======================
    const int m = role;
    const int h = p.members[n * kG + m];
    SigSt st;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) st.o1[cb] = f32x16{};
    st.o2[0] = st.o2[1] = f32x16{};
    st.m = -1e30f;
    st.l = 0.f;
    read_q(st.qf);
    {
      bf16x8 kf[NKS];
      read_k(kf, c, 0);
      st.s[0] = score_products(kf, st.qf);
    }
    tile_sync(0);
    if (jm > 0)
      sig_step<0, false, true>(st, c, m, 0);
    else
      sig_step<0, true, true>(st, c, m, 0);
    int j = 1;
    for (; j + 1 < jm; j += 2) {
      tile_sync(j);
      sig_step<1, false>(st, c, m, j);
      tile_sync(j + 1);
      sig_step<0, false>(st, c, m, j + 1);
    }
    if (j < jm) {
      tile_sync(j);
      sig_step<1, false>(st, c, m, j);
      ++j;
    }
    if ((j & 1) && j < nb) {
      tile_sync(j);
      sig_step<1, true>(st, c, m, j);
      ++j;
    }
    for (; j < nb; j += 2) {
      tile_sync(j);
      sig_step<0, true>(st, c, m, j);
      if (j + 1 < nb) {
        tile_sync(j + 1);
        sig_step<1, true>(st, c, m, j + 1);
      }
    }
    // drain: P.V of the last block, map 2 with the noise weights published in it
    wait_vmcnt<0>();
    wait_lds_and_barrier();
    if ((nb - 1) & 1)
      sig_pv(st, c, m, nb - 1, 1, st.p[1][0], st.p[1][1]);
    else
      sig_pv(st, c, m, nb - 1, 0, st.p[0][0], st.p[0][1]);
    wait_lds_and_barrier();  // ring reads done: the noise wavefronts fill the hand-off
    wait_lds_and_barrier();  // hand-off written

    const float lsum = half_swap_sum(st.l);
    const float inv1 = 1.0f / lsum;
    const int q = qw0 + l32;
    if (p.lse && hh == 0 && q < N) {
      constexpr float kLn2 = 0.69314718055994531f;
      p.lse[((int64_t)b * p.Hs + h) * p.N + q] = (st.m + __log2f(lsum)) * kLn2;
    }
    if (qw0 >= N) return;
    const lds_u8* xo = xo_base + (m * 2 * 16 * 64 * 4 + lane * 4);
    const float inv2 = lds_ldf(xo_base + (kG * 2 * 16 * 64 + lane) * 4);
    // o2 by channel block: 0, 1 from this wavefront (times 1/l2), 2, 3 from the hand-off
    auto o2n = [&](int cb, int r) {
      return cb < 2 ? __fmul_rn(st.o2[cb & 1][r], inv2) : lds_ldf(xo + ((cb - 2) * 16 + r) * 64 * 4);
    };
    if (p.o_maps && q < N) {  // each map's own output, A1 V and A2 V, in fp32
      float* om1 = p.o_maps + ((((int64_t)b * p.N + q) * p.Hs + h) * DV);
      float* om2 = om1 + (int64_t)p.B * p.N * p.Hs * DV;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int ch = cb * 32 + 8 * g4 + 4 * hh;
          f32x4 a, z;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = __fmul_rn(st.o1[cb][4 * g4 + e], inv1);
            z[e] = o2n(cb, 4 * g4 + e);
          }
          *(f32x4*)(om1 + ch) = a;
          *(f32x4*)(om2 + ch) = z;
        }
    }
    // o = O1/l1 - lambda O2/l2 (both maps take identical operations: identical
    // maps with lambda = 1 give exact zeros), then the head RMS norm
    float ss = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = __builtin_fmaf(-lam, o2n(cb, r), __fmul_rn(st.o1[cb][r], inv1));
        st.o1[cb][r] = x;
        ss = __builtin_fmaf(x, x, ss);
      }
    float scale = 1.0f;
    if (p.normalize) {
      ss = half_swap_sum(ss);
      scale = (1.0f - p.lam_init) / sqrtf(ss * (1.0f / DV) + p.eps);
    }
    if (q < N) {
      __bf16* out = (__bf16*)p.out + b * p.so[0] + q * p.so[1] + h * p.so[2];
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
          const int ch = cb * 32 + 8 * g4 + 4 * hh;  // channels ch..ch+3 live in o1[cb][4 g4 .. 4 g4 + 3]
          const f32x4 w = wv[cb][g4];
          f32x4 y = {st.o1[cb][4 * g4] * scale * w[0], st.o1[cb][4 * g4 + 1] * scale * w[1],
                     st.o1[cb][4 * g4 + 2] * scale * w[2], st.o1[cb][4 * g4 + 3] * scale * w[3]};
          *(bf16x4*)(out + ch) = __builtin_convertvector(y, bf16x4);
        }
    }
  } else {
    // ======================= noise wavefront =======================
    NzSt st;
#pragma unroll
    for (int m = 0; m < kG; ++m) st.o[m][0] = st.o[m][1] = f32x16{};
    st.m = -1e30f;
    st.l = 0.f;
    read_q(st.qf);
    {
      bf16x8 kf[NKS];
      read_k(kf, c, 0);
      st.s[0] = score_products(kf, st.qf);
    }
    tile_sync(0);
    if (jm > 0)
      nz_step<0, false, true>(st, c, 0);
    else
      nz_step<0, true, true>(st, c, 0);
    int j = 1;
    for (; j + 1 < jm; j += 2) {
      tile_sync(j);
      nz_step<1, false>(st, c, j);
      tile_sync(j + 1);
      nz_step<0, false>(st, c, j + 1);
    }
    if (j < jm) {
      tile_sync(j);
      nz_step<1, false>(st, c, j);
      ++j;
    }
    if ((j & 1) && j < nb) {
      tile_sync(j);
      nz_step<1, true>(st, c, j);
      ++j;
    }
    for (; j < nb; j += 2) {
      tile_sync(j);
      nz_step<0, true>(st, c, j);
      if (j + 1 < nb) {
        tile_sync(j + 1);
        nz_step<1, true>(st, c, j + 1);
      }
    }
    wait_vmcnt<0>();
    wait_lds_and_barrier();  // the signal wavefronts read the last block's weights
    if ((nb - 1) & 1)
      nz_pv(st, c, nb - 1, st.p[1][0], st.p[1][1]);
    else
      nz_pv(st, c, nb - 1, st.p[0][0], st.p[0][1]);
    wait_lds_and_barrier();  // ring reads done
    const float lsum = half_swap_sum(st.l);
    const float inv2 = 1.0f / lsum;
    // hand-off in the accumulator layout: member m, block cc, register r of lane l
    // at float ((m 2 + cc) 16 + r) 64 + l; then 1/l2 per lane
#pragma unroll
    for (int m = 0; m < kG; ++m)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          lds_stf(xo_base + (((m * 2 + cc) * 16 + r) * 64 + lane) * 4, __fmul_rn(st.o[m][cc][r], inv2));
    lds_stf(xo_base + (kG * 2 * 16 * 64 + lane) * 4, inv2);
    const int q = qw0 + l32;
    if (p.lse && hh == 0 && q < N) {
      constexpr float kLn2 = 0.69314718055994531f;
      const float v = (st.m + __log2f(lsum)) * kLn2;
#pragma unroll
      for (int m = 0; m < kG; ++m)
        p.lse[(int64_t)p.B * p.Hs * p.N + ((int64_t)b * p.Hs + p.members[n * kG + m]) * p.N + q] = v;
    }
    wait_lds_and_barrier();  // hand-off written
  }
}

}  // namespace

// The grouped kernel applies when every noise group has three signal heads on
// three distinct key/value heads (d = 64); other layouts take fwd_bf16_kernel.
// Fixed-length batches only: packed sequences of unequal lengths take the
// general kernel, whose 128-query blocks of every (signal head, sequence)
// spread each sequence over all XCDs; at this kernel's granularity an XCD's
// contiguous share held 6 of the 8 sequences of a noise group and the XCDs'
// work differed by 29% (packed 3:1 workload 0.78 ms here, 0.70 ms there).
bool gda3_applies(const FwdParams& p) {
  if (p.d != 64 || p.g != kG || p.cu_seqlens) return false;
  for (int n = 0; n < p.Hn; ++n) {
    const int a = p.kv[p.members[n * kG]], b = p.kv[p.members[n * kG + 1]], c = p.kv[p.members[n * kG + 2]];
    if (a == b || a == c || b == c) return false;
  }
  return true;
}

hipError_t launch_fwd_gda3_bf16(const FwdParams& p, hipStream_t s) {
  const int64_t nq = (p.N + kQB - 1) / kQB;
  const int64_t total = (int64_t)p.B * p.Hn * nq;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_gda3_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

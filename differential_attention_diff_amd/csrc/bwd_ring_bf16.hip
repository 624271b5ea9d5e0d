// bf16 backward score passes for d = 64 (dv = 128) on gfx950: the dQ pass and
// the dK/dV pass with their streamed operands in an LDS ring filled by DMA,
// sized so that several workgroups share a compute unit.
//
// Gradients of "Differential Attention in Large Language Models: How
// Denoising Subtraction Eliminates Attention Noise and Outlier Activations"
// (llms.blog), "Differential Attention Architecture", DiffAttn equation, with
// the noise heads of "Grouped Differential Attention" (mlsanity.com),
// "Abstract".  With do and the row statistics of the prep pass (lse1', lse2'
// in log2 units, D1 = do . o1, D2 = do . o2), per query i, visible key j:
//   p1 = 2^(s1 sc - lse1'), p2 = 2^(s2 sc - lse2'), dp = do_i . v_j
//   ds1 = p1 (dp - D1),  ds2 = -lambda p2 (dp - D2)
//   dQ1 = dS1 K1 / sqrt(d), dK1 = dS1^T Q1 / sqrt(d), dV = (P1 - lambda P2)^T do,
//   dQ2 = dS2 K2 / sqrt(d), dK2 = dS2^T Q2 / sqrt(d)
// (the prep pass stores lse2' - log2|lambda| and sgn D2 with -lambda = sgn
// |lambda|, so the kernels form |lambda| p2 and ds2 = (|lambda| p2)(sgn dp -
// sgn D2) directly; P1 - lambda P2 = p1 + sgn (|lambda| p2)).
//
// Work decomposition: a workgroup owns the rows of one (batch, noise group)
// -- 16 per wavefront -- and walks the group's signal heads in turn; the noise
// head's sums stay in registers, every gradient row is written once.  The
// other side streams through LDS in blocks of 32 rows:
//   dQ pass (8 wavefronts, 128 queries): K1, K2 and V of a block, 16 KiB;
//   dK/dV pass (4 wavefronts, 64 keys): Q1, Q2, do and the row statistics,
//     16.5 KiB.
// A ring of slots holds the blocks of all signal heads in one sequence: at the
// barrier before block f, block f has landed and the next block is issued
// into the slot block f - 1 left (global_load_lds_dwordx4, 16 B per lane,
// 1 KiB per wavefront load).  The 16-byte chunks of a row are XOR-swizzled by
// row (the swizzle is the global chunk each lane fetches), so the row-wise
// operand reads (16 rows at one chunk) and the transposing reads (8 rows x
// 32 B per 32 lanes) spread over the banks.
//
// Occupancy carries the overlap: a dQ workgroup needs at most 128 registers
// per lane and 64 KiB of LDS, so two share a compute unit (four wavefronts
// per SIMD); a dK/dV workgroup at most 168 registers (its key-side operands
// and dK1/dK2/dV sums stay in registers) and 49.5 KiB, so three share one
// (three per SIMD).  While one wavefront waits for its products or its
// barrier, the others issue.
//
// v_mfma_f32_16x16x32_bf16 throughout (lane l: A row l%16, B column l%16,
// k 8 (l/16) .. +7; accumulator rows 4 (l/16) + r of column l%16); operands
// that must be transposed are read with ds_read_b64_tr_b16.
//   dQ pass: S^T = K Q^T (lane = query), so dS^T is the B operand of
//     dQ^T = K^T dS^T.
//   dKV pass: S = Q K^T (lane = key), so dS and P1 - lambda P2 are the B
//     operands of dK^T = Q^T dS and dV^T = do^T (P1 - lambda P2); the
//     per-query statistics are LDS broadcasts.
// In the dKV pass the signal heads of a key/value head must be consecutive in
// the group (checked on the host): dK1/dV accumulate over that run and are
// stored when the key/value head changes.
#include <math.h>

#include <stddef.h>

#include <type_traits>

#include "fwd_common.h"
#include "kernels.h"

namespace da {
namespace {

using namespace fwdc;

constexpr int kRW = 16;   // rows per wavefront
constexpr int kBK = 32;   // rows of the streamed side per block
constexpr int D = 64, DV = 128;
constexpr int KROW = 2 * D, VROW = 2 * DV;          // bytes per row
constexpr int KBLK = kBK * KROW, VBLK = kBK * VROW;  // 4 KiB, 8 KiB
constexpr int NS = D / 32, NVS = DV / 32;            // 32-wide k steps over d, dv
constexpr int NDT = D / 16, NVT = DV / 16;           // 16-column output tiles over d, dv
static_assert(offsetof(BwdParams, members) % 4 == 0 && offsetof(BwdParams, kv) % 4 == 0,
              "head tables are read 4 bytes at a time");

// Swizzles (r = row mod 16).  128-byte rows: chunk c of row r sits at chunk
// c ^ hk(r); the 8 even (odd) rows of 16 take distinct values, and the 4 even
// (odd) rows of 8 distinct values of hk >> 1, which is what the row-wise and
// the transposing reads need.  256-byte rows (a row covers all banks): chunk
// c ^ hv(r), hv distinct over 16 rows and hv >> 1 distinct over 8.
__device__ __forceinline__ int hk(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int hv(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed operand of a 16 x 32 step: rows {4 (l/16) + 0..3} of the block
// and the same rows + 16 (the order of two 16-row accumulator tiles), columns
// 16 ct + l%16; `a` points at this lane's 8 bytes of the first read.
__device__ __forceinline__ bf16x8 rd_tr(const lds_u8* a, int hi) {
  const bf16x4 lo = lds_ld_tr8(a), up = lds_ld_tr8(a + hi);
  return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane offsets of the two read patterns within a block of 16-row halves:
// row-wise A operand (lane reads row l%16 at chunk 4 s + l/16), and the
// transposing read (lane i of 16-lane group g reads row 4 g + i/4 at columns
// 16 ct + 4 (i%4)).
__device__ __forceinline__ uint32_t row_off(int lane, int s, int rowbytes, bool wide) {
  const int r = lane & 15, jg = lane >> 4;
  const int h = wide ? hv(r) : hk(r);
  return (uint32_t)(r * rowbytes + (((jg ^ h) ^ (4 * s)) << 4));
}
__device__ __forceinline__ uint32_t tr_off(int lane, int ct, int rowbytes, bool wide) {
  const int i = lane & 15, r = 4 * (lane >> 4) + (i >> 2), x = (i & 3) >> 1;
  const int h = wide ? hv(r) : hk(r);
  return (uint32_t)(r * rowbytes + (((x ^ h) ^ (2 * ct)) << 4) + ((i & 1) << 3));
}
// Source offset of lane l's chunk in a 1-KiB load of rows [r0, r0 + 8) of 128-byte
// rows or [r0, r0 + 4) of 256-byte rows (r0 a multiple of 4), rows clamped to lim.
__device__ __forceinline__ uint32_t src_off(int lane, int r0, bool wide, uint32_t rowstride, int lim) {
  const int r = r0 + (wide ? lane >> 4 : lane >> 3), c = wide ? lane & 15 : lane & 7;
  return (uint32_t)min(r, lim) * rowstride + (uint32_t)((c ^ (wide ? hv(r) : hk(r))) << 4);
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

// Work item `logical` of ngroups (batch, noise group) pairs x nblk blocks.
// Clusters of up to four pairs of one XCD's share (xcd_logical hands each XCD
// a contiguous range) are walked block-major: block 0 of every pair of the
// cluster, then block 1, ..., so the longest causal blocks start first and
// the XCD's workgroups finish together (walking each pair's blocks in turn
// left the longest blocks of an XCD's last pairs to start late: 8-10% longer
// passes with three grouped pairs per XCD).  Four pairs keep their streamed
// operands mostly in the XCD's L2: with all twelve pairs of the 24-head
// layers in one cluster the passes fetched twice the bytes from beyond the
// L2 and took 1% longer.  blk counts from the first block walked.
__device__ __forceinline__ void bwd_item(int logical, int ngroups, int nblk, int& grp, int& blk) {
  const int cl = min((ngroups + 7) / 8, 4);
  const int per = cl * nblk, c = logical / per, idx = logical % per;
  const int cs = min(cl, ngroups - c * cl);  // the last cluster may be smaller
  blk = idx / cs;
  grp = c * cl + idx % cs;
}

// s_waitcnt vmcnt(0) as an instruction the compiler's own counter tracking
// sees (simm16: expcnt 7, lgkmcnt 15, vmcnt 0).  The operand rows a wavefront
// loads into registers before walking the ring are drained with it: the
// compiler does not see the inline-assembly waits of the ring, so it would
// otherwise guard their uses in every block with vmcnt waits of its own, and
// those count the ring's DMA loads too (one counter), holding each block until
// the block issued at its own barrier had landed.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most `after` blocks' loads (PER per wavefront each) are in
// flight; `after` never exceeds MAXA (the ring's depth less two), which keeps
// the choice of wait to MAXA + 1 cases instead of five.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_blocks(int after) {
  static_assert(MAXA >= 0 && MAXA <= 4, "at most four blocks in flight");
  if (MAXA >= 4 && after >= 4)
    wait_vmcnt<4 * PER>();
  else if (MAXA >= 3 && after >= 3)
    wait_vmcnt<3 * PER>();
  else if (MAXA >= 2 && after >= 2)
    wait_vmcnt<2 * PER>();
  else if (MAXA >= 1 && after >= 1)
    wait_vmcnt<PER>();
  else
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// dQ pass: workgroup = (b, noise group n, 128 queries); slot = K1 | K2 | V
// ---------------------------------------------------------------------------
constexpr int kQWaves = 8, kQThreads = 64 * kQWaves, kQRB = kQWaves * kRW;
constexpr int kQSlots = 4;
constexpr int QSLOT = 2 * KBLK + VBLK;
static_assert(kQSlots - 2 <= 4, "wait_blocks covers four blocks in flight");

// Per-lane read offsets of step 0 / column tile 0.  The other steps and tiles
// differ only in the chunk bits of the XOR swizzle: step s of a row read is
// offset ^ (s << 6), column tile c of a transposing read offset ^ (c << 5);
// slot offsets are multiples of 512 and the tensor offsets of 8 KiB, so the
// XOR can follow the slot and tensor terms.
struct DqLane {
  uint32_t kr;   // K rows
  uint32_t kt;   // K^T (rows 0-15; + 16 rows for the second read)
  uint32_t vr;   // V rows (V tensor offset included)
};

// One 32-key block in slot offset sb (keys key0 ..): S1^T, S2^T, dP^T, the
// weights and dS^T, then dQ1^T += K1^T dS1^T and dQ2^T += K2^T dS2^T.  rs
// holds the lane's query statistics as {lse1', lse2', -D1, sgn (D1 - D2)}: the
// dP^T products accumulate onto -D1, so dS1 = P1 (dP - D1) takes one multiply
// and sgn (dP - D2) = sgn (dP - D1) + sgn (D1 - D2) one FMA.
template <bool MASK>
__device__ __forceinline__ void dq_block(f32x4 (&dq1)[NDT], f32x4 (&dq2)[NDT], const bf16x8 (&q1f)[NS],
                                         const bf16x8 (&q2f)[NS], const bf16x8 (&dof)[NVS], const float4& rs,
                                         const lds_u8* lds, const DqLane& L, uint32_t sb, float sc, float sgn,
                                         int key0, int kvis, int jg) {
  // product i of the first phase, 8 per 16-key half t = i / 8: S1^T and S2^T
  // of step 0, of step 1, then the four dP^T steps; each product's LDS operand
  // is read one product ahead (two reads in flight)
  f32x4 s1[2], s2[2], dp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s1[t] = s2[t] = f32x4{};
    dp[t] = f32x4{rs.z, rs.z, rs.z, rs.z};  // -D1: the products accumulate dP - D1
  }
  auto rop = [&](int i) -> bf16x8 {
    const int t = i >> 3, k = i & 7;
    if (k < 4) return lds_ld16(lds + ((sb + L.kr) ^ ((k >> 1) << 6)) + t * 16 * KROW + ((k & 1) ? KBLK : 0));
    return lds_ld16(lds + ((sb + L.vr) ^ ((k - 4) << 6)) + t * 16 * VROW);
  };
  bf16x8 rc = rop(0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bf16x8 rn;
    if (i + 1 < 16) rn = rop(i + 1);
    const int t = i >> 3, k = i & 7;
    if (k >= 4)
      dp[t] = mfma16(rc, dof[k - 4], dp[t]);
    else if (k & 1)
      s2[t] = mfma16(rc, q2f[k >> 1], s2[t]);
    else
      s1[t] = mfma16(rc, q1f[k >> 1], s1[t]);
    rc = rn;
  }
  // k order of the dS^T operand: slots 0-3 = keys 4 (l/16) + r, slots 4-7 = + 16
  bf16x8 b1, b2;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[t][r], sc, -rs.x));
      float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[t][r], sc, -rs.y));  // |lambda| P2
      if (MASK) {
        const bool vis = key0 + 16 * t + 4 * jg + r <= kvis;
        p1 = vis ? p1 : 0.f;
        p2 = vis ? p2 : 0.f;
      }
      b1[4 * t + r] = (__bf16)(p1 * dp[t][r]);
      b2[4 * t + r] = (__bf16)(p2 * __builtin_fmaf(sgn, dp[t][r], rs.w));  // sgn (dP - D2)
    }
  // product i of the second phase: K1^T (even i) or K2^T (odd i) of column
  // tile i / 2, read one product ahead
  auto top = [&](int i) -> bf16x8 { return rd_tr(lds + ((sb + L.kt) ^ ((i >> 1) << 5)) + ((i & 1) ? KBLK : 0), 16 * KROW); };
  bf16x8 tc = top(0);
#pragma unroll
  for (int i = 0; i < 2 * NDT; ++i) {
    bf16x8 tn;
    if (i + 1 < 2 * NDT) tn = top(i + 1);
    if (i & 1)
      dq2[i >> 1] = mfma16(tc, b2, dq2[i >> 1]);
    else
      dq1[i >> 1] = mfma16(tc, b1, dq1[i >> 1]);
    tc = tn;
  }
}

__global__ __launch_bounds__(kQThreads, 4) void bwd_dq_ring_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[kQSlots * QSLOT];
  const lds_u8* lds = (const lds_u8*)lds_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;
  const int lane = threadIdx.x & 63, jg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int N = p.N, g = p.g;
  const int nq = (N + kQRB - 1) / kQRB;
  int t0, blk;
  bwd_item(xcd_logical(blockIdx.x, (int)gridDim.x), p.B * p.Hn, nq, t0, blk);
  const int qb = nq - 1 - blk;  // longest causal range first
  const int n = t0 % p.Hn, b = t0 / p.Hn;
  const int q0 = qb * kQRB, qw = q0 + wave * kRW, q = qw + (lane & 15), qc = min(q, N - 1);
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;  // -lambda = sgn |lambda|
  const float sc = p.sm_scale_log2;
  const int kend = p.causal ? min(q0 + kQRB, N) : N;
  const int nb = (kend + kBK - 1) / kBK;                          // blocks the workgroup walks
  const int klast = p.causal ? min(qw + kRW - 1, N - 1) : N - 1;  // last key this wavefront sees
  const int kfree = p.causal ? min(qw, N - 1) : N - 1;            // keys every query sees: <= kfree
  const int kvis = p.causal ? min(q, N - 1) : N - 1;              // last key this lane sees
  const int nbw = qw < N ? klast / kBK + 1 : 0;                   // blocks this wavefront needs
  const int jfull = min((kfree + 1) / kBK, nbw);                  // ... without a mask

  // ---- DMA of one block: load 0 = 1 KiB of K1 (waves 0-3) or K2 (waves 4-7),
  // rows 8 (wave % 4) ..; load 1 = 1 KiB of V, rows 4 wave ..  Lane l writes
  // LDS bytes [16 l, 16 l + 16) of its KiB, so the chunk it fetches implements
  // the swizzle.  Rows past N re-read row N - 1 (in bounds; such keys are
  // always masked).
  const bool isk2 = wave >= 4;
  const uint32_t kbs = (uint32_t)(isk2 ? p.sk2[1] : p.sk1[1]) * 2u, vbs = (uint32_t)p.sv[1] * 2u;  // bytes per row
  const int kr0 = 8 * (wave & 3), vr0 = 4 * wave;
  const uint32_t koff = src_off(lane, kr0, false, kbs, kBK), voff = src_off(lane, vr0, true, vbs, kBK);
  const uint32_t kdst = (isk2 ? KBLK : 0) + (wave & 3) * 1024, vdst = 2 * KBLK + wave * 1024;
  const int F = g * nb;  // blocks of all signal heads, in walk order
  // the blocks are issued in order: running sources (rows of the next block) and slot
  int im = 0, ij = 0;
  uint32_t idst = lds_base;
  const char* ksrc;
  const char* vsrc;
  auto head_sources = [&]() {
    const int kh = arg16(p.kv, arg16(p.members, n * g + im));
    ksrc = isk2 ? (const char*)((const __bf16*)p.k2 + b * p.sk2[0] + n * p.sk2[2])
                : (const char*)((const __bf16*)p.k1 + b * p.sk1[0] + kh * p.sk1[2]);
    vsrc = (const char*)((const __bf16*)p.v + b * p.sv[0] + kh * p.sv[2]);
  };
  head_sources();
  auto issue = [&]() {
    if (ij * kBK + kBK <= N) {
      dma16(ksrc, koff, idst + kdst);
      dma16(vsrc, voff, idst + vdst);
    } else {  // the block that holds row N - 1
      const int lim = N - 1 - ij * kBK;
      dma16(ksrc, src_off(lane, kr0, false, kbs, lim), idst + kdst);
      dma16(vsrc, src_off(lane, vr0, true, vbs, lim), idst + vdst);
    }
    ksrc += (size_t)kBK * kbs;
    vsrc += (size_t)kBK * vbs;
    if (++ij == nb) {
      ij = 0;
      if (++im < g) head_sources();
    }
    idst = idst == lds_base + (kQSlots - 1) * QSLOT ? lds_base : idst + QSLOT;
  };
  // barrier before block f: f has landed; then f + kQSlots - 1 is issued into
  // the slot of block f - 1, which every wavefront has finished with
  auto sync = [&](int f) {
    wait_blocks<2, kQSlots - 2>(min(F - 1, f + kQSlots - 2) - f);
    wait_lds_and_barrier();
    if (f + kQSlots - 1 < F) issue();
  };
  auto next_slot = [](uint32_t sl) { return sl == (kQSlots - 1) * QSLOT ? 0u : sl + QSLOT; };

  DqLane L;
  L.kr = row_off(lane, 0, KROW, false);
  L.kt = tr_off(lane, 0, KROW, false);
  L.vr = 2 * KBLK + row_off(lane, 0, VROW, true);

  bf16x8 q2f[NS];
  {
    const __bf16* Q2 = (const __bf16*)p.q2 + b * p.sq2[0] + (int64_t)qc * p.sq2[1] + n * p.sq2[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) q2f[s] = *(const bf16x8*)(Q2 + 32 * s + 8 * jg);
  }
  f32x4 dq2[NDT];
#pragma unroll
  for (int ct = 0; ct < NDT; ++ct) dq2[ct] = f32x4{};

  for (int t = 0; t < min(F, kQSlots - 1); ++t) issue();  // blocks 0 .. kQSlots - 2

  uint32_t sl = 0;  // slot offset of the next block walked
  int f0 = 0;
  for (int mem = 0; mem < g; ++mem, f0 += nb) {
    const int h = arg16(p.members, n * g + mem);
    // the lane's row index made opaque: its row addresses are formed here for
    // each member rather than held (in registers the walk needs) across the walk
    const int qm = (int)opaque((uint32_t)qc);
    bf16x8 q1f[NS], dof[NVS];
    {
      const __bf16* Q1 = (const __bf16*)p.q1 + b * p.sq1[0] + (int64_t)qm * p.sq1[1] + h * p.sq1[2];
      const __bf16* DO = (const __bf16*)p.dop + (((int64_t)b * N + qm) * p.Hs + h) * DV;
#pragma unroll
      for (int s = 0; s < NS; ++s) q1f[s] = *(const bf16x8*)(Q1 + 32 * s + 8 * jg);
#pragma unroll
      for (int s = 0; s < NVS; ++s) dof[s] = *(const bf16x8*)(DO + 32 * s + 8 * jg);
    }
    float4 rs = *(const float4*)(p.rowstat + 4 * (((int64_t)b * p.Hs + h) * N + qm));
    rs.w = __builtin_fmaf(sgn, rs.z, -rs.w);  // sgn (D1 - D2)
    rs.z = -rs.z;
    vm_drain();  // the member's operands (and the ring's blocks in flight) have landed
    f32x4 dq1[NDT];
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) dq1[ct] = f32x4{};

    int j = 0;
    for (; j < jfull; ++j) {
      sync(f0 + j);
      dq_block<false>(dq1, dq2, q1f, q2f, dof, rs, lds, L, sl, sc, sgn, j * kBK, kvis, jg);
      sl = next_slot(sl);
    }
    for (; j < nbw; ++j) {  // at most one: the block of the wavefront's diagonal or of key N - 1
      sync(f0 + j);
      dq_block<true>(dq1, dq2, q1f, q2f, dof, rs, lds, L, sl, sc, sgn, j * kBK, kvis, jg);
      sl = next_slot(sl);
    }
    for (; j < nb; ++j) {
      sync(f0 + j);
      sl = next_slot(sl);
    }
    const int qs = (int)opaque((uint32_t)q);
    if (qs < N)
      store_row16((__bf16*)p.gq1 + b * p.sgq1[0] + (int64_t)qs * p.sgq1[1] + h * p.sgq1[2], dq1, p.sm_scale, jg);
  }
  const int qs = (int)opaque((uint32_t)q);
  if (qs < N)
    store_row16((__bf16*)p.gq2 + b * p.sgq2[0] + (int64_t)qs * p.sgq2[1] + n * p.sgq2[2], dq2, p.sm_scale, jg);
}

// ---------------------------------------------------------------------------
// dK/dV pass: workgroup = (b, noise group n, 64 keys); slot = Q1 | Q2 | do | stats
// ---------------------------------------------------------------------------
constexpr int kKWaves = 4, kKThreads = 64 * kKWaves, kKRB = kKWaves * kRW;
constexpr int kKSlots = 3;
constexpr int RSOFF = 2 * KBLK + VBLK;           // row statistics: 32 x float4
constexpr int KSLOT = RSOFF + kBK * 16;          // 16.5 KiB
static_assert(QSLOT % 512 == 0 && KSLOT % 512 == 0 && KBLK % 256 == 0, "slot offsets keep the swizzle bits");
static_assert(kKSlots - 2 <= 4, "wait_blocks covers four blocks in flight");

// per-lane read offsets of step 0 / column tile 0 (others: XOR, as for DqLane)
struct DkvLane {
  uint32_t qr;    // Q rows
  uint32_t qt;    // Q^T
  uint32_t orow;  // do rows (do tensor offset included)
  uint32_t ot;    // do^T (do tensor offset included)
};

struct DkvAcc {
  f32x4 dk1[NDT], dk2[NDT], dv[NVT];
};

// One 32-query block in slot offset sb: S1, S2, dP (lane = key), the weights,
// dS and P1 - lambda P2, then dV^T += do^T (P1 - lambda P2), dK1^T += Q1^T dS1,
// dK2^T += Q2^T dS2.  Query qs0 + 16 t + 4 (l/16) + r is visible to the lane's
// key iff vd0 + 16 t + r < vrange (unsigned; vd0 = qs0 + 4 (l/16) - first
// visible query).
template <bool MASK>
__device__ __forceinline__ void dkv_block(DkvAcc& A, const bf16x8 (&kf1)[NS], const bf16x8 (&kf2)[NS],
                                          const bf16x8 (&vf)[NVS], const lds_u8* lds, const DkvLane& L,
                                          uint32_t sb, float sc, float sgn, int vd0, uint32_t vrange, int jg) {
  // product i of the first phase, 8 per 16-query half t = i / 8: S1 and S2 of
  // step 0, of step 1, then the four dP steps; each product's LDS operand is
  // read one product ahead (two reads in flight)
  f32x4 s1[2], s2[2], dp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) s1[t] = s2[t] = dp[t] = f32x4{};
  auto rop = [&](int i) -> bf16x8 {
    const int t = i >> 3, k = i & 7;
    if (k < 4) return lds_ld16(lds + ((sb + L.qr) ^ ((k >> 1) << 6)) + t * 16 * KROW + ((k & 1) ? KBLK : 0));
    return lds_ld16(lds + ((sb + L.orow) ^ ((k - 4) << 6)) + t * 16 * VROW);
  };
  bf16x8 rc = rop(0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bf16x8 rn;
    if (i + 1 < 16) rn = rop(i + 1);
    const int t = i >> 3, k = i & 7;
    if (k >= 4)
      dp[t] = mfma16(rc, vf[k - 4], dp[t]);
    else if (k & 1)
      s2[t] = mfma16(rc, kf2[k >> 1], s2[t]);
    else
      s1[t] = mfma16(rc, kf1[k >> 1], s1[t]);
    rc = rn;
  }
  // k order of the B operands: slots 0-3 = queries 4 (l/16) + r, slots 4-7 = + 16
  const lds_u8* rsb = lds + (sb + RSOFF + 64 * jg);
  bf16x8 bc, b1, b2;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 st = *(const __attribute__((address_space(3))) f32x4*)(rsb + 256 * t + 16 * r);
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[t][r], sc, -st[0]));
      float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[t][r], sc, -st[1]));  // |lambda| P2
      if (MASK) {
        const bool vis = (uint32_t)(vd0 + 16 * t + r) < vrange;
        p1 = vis ? p1 : 0.f;
        p2 = vis ? p2 : 0.f;
      }
      bc[4 * t + r] = (__bf16)__builtin_fmaf(sgn, p2, p1);
      b1[4 * t + r] = (__bf16)(p1 * (dp[t][r] - st[2]));
      b2[4 * t + r] = (__bf16)(p2 * __builtin_fmaf(sgn, dp[t][r], -st[3]));
    }
  // product i of the second phase: do^T column tiles 0-7 for dV, then Q1^T
  // (even) and Q2^T (odd) of column tiles 0-3 for dK1 and dK2, read one
  // product ahead
  auto top = [&](int i) -> bf16x8 {
    if (i < NVT) return rd_tr(lds + ((sb + L.ot) ^ (i << 5)), 16 * VROW);
    const int ct = (i - NVT) >> 1;
    return rd_tr(lds + ((sb + L.qt) ^ (ct << 5)) + ((i & 1) ? KBLK : 0), 16 * KROW);
  };
  bf16x8 tc = top(0);
#pragma unroll
  for (int i = 0; i < NVT + 2 * NDT; ++i) {
    bf16x8 tn;
    if (i + 1 < NVT + 2 * NDT) tn = top(i + 1);
    if (i < NVT)
      A.dv[i] = mfma16(tc, bc, A.dv[i]);
    else if (i & 1)
      A.dk2[(i - NVT) >> 1] = mfma16(tc, b2, A.dk2[(i - NVT) >> 1]);
    else
      A.dk1[(i - NVT) >> 1] = mfma16(tc, b1, A.dk1[(i - NVT) >> 1]);
    tc = tn;
  }
}

__global__ __launch_bounds__(kKThreads, 3) void bwd_dkv_ring_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[kKSlots * KSLOT];
  const lds_u8* lds = (const lds_u8*)lds_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;
  const int lane = threadIdx.x & 63, jg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int N = p.N, g = p.g;
  const int nk = (N + kKRB - 1) / kKRB;
  int t0, blk;
  bwd_item(xcd_logical(blockIdx.x, (int)gridDim.x), p.B * p.Hn, nk, t0, blk);
  const int kb = p.causal ? blk : nk - 1 - blk;  // causal: most queries first
  const int n = t0 % p.Hn, b = t0 / p.Hn;
  const int k0 = kb * kKRB, kw = k0 + wave * kRW, key = kw + (lane & 15), kc = min(key, N - 1);
  const float sgn = lambda_of(p.lam_dev, p.lam) > 0.f ? -1.f : 1.f;  // -lambda = sgn |lambda|
  const float sc = p.sm_scale_log2;
  const int nbq = (N + kBK - 1) / kBK;
  const int j0 = p.causal ? k0 / kBK : 0;  // first query block the workgroup walks
  const int nb = nbq - j0;                 // blocks per signal head
  // this wavefront: blocks [jlo, nbq) hold visible queries; the first is masked
  // in the causal case (the diagonal), the last when it holds query N - 1 and N
  // is not a multiple of 32
  const int jlo = kw >= N ? nbq : (p.causal ? kw / kBK : 0);
  const int jm0 = p.causal ? jlo + 1 : jlo;     // first unmasked block
  const int jm1 = (N % kBK) ? nbq - 1 : nbq;    // unmasked blocks end before this one
  const int vis_lo = p.causal ? key : 0;        // first query that sees this lane's key
  const uint32_t vrange = (uint32_t)(N - vis_lo);  // visible queries: [vis_lo, N)

  // ---- DMA of one block (32 queries): wave w loads Q1 rows 8w .., Q2 rows
  // 8w .., do rows 8w .. 8w + 7 (two KiB) and the statistics of rows 8w ..
  // 8w + 7 (lanes 0-7, 16 B each): five loads per block and wavefront, so the
  // ring waits are the same in every wavefront.  Rows past N re-read row
  // N - 1 (never visible).
  const uint32_t q1s = (uint32_t)p.sq1[1] * 2u, q2s = (uint32_t)p.sq2[1] * 2u;
  const uint32_t dos = (uint32_t)(p.Hs * DV) * 2u;  // do rows are dense [B][N][Hs][dv]
  const int qr0 = 8 * wave;
  constexpr int kRsRows = kBK / kKWaves;  // statistics rows per wavefront
  static_assert(kRsRows * kKWaves == kBK, "the statistics split evenly over the wavefronts");
  const uint32_t rs_dst = RSOFF + 16u * kRsRows * wave;
  const int F = g * nb;
  int im = 0, ij = j0;
  uint32_t idst = lds_base;
  const char *s_q1, *s_q2, *s_do, *s_rs;
  auto head_sources = [&]() {
    const int h = arg16(p.members, n * g + im);
    const int64_t r0 = (int64_t)j0 * kBK;
    s_q1 = (const char*)((const __bf16*)p.q1 + b * p.sq1[0] + r0 * p.sq1[1] + h * p.sq1[2]);
    s_q2 = (const char*)((const __bf16*)p.q2 + b * p.sq2[0] + r0 * p.sq2[1] + n * p.sq2[2]);
    s_do = (const char*)((const __bf16*)p.dop + (((int64_t)b * N + r0) * p.Hs + h) * DV);
    s_rs = (const char*)(p.rowstat + 4 * (((int64_t)b * p.Hs + h) * N + r0));
  };
  head_sources();
  const uint32_t o_q1 = src_off(lane, qr0, false, q1s, kBK), o_q2 = src_off(lane, qr0, false, q2s, kBK);
  const uint32_t o_d0 = src_off(lane, qr0, true, dos, kBK), o_d1 = src_off(lane, qr0 + 4, true, dos, kBK);
  auto issue = [&]() {
    const uint32_t dst = idst;
    if (ij * kBK + kBK <= N) {
      dma16(s_q1, o_q1, dst + wave * 1024);
      dma16(s_q2, o_q2, dst + KBLK + wave * 1024);
      dma16(s_do, o_d0, dst + 2 * KBLK + 2 * wave * 1024);
      dma16(s_do, o_d1, dst + 2 * KBLK + (2 * wave + 1) * 1024);
      if (lane < kRsRows) dma16(s_rs, (uint32_t)(kRsRows * wave + lane) * 16u, dst + rs_dst);
    } else {  // the block that holds row N - 1
      const int lim = N - 1 - ij * kBK;
      dma16(s_q1, src_off(lane, qr0, false, q1s, lim), dst + wave * 1024);
      dma16(s_q2, src_off(lane, qr0, false, q2s, lim), dst + KBLK + wave * 1024);
      dma16(s_do, src_off(lane, qr0, true, dos, lim), dst + 2 * KBLK + 2 * wave * 1024);
      dma16(s_do, src_off(lane, qr0 + 4, true, dos, lim), dst + 2 * KBLK + (2 * wave + 1) * 1024);
      if (lane < kRsRows) dma16(s_rs, (uint32_t)min(kRsRows * wave + lane, lim) * 16u, dst + rs_dst);
    }
    s_q1 += (size_t)kBK * q1s;
    s_q2 += (size_t)kBK * q2s;
    s_do += (size_t)kBK * dos;
    s_rs += kBK * 16;
    if (++ij == nbq) {
      ij = j0;
      if (++im < g) head_sources();
    }
    idst = idst == lds_base + (kKSlots - 1) * KSLOT ? lds_base : idst + KSLOT;
  };
  auto sync = [&](int f) {
    wait_blocks<5, kKSlots - 2>(min(F - 1, f + kKSlots - 2) - f);
    wait_lds_and_barrier();
    if (f + kKSlots - 1 < F) issue();
  };
  auto next_slot = [](uint32_t sl) { return sl == (kKSlots - 1) * KSLOT ? 0u : sl + KSLOT; };

  DkvLane L;
  L.qr = row_off(lane, 0, KROW, false);
  L.qt = tr_off(lane, 0, KROW, false);
  L.orow = 2 * KBLK + row_off(lane, 0, VROW, true);
  L.ot = 2 * KBLK + tr_off(lane, 0, VROW, true);

  for (int t = 0; t < min(F, kKSlots - 1); ++t) issue();  // blocks 0 .. kKSlots - 2

  // key-side operands: K2 of the noise head, K1 and V of the run's key/value head
  bf16x8 kf2[NS], kf1[NS], vf[NVS];
  auto load_kv = [&](int kh) {
    const int km = (int)opaque((uint32_t)kc);  // row address formed here, not held across the walk
    const __bf16* K1 = (const __bf16*)p.k1 + b * p.sk1[0] + (int64_t)km * p.sk1[1] + kh * p.sk1[2];
    const __bf16* V = (const __bf16*)p.v + b * p.sv[0] + (int64_t)km * p.sv[1] + kh * p.sv[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) kf1[s] = *(const bf16x8*)(K1 + 32 * s + 8 * jg);
#pragma unroll
    for (int s = 0; s < NVS; ++s) vf[s] = *(const bf16x8*)(V + 32 * s + 8 * jg);
  };
  {
    const __bf16* K2 = (const __bf16*)p.k2 + b * p.sk2[0] + (int64_t)kc * p.sk2[1] + n * p.sk2[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) kf2[s] = *(const bf16x8*)(K2 + 32 * s + 8 * jg);
  }
  int cur = arg16(p.kv, arg16(p.members, n * g));  // key/value head of the accumulating run
  load_kv(cur);
  vm_drain();
  DkvAcc A;
#pragma unroll
  for (int ct = 0; ct < NDT; ++ct) A.dk2[ct] = A.dk1[ct] = f32x4{};
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) A.dv[vt] = f32x4{};

  uint32_t sl = 0;  // slot offset of the next block walked
  int f0 = 0;
  for (int mem = 0; mem < g; ++mem, f0 += nb) {
    const int kh = arg16(p.kv, arg16(p.members, n * g + mem));
    if (kh != cur) {
      const int ks = (int)opaque((uint32_t)key);
      if (ks < N) {
        store_row16((__bf16*)p.gk1 + b * p.sgk1[0] + (int64_t)ks * p.sgk1[1] + cur * p.sgk1[2], A.dk1, p.sm_scale,
                    jg);
        store_row16((__bf16*)p.gv + b * p.sgv[0] + (int64_t)ks * p.sgv[1] + cur * p.sgv[2], A.dv, 1.0f, jg);
      }
#pragma unroll
      for (int ct = 0; ct < NDT; ++ct) A.dk1[ct] = f32x4{};
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) A.dv[vt] = f32x4{};
      cur = kh;
      load_kv(kh);
      vm_drain();
    }
    // ring block f0 + i is query block j0 + i of this head
    int j = j0;
    auto walk = [&](auto mask, int jend) {
      for (; j < jend; ++j) {
        sync(f0 + j - j0);
        dkv_block<decltype(mask)::value>(A, kf1, kf2, vf, lds, L, sl, sc, sgn, j * kBK + 4 * jg - vis_lo, vrange,
                                         jg);
        sl = next_slot(sl);
      }
    };
    for (; j < jlo; ++j) {  // blocks before this wavefront's keys: no visible query
      sync(f0 + j - j0);
      sl = next_slot(sl);
    }
    walk(std::true_type{}, min(jm0, nbq));
    walk(std::false_type{}, max(jm1, j));
    walk(std::true_type{}, nbq);
  }
  const int ks = (int)opaque((uint32_t)key);
  if (ks < N) {
    store_row16((__bf16*)p.gk1 + b * p.sgk1[0] + (int64_t)ks * p.sgk1[1] + cur * p.sgk1[2], A.dk1, p.sm_scale, jg);
    store_row16((__bf16*)p.gv + b * p.sgv[0] + (int64_t)ks * p.sgv[1] + cur * p.sgv[2], A.dv, 1.0f, jg);
    store_row16((__bf16*)p.gk2 + b * p.sgk2[0] + (int64_t)ks * p.sgk2[1] + n * p.sgk2[2], A.dk2, p.sm_scale, jg);
  }
}

}  // namespace

bool bwd_ring_applies(const BwdParams& p) { return p.d == D && p.dv == DV; }

hipError_t launch_bwd_ring_bf16(const BwdParams& p, hipStream_t s) {
  const int64_t gq = (int64_t)p.B * p.Hn * ((p.N + kQRB - 1) / kQRB);
  const int64_t gk = (int64_t)p.B * p.Hn * ((p.N + kKRB - 1) / kKRB);
  if (!bwd_ring_applies(p) || gq > INT32_MAX || gk > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_ring_kernel, dim3((unsigned)gq), dim3(kQThreads), 0, s, p);
  hipLaunchKernelGGL(bwd_dkv_ring_kernel, dim3((unsigned)gk), dim3(kKThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace da

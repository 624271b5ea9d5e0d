// C-ABI layer of libdiffattn.so: argument validation (pure host code, run
// before any HIP call), head-map resolution and kernel dispatch.
//
// The operations and their arguments follow "Differential Attention in Large
// Language Models: How Denoising Subtraction Eliminates Attention Noise and
// Outlier Activations" (llms.blog), sections "Differential Attention
// Architecture" (Q1/Q2, K1/K2 of width d, V of width 2d, the DiffAttn
// equation), "Learnable Lambda Re-parameterization" and "Headwise
// Normalization", and the head grouping of "Grouped Differential Attention"
// (mlsanity.com), "Abstract".
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

da_status fail(da_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
da_status fail(da_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

da_status hip_fail(hipError_t e, const char* what) {
  return fail(DA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Byte extent [lo, hi) of a strided tensor whose last dim is contiguous.
struct Extent {
  uintptr_t lo, hi;
};

Extent extent(const void* p, const int64_t* dims, const int64_t* strides, int nlead, int64_t last, int esize) {
  int64_t maxoff = last - 1;
  for (int i = 0; i < nlead; ++i) maxoff += (dims[i] - 1) * strides[i];
  return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)((maxoff + 1) * esize)};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

// A strided [B, N, heads, last] view (last dim contiguous, strides of (b, n, head) in elements).
struct View {
  const void* p;
  int64_t dims[3];
  const int64_t* s;
  int64_t last;
  int es;
};

// Whether two views may share a byte.  Disjoint byte extents never do.  Nor do
// two views that repeat with the same token stride (batch strides multiples
// of it) when their footprints within one token row -- heads and channels --
// are disjoint intervals modulo that stride: the interleaved views of one
// packed buffer, e.g. the projections of a fused QKV layer and their
// gradients.  Otherwise they are taken to overlap.
bool views_overlap(const View& x, const View& y) {
  if (!overlaps(extent(x.p, x.dims, x.s, 3, x.last, x.es), extent(y.p, y.dims, y.s, 3, y.last, y.es))) return false;
  const int64_t ts = x.s[1];
  if (x.es != y.es || ts <= 0 || y.s[1] != ts) return true;
  if ((x.dims[0] > 1 && x.s[0] % ts) || (y.dims[0] > 1 && y.s[0] % ts)) return true;
  const int64_t R = ts * x.es;  // bytes per token row
  const int64_t fx = ((x.dims[2] - 1) * x.s[2] + x.last) * x.es, fy = ((y.dims[2] - 1) * y.s[2] + y.last) * y.es;
  if (fx > R || fy > R) return true;
  const int64_t x0 = (int64_t)((uintptr_t)x.p % (uint64_t)R), y0 = (int64_t)((uintptr_t)y.p % (uint64_t)R);
  return !(((y0 - x0 + R) % R) >= fx && ((x0 - y0 + R) % R) >= fy);
}

da_status check_strides(const char* name, const void* p, const int64_t* s, int n, int esize) {
  if (!p) return fail(DA_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(DA_EINVAL, "%s is not 16-byte aligned", name);
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(DA_EINVAL, "%s has a negative stride", name);
    if ((s[i] * esize) % 16 != 0) return fail(DA_EINVAL, "%s stride %d (%lld elements) is not a multiple of 16 bytes",
                                              name, i, (long long)s[i]);
  }
  return DA_OK;
}

// Resolve and check the head maps.  Each noise head must serve exactly g
// signal heads and each kv head exactly H_s/H_kv (GQA-style repetition).
da_status resolve_maps(int Hs, int Hn, int Hkv, const int32_t* nzmap, const int32_t* kvmap, int16_t* nz,
                       int16_t* kv, int16_t* members) {
  const int g = Hs / Hn, gk = Hs / Hkv;
  int cnt_n[DA_MAX_HEADS] = {0}, cnt_k[DA_MAX_HEADS] = {0};
  for (int h = 0; h < Hs; ++h) {
    int n = nzmap ? nzmap[h] : h / g;
    int k = kvmap ? kvmap[h] : h / gk;
    if (n < 0 || n >= Hn) return fail(DA_EINVAL, "noise_of_signal[%d] = %d out of [0, %d)", h, n, Hn);
    if (k < 0 || k >= Hkv) return fail(DA_EINVAL, "kv_of_signal[%d] = %d out of [0, %d)", h, k, Hkv);
    nz[h] = (int16_t)n;
    kv[h] = (int16_t)k;
    cnt_n[n]++;
    cnt_k[k]++;
  }
  for (int n = 0; n < Hn; ++n)
    if (cnt_n[n] != g) return fail(DA_EINVAL, "noise head %d serves %d signal heads, expected %d", n, cnt_n[n], g);
  for (int k = 0; k < Hkv; ++k)
    if (cnt_k[k] != gk) return fail(DA_EINVAL, "kv head %d serves %d signal heads, expected %d", k, cnt_k[k], gk);
  int fill[DA_MAX_HEADS] = {0};
  for (int h = 0; h < Hs; ++h) {
    int n = nz[h];
    members[n * g + fill[n]++] = (int16_t)h;
  }
  return DA_OK;
}

da_status check_common_shapes(int64_t B, int64_t N, int64_t Hs, int64_t Hn, int64_t Hkv, int64_t d, int64_t dv,
                              int32_t dtype, float lam, float lam_init, float eps) {
  if (dtype != DA_F32 && dtype != DA_BF16) return fail(DA_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 0 || N < 0) return fail(DA_EINVAL, "negative batch or length");
  if (B > INT32_MAX || N > INT32_MAX) return fail(DA_EINVAL, "batch or length exceeds int32");
  if (Hs < 1 || Hn < 1 || Hkv < 1) return fail(DA_EINVAL, "head counts must be >= 1");
  if (Hs > DA_MAX_HEADS) return fail(DA_EINVAL, "H_s = %lld exceeds %d", (long long)Hs, DA_MAX_HEADS);
  if (Hs % Hn != 0) return fail(DA_EINVAL, "H_s (%lld) is not a multiple of H_n (%lld)", (long long)Hs, (long long)Hn);
  if (Hs % Hkv != 0)
    return fail(DA_EINVAL, "H_s (%lld) is not a multiple of H_kv (%lld)", (long long)Hs, (long long)Hkv);
  if (dv != 2 * d) return fail(DA_EINVAL, "dv (%lld) must equal 2*d (d = %lld)", (long long)dv, (long long)d);
  if (d != 32 && d != 64) return fail(DA_EUNSUPPORTED, "d = %lld: kernels exist for d in {32, 64}", (long long)d);
  if (!isfinite(lam) || !isfinite(lam_init)) return fail(DA_EINVAL, "lambda and lambda_init must be finite");
  // eps > 0 keeps the head norm finite on rows whose difference is exactly zero
  // (identical maps with lambda = 1 give o = 0, and 0 / sqrt(0 + eps) = 0)
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(DA_EINVAL, "eps must be finite and > 0");
  return DA_OK;
}

// Packed sequences of the varlen entry point (cu == nullptr: fixed-length batch).
struct Packing {
  const int32_t* cu;
  int64_t nseq, max_seqlen;
};

constexpr int kMaxGridYZ = 65535;  // grid y/z limit of the fp32 kernel's and the decode's launches
// bf16 prefill: a tile or query block spans at most 128 rows; their byte offsets
// from the block's first row (row x stride x 2 + the 256-byte row) stay below 2^32
constexpr int64_t kMaxTileRows = 128;
constexpr int64_t kMaxTokenStride = (((int64_t)1 << 32) - 256) / (2 * kMaxTileRows);

da_status fwd_impl(const da_fwd_args* a, void* stream, bool plain, const Packing* pk = nullptr) {
  if (!a) return fail(DA_EINVAL, "args is NULL");
  da_status st = check_common_shapes(a->B, a->N, a->H_s, a->H_n, a->H_kv, a->d, a->dv, a->dtype, a->lambda,
                                     a->lambda_init, a->eps);
  if (st != DA_OK) return st;
  if (pk) {
    if (a->B != 1) return fail(DA_EINVAL, "packed sequences need B == 1 (got %lld)", (long long)a->B);
    if (pk->nseq < 0 || pk->nseq > INT32_MAX) return fail(DA_EINVAL, "nseq = %lld out of range", (long long)pk->nseq);
    if (pk->max_seqlen < 0 || pk->max_seqlen > a->N)
      return fail(DA_EINVAL, "max_seqlen = %lld outside [0, N = %lld]", (long long)pk->max_seqlen, (long long)a->N);
    if (pk->nseq > 0 && !pk->cu) return fail(DA_EINVAL, "cu_seqlens is NULL");
    if (pk->cu && ((uintptr_t)pk->cu & 3u)) return fail(DA_EINVAL, "cu_seqlens is not 4-byte aligned");
  }
  const int64_t nseq = pk ? pk->nseq : a->B, max_seqlen = pk ? pk->max_seqlen : a->N;
  if (a->dtype == DA_F32 && nseq > kMaxGridYZ)
    return fail(DA_EUNSUPPORTED, "the fp32 kernel takes at most %d sequences per call", kMaxGridYZ);
  if (a->flags & ~(uint32_t)(DA_CAUSAL | DA_NO_NORM)) return fail(DA_EINVAL, "unknown flag bits 0x%x", a->flags);
  if (plain) {
    if (a->H_n != a->H_s || a->H_kv != a->H_s)
      return fail(DA_EINVAL, "diffattn_fwd needs H_n == H_kv == H_s (use gda_fwd for grouped heads)");
    if (a->noise_of_signal || a->kv_of_signal) return fail(DA_EINVAL, "diffattn_fwd takes no head maps");
  }
  da::FwdParams p;
  memset(&p, 0, sizeof p);
  if ((st = resolve_maps((int)a->H_s, (int)a->H_n, (int)a->H_kv, a->noise_of_signal, a->kv_of_signal, p.nz, p.kv,
                         p.members)) != DA_OK)
    return st;
  if (a->B == 0 || a->N == 0 || nseq == 0 || max_seqlen == 0)
    return DA_OK;  // empty: no pointer is touched (torch gives NULL for empty tensors)

  const int es = a->dtype == DA_BF16 ? 2 : 4;
  struct T {
    const char* name;
    const void* p;
    const int64_t* s;
    int64_t heads, last;
  } ts[6] = {{"q1", a->q1, a->s_q1, a->H_s, a->d},   {"q2", a->q2, a->s_q2, a->H_n, a->d},
             {"k1", a->k1, a->s_k1, a->H_kv, a->d},  {"k2", a->k2, a->s_k2, a->H_n, a->d},
             {"v", a->v, a->s_v, a->H_kv, a->dv},    {"out", a->out, a->s_out, a->H_s, a->dv}};
  for (auto& t : ts)
    if ((st = check_strides(t.name, t.p, t.s, 3, es)) != DA_OK) return st;
  if (a->dtype == DA_BF16) {
    // the bf16 kernels address the rows of one tile or query block (at most
    // kMaxTileRows rows) from a 64-bit base with 32-bit per-lane byte offsets
    for (int i = 0; i < 5; ++i)
      if (ts[i].s[1] > kMaxTokenStride)
        return fail(DA_EUNSUPPORTED, "%s token stride %lld exceeds %lld elements", ts[i].name,
                    (long long)ts[i].s[1], (long long)kMaxTokenStride);
  }
  if (a->norm_w && ((uintptr_t)a->norm_w & 3u)) return fail(DA_EINVAL, "norm_w is not 4-byte aligned");
  if (a->lse && ((uintptr_t)a->lse & 3u)) return fail(DA_EINVAL, "lse is not 4-byte aligned");
  if (a->o_maps && !aligned16(a->o_maps)) return fail(DA_EINVAL, "o_maps is not 16-byte aligned");

  Extent eo;
  {
    int64_t dims[3] = {a->B, a->N, a->H_s};
    eo = extent(a->out, dims, a->s_out, 3, a->dv, es);
  }
  const View vo{a->out, {a->B, a->N, a->H_s}, a->s_out, a->dv, es};
  for (int i = 0; i < 5; ++i)
    if (views_overlap(vo, View{ts[i].p, {a->B, a->N, ts[i].heads}, ts[i].s, ts[i].last, es}))
      return fail(DA_EINVAL, "out overlaps %s", ts[i].name);
  if (a->lse) {
    Extent el{(uintptr_t)a->lse, (uintptr_t)(a->lse + 2 * a->B * a->H_s * a->N)};
    if (overlaps(el, eo)) return fail(DA_EINVAL, "lse overlaps out");
    for (int i = 0; i < 5; ++i) {
      int64_t dims[3] = {a->B, a->N, ts[i].heads};
      if (overlaps(el, extent(ts[i].p, dims, ts[i].s, 3, ts[i].last, es)))
        return fail(DA_EINVAL, "lse overlaps %s", ts[i].name);
    }
  }
  if (a->o_maps) {
    const uintptr_t lo = (uintptr_t)a->o_maps;
    Extent em{lo, lo + (uintptr_t)(2 * a->B * a->N * a->H_s * a->dv * 4)};
    if (overlaps(em, eo)) return fail(DA_EINVAL, "o_maps overlaps out");
    if (a->lse && overlaps(em, Extent{(uintptr_t)a->lse, (uintptr_t)(a->lse + 2 * a->B * a->H_s * a->N)}))
      return fail(DA_EINVAL, "o_maps overlaps lse");
    for (int i = 0; i < 5; ++i) {
      int64_t dims[3] = {a->B, a->N, ts[i].heads};
      if (overlaps(em, extent(ts[i].p, dims, ts[i].s, 3, ts[i].last, es)))
        return fail(DA_EINVAL, "o_maps overlaps %s", ts[i].name);
    }
  }

  p.q1 = a->q1;
  p.q2 = a->q2;
  p.k1 = a->k1;
  p.k2 = a->k2;
  p.v = a->v;
  p.out = a->out;
  p.norm_w = a->norm_w;
  p.lse = a->lse;
  p.o_maps = (float*)a->o_maps;
  p.lam_dev = a->lambda_dev;
  p.cu_seqlens = pk ? pk->cu : nullptr;
  p.nseq = (int)nseq;
  p.max_seqlen = (int)max_seqlen;
  for (int i = 0; i < 3; ++i) {
    p.sq1[i] = a->s_q1[i];
    p.sq2[i] = a->s_q2[i];
    p.sk1[i] = a->s_k1[i];
    p.sk2[i] = a->s_k2[i];
    p.sv[i] = a->s_v[i];
    p.so[i] = a->s_out[i];
  }
  p.B = (int)a->B;
  p.N = (int)a->N;
  p.Hs = (int)a->H_s;
  p.Hn = (int)a->H_n;
  p.Hkv = (int)a->H_kv;
  p.d = (int)a->d;
  p.dv = (int)a->dv;
  p.g = (int)(a->H_s / a->H_n);
  p.causal = (a->flags & DA_CAUSAL) ? 1 : 0;
  p.normalize = (a->flags & DA_NO_NORM) ? 0 : 1;
  p.lam = a->lambda;
  p.lam_init = a->lambda_init;
  p.eps = a->eps;
  p.sm_scale = (float)(1.0 / sqrt((double)a->d));
  p.sm_scale_log2 = (float)(1.4426950408889634 / sqrt((double)a->d));

  hipError_t e;
  if (a->dtype == DA_BF16)
    e = da::shared_kv_plan(p)    ? da::launch_fwd_shared_bf16(p, (hipStream_t)stream)
        : da::gda3_applies(p)    ? da::launch_fwd_gda3_bf16(p, (hipStream_t)stream)
                                 : da::launch_fwd_bf16(p, (hipStream_t)stream);
  else
    e = da::launch_fwd_f32(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return DA_OK;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// default split: about kDefaultPartials partial workgroups (a little over three rounds of
// the ~768 that run at once, 3 per CU; measured on 64 sequences of 4096..8192 positions,
// where 2048 partials leave the last round a third full), with the split between one
// sub-chunk and kMaxChunk positions
constexpr int64_t kDefaultPartials = 2560;
constexpr int kChunkQuantum = 128;  // positions per decode sub-chunk
constexpr int kMaxChunk = 2048;
constexpr int kDecodeMaxQueries = 8;  // g + 1 scored queries per noise group
constexpr int kDecodeMaxOutputs = 8;  // g + u outputs per noise group (u: its distinct key/value heads)
constexpr int64_t kMaxPosStride = 1 << 19;  // elements; 2048 positions x 2 B x 2^19 < 2^31

da_status decode_prepare(const da_decode_args* a, da::DecodeParams* p, bool check_pointers) {
  memset(p, 0, sizeof *p);  // B == 0 exits early with an all-zero (empty) parameter block
  if (!a) return fail(DA_EINVAL, "args is NULL");
  da_status st = check_common_shapes(a->B, a->Lmax, a->H_s, a->H_n, a->H_kv, a->d, a->dv, a->dtype, a->lambda,
                                     a->lambda_init, a->eps);
  if (st != DA_OK) return st;
  if (a->dtype != DA_BF16) return fail(DA_EUNSUPPORTED, "gda_decode has a bf16 kernel only");
  const bool fp8 = a->cache_dtype == DA_FP8_E4M3;
  if (fp8) {
    const float sc[3] = {a->k1_scale, a->k2_scale, a->v_scale};
    for (float x : sc)
      if (!(x > 0.0f) || !isfinite(x)) return fail(DA_EINVAL, "fp8 cache scales must be finite and > 0");
  }
  if (a->d != 64) return fail(DA_EUNSUPPORTED, "gda_decode has a d = 64 kernel only");
  if (a->flags & ~(uint32_t)DA_NO_NORM) return fail(DA_EINVAL, "gda_decode accepts only DA_NO_NORM");
  if (a->chunk < 0 || a->chunk % kChunkQuantum != 0)
    return fail(DA_EINVAL, "chunk must be 0 or a positive multiple of %d", kChunkQuantum);
  if (a->chunk > kMaxChunk) return fail(DA_EUNSUPPORTED, "chunk %lld exceeds %d", (long long)a->chunk, kMaxChunk);
  if (a->H_s / a->H_n + 1 > kDecodeMaxQueries)
    return fail(DA_EUNSUPPORTED, "gda_decode supports up to %d signal heads per noise head", kDecodeMaxQueries - 1);
  if (a->B == 0) return DA_OK;  // empty batch: nothing is validated further or touched
  if (a->B > kMaxGridYZ)  // the batch is a grid dimension of both decode kernels
    return fail(DA_EUNSUPPORTED, "gda_decode takes at most %d sequences per call", kMaxGridYZ);
  // the partial kernel addresses a chunk's rows with 32-bit byte offsets
  if (a->s_k1[2] > kMaxPosStride || a->s_k2[2] > kMaxPosStride || a->s_v[2] > kMaxPosStride)
    return fail(DA_EUNSUPPORTED, "cache position stride exceeds %d elements", kMaxPosStride);
  const int es = 2, ces = fp8 ? 1 : 2;  // element bytes of queries / output, of the caches
  struct T {
    const char* name;
    const void* p;
    const int64_t* s;
    int nlead, es;
  } ts[6] = {{"q1", a->q1, a->s_q1, 2, es},         {"q2", a->q2, a->s_q2, 2, es},
             {"k1_cache", a->k1_cache, a->s_k1, 3, ces}, {"k2_cache", a->k2_cache, a->s_k2, 3, ces},
             {"v_cache", a->v_cache, a->s_v, 3, ces},    {"out", a->out, a->s_out, 2, es}};
  if (check_pointers) {
    for (auto& t : ts)
      if ((st = check_strides(t.name, t.p, t.s, t.nlead, t.es)) != DA_OK) return st;
    if (!a->seq_lens) return fail(DA_EINVAL, "seq_lens is NULL");
    if ((uintptr_t)a->seq_lens & 3u) return fail(DA_EINVAL, "seq_lens is not 4-byte aligned");
    if (a->norm_w && ((uintptr_t)a->norm_w & 3u)) return fail(DA_EINVAL, "norm_w is not 4-byte aligned");
  }

  int16_t nz[DA_MAX_HEADS];
  if ((st = resolve_maps((int)a->H_s, (int)a->H_n, (int)a->H_kv, a->noise_of_signal, a->kv_of_signal, nz, p->kv,
                         p->members)) != DA_OK)
    return st;
  const int Hs = (int)a->H_s, Hn = (int)a->H_n, g = Hs / Hn;
  int umax = 0;
  for (int n = 0; n < Hn; ++n) {
    int u = 0;
    for (int j = 0; j < g; ++j) {
      int h = p->members[n * g + j];
      int k = p->kv[h], idx = -1;
      for (int t = 0; t < u; ++t)
        if (p->ukv[n * g + t] == k) idx = t;
      if (idx < 0) {
        idx = u;
        p->ukv[n * g + u++] = (int16_t)k;
      }
      p->uidx[h] = (int16_t)idx;
    }
    p->nu[n] = (int16_t)u;
    umax = std::max(umax, u);
  }
  if (g + umax > kDecodeMaxOutputs)
    return fail(DA_EUNSUPPORTED,
                "gda_decode keeps at most %d outputs per noise group: its %d signal heads plus the %d distinct "
                "key/value heads they read",
                kDecodeMaxOutputs, g, umax);
  // fp8 caches are walked in sub-chunks of 2 x 128 positions
  const int64_t quantum = fp8 ? 2 * kChunkQuantum : kChunkQuantum;
  if (a->block_table) {  // paged caches: every sub-chunk inside one block
    if (a->block_size < quantum || a->block_size % quantum != 0 || a->block_size > INT32_MAX)
      return fail(DA_EUNSUPPORTED, "block_size %lld: paged caches need a multiple of %lld positions",
                  (long long)a->block_size, (long long)quantum);
    if (a->max_blocks < 1 || a->num_blocks < 1 || a->max_blocks > INT32_MAX || a->num_blocks > INT32_MAX)
      return fail(DA_EINVAL, "max_blocks and num_blocks must be in [1, 2^31)");
    if (a->Lmax > a->max_blocks * a->block_size)
      return fail(DA_EINVAL, "Lmax %lld exceeds max_blocks x block_size", (long long)a->Lmax);
    if (check_pointers && ((uintptr_t)a->block_table & 3u))
      return fail(DA_EINVAL, "block_table is not 4-byte aligned");
  }
  if (a->chunk % quantum != 0)
    return fail(DA_EINVAL, "chunk must be 0 or a positive multiple of %lld for these caches", (long long)quantum);
  int64_t chunk = a->chunk;
  if (!chunk) {  // partials of B x H_n x (Lmax / chunk) ~ kDefaultPartials, rounded up to the quantum
    // (128-bit: B and Lmax may each reach 2^31)
    const __int128 work = (__int128)a->B * a->H_n * a->Lmax;
    const __int128 c = (work / kDefaultPartials + quantum - 1) / quantum * quantum;
    chunk = (int64_t)std::min<__int128>(std::max<__int128>(c, quantum), kMaxChunk);
  }
  int64_t lmax_r = (a->Lmax + quantum - 1) / quantum * quantum;
  if (chunk > lmax_r) chunk = std::max<int64_t>(quantum, lmax_r);
  p->chunk = (int)chunk;
  p->nchunks = (int)((a->Lmax + chunk - 1) / chunk);
  p->slots = g + umax;
  {  // the workspace size must be representable (sizes near the int32 limits would wrap it)
    const __int128 ws = (__int128)a->B * a->H_n * p->nchunks *
                        (__int128)da::decode_ws_floats_per_chunk(p->slots, (int)a->dv) * (__int128)sizeof(float);
    if (ws > ((__int128)1 << 62)) return fail(DA_EINVAL, "the decode workspace for these shapes exceeds 2^62 bytes");
  }
  p->q1 = a->q1;
  p->q2 = a->q2;
  p->k1 = a->k1_cache;
  p->k2 = a->k2_cache;
  p->v = a->v_cache;
  p->seq_lens = a->seq_lens;
  p->lam_dev = a->lambda_dev;
  p->out = a->out;
  p->norm_w = a->norm_w;
  for (int i = 0; i < 2; ++i) {
    p->sq1[i] = a->s_q1[i];
    p->sq2[i] = a->s_q2[i];
    p->so[i] = a->s_out[i];
  }
  for (int i = 0; i < 3; ++i) {
    p->sk1[i] = a->s_k1[i];
    p->sk2[i] = a->s_k2[i];
    p->sv[i] = a->s_v[i];
  }
  p->B = (int)a->B;
  p->Lmax = (int)a->Lmax;
  p->Hs = Hs;
  p->Hn = Hn;
  p->Hkv = (int)a->H_kv;
  p->d = (int)a->d;
  p->dv = (int)a->dv;
  p->g = g;
  p->fp8 = fp8 ? 1 : 0;
  p->block_table = a->block_table;
  p->block_size = a->block_table ? (int)a->block_size : 0;
  p->max_blocks = a->block_table ? (int)a->max_blocks : 0;
  p->num_blocks = a->block_table ? (int)a->num_blocks : 0;
  p->k1_scale = fp8 ? a->k1_scale : 1.0f;
  p->k2_scale = fp8 ? a->k2_scale : 1.0f;
  p->v_scale = fp8 ? a->v_scale : 1.0f;
  p->normalize = (a->flags & DA_NO_NORM) ? 0 : 1;
  p->lam = a->lambda;
  p->lam_init = a->lambda_init;
  p->eps = a->eps;
  p->sm_scale_log2 = (float)(1.4426950408889634 / sqrt((double)a->d));
  return DA_OK;
}

size_t decode_ws_bytes(const da::DecodeParams& p) {
  return (size_t)p.B * p.Hn * p.nchunks * da::decode_ws_floats_per_chunk(p.slots, p.dv) * sizeof(float);
}

// The decode's outputs (out, and the workspace when given) must not overlap
// its inputs or each other.
da_status decode_check_overlap(const da_decode_args* a, const void* ws, size_t ws_bytes) {
  const bool fp8 = a->cache_dtype == DA_FP8_E4M3;
  const int ces = fp8 ? 1 : 2;
  const bool paged = a->block_table != nullptr;
  auto cache = [&](const void* p, const int64_t* s, int64_t heads, int64_t width) {
    int64_t dims[3] = {paged ? a->num_blocks : a->B, heads, paged ? a->block_size : a->Lmax};
    return extent(p, dims, s, 3, width, ces);
  };
  int64_t dq1[2] = {a->B, a->H_s}, dq2[2] = {a->B, a->H_n}, dout[2] = {a->B, a->H_s};
  const Extent in[8] = {extent(a->q1, dq1, a->s_q1, 2, a->d, 2),
                        extent(a->q2, dq2, a->s_q2, 2, a->d, 2),
                        cache(a->k1_cache, a->s_k1, a->H_kv, a->d),
                        cache(a->k2_cache, a->s_k2, a->H_n, a->d),
                        cache(a->v_cache, a->s_v, a->H_kv, a->dv),
                        {(uintptr_t)a->seq_lens, (uintptr_t)(a->seq_lens + a->B)},
                        {(uintptr_t)a->norm_w, (uintptr_t)(a->norm_w ? a->norm_w + a->dv : a->norm_w)},
                        {(uintptr_t)a->block_table,
                         (uintptr_t)(paged ? a->block_table + a->B * a->max_blocks : a->block_table)}};
  const char* names[8] = {"q1", "q2", "k1_cache", "k2_cache", "v_cache", "seq_lens", "norm_w", "block_table"};
  const Extent eo = extent(a->out, dout, a->s_out, 2, a->dv, 2);
  const Extent ew{(uintptr_t)ws, (uintptr_t)ws + (ws ? ws_bytes : 0)};
  for (int i = 0; i < 8; ++i) {
    if (overlaps(eo, in[i])) return fail(DA_EINVAL, "out overlaps %s", names[i]);
    if (ws && overlaps(ew, in[i])) return fail(DA_EINVAL, "workspace overlaps %s", names[i]);
  }
  if (a->lambda_dev) {
    const Extent el{(uintptr_t)a->lambda_dev, (uintptr_t)(a->lambda_dev + 1)};
    if (overlaps(eo, el)) return fail(DA_EINVAL, "out overlaps lambda_dev");
    if (ws && overlaps(ew, el)) return fail(DA_EINVAL, "workspace overlaps lambda_dev");
  }
  if (ws && overlaps(ew, eo)) return fail(DA_EINVAL, "workspace overlaps out");
  return DA_OK;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t dop, rowstat, partial, total;
};

BwdLayout bwd_layout(const da::BwdParams& p, int es) {
  BwdLayout l;
  l.dop = 0;
  l.rowstat = round256((size_t)p.B * p.N * p.Hs * p.dv * es);
  l.partial = l.rowstat + round256((size_t)p.B * p.Hs * p.N * 16);
  l.total = l.partial + round256((size_t)p.nprep * (1 + p.dv) * 8);
  return l;
}

da_status bwd_prepare(const da_bwd_args* a, da::BwdParams* p, bool check_pointers) {
  memset(p, 0, sizeof *p);
  if (!a) return fail(DA_EINVAL, "args is NULL");
  da_status st = check_common_shapes(a->B, a->N, a->H_s, a->H_n, a->H_kv, a->d, a->dv, a->dtype, a->lambda,
                                     a->lambda_init, a->eps);
  if (st != DA_OK) return st;
  if (a->flags & ~(uint32_t)(DA_CAUSAL | DA_NO_NORM)) return fail(DA_EINVAL, "unknown flag bits 0x%x", a->flags);
  if (a->dtype == DA_F32 && a->B > kMaxGridYZ)
    return fail(DA_EUNSUPPORTED, "the fp32 backward takes at most %d batches per call", kMaxGridYZ);
  if ((st = resolve_maps((int)a->H_s, (int)a->H_n, (int)a->H_kv, a->noise_of_signal, a->kv_of_signal, p->nz, p->kv,
                         p->members)) != DA_OK)
    return st;
  const int Hs = (int)a->H_s, Hn = (int)a->H_n, Hkv = (int)a->H_kv, g = Hs / Hn, gk = Hs / Hkv;
  {
    int fill[DA_MAX_HEADS] = {0};
    for (int h = 0; h < Hs; ++h) p->kvmembers[p->kv[h] * gk + fill[p->kv[h]]++] = (int16_t)h;
  }
  if (a->dtype == DA_BF16) {
    // each key/value head's signal heads form one run in one noise group's member order
    int runs[DA_MAX_HEADS] = {0};
    for (int n = 0; n < Hn; ++n)
      for (int t = 0; t < g; ++t) {
        const int k = p->kv[p->members[n * g + t]];
        if (t == 0 || p->kv[p->members[n * g + t - 1]] != k) runs[k]++;
      }
    for (int k = 0; k < Hkv; ++k)
      if (runs[k] != 1)
        return fail(DA_EUNSUPPORTED,
                    "bf16 backward: the signal heads of kv head %d are not one run inside one noise group", k);
  }
  const int64_t rows = a->B * a->N * a->H_s;
  p->nprep = (int)std::max<int64_t>(1, std::min<int64_t>(da::kBwdPrepBlocks, (rows + 3) / 4));
  p->B = (int)a->B;
  p->N = (int)a->N;
  p->Hs = Hs;
  p->Hn = Hn;
  p->Hkv = Hkv;
  p->d = (int)a->d;
  p->dv = (int)a->dv;
  p->g = g;
  p->gk = gk;
  p->causal = (a->flags & DA_CAUSAL) ? 1 : 0;
  p->normalize = (a->flags & DA_NO_NORM) ? 0 : 1;
  p->lam = a->lambda;
  p->lam_init = a->lambda_init;
  p->eps = a->eps;
  p->sm_scale = (float)(1.0 / sqrt((double)a->d));
  p->sm_scale_log2 = (float)(1.4426950408889634 / sqrt((double)a->d));
  if (!check_pointers) return DA_OK;

  if (!a->dlambda) return fail(DA_EINVAL, "dlambda is NULL");
  if ((uintptr_t)a->dlambda & 3u) return fail(DA_EINVAL, "dlambda is not 4-byte aligned");
  if (a->dnorm_w) {
    if ((uintptr_t)a->dnorm_w & 3u) return fail(DA_EINVAL, "dnorm_w is not 4-byte aligned");
    if (!a->norm_w || !p->normalize) return fail(DA_EINVAL, "dnorm_w needs norm_w and the head norm");
  }
  if (a->norm_w && ((uintptr_t)a->norm_w & 3u)) return fail(DA_EINVAL, "norm_w is not 4-byte aligned");
  p->dlambda = a->dlambda;
  p->dnorm_w = a->dnorm_w;
  p->norm_w = a->norm_w;
  if (a->B == 0 || a->N == 0) return DA_OK;  // empty: only dlambda / dnorm_w are written (zeros)

  const int es = a->dtype == DA_BF16 ? 2 : 4;
  struct T {
    const char* name;
    const void* p;
    const int64_t* s;
    int64_t heads, last;
  } ins[6] = {{"q1", a->q1, a->s_q1, a->H_s, a->d},       {"q2", a->q2, a->s_q2, a->H_n, a->d},
              {"k1", a->k1, a->s_k1, a->H_kv, a->d},      {"k2", a->k2, a->s_k2, a->H_n, a->d},
              {"v", a->v, a->s_v, a->H_kv, a->dv},        {"dout", a->dout, a->s_dout, a->H_s, a->dv}},
    outs[5] = {{"grad_q1", a->grad_q1, a->s_gq1, a->H_s, a->d}, {"grad_q2", a->grad_q2, a->s_gq2, a->H_n, a->d},
               {"grad_k1", a->grad_k1, a->s_gk1, a->H_kv, a->d}, {"grad_k2", a->grad_k2, a->s_gk2, a->H_n, a->d},
               {"grad_v", a->grad_v, a->s_gv, a->H_kv, a->dv}};
  for (auto& t : ins)
    if ((st = check_strides(t.name, t.p, t.s, 3, es)) != DA_OK) return st;
  for (auto& t : outs)
    if ((st = check_strides(t.name, t.p, t.s, 3, es)) != DA_OK) return st;
  if (a->dtype == DA_BF16) {
    // the bf16 passes address the rows of one streamed block from a 64-bit base
    // with 32-bit per-lane byte offsets (same bound as the prefill's)
    for (int i = 0; i < 5; ++i)
      if (ins[i].s[1] > kMaxTokenStride)
        return fail(DA_EUNSUPPORTED, "%s token stride %lld exceeds %lld elements", ins[i].name,
                    (long long)ins[i].s[1], (long long)kMaxTokenStride);
  }
  if (!a->o_maps) return fail(DA_EINVAL, "o_maps is NULL");
  if (!aligned16(a->o_maps)) return fail(DA_EINVAL, "o_maps is not 16-byte aligned");
  if (!a->lse) return fail(DA_EINVAL, "lse is NULL");
  if ((uintptr_t)a->lse & 3u) return fail(DA_EINVAL, "lse is not 4-byte aligned");
  auto view = [&](const T& t) { return View{t.p, {a->B, a->N, t.heads}, t.s, t.last, es}; };
  const Extent e_maps{(uintptr_t)a->o_maps, (uintptr_t)a->o_maps + (uintptr_t)(2 * a->B * a->N * a->H_s * a->dv * 4)};
  const Extent e_lse{(uintptr_t)a->lse, (uintptr_t)(a->lse + 2 * a->B * a->H_s * a->N)};
  for (int i = 0; i < 5; ++i) {
    const View vi = view(outs[i]);
    for (int j = 0; j < 6; ++j)
      if (views_overlap(vi, view(ins[j]))) return fail(DA_EINVAL, "%s overlaps %s", outs[i].name, ins[j].name);
    const Extent ei = extent(vi.p, vi.dims, vi.s, 3, vi.last, es);
    if (overlaps(ei, e_maps)) return fail(DA_EINVAL, "%s overlaps o_maps", outs[i].name);
    if (overlaps(ei, e_lse)) return fail(DA_EINVAL, "%s overlaps lse", outs[i].name);
    for (int j = 0; j < i; ++j)
      if (views_overlap(vi, view(outs[j]))) return fail(DA_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  p->q1 = a->q1;
  p->q2 = a->q2;
  p->k1 = a->k1;
  p->k2 = a->k2;
  p->v = a->v;
  p->o_maps = (const float*)a->o_maps;
  p->lam_dev = a->lambda_dev;
  p->lse = a->lse;
  p->dout = a->dout;
  p->gq1 = a->grad_q1;
  p->gq2 = a->grad_q2;
  p->gk1 = a->grad_k1;
  p->gk2 = a->grad_k2;
  p->gv = a->grad_v;
  for (int i = 0; i < 3; ++i) {
    p->sq1[i] = a->s_q1[i];
    p->sq2[i] = a->s_q2[i];
    p->sk1[i] = a->s_k1[i];
    p->sk2[i] = a->s_k2[i];
    p->sv[i] = a->s_v[i];
    p->sdo[i] = a->s_dout[i];
    p->sgq1[i] = a->s_gq1[i];
    p->sgq2[i] = a->s_gq2[i];
    p->sgk1[i] = a->s_gk1[i];
    p->sgk2[i] = a->s_gk2[i];
    p->sgv[i] = a->s_gv[i];
  }
  return DA_OK;
}

da_status check_vec(const char* name, const float* p) {
  if (!p) return fail(DA_EINVAL, "%s is NULL", name);
  if ((uintptr_t)p & 3u) return fail(DA_EINVAL, "%s is not 4-byte aligned", name);
  return DA_OK;
}

}  // namespace

extern "C" {

da_status diffattn_fwd(const da_fwd_args* args, void* stream) { return fwd_impl(args, stream, true); }

da_status gda_fwd(const da_fwd_args* args, void* stream) { return fwd_impl(args, stream, false); }

da_status gda_fwd_varlen(const da_fwd_args* args, const int32_t* cu_seqlens, int64_t nseq, int64_t max_seqlen,
                         void* stream) {
  const Packing pk{cu_seqlens, nseq, max_seqlen};
  return fwd_impl(args, stream, false, &pk);
}

size_t gda_decode_workspace_bytes(const da_decode_args* args) {
  da::DecodeParams p;
  if (decode_prepare(args, &p, /*check_pointers=*/false) != DA_OK) return 0;  // shapes only
  return decode_ws_bytes(p);
}

da_status gda_decode(const da_decode_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  da::DecodeParams p;
  da_status st = decode_prepare(args, &p, /*check_pointers=*/true);
  if (st != DA_OK) return st;
  if (p.B == 0) return DA_OK;  // Lmax == 0 still launches: every output row is zero
  const size_t need = decode_ws_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DA_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? workspace_bytes : (size_t)0);
  if (workspace && ((uintptr_t)workspace & 15u)) return fail(DA_EINVAL, "workspace is not 16-byte aligned");
  if ((st = decode_check_overlap(args, workspace, need)) != DA_OK) return st;
  p.ws = (float*)workspace;
  hipError_t e = da::launch_decode(p, args->dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return DA_OK;
}

da_status gda_decode_noalloc(const da_decode_args* args, void* stream) {
  da::DecodeParams p;
  da_status st = decode_prepare(args, &p, /*check_pointers=*/true);
  if (st != DA_OK) return st;
  if (p.B == 0) return DA_OK;
  const size_t need = decode_ws_bytes(p);
  if (need > da::kDecodeScratchBytes)
    return fail(DA_EUNSUPPORTED, "these shapes need %zu bytes of decode partials; the fixed scratch holds %zu",
                need, (size_t)da::kDecodeScratchBytes);
  if ((st = decode_check_overlap(args, nullptr, 0)) != DA_OK) return st;
  // the scratch belongs to the current device: the stream must run on it
  int dev = -1, sdev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "current device");
  if (stream) {
    if ((e = hipStreamGetDevice((hipStream_t)stream, &sdev)) != hipSuccess) return hip_fail(e, "stream device");
    if (sdev != dev)
      return fail(DA_EINVAL, "stream runs on device %d, the current device is %d", sdev, dev);
  }
  if ((e = da::decode_scratch(&p.ws)) != hipSuccess) return hip_fail(e, "decode scratch address");
  e = da::launch_decode(p, args->dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return DA_OK;
}

size_t gda_bwd_workspace_bytes(const da_bwd_args* args) {
  da::BwdParams p;
  if (bwd_prepare(args, &p, /*check_pointers=*/false) != DA_OK) return 0;  // shapes only
  if (p.B == 0 || p.N == 0) return 0;
  return bwd_layout(p, args->dtype == DA_BF16 ? 2 : 4).total;
}

da_status gda_bwd(const da_bwd_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  da::BwdParams p;
  da_status st = bwd_prepare(args, &p, /*check_pointers=*/true);
  if (st != DA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (p.B == 0 || p.N == 0) {
    if ((e = da::launch_bwd_zero(p, s)) != hipSuccess) return hip_fail(e, "backward launch");
    return DA_OK;
  }
  const BwdLayout l = bwd_layout(p, args->dtype == DA_BF16 ? 2 : 4);
  if (!workspace || workspace_bytes < l.total)
    return fail(DA_EWORKSPACE, "workspace needs %zu bytes, got %zu", l.total, workspace ? workspace_bytes : (size_t)0);
  if ((uintptr_t)workspace & 15u) return fail(DA_EINVAL, "workspace is not 16-byte aligned");
  unsigned char* ws = (unsigned char*)workspace;
  p.dop = ws + l.dop;
  p.rowstat = (float*)(ws + l.rowstat);
  p.partial = (double*)(ws + l.partial);
  if ((e = da::launch_bwd_prep(p, args->dtype, s)) != hipSuccess) return hip_fail(e, "backward row pass");
  e = args->dtype == DA_BF16 ? da::launch_bwd_bf16(p, s) : da::launch_bwd_f32(p, s);
  if (e != hipSuccess) return hip_fail(e, "backward score passes");
  if ((e = da::launch_bwd_finalize(p, s)) != hipSuccess) return hip_fail(e, "backward reduction");
  return DA_OK;
}

da_status da_lambda_reparam(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int64_t dim,
                            float lambda_init, float* lambda_out, void* stream) {
  if (dim < 1 || dim > 65536) return fail(DA_EINVAL, "dim = %lld outside [1, 65536]", (long long)dim);
  if (!isfinite(lambda_init)) return fail(DA_EINVAL, "lambda_init must be finite");
  const char* names[5] = {"lq1", "lk1", "lq2", "lk2", "lambda_out"};
  const float* ptrs[5] = {lq1, lk1, lq2, lk2, lambda_out};
  da_status st;
  for (int i = 0; i < 5; ++i)
    if ((st = check_vec(names[i], ptrs[i])) != DA_OK) return st;
  const Extent eo{(uintptr_t)lambda_out, (uintptr_t)(lambda_out + 1)};
  for (int i = 0; i < 4; ++i)
    if (overlaps(eo, Extent{(uintptr_t)ptrs[i], (uintptr_t)(ptrs[i] + dim)}))
      return fail(DA_EINVAL, "lambda_out overlaps %s", names[i]);
  hipError_t e = da::launch_lambda_reparam(lq1, lk1, lq2, lk2, (int)dim, lambda_init, lambda_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "lambda launch");
  return DA_OK;
}

da_status da_lambda_reparam_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int64_t dim,
                                const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                                void* stream) {
  if (dim < 1 || dim > 65536) return fail(DA_EINVAL, "dim = %lld outside [1, 65536]", (long long)dim);
  const char* names[9] = {"lq1", "lk1", "lq2", "lk2", "dlambda", "dlq1", "dlk1", "dlq2", "dlk2"};
  const float* ptrs[9] = {lq1, lk1, lq2, lk2, dlambda, dlq1, dlk1, dlq2, dlk2};
  da_status st;
  for (int i = 0; i < 9; ++i)
    if ((st = check_vec(names[i], ptrs[i])) != DA_OK) return st;
  for (int i = 5; i < 9; ++i) {
    const Extent eo{(uintptr_t)ptrs[i], (uintptr_t)(ptrs[i] + dim)};
    for (int j = 0; j < i; ++j) {
      const Extent ej{(uintptr_t)ptrs[j], (uintptr_t)(ptrs[j] + (j == 4 ? 1 : dim))};
      if (overlaps(eo, ej)) return fail(DA_EINVAL, "%s overlaps %s", names[i], names[j]);
    }
  }
  hipError_t e = da::launch_lambda_reparam_bwd(lq1, lk1, lq2, lk2, (int)dim, dlambda, dlq1, dlk1, dlq2, dlk2,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "lambda backward launch");
  return DA_OK;
}

const char* da_status_str(int status) {
  switch (status) {
    case DA_OK: return "DA_OK: success";
    case DA_EINVAL: return "DA_EINVAL: invalid argument";
    case DA_EUNSUPPORTED: return "DA_EUNSUPPORTED: no kernel for this request";
    case DA_EHIP: return "DA_EHIP: HIP runtime or launch failure";
    case DA_EWORKSPACE: return "DA_EWORKSPACE: workspace missing or too small";
    default: return "unknown status";
  }
}

const char* da_last_error(void) { return g_last_error.c_str(); }

int da_abi_version(void) { return DA_ABI_VERSION; }

}  // extern "C"

/*
 * diffattn.h -- C ABI of libdiffattn.so: fused causal differential attention
 * and Grouped Differential Attention (GDA) on AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by title and section):
 *   [DA-blog] "Differential Attention in Large Language Models: How Denoising
 *             Subtraction Eliminates Attention Noise and Outlier Activations"
 *             (llms.blog): "Differential Attention Architecture" (the
 *             projections into Q1/Q2, K1/K2 halves of width d and V of width
 *             2d, and the DiffAttn equation), "Learnable Lambda
 *             Re-parameterization" (lambda, lambda_init), "Headwise
 *             Normalization" (head_bar_i = (1 - lambda_init) RMSNorm(head_i)).
 *   [GDA]     "Grouped Differential Attention" (mlsanity.com), "Abstract":
 *             more signal heads than noise-control heads, the noise heads
 *             repeated the way GQA repeats key/value heads.
 *
 * Per signal head h, query i and visible keys j (j <= i when causal):
 *   A1 = softmax_j(Q1[i,h] . K1[j,kv(h)] / sqrt(d))
 *   A2 = softmax_j(Q2[i,nz(h)] . K2[j,nz(h)] / sqrt(d))
 *   o  = sum_j (A1_j - lambda A2_j) V[j,kv(h)]                       [DA-blog] DiffAttn
 *   out[i,h,:] = (1 - lambda_init) * w * o / sqrt(mean_c(o_c^2) + eps) [DA-blog] head_bar_i
 * with nz(h) = h / (H_s/H_n) and kv(h) = h / (H_s/H_kv) unless explicit maps
 * are given.  Plain differential attention is H_n = H_kv = H_s.
 *
 * Conventions shared by every entry point
 *   Memory   All tensor pointers are DEVICE pointers owned by the caller.  The
 *            library never allocates or frees device memory and keeps no
 *            state between calls.  Head maps are HOST arrays read during the
 *            call.  Outputs must not overlap inputs.
 *   Layout   Element strides (not bytes) for the listed leading dims; the last
 *            dim is contiguous (stride 1).  Every row start must be 16-byte
 *            aligned (pointer % 16 == 0, strides multiples of 16 bytes).
 *   Dtypes   DA_BF16: bf16 storage, fp32 accumulation, bf16 output rounded to
 *            nearest even.  DA_F32: fp32 throughout.
 *   Shapes   dv == 2*d ([DA-blog]: W^V maps to 2d); d in {32, 64}.
 *   Errors   A status code is returned; nothing is thrown and nothing aborts.
 *            Arguments are validated on the host before any HIP call
 *            (DA_EINVAL / DA_EUNSUPPORTED, nothing launched); launch failures
 *            return DA_EHIP.  da_last_error() gives a thread-local message.
 *   Streams  `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *            asynchronous on it; there is no host synchronisation.  Calls are
 *            thread-safe; calls that write the same output race.
 *   Empty    B == 0 or N == 0 is a valid no-op returning DA_OK.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DA_ABI_VERSION 3
#define DA_MAX_HEADS 256

typedef enum {
  DA_OK = 0,
  DA_EINVAL = 1,        /* bad pointer, shape, stride, alignment, map or overlap */
  DA_EUNSUPPORTED = 2,  /* valid request with no kernel (e.g. d not in {32,64}) */
  DA_EHIP = 3,          /* a HIP runtime call or kernel launch failed */
  DA_EWORKSPACE = 4     /* decode workspace missing or too small */
} da_status;

typedef enum { DA_F32 = 0, DA_BF16 = 1, DA_FP8_E4M3 = 2 } da_dtype;  /* FP8: OCP e4m3 (fn), caches only */

enum {
  DA_CAUSAL = 1u,   /* query i sees keys 0..i (decoder self-attention); without
                       it every query sees all N keys (the equation as printed) */
  DA_NO_NORM = 2u   /* store the raw DiffAttn output o (no head norm, no
                       (1 - lambda_init) factor) */
};

/* Prefill forward arguments (diffattn_fwd, gda_fwd).
 *   q1  [B,N,H_s,d]   q2 [B,N,H_n,d]    k1 [B,N,H_kv,d]   k2 [B,N,H_n,d]
 *   v   [B,N,H_kv,dv] out [B,N,H_s,dv]   (dtype `dtype`, device)
 *   s_* element strides of dims (b, n, head) of each tensor.
 *   noise_of_signal / kv_of_signal: host int32[H_s] or NULL (consecutive
 *     grouping).  H_s must be a multiple of H_n and of H_kv (DA_EINVAL
 *     otherwise), with explicit maps too; each noise head must serve exactly
 *     H_s/H_n signal heads.
 *   lambda: the folded per-layer scalar of [DA-blog] "Learnable Lambda
 *     Re-parameterization" (any real value).  lambda_init: the same section's
 *     per-layer constant, used only by the head norm.  eps > 0: added to the
 *     mean of squares.  norm_w: device fp32 [dv] or NULL (unit weight).
 *   lse: device fp32 [2][B][H_s][N] or NULL.  When given, receives the natural
 *     log-sum-exp of each map's scaled logits per (b, h, i): lse[0] for A1,
 *     lse[1] for A2 (what a backward pass re-uses).
 *   lambda_dev: device fp32 [1] or NULL.  When given, lambda is read from it
 *     when the kernels run (the host `lambda` is then ignored), e.g. the output
 *     of da_lambda_reparam: no host round trip per call.
 *   o_maps: device fp32 [2][B][N][H_s][dv] (dense, any dtype) or NULL.  When
 *     given, receives each map's own output A1 V and A2 V per (b, i, h), the
 *     two terms of the DiffAttn difference (what gda_bwd needs besides lse;
 *     fp32 because the head norm's backward differences them). */
typedef struct da_fwd_args {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  void* out;
  int64_t B, N, H_s, H_n, H_kv, d, dv;
  int64_t s_q1[3], s_q2[3], s_k1[3], s_k2[3], s_v[3], s_out[3];
  const int32_t* noise_of_signal;
  const int32_t* kv_of_signal;
  float lambda, lambda_init, eps;
  const float* norm_w;
  float* lse;
  int32_t dtype;    /* da_dtype */
  uint32_t flags;   /* DA_CAUSAL | DA_NO_NORM */
  void* o_maps;
  const float* lambda_dev;
} da_fwd_args;

/* Plain differential attention ([DA-blog] DiffAttn + head_bar_i): requires
 * H_n == H_kv == H_s and no explicit maps. */
da_status diffattn_fwd(const da_fwd_args* args, void* stream);

/* Grouped differential attention ([GDA] Abstract, GQA-style repetition of the
 * noise heads; GQA key/value heads for K1/V): requires H_s % H_n == 0 and
 * H_s % H_kv == 0.  With H_n == H_kv == H_s it equals diffattn_fwd.
 * Signal heads that share a noise head and a key/value head have one map-2
 * output; for bf16 at d = 64 with such heads in combos of 2, 4 or 8 and
 * nested row-major `out` strides, the call runs as two launches and `out`
 * holds intermediate values (each combo's A2 V) between them: its contents
 * are defined only once the stream has passed the call. */
da_status gda_fwd(const da_fwd_args* args, void* stream);

/* Packed variable-length GDA prefill: the same operation as gda_fwd applied
 * to each of `nseq` sequences packed one after another along the token axis
 * (the serving-side prefill batch; [GDA] Abstract for the head grouping,
 * [DA-blog] DiffAttn and head_bar_i per sequence).  Attention never crosses
 * a sequence boundary; DA_CAUSAL applies within each sequence.
 *   args: as for gda_fwd with B == 1 and N = the packed token count; every
 *     tensor is [1, N, heads, width] (the batch stride is not used).
 *   cu_seqlens: DEVICE int32[nseq + 1]; sequence s is tokens
 *     [cu_seqlens[s], cu_seqlens[s+1]).  Caller contract: cu_seqlens[0] >= 0,
 *     non-decreasing, cu_seqlens[nseq] <= N, every length <= max_seqlen.  The
 *     kernels clamp starts to [0, N] and lengths to [0, min(max_seqlen, N -
 *     start)], so a broken contract truncates sequences but never reads or
 *     writes outside the tensors.  Tokens outside every sequence are not
 *     written.
 *   max_seqlen: HOST bound on the sequence lengths, 0 <= max_seqlen <= N
 *     (sizes the launch grid).
 *   lse (optional): fp32 [2][H_s][N], indexed by packed token.
 * nseq == 0, max_seqlen == 0 or N == 0 is a no-op returning DA_OK.  Errors as
 * for gda_fwd, plus DA_EINVAL for B != 1, nseq < 0, a NULL or misaligned
 * cu_seqlens, or max_seqlen outside [0, N]. */
da_status gda_fwd_varlen(const da_fwd_args* args, const int32_t* cu_seqlens, int64_t nseq, int64_t max_seqlen,
                         void* stream);

/* Backward arguments (gda_bwd): gradients of L = sum(dout * out) for the
 * forward of the same arguments (the derivative of [DA-blog] DiffAttn and
 * head_bar_i; [GDA] Abstract for the sums over shared heads).
 *   q1, q2, k1, k2, v: the forward's inputs, layouts and strides as in
 *     da_fwd_args.
 *   o_maps: fp32 [2][B][N][H_s][dv] dense, lse: fp32 [2][B][H_s][N]: what
 *     the forward stored through its o_maps and lse arguments.
 *   dout [B,N,H_s,dv]: the incoming gradient (dtype `dtype`).
 *   grad_q1 .. grad_v: the gradients, shapes of q1 .. v, written in full
 *     (never accumulated into); strides s_g*.  A noise head's dQ2/dK2 sum its
 *     signal heads' contributions, a key/value head's dK1/dV its heads'.
 *   dlambda: device fp32 [1], receives dL/dlambda.  dnorm_w: device fp32 [dv]
 *     or NULL; receives dL/dw when the head norm is on and norm_w is given.
 *     lambda_init is a per-layer constant ([DA-blog] lambda_init schedule):
 *     no gradient.
 *   Everything else as in da_fwd_args (lambda_dev included); DA_CAUSAL and
 *     DA_NO_NORM must match the forward.  With dtype DA_BF16 the key/value map must keep the heads that
 *     share a key/value head together: every key/value head's signal heads
 *     lie in one noise group (true for consecutive maps with H_kv >= H_n);
 *     otherwise DA_EUNSUPPORTED. */
typedef struct da_bwd_args {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  const void* o_maps;
  const float* lse;
  const void* dout;
  void* grad_q1;
  void* grad_q2;
  void* grad_k1;
  void* grad_k2;
  void* grad_v;
  float* dlambda;
  float* dnorm_w;
  int64_t B, N, H_s, H_n, H_kv, d, dv;
  int64_t s_q1[3], s_q2[3], s_k1[3], s_k2[3], s_v[3], s_dout[3];
  int64_t s_gq1[3], s_gq2[3], s_gk1[3], s_gk2[3], s_gv[3];
  const int32_t* noise_of_signal;
  const int32_t* kv_of_signal;
  float lambda, lambda_init, eps;
  const float* norm_w;
  int32_t dtype;
  uint32_t flags;
  const float* lambda_dev;
} da_bwd_args;

/* Bytes of device workspace gda_bwd needs (shapes and dtype only; pointers
 * may be NULL).  0 for empty inputs and on invalid shapes (then
 * da_last_error() says why). */
size_t gda_bwd_workspace_bytes(const da_bwd_args* args);

/* Backward of gda_fwd / diffattn_fwd (plain differential attention is H_n ==
 * H_kv == H_s).  Kernels: a row pass (head-norm backward, the per-row dot
 * products dout' . o1 and dout' . o2, partial sums of dlambda and dw), a
 * query-major pass (dQ1, dQ2), a key-major pass (dK1, dK2, dV) and a final
 * reduction (dlambda, dw); scores and weights are recomputed from lse.
 * workspace: device, caller-owned, 16-byte aligned, >= gda_bwd_workspace_bytes
 * (DA_EWORKSPACE otherwise).  Outputs must not overlap inputs or each other
 * (DA_EINVAL): strided views of one buffer pass when they repeat with the same
 * token stride and their columns within a token are disjoint -- the gradient
 * of a fused projection written in its own layout; otherwise their byte
 * ranges must be disjoint. */
da_status gda_bwd(const da_bwd_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* Decode arguments (gda_decode): one new query per sequence against caches
 * that already hold the current token, as in a serving step.
 *   q1 [B,H_s,d]  q2 [B,H_n,d]  out [B,H_s,dv]        strides of (b, head)
 *   k1_cache [B,H_kv,Lmax,d]  k2_cache [B,H_n,Lmax,d]  v_cache [B,H_kv,Lmax,dv]
 *                                                     strides of (b, head, pos)
 *   seq_lens: device int32[B]; sequence b's query sees positions 0..L_b-1.
 *     0 <= L_b <= Lmax is the caller's contract (the kernels clamp to
 *     [0, Lmax]); L_b == 0 yields a zero output row.
 *   chunk: cached positions per split-K partial (a multiple of 128, of 256
 *     for e4m3 caches; at most 2048), 0 = automatic: about 2560 partials in
 *     all (B x H_n x Lmax / chunk), rounded up to that multiple and capped at
 *     2048.  The result does not depend on it beyond rounding order.
 *   block_table: device int32 [B][max_blocks] or NULL.  When given the caches
 *     are paged: each cache is a pool [num_blocks][heads][block_size][width]
 *     (strides of (block, head, position) in s_k1 / s_k2 / s_v) and position p
 *     of sequence b is row p % block_size of block block_table[b][p /
 *     block_size] (the paged KV cache of serving engines).  block_size is a
 *     multiple of 128 (of 256 for e4m3 caches) so that every sub-chunk of 128
 *     (256) positions lies in one block; Lmax <= max_blocks * block_size; block
 *     indices are clamped to [0, num_blocks - 1] (a broken table never reads
 *     outside the pool); DA_EUNSUPPORTED for other block sizes.
 *   cache_dtype: DA_FP8_E4M3 for caches of OCP e4m3 bytes (1 byte per element,
 *     strides in elements = bytes), each cache read as value * its scale
 *     (k1_scale, k2_scale, v_scale: finite, > 0; the low-bit KV cache of
 *     [DA-blog] "Hardware Implementations and Serving Considerations"); any
 *     other value (0 included) means the caches are in `dtype` and the scales
 *     are ignored.
 *   Everything else as in da_fwd_args (the causal flag is implied; lambda_dev
 *     included).
 *   Limits (DA_EUNSUPPORTED otherwise, before any HIP call): d = 64, bf16
 *     queries, bf16 or e4m3 caches; per noise group at most 7 signal heads
 *     and at most 8 outputs, its g signal heads plus the u distinct key/value
 *     heads they read (g + u <= 8: 3:1 GDA on distinct key/value heads is
 *     3 + 3, 4:1 GDA on 2:1 GQA 4 + 2); at most 65535 sequences. */
typedef struct da_decode_args {
  const void* q1;
  const void* q2;
  const void* k1_cache;
  const void* k2_cache;
  const void* v_cache;
  const int32_t* seq_lens;
  void* out;
  int64_t B, Lmax, H_s, H_n, H_kv, d, dv, chunk;
  int64_t s_q1[2], s_q2[2], s_out[2];
  int64_t s_k1[3], s_k2[3], s_v[3];
  const int32_t* noise_of_signal;
  const int32_t* kv_of_signal;
  float lambda, lambda_init, eps;
  const float* norm_w;
  int32_t dtype;
  uint32_t flags;   /* DA_NO_NORM only */
  const float* lambda_dev;
  int32_t cache_dtype;
  float k1_scale, k2_scale, v_scale;
  const int32_t* block_table;
  int64_t block_size, max_blocks, num_blocks;
} da_decode_args;

/* Bytes of device workspace gda_decode needs for these arguments.  Depends on
 * the shapes, head maps and chunk only: data pointers may be NULL.  Returns 0
 * for an empty batch and on invalid shapes (then da_last_error() says why). */
size_t gda_decode_workspace_bytes(const da_decode_args* args);

/* Split-K GDA decode: a partial kernel streams each cached K1/V/K2 byte once
 * per noise group and writes per-chunk (max, sum, unnormalised output) of both
 * maps to `workspace` (device, caller-owned, >= gda_decode_workspace_bytes);
 * a combine kernel merges the chunks, applies the lambda difference and the
 * head norm.  Returns DA_EWORKSPACE if the workspace is NULL or too small. */
da_status gda_decode(const da_decode_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* gda_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and result, with the chunk partials in a fixed device array of
 * DA_DECODE_SCRATCH_BYTES inside the library instead of a caller workspace.
 * Nothing is allocated or freed by the call.  One array per GPU, created when
 * the library is loaded on that GPU and held until the process ends; its
 * address is looked up on the first call on each device.  The array belongs to
 * the current device (hipGetDevice): `stream` must run on it (DA_EINVAL
 * otherwise).  Calls on one GPU share the array, so calls that overlap in time
 * on one GPU (different streams, or host threads) race and must be serialised
 * by the caller; consecutive calls on one stream are safe.  Shapes whose
 * partials exceed the array (gda_decode_workspace_bytes > DA_DECODE_SCRATCH_BYTES)
 * return DA_EUNSUPPORTED before any HIP call.  Other errors as for gda_decode. */
#define DA_DECODE_SCRATCH_BYTES (32u << 20)
da_status gda_decode_noalloc(const da_decode_args* args, void* stream);

/* lambda on the device ([DA-blog] "Learnable Lambda Re-parameterization",
 * lambda equation): lambda_out[0] = exp(lq1 . lk1) - exp(lq2 . lk2) +
 * lambda_init, with lq1, lk1, lq2, lk2 device fp32 vectors of `dim` entries
 * (the per-layer learnable vectors, dim = the head dimension).  lambda_out is a
 * device fp32 [1] that the prefill, backward and decode calls can read through
 * lambda_dev.  DA_EINVAL for NULL or misaligned pointers, dim outside [1, 65536],
 * a non-finite lambda_init or lambda_out overlapping an input. */
da_status da_lambda_reparam(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int64_t dim,
                            float lambda_init, float* lambda_out, void* stream);

/* Gradients of da_lambda_reparam given dlambda (device fp32 [1], e.g. what
 * gda_bwd wrote): dlq1 = dlambda e1 lk1, dlk1 = dlambda e1 lq1,
 * dlq2 = -dlambda e2 lk2, dlk2 = -dlambda e2 lq2 with e1 = exp(lq1 . lk1),
 * e2 = exp(lq2 . lk2); outputs device fp32 [dim] each, written in full.
 * Errors as for da_lambda_reparam; outputs must not overlap inputs or each other. */
da_status da_lambda_reparam_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int64_t dim,
                                const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                                void* stream);

/* Static description of a status code. */
const char* da_status_str(int status);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char* da_last_error(void);

/* DA_ABI_VERSION of the loaded library. */
int da_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */

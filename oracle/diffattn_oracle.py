"""Plain fp64 CPU oracle for causal differential attention and Grouped
Differential Attention (GDA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module; only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP kernels.

Pages this file follows (cited by title and section):

* [DA-blog]  "Differential Attention in Large Language Models: How Denoising
  Subtraction Eliminates Attention Noise and Outlier Activations" (llms.blog):
  section "The Mechanics of Attention Noise" (standard attention equation),
  section "Differential Attention Architecture" (projection equations and the
  DiffAttn equation), section "Learnable Lambda Re-parameterization" (lambda
  and lambda_init equations), section "Headwise Normalization" (head_bar_i
  equation).
* [GDA]  "Grouped Differential Attention" (mlsanity.com), "Abstract": signal
  heads outnumber noise-control heads, and the noise heads are repeated the
  way GQA repeats key/value heads.
* [DT-summary]  "Differential Transformer" (atlas.scime.ai), "Approach" and
  the "Measured effects" table (the per-head norm is called GroupNorm there).

What the method computes is exact: a fused kernel reaches the same real-valued
function, only the rounding order differs.  So this oracle is the definition
written out, in float64, with a full-row softmax (no online rescaling, no
blocking over keys).  Readings taken where the pages are silent:

* causal masking (query i sees keys 0..i) unless ``causal=False``;
* the softmax scale is 1/sqrt(d) with d the width of one Q/K half, for both maps;
* lambda and lambda_init are one scalar each per call (per layer);
* the per-head norm is RMS (no mean subtraction) over the dv output channels,
  with eps added to the mean of squares, then times (1 - lambda_init) and an
  optional per-channel weight;
* in GDA each noise head owns both its Q2 and its K2; signal head h uses noise
  head noise_of_signal[h] (default h // (H_s / H_n)) and key/value head
  kv_of_signal[h] (default h // (H_s / H_kv));
* the backward is the derivative of this forward (chain rule written out in
  ``diff_attention_backward``): the pages state no training kernel, and the
  gradient of a stated function has one value.  lambda_init is a per-layer
  constant (its schedule), so it has no gradient;
* a packed batch of sequences (the serving-side prefill) is the same
  forward applied to each sequence on its own: no query attends across a
  sequence boundary, and causality counts positions from the sequence start.

Every function here is pinned by the CPU tests against closed forms, library
routines and brute force; none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lambda_init_schedule",
    "lambda_reparam",
    "lambda_reparam_grad",
    "consecutive_map",
    "softmax_rows",
    "head_rms_norm",
    "diff_attention",
    "diff_attention_rows",
    "diff_attention_lse",
    "diff_attention_packed",
    "diff_attention_packed_lse",
    "diff_attention_maps",
    "diff_attention_backward",
    "gda_decode",
    "fp8_e4m3_decode",
    "gda_decode_fp8",
    "brute_diff_attention",
    "causal_pairs",
    "flops_alg",
    "flops_exec",
]


# ---------------------------------------------------------------------------
# Scalars: [DA-blog] "Learnable Lambda Re-parameterization"
# ---------------------------------------------------------------------------

def lambda_init_schedule(layer: int) -> float:
    """lambda_init for 1-based layer index ``layer``: 0.8 minus 0.6 times
    exp(-0.3 (layer - 1)) ([DA-blog], lambda_init equation)."""
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def lambda_reparam(lq1, lk1, lq2, lk2, lambda_init: float) -> float:
    """lambda from the four learnable vectors: exp(lq1 . lk1) - exp(lq2 . lk2)
    + lambda_init ([DA-blog], lambda equation).  The kernels take the folded
    scalar; this exists so the tests can state where that scalar comes from."""
    a = float(np.dot(_as64(lq1).reshape(-1), _as64(lk1).reshape(-1)))
    b = float(np.dot(_as64(lq2).reshape(-1), _as64(lk2).reshape(-1)))
    return math.exp(a) - math.exp(b) + lambda_init


def lambda_reparam_grad(lq1, lk1, lq2, lk2, dlambda: float):
    """Gradients of ``lambda_reparam`` times dlambda (the chain rule of the
    lambda equation): d/dlq1 = exp(lq1 . lk1) lk1, d/dlk1 = exp(lq1 . lk1) lq1,
    d/dlq2 = -exp(lq2 . lk2) lk2, d/dlk2 = -exp(lq2 . lk2) lq2.  Returns float64
    arrays (dlq1, dlk1, dlq2, dlk2)."""
    lq1, lk1, lq2, lk2 = (np.asarray(_as64(x), np.float64).reshape(-1) for x in (lq1, lk1, lq2, lk2))
    e1 = math.exp(float(np.dot(lq1, lk1)))
    e2 = math.exp(float(np.dot(lq2, lk2)))
    return dlambda * e1 * lk1, dlambda * e1 * lq1, -dlambda * e2 * lk2, -dlambda * e2 * lq2


# ---------------------------------------------------------------------------
# Head maps: [GDA] "Abstract" (noise heads repeated GQA-style)
# ---------------------------------------------------------------------------

def consecutive_map(h_s: int, h_x: int) -> np.ndarray:
    """Signal head h -> shared head h // (h_s / h_x): consecutive grouping,
    the GQA convention the GDA abstract refers to."""
    if h_x <= 0 or h_s % h_x != 0:
        raise ValueError(f"{h_s} signal heads cannot be grouped over {h_x} heads")
    return np.arange(h_s, dtype=np.int64) // (h_s // h_x)


# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------

def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis; -inf entries get weight 0.  Each row is a
    strictly positive distribution over its unmasked entries that sums to one
    ([DA-blog] introduction).  The row max is subtracted before exp, which
    changes nothing mathematically."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def head_rms_norm(o: np.ndarray, lambda_init: float, eps: float,
                  weight: np.ndarray | None = None) -> np.ndarray:
    """(1 - lambda_init) * RMSNorm(o) over the last axis ([DA-blog] "Headwise
    Normalization", head_bar_i equation): o / sqrt(mean(o^2) + eps), times an
    optional per-channel weight, times (1 - lambda_init)."""
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, np.float64)
    return (1.0 - lambda_init) * y


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor handed in by a test
        x = x.detach().to("cpu")
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def _maps(h_s, h_n, h_kv, noise_of_signal, kv_of_signal):
    nz = consecutive_map(h_s, h_n) if noise_of_signal is None else np.asarray(noise_of_signal, np.int64)
    kv = consecutive_map(h_s, h_kv) if kv_of_signal is None else np.asarray(kv_of_signal, np.int64)
    if nz.shape != (h_s,) or kv.shape != (h_s,):
        raise ValueError("head maps must have one entry per signal head")
    if nz.min(initial=0) < 0 or nz.max(initial=0) >= h_n or kv.min(initial=0) < 0 or kv.max(initial=0) >= h_kv:
        raise ValueError("head map entry out of range")
    return nz, kv


# ---------------------------------------------------------------------------
# The forward: [DA-blog] DiffAttn equation + head_bar_i equation, [GDA] grouping
# ---------------------------------------------------------------------------

def diff_attention_rows(q1, q2, k1, k2, v, lam: float, lambda_init: float, *,
                        rows, eps: float = 1e-5, norm_weight=None, causal: bool = True,
                        noise_of_signal=None, kv_of_signal=None, normalize: bool = True,
                        heads=None, batches=None, block: int = 256) -> np.ndarray:
    """Output rows ``rows`` (query positions) of the forward, for the batches
    ``batches`` and signal heads ``heads`` (default: all).

    Shapes (BSHD, last dim contiguous):
      q1 [B,N,H_s,d]   q2 [B,N,H_n,d]   k1 [B,N,H_kv,d]   k2 [B,N,H_n,d]
      v  [B,N,H_kv,dv]
    Returns float64 [len(batches), len(rows), len(heads), dv].

    Per signal head h and query i ([DA-blog] DiffAttn equation):
      s1_j = q1[i,h] . k1[j,kv(h)] / sqrt(d),  s2_j = q2[i,nz(h)] . k2[j,nz(h)] / sqrt(d)
      a1 = softmax(s1), a2 = softmax(s2)  over visible keys j (j <= i if causal)
      o  = sum_j (a1_j - lam * a2_j) v[j,kv(h)]
    then ([DA-blog] head_bar_i equation) y = (1 - lambda_init) RMSNorm(o),
    skipped when ``normalize`` is False (the raw DiffAttn output).
    """
    q1, q2, k1, k2, v = (_as64(t) for t in (q1, q2, k1, k2, v))
    B, N, h_s, d = q1.shape
    h_n = q2.shape[2]
    h_kv = k1.shape[2]
    dv = v.shape[3]
    if q2.shape != (B, N, h_n, d) or k2.shape != (B, N, h_n, d):
        raise ValueError("q2/k2 must be [B,N,H_n,d]")
    if k1.shape != (B, N, h_kv, d) or v.shape[:3] != (B, N, h_kv):
        raise ValueError("k1 must be [B,N,H_kv,d] and v [B,N,H_kv,dv]")
    nz, kv = _maps(h_s, h_n, h_kv, noise_of_signal, kv_of_signal)
    rows = np.asarray(rows, np.int64).reshape(-1)
    heads = np.arange(h_s) if heads is None else np.asarray(heads, np.int64).reshape(-1)
    batches = np.arange(B) if batches is None else np.asarray(batches, np.int64).reshape(-1)
    w = None if norm_weight is None else _as64(norm_weight).reshape(dv)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((len(batches), len(rows), len(heads), dv), np.float64)
    keys = np.arange(N)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            for r0 in range(0, len(rows), block):
                rr = rows[r0:r0 + block]
                s1 = (q1[b, rr, h, :] @ k1[b, :, kv[h], :].T) * scale
                s2 = (q2[b, rr, nz[h], :] @ k2[b, :, nz[h], :].T) * scale
                if causal:
                    hidden = keys[None, :] > rr[:, None]
                    s1 = np.where(hidden, -np.inf, s1)
                    s2 = np.where(hidden, -np.inf, s2)
                a = softmax_rows(s1) - lam * softmax_rows(s2)
                o = a @ v[b, :, kv[h], :]
                out[bi, r0:r0 + len(rr), hi, :] = (
                    head_rms_norm(o, lambda_init, eps, w) if normalize else o)
    return out


def diff_attention(q1, q2, k1, k2, v, lam: float, lambda_init: float, **kw) -> np.ndarray:
    """All rows of the forward: float64 [B,N,H_s,dv].  Plain differential
    attention is the case H_n = H_kv = H_s; GDA is H_s > H_n."""
    n = _as64(q1).shape[1] if not hasattr(q1, "shape") else q1.shape[1]
    return diff_attention_rows(q1, q2, k1, k2, v, lam, lambda_init, rows=np.arange(n), **kw)


def diff_attention_lse(q1, q2, k1, k2, *, rows, causal: bool = True, noise_of_signal=None,
                       kv_of_signal=None, heads=None, batches=None) -> np.ndarray:
    """Natural log-sum-exp of each map's scaled logits over the visible keys:
    float64 [2, len(batches), len(rows), len(heads)], index 0 for the first
    map (Q1 K1^T / sqrt(d)), 1 for the second.  softmax_j = exp(s_j - lse)."""
    q1, q2, k1, k2 = (_as64(t) for t in (q1, q2, k1, k2))
    B, N, h_s, d = q1.shape
    h_n, h_kv = q2.shape[2], k1.shape[2]
    nz, kv = _maps(h_s, h_n, h_kv, noise_of_signal, kv_of_signal)
    rows = np.asarray(rows, np.int64).reshape(-1)
    heads = np.arange(h_s) if heads is None else np.asarray(heads, np.int64).reshape(-1)
    batches = np.arange(B) if batches is None else np.asarray(batches, np.int64).reshape(-1)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((2, len(batches), len(rows), len(heads)))
    keys = np.arange(N)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            for t, (qq, kk, hq, hk) in enumerate(((q1, k1, h, kv[h]), (q2, k2, nz[h], nz[h]))):
                s = (qq[b, rows, hq, :] @ kk[b, :, hk, :].T) * scale
                if causal:
                    s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
                m = np.max(s, axis=-1)
                out[t, bi, :, hi] = m + np.log(np.sum(np.exp(s - m[:, None]), axis=-1))
    return out


def _packed_segments(cu_seqlens, T: int, tokens):
    """(start, length, positions of ``tokens`` inside this sequence, their
    indices in ``tokens``) per sequence of the packing ``cu_seqlens``."""
    cu = np.asarray(cu_seqlens, np.int64).reshape(-1)
    if cu.size < 1 or cu[0] < 0 or np.any(np.diff(cu) < 0) or cu[-1] > T:
        raise ValueError("cu_seqlens must be non-decreasing offsets within [0, T]")
    tokens = np.asarray(tokens, np.int64).reshape(-1)
    segs = []
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        idx = np.nonzero((tokens >= a) & (tokens < b))[0]
        if b > a and idx.size:
            segs.append((a, b - a, tokens[idx] - a, idx))
    return segs


def diff_attention_packed(q1, q2, k1, k2, v, cu_seqlens, lam: float, lambda_init: float, *,
                          tokens=None, **kw) -> np.ndarray:
    """Packed variable-length forward: sequence s is tokens
    [cu_seqlens[s], cu_seqlens[s+1]) of the packed tensors
      q1 [T,H_s,d]  q2 [T,H_n,d]  k1 [T,H_kv,d]  k2 [T,H_n,d]  v [T,H_kv,dv]
    and each sequence gets ``diff_attention_rows`` of its own slice (a batch
    of one); keyword arguments are passed through.  Returns float64
    [len(tokens), H_s, dv] for the packed token indices ``tokens`` (default:
    all); a token outside every sequence gives NaN."""
    q1, q2, k1, k2, v = (_as64(t) for t in (q1, q2, k1, k2, v))
    T, h_s = q1.shape[0], q1.shape[1]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64).reshape(-1)
    out = np.full((len(tokens), h_s, v.shape[2]), np.nan)
    for a, n, rows, idx in _packed_segments(cu_seqlens, T, tokens):
        sl = slice(a, a + n)
        out[idx] = diff_attention_rows(q1[None, sl], q2[None, sl], k1[None, sl], k2[None, sl], v[None, sl],
                                       lam, lambda_init, rows=rows, **kw)[0]
    return out


def diff_attention_packed_lse(q1, q2, k1, k2, cu_seqlens, *, tokens=None, **kw) -> np.ndarray:
    """``diff_attention_lse`` per sequence of a packing: float64
    [2, len(tokens), H_s], NaN for tokens outside every sequence."""
    q1, q2, k1, k2 = (_as64(t) for t in (q1, q2, k1, k2))
    T, h_s = q1.shape[0], q1.shape[1]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64).reshape(-1)
    out = np.full((2, len(tokens), h_s), np.nan)
    for a, n, rows, idx in _packed_segments(cu_seqlens, T, tokens):
        sl = slice(a, a + n)
        out[:, idx] = diff_attention_lse(q1[None, sl], q2[None, sl], k1[None, sl], k2[None, sl], rows=rows,
                                         **kw)[:, 0]
    return out


def gda_decode(q1, q2, k1_cache, k2_cache, v_cache, seq_lens, lam: float, lambda_init: float, *,
               eps: float = 1e-5, norm_weight=None, noise_of_signal=None, kv_of_signal=None,
               normalize: bool = True, batches=None) -> np.ndarray:
    """One new query per sequence against its cache (the serving step).

      q1 [B,H_s,d]  q2 [B,H_n,d]
      k1_cache [B,H_kv,Lmax,d]  k2_cache [B,H_n,Lmax,d]  v_cache [B,H_kv,Lmax,dv]
      seq_lens [B]: the query sees cache positions 0..L_b-1 (the cache already
      holds the current token, so this is the last row of a causal prefill).
    Returns float64 [len(batches), H_s, dv]; a sequence with L_b = 0 gives zeros.
    Same formulas as ``diff_attention_rows``.
    """
    q1, q2, k1c, k2c, vc = (_as64(t) for t in (q1, q2, k1_cache, k2_cache, v_cache))
    lens = np.asarray(_as64(seq_lens), np.int64).reshape(-1)
    B, h_s, d = q1.shape
    h_n = q2.shape[1]
    h_kv = k1c.shape[1]
    dv = vc.shape[3]
    nz, kv = _maps(h_s, h_n, h_kv, noise_of_signal, kv_of_signal)
    w = None if norm_weight is None else _as64(norm_weight).reshape(dv)
    batches = np.arange(B) if batches is None else np.asarray(batches, np.int64).reshape(-1)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((len(batches), h_s, dv), np.float64)
    for bi, b in enumerate(batches):
        L = int(lens[b])
        if L <= 0:
            continue
        for h in range(h_s):
            s1 = (k1c[b, kv[h], :L, :] @ q1[b, h, :]) * scale
            s2 = (k2c[b, nz[h], :L, :] @ q2[b, nz[h], :]) * scale
            a = softmax_rows(s1) - lam * softmax_rows(s2)
            o = a @ vc[b, kv[h], :L, :]
            out[bi, h, :] = head_rms_norm(o, lambda_init, eps, w) if normalize else o
    return out


# ---------------------------------------------------------------------------
# Gradients: the derivative of the forward above, by the chain rule
# ---------------------------------------------------------------------------

def diff_attention_maps(q1, q2, k1, k2, v, *, causal: bool = True, noise_of_signal=None, kv_of_signal=None):
    """Each map's normalised output, o1 = A1 V and o2 = A2 V, per signal head:
    float64 [2, B, N, H_s, dv] (index 0: the Q1 K1^T map, 1: the Q2 K2^T map).
    The forward's raw output is o1 - lambda o2 ([DA-blog] DiffAttn equation)."""
    one = diff_attention(q1, q2, k1, k2, v, 0.0, 0.0, causal=causal, noise_of_signal=noise_of_signal,
                         kv_of_signal=kv_of_signal, normalize=False)
    diff = diff_attention(q1, q2, k1, k2, v, 1.0, 0.0, causal=causal, noise_of_signal=noise_of_signal,
                          kv_of_signal=kv_of_signal, normalize=False)
    return np.stack([one, one - diff])


def diff_attention_backward(q1, q2, k1, k2, v, dout, lam: float, lambda_init: float, *, eps: float = 1e-5,
                            norm_weight=None, causal: bool = True, noise_of_signal=None, kv_of_signal=None,
                            normalize: bool = True) -> dict:
    """Gradients of L = sum(dout * out) for the forward ``diff_attention``
    (same arguments; dout [B,N,H_s,dv]).  Returns float64 arrays dq1, dq2,
    dk1, dk2, dv (shapes of the inputs), the scalar dlambda, the L2 norm of
    the terms dlambda sums (dlambda_scale: the scale of its rounding error,
    whose terms cancel) and, when a norm weight is given, dnorm_weight [dv].

    Steps, per batch b and signal head h (n = nz(h), k = kv(h)):
      forward pieces: s1 = q1 k1^T / sqrt(d), s2 = q2 k2^T / sqrt(d), a1 =
        softmax(s1), a2 = softmax(s2) (masked keys weigh 0), o1 = a1 v,
        o2 = a2 v, o = o1 - lam o2 ([DA-blog] DiffAttn equation);
      head norm ([DA-blog] head_bar_i): y = c w o / r, c = 1 - lambda_init,
        r = sqrt(mean(o^2) + eps), so do = c w dy / r - o sum(c w dy o) / (dv r^3)
        and dw = sum over rows of dy c o / r (do = dy without the norm);
      lambda: do/dlam = -o2, so dlam = -sum(do . o2);
      the difference: da1 = do v^T, da2 = -lam do v^T, dv += (a1 - lam a2)^T do;
      softmax: ds = a (da - rowsum(a da)) for each map;
      scores: dq1 += ds1 k1 / sqrt(d), dk1 += ds1^T q1 / sqrt(d), and the same
        for the second map into dq2[n], dk2[n] (shared by the group's heads).
    """
    q1, q2, k1, k2, v, dy = (_as64(t) for t in (q1, q2, k1, k2, v, dout))
    B, N, h_s, d = q1.shape
    h_n, h_kv, dv_ = q2.shape[2], k1.shape[2], v.shape[3]
    nz, kv = _maps(h_s, h_n, h_kv, noise_of_signal, kv_of_signal)
    w = np.ones(dv_) if norm_weight is None else _as64(norm_weight).reshape(dv_)
    c = 1.0 - lambda_init
    scale = 1.0 / math.sqrt(d)
    g = {k: np.zeros_like(x) for k, x in (("dq1", q1), ("dq2", q2), ("dk1", k1), ("dk2", k2), ("dv", v))}
    dlam = 0.0
    dlam_sq = 0.0
    dw = np.zeros(dv_)
    hidden = np.triu(np.ones((N, N), bool), 1) if causal else np.zeros((N, N), bool)
    for b in range(B):
        for h in range(h_s):
            n, k = nz[h], kv[h]
            s1 = np.where(hidden, -np.inf, (q1[b, :, h] @ k1[b, :, k].T) * scale)
            s2 = np.where(hidden, -np.inf, (q2[b, :, n] @ k2[b, :, n].T) * scale)
            a1, a2 = softmax_rows(s1), softmax_rows(s2)
            vv = v[b, :, k]
            o1, o2 = a1 @ vv, a2 @ vv
            o = o1 - lam * o2
            gy = dy[b, :, h]
            if normalize:
                r = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
                gw = c * w * gy
                do = gw / r - o * np.sum(gw * o, axis=-1, keepdims=True) / (dv_ * r ** 3)
                dw += np.sum(gy * c * o / r, axis=0)
            else:
                do = gy
            dlam -= float(np.sum(do * o2))
            dlam_sq += float(np.sum((do * o2) ** 2))
            dp = do @ vv.T
            g["dv"][b, :, k] += (a1 - lam * a2).T @ do
            ds1 = a1 * (dp - np.sum(a1 * dp, axis=-1, keepdims=True))
            da2 = -lam * dp
            ds2 = a2 * (da2 - np.sum(a2 * da2, axis=-1, keepdims=True))
            g["dq1"][b, :, h] += ds1 @ k1[b, :, k] * scale
            g["dk1"][b, :, k] += ds1.T @ q1[b, :, h] * scale
            g["dq2"][b, :, n] += ds2 @ k2[b, :, n] * scale
            g["dk2"][b, :, n] += ds2.T @ q2[b, :, n] * scale
    g["dlambda"] = dlam
    g["dlambda_scale"] = math.sqrt(dlam_sq)
    if norm_weight is not None and normalize:
        g["dnorm_weight"] = dw
    return g


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP 8-bit e4m3 ("fn") codes, the low-bit KV cache format the
    serving section of [DA-blog] ("Hardware Implementations and Serving
    Considerations") points at: bit 7 the sign, bits 6-3 the exponent with
    bias 7, bits 2-0 the mantissa; exponent 0 is subnormal (m/8 * 2^-6); the
    all-ones exponent and mantissa is NaN; there are no infinities."""
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(sign == 1, -val, val)


def gda_decode_fp8(q1, q2, k1_codes, k2_codes, v_codes, scales, seq_lens, lam: float, lambda_init: float,
                   **kw) -> np.ndarray:
    """``gda_decode`` on caches stored as e4m3 codes: each cache is read as its
    decoded value times its scale (scales = (k1, k2, v))."""
    k1, k2, v = (fp8_e4m3_decode(_as_codes(c)) * float(sc) for c, sc in zip((k1_codes, k2_codes, v_codes), scales))
    return gda_decode(q1, q2, k1, k2, v, seq_lens, lam, lambda_init, **kw)


def _as_codes(x) -> np.ndarray:
    """uint8 codes from a NumPy array or a (CPU or device) uint8 torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x)


# ---------------------------------------------------------------------------
# Brute force: literal loops for tiny inputs (pins the vectorised oracle)
# ---------------------------------------------------------------------------

def brute_diff_attention(q1, q2, k1, k2, v, lam, lambda_init, *, eps=1e-5, causal=True,
                         noise_of_signal=None, kv_of_signal=None, normalize=True):
    """Pure-Python scalar loops over the same definition; only for N, d tiny."""
    q1, q2, k1, k2, v = (_as64(t).tolist() for t in (q1, q2, k1, k2, v))
    B, N, h_s, d = len(q1), len(q1[0]), len(q1[0][0]), len(q1[0][0][0])
    h_n, h_kv, dv = len(q2[0][0]), len(k1[0][0]), len(v[0][0][0])
    nz = [h // (h_s // h_n) for h in range(h_s)] if noise_of_signal is None else list(noise_of_signal)
    kv = [h // (h_s // h_kv) for h in range(h_s)] if kv_of_signal is None else list(kv_of_signal)
    out = [[[[0.0] * dv for _ in range(h_s)] for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for h in range(h_s):
            for i in range(N):
                last = i if causal else N - 1
                s1, s2 = [], []
                for j in range(last + 1):
                    t1 = 0.0
                    t2 = 0.0
                    for c in range(d):
                        t1 += q1[b][i][h][c] * k1[b][j][kv[h]][c]
                        t2 += q2[b][i][nz[h]][c] * k2[b][j][nz[h]][c]
                    s1.append(t1 / math.sqrt(d))
                    s2.append(t2 / math.sqrt(d))
                e1 = [math.exp(x - max(s1)) for x in s1]
                e2 = [math.exp(x - max(s2)) for x in s2]
                z1, z2 = sum(e1), sum(e2)
                o = [0.0] * dv
                for j in range(last + 1):
                    wgt = e1[j] / z1 - lam * e2[j] / z2
                    for c in range(dv):
                        o[c] += wgt * v[b][j][kv[h]][c]
                if normalize:
                    ms = sum(x * x for x in o) / dv
                    o = [(1.0 - lambda_init) * x / math.sqrt(ms + eps) for x in o]
                out[b][i][h] = o
    return np.asarray(out, np.float64)


# ---------------------------------------------------------------------------
# Work accounting used by the benchmark's roofline
# ---------------------------------------------------------------------------

def causal_pairs(B: int, N: int) -> int:
    """Number of (query, key) pairs with key <= query: B * N (N + 1) / 2."""
    return B * N * (N + 1) // 2


def flops_alg(B, N, h_s, h_n, d, dv, causal=True) -> int:
    """Products the DiffAttn equation names, each counted once: Q1K1^T per
    signal head (2d per pair), Q2K2^T once per noise head (2d per pair), one
    (A1 - lam A2) V per signal head (2 dv per pair)."""
    pairs = causal_pairs(B, N) if causal else B * N * N
    return pairs * (h_s * 2 * d + h_n * 2 * d + h_s * 2 * dv)


def flops_exec(B, N, h_s, h_n, h_kv, d, dv, causal=True, noise_of_signal=None, kv_of_signal=None) -> int:
    """flops_alg plus the second P.V an exact one-pass kernel must issue: one
    more 2 dv per pair for every distinct (noise head, kv head) combination."""
    nz, kv = _maps(h_s, h_n, h_kv, noise_of_signal, kv_of_signal)
    distinct = len({(int(a), int(b)) for a, b in zip(nz, kv)})
    pairs = causal_pairs(B, N) if causal else B * N * N
    return flops_alg(B, N, h_s, h_n, d, dv, causal) + pairs * distinct * 2 * dv

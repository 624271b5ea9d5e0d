"""Seeded synthetic workloads: shapes, scalars and input generators.

Holds none of the method's arithmetic: it only draws seeded random tensors of
the shapes the differential-attention pages work with (3B-scale layers at 4K
tokens, long contexts, a serving batch) and names the per-call scalars.  Both
the oracle-side tests and the HIP side use these generators, so the two see
bit-identical inputs.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; float32 ``randn`` draws
in the order q1, q2, k1, k2, v (decode: q1, q2, k1_cache, k2_cache, v_cache,
then the cache lengths), each scaled by its standard deviation and then
rounded to the storage dtype (round-to-nearest-even for bf16).  Layout BSHD
(last dim contiguous) for prefill; [B, H, Lmax, D] caches for decode.  A
packed (varlen) prefill batch draws its B sequence lengths first (uniform
integers in len_range), then q1, q2, k1, k2, v as [T, H, D] with T the sum of
the lengths.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

# lambda_init of layer 12 under the depth schedule of the "Learnable Lambda
# Re-parameterization" section (0.8 - 0.6 exp(-0.3 * 11)); the 3B-like layer
# uses lambda = lambda_init + 0.05.  The CPU tests re-derive this constant
# from the oracle's schedule.
LAMBDA_INIT_L12 = 0.777870099559256


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill", "varlen" (packed prefill) or "decode"
    dtype: str           # "f32" or "bf16"
    B: int
    N: int               # prefill: sequence length; varlen: bound on lengths; decode: Lmax
    H_s: int
    H_n: int
    H_kv: int
    d: int
    dv: int
    lam: float
    lam_init: float
    eps: float = 1e-5
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0
    causal: bool = True
    len_range: tuple = field(default=(0, 0))   # decode / varlen: inclusive [lo, hi] of the lengths
    seed: int = 0
    cache: str = "same"  # decode: "same" (caches in dtype) or "fp8" (OCP e4m3 codes with per-cache scales)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    # tiny exact-path check: 1 x 128 tokens, 4 heads, d=32, fp32
    "tiny_diff_f32": Workload("tiny_diff_f32", "prefill", "f32", B=1, N=128, H_s=4, H_n=4, H_kv=4,
                              d=32, dv=64, lam=0.8, lam_init=0.8, seed=1000),
    # 3B-like Diff Transformer layer: d_model 3072 = 24 heads x 2 x 64, 4 x 4096 tokens
    "diff3b_bf16_n4096": Workload("diff3b_bf16_n4096", "prefill", "bf16", B=4, N=4096, H_s=24, H_n=24,
                                  H_kv=24, d=64, dv=128, lam=LAMBDA_INIT_L12 + 0.05,
                                  lam_init=LAMBDA_INIT_L12, seed=1001),
    # GDA 3:1 (18 signal heads over 6 noise heads), 4 x 4096 tokens
    "gda3to1_bf16_n4096": Workload("gda3to1_bf16_n4096", "prefill", "bf16", B=4, N=4096, H_s=18, H_n=6,
                                   H_kv=18, d=64, dv=128, lam=0.7, lam_init=0.7, seed=1002),
    # long-context GDA 4:1 with 8 GQA key/value heads, 32768 tokens, V ~ N(0, 0.5^2)
    "gda4to1_gqa_bf16_n32768": Workload("gda4to1_gqa_bf16_n32768", "prefill", "bf16", B=1, N=32768, H_s=16,
                                        H_n=4, H_kv=8, d=64, dv=128, lam=0.8, lam_init=0.8, v_std=0.5,
                                        seed=1003),
    # GDA serving step: 64 sequences, one new token each, caches of 4096..8192 positions
    "gda_decode_bf16_b64_l8192": Workload("gda_decode_bf16_b64_l8192", "decode", "bf16", B=64, N=8192, H_s=18,
                                          H_n=6, H_kv=6, d=64, dv=128, lam=0.75, lam_init=0.75,
                                          len_range=(4096, 8192), seed=1004),
    # the same serving step with fp8 (e4m3) caches, one scale per cache tensor
    "gda_decode_fp8_b64_l8192": Workload("gda_decode_fp8_b64_l8192", "decode", "bf16", B=64, N=8192, H_s=18,
                                         H_n=6, H_kv=6, d=64, dv=128, lam=0.75, lam_init=0.75,
                                         len_range=(4096, 8192), seed=1004, cache="fp8"),
    # serving-side prefill: 8 GDA 3:1 sequences of 256..4096 tokens packed in one call
    "gda3to1_varlen_bf16_8x4096": Workload("gda3to1_varlen_bf16_8x4096", "varlen", "bf16", B=8, N=4096, H_s=18,
                                           H_n=6, H_kv=18, d=64, dv=128, lam=0.7, lam_init=0.7,
                                           len_range=(256, 4096), seed=1005),
}

# workload order used by tests and docs (index = position in this list)
ORDER = ["tiny_diff_f32", "diff3b_bf16_n4096", "gda3to1_bf16_n4096",
         "gda4to1_gqa_bf16_n32768", "gda_decode_bf16_b64_l8192"]


def _draw(gen, shape, std, dtype):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype).contiguous()


def make_prefill_inputs(w: Workload, *, seed: int | None = None, N: int | None = None, B: int | None = None):
    """Seeded prefill inputs on the CPU: dict q1,q2,k1,k2,v in the storage dtype."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    B = w.B if B is None else B
    N = w.N if N is None else N
    dt = w.torch_dtype
    return {
        "q1": _draw(g, (B, N, w.H_s, w.d), w.q_std, dt),
        "q2": _draw(g, (B, N, w.H_n, w.d), w.q_std, dt),
        "k1": _draw(g, (B, N, w.H_kv, w.d), w.k_std, dt),
        "k2": _draw(g, (B, N, w.H_n, w.d), w.k_std, dt),
        "v": _draw(g, (B, N, w.H_kv, w.dv), w.v_std, dt),
    }


def make_varlen_inputs(w: Workload, *, seed: int | None = None, lengths=None):
    """Seeded packed-prefill inputs on the CPU: the B sequence lengths (drawn
    uniformly from len_range unless given), q1 [T,H_s,d], q2/k2 [T,H_n,d],
    k1 [T,H_kv,d], v [T,H_kv,dv] in the storage dtype, int32 cu_seqlens [B+1]
    and max_seqlen (the longest length, a host int)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    if lengths is None:
        lo, hi = w.len_range
        lengths = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64)
    lengths = torch.as_tensor(lengths, dtype=torch.int64).reshape(-1)
    T = int(lengths.sum())
    dt = w.torch_dtype
    out = {
        "q1": _draw(g, (T, w.H_s, w.d), w.q_std, dt),
        "q2": _draw(g, (T, w.H_n, w.d), w.q_std, dt),
        "k1": _draw(g, (T, w.H_kv, w.d), w.k_std, dt),
        "k2": _draw(g, (T, w.H_n, w.d), w.k_std, dt),
        "v": _draw(g, (T, w.H_kv, w.dv), w.v_std, dt),
    }
    out["cu_seqlens"] = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lengths, 0)]).to(torch.int32)
    out["max_seqlen"] = int(lengths.max()) if lengths.numel() else 0
    return out


def _fp8_codes(x: torch.Tensor):
    """OCP e4m3 codes of x / scale (round to nearest even) with scale = max|x| / 448,
    the largest finite e4m3 value; returns (uint8 codes, scale)."""
    scale = float(x.abs().max()) / 448.0 or 1.0
    return (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), scale


def make_decode_inputs(w: Workload, *, seed: int | None = None, B: int | None = None, Lmax: int | None = None,
                       len_range: tuple | None = None):
    """Seeded decode inputs on the CPU: q1 [B,H_s,d], q2 [B,H_n,d], caches
    [B,H,Lmax,D] and int32 seq_lens [B] drawn uniformly from len_range.  With
    fp8 caches the same fp32 draws are stored as e4m3 codes (uint8) and the
    per-cache scales are returned as "cache_scales" (k1, k2, v)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    B = w.B if B is None else B
    L = w.N if Lmax is None else Lmax
    lo, hi = w.len_range if len_range is None else len_range
    dt = w.torch_dtype
    cdt = torch.float32 if w.cache == "fp8" else dt
    out = {
        "q1": _draw(g, (B, w.H_s, w.d), w.q_std, dt),
        "q2": _draw(g, (B, w.H_n, w.d), w.q_std, dt),
        "k1_cache": _draw(g, (B, w.H_kv, L, w.d), w.k_std, cdt),
        "k2_cache": _draw(g, (B, w.H_n, L, w.d), w.k_std, cdt),
        "v_cache": _draw(g, (B, w.H_kv, L, w.dv), w.v_std, cdt),
    }
    out["seq_lens"] = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    if w.cache == "fp8":
        scales = []
        for k in ("k1_cache", "k2_cache", "v_cache"):
            out[k], sc = _fp8_codes(out[k])
            scales.append(sc)
        out["cache_scales"] = tuple(scales)
    return out

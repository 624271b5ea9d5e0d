"""GPU parity of the prefill entry points (diffattn_fwd, gda_fwd) against the
fp64 oracle, through the C ABI.

Small cases are compared element by element on every output (they span
several 128-query blocks / 64-key tiles and end on a ragged tail); the full
workloads run in the launch configuration the benchmark times and are compared
on sampled rows (block and tile edges plus random rows) that the oracle
computes one by one."""

import numpy as np
import pytest
import torch

from differential_attention_diff_amd import ops
from differential_attention_diff_amd import workloads as W
from oracle import diffattn_oracle as O
from tests.helpers import as64, assert_parity, norm_scale, rand_inputs, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def run(inp, lam, li, entry="gda", **kw):
    d = to_dev(inp)
    f = ops.gda_fwd if entry == "gda" else ops.diffattn_fwd
    out = f(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], lam, li, **kw)
    torch.cuda.synchronize()
    return out


def test_tiny_fp32_workload_full():
    w = W.WORKLOADS["tiny_diff_f32"]
    inp = W.make_prefill_inputs(w)
    out = run(inp, w.lam, w.lam_init, entry="diff")
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], w.lam, w.lam_init, eps=w.eps)
    print("tiny fp32 max-abs %.3e rel %.3e" % assert_parity(as64(out), want, "f32", "tiny fp32"))


@pytest.mark.parametrize("shape", [
    dict(B=1, N=77, hs=4, hn=2, hkv=2, d=32),
    dict(B=2, N=130, hs=6, hn=2, hkv=3, d=64),
])
@pytest.mark.parametrize("causal", [True, False])
def test_fp32_variants(shape, causal):
    inp = rand_inputs(**shape, dtype=torch.float32, seed=3)
    w = torch.linspace(0.5, 1.5, 2 * shape["d"], device="cuda")
    out = run(inp, 0.6, 0.3, causal=causal, norm_weight=w)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.6, 0.3, causal=causal,
                            norm_weight=as64(w))
    assert_parity(as64(out), want, "f32", f"fp32 {shape} causal={causal}")


BF16_SMALL = [
    dict(B=2, N=300, hs=4, hn=4, hkv=4, d=64),    # plain diff, ragged tail
    dict(B=1, N=257, hs=6, hn=2, hkv=6, d=64),    # GDA 3:1
    dict(B=1, N=200, hs=8, hn=2, hkv=4, d=64),    # GDA 4:1 + GQA
    dict(B=2, N=190, hs=4, hn=2, hkv=2, d=32),    # d = 32
    dict(B=1, N=1, hs=2, hn=2, hkv=2, d=64),      # one token
    dict(B=1, N=33, hs=3, hn=1, hkv=1, d=64),     # one noise head for all, MQA
]


@pytest.mark.parametrize("shape", BF16_SMALL, ids=lambda s: "B{B}N{N}hs{hs}hn{hn}hkv{hkv}d{d}".format(**s))
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_small_full(shape, causal):
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=11)
    out = run(inp, 0.8, 0.7, causal=causal)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.8, 0.7, causal=causal)
    ma, rel = assert_parity(as64(out), want, "bf16", f"bf16 {shape} causal={causal}")
    print(f"{shape} causal={causal}: max-abs {ma:.3e} rel-L2 {rel:.3e}")


def test_bf16_plain_entry_matches_gda_entry():
    inp = rand_inputs(B=1, N=150, hs=4, hn=4, hkv=4, d=64, dtype=torch.bfloat16, seed=12)
    a = run(inp, 0.5, 0.5, entry="diff")
    b = run(inp, 0.5, 0.5, entry="gda")
    assert torch.equal(a, b)


def test_bf16_no_norm_and_weight_and_lse():
    shape = dict(B=2, N=160, hs=6, hn=3, hkv=2, d=64)
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=13)
    raw = run(inp, 0.7, 0.7, normalize=False)
    want_raw = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.7, 0.7, normalize=False)
    sc = norm_scale(want_raw, 0.7)
    ma, rel = assert_parity(as64(raw) * sc, want_raw * sc, "bf16", "raw DiffAttn output")
    w = torch.linspace(-1.0, 2.0, 128, device="cuda")
    lse = torch.empty(2, 2, 6, 160, device="cuda")
    out = run(inp, 0.7, 0.7, norm_weight=w, lse=lse)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.7, 0.7, norm_weight=as64(w))
    assert_parity(as64(out), want, "bf16", "norm weight")
    want_lse = O.diff_attention_lse(inp["q1"], inp["q2"], inp["k1"], inp["k2"], rows=np.arange(160))
    got_lse = as64(lse).transpose(0, 1, 3, 2)  # [2,B,H,N] -> [2,B,N,H]
    # l sums the bf16-rounded weights (relative rounding <= 2^-9 each), so |d lse| <= log(1 + 2^-9)
    # plus fp32 accumulation: bound 2^-8
    assert np.max(np.abs(got_lse - want_lse)) <= 2.0 ** -8


def test_bf16_explicit_maps():
    shape = dict(B=1, N=140, hs=6, hn=2, hkv=3, d=64)
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=14)
    nz, kv = [1, 0, 1, 0, 0, 1], [2, 2, 0, 1, 0, 1]
    out = run(inp, 0.9, 0.6, noise_of_signal=nz, kv_of_signal=kv)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.9, 0.6,
                            noise_of_signal=nz, kv_of_signal=kv)
    assert_parity(as64(out), want, "bf16", "explicit maps")


def test_bf16_packed_projection_views():
    # Q1|Q2 and K1|K2 as the two halves of packed [B,N,H,2d] projections (non-contiguous views)
    B, N, H, d = 2, 180, 4, 64
    g = torch.Generator("cpu").manual_seed(15)
    qp = torch.randn(B, N, H, 2 * d, generator=g).bfloat16()
    kp = torch.randn(B, N, H, 2 * d, generator=g).bfloat16()
    v = torch.randn(B, N, H, 2 * d, generator=g).bfloat16()
    out_dev = torch.empty(B, N, H, 2 * d, dtype=torch.bfloat16, device="cuda")
    qd, kd, vd = qp.cuda(), kp.cuda(), v.cuda()
    ops.diffattn_fwd(qd[..., :d], qd[..., d:], kd[..., :d], kd[..., d:], vd, 0.8, 0.8, out=out_dev)
    torch.cuda.synchronize()
    want = O.diff_attention(qp[..., :d], qp[..., d:], kp[..., :d], kp[..., d:], v, 0.8, 0.8)
    assert_parity(as64(out_dev), want, "bf16", "packed views")
    ref = run({"q1": qp[..., :d].contiguous(), "q2": qp[..., d:].contiguous(), "k1": kp[..., :d].contiguous(),
               "k2": kp[..., d:].contiguous(), "v": v}, 0.8, 0.8, entry="diff")
    assert torch.equal(ref, out_dev)


def test_empty_inputs_are_noops():
    for B, N in ((0, 64), (2, 0)):
        inp = rand_inputs(B=B, N=N, hs=2, hn=2, hkv=2, d=64, dtype=torch.bfloat16, seed=1)
        out = run(inp, 0.5, 0.5)
        assert out.numel() == 0


@pytest.mark.parametrize("name", ["diff3b_bf16_n4096", "gda3to1_bf16_n4096", "gda4to1_gqa_bf16_n32768"])
def test_full_workload_sampled_rows(name):
    w = W.WORKLOADS[name]
    inp = W.make_prefill_inputs(w)
    print(f"[{name}] inputs ready", flush=True)
    # completeness: every output element is written (a NaN sentinel must not survive anywhere)
    out = torch.full((w.B, w.N, w.H_s, w.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    run(inp, w.lam, w.lam_init, entry="diff" if w.H_n == w.H_s and w.H_kv == w.H_s else "gda", out=out)
    assert bool(torch.isfinite(out).all()), f"{name}: some outputs were not written"
    rows = sample_rows(w.N, 12 if w.N > 8192 else 24, seed=w.seed)
    heads = list(range(w.H_s))
    want = O.diff_attention_rows(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], w.lam, w.lam_init,
                                 rows=rows, heads=heads, eps=w.eps)
    got = as64(out[:, rows])
    ma, rel = assert_parity(got, want, "bf16", name)
    print(f"[{name}] {len(rows)} rows x {w.B} x {w.H_s} heads: max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)


def test_gda3to1_whole_noise_group_element_by_element():
    # every output of one (batch, noise group) slab of the 3:1 workload -- its three
    # signal heads over all 4096 queries -- against the oracle, in the bench's launch
    w = W.WORKLOADS["gda3to1_bf16_n4096"]
    inp = W.make_prefill_inputs(w)
    out = run(inp, w.lam, w.lam_init)
    b, n = 2, 4  # batch 2, noise group 4: signal heads 12, 13, 14
    heads = [3 * n, 3 * n + 1, 3 * n + 2]
    want = O.diff_attention_rows(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], w.lam, w.lam_init,
                                 rows=np.arange(w.N), heads=heads, batches=[b], eps=w.eps)
    got = as64(out[b:b + 1, :, heads[0]:heads[-1] + 1])
    ma, rel = assert_parity(got, want, "bf16", "3:1 slab")
    print(f"[gda3to1 slab b={b} group={n}] {w.N} rows x 3 heads: max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)


@pytest.mark.parametrize("lam", [0.958, 0.99, 0.999])
@pytest.mark.parametrize("shape", [dict(B=1, N=384, hs=9, hn=3, hkv=9, d=64), dict(B=2, N=300, hs=4, hn=4, hkv=4, d=64)],
                         ids=["gda3to1", "plain"])
def test_bf16_near_lambda_one_within_conditioned_bar(shape, lam):
    """As lambda approaches 1 the two maps nearly cancel on some early causal
    rows, and the head norm ("Headwise Normalization", head_bar_i equation)
    divides such a row by its small RMS.  The bf16 rounding of each map's
    weights enters o1 and o2 separately, so on the normalised output it grows
    with the row's conditioning kappa = (rms(o1) + |lambda| rms(o2)) /
    rms(o1 - lambda o2).  The fixed bf16 bar is the one for rows with kappa <= 3
    (the median row here has kappa ~1.8); past that it scales with kappa.  A
    CPU emulation of the bf16 weights (row-max reference) stays within 0.74 of
    this bar at lambda 0.5 ... 0.999 on these shapes, and reproduces the 0.105
    error that the 3:1 layer with seed 1038 shows at lambda = 0.958."""
    li = 0.22
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=1038 if shape["hs"] == 9 else 15)
    got = as64(run(inp, lam, li, causal=True))
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], lam, li, causal=True)
    o1, o2 = O.diff_attention_maps(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], causal=True)
    rms = lambda x: np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    diff = o1 - lam * o2
    kappa = (rms(o1) + abs(lam) * rms(o2)) / np.sqrt(rms(diff) ** 2 + 1e-5)
    bar = 2e-2 * np.maximum(1.0, kappa / 3.0)
    assert np.all(np.isfinite(got))
    ratio = np.abs(got - want) / bar
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    print(f"{shape} lam={lam}: max err/bar {ratio.max():.3f}, max kappa {kappa.max():.1f}, rel-L2 {rel:.3e}")
    worst = np.unravel_index(ratio.argmax(), ratio.shape)
    assert ratio.max() <= 1.0, f"max err/bar {ratio.max():.3f} at {worst}, kappa {kappa[worst[:-1]][0]:.1f}"
    assert rel <= 5e-3, f"rel-L2 {rel:.3e}"

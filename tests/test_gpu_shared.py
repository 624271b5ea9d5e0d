"""GPU parity of the bf16 prefill for layers whose signal heads share noise and
key/value heads ("combos" of 2, 4 or 8 heads with the same noise head and the
same key/value head: GQA key/value heads under GDA noise heads), through
gda_fwd, against the fp64 oracle.

That path forms A2 V once per combo in a first launch, parks it in the combo's
own output rows, and a second launch forms every member's map 1 over shared
K1/V tiles and combines the two.  The tests aim at what this can get wrong:
each combo size (32, 64 and 128 queries per signal workgroup), ragged query
blocks of both launches (256 queries for the map-2 launch), several combos per
noise group and explicit head maps, the parked rows (every output written
after every parked row was read), the per-map outputs and LSE the backward
reads, the exact cancellation of identical maps (both launches must take
identical arithmetic), and bit-identity with the general kernel, which the
same call takes when the output rows are not nested row-major.

Pages: "Grouped Differential Attention" (mlsanity.com), "Abstract" (noise heads
shared GQA-style); "Differential Attention in Large Language Models: How
Denoising Subtraction Eliminates Attention Noise and Outlier Activations"
(llms.blog), "Differential Attention Architecture" (DiffAttn equation) and
"Headwise Normalization" (head_bar_i)."""

import numpy as np
import pytest
import torch

from differential_attention_diff_amd import ops
from oracle import diffattn_oracle as O
from tests.helpers import as64, assert_parity, norm_scale, rand_inputs, to_dev

pytestmark = pytest.mark.gpu


def fwd(inp, lam, li, **kw):
    d = to_dev(inp)
    out = ops.gda_fwd(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], lam, li, **kw)
    torch.cuda.synchronize()
    return out


SHAPES = [
    dict(B=2, N=1, hs=2, hn=1, hkv=1, d=64),      # combos of 2, one token
    dict(B=1, N=33, hs=4, hn=1, hkv=1, d=64),     # combos of 4, one key past a tile
    dict(B=1, N=97, hs=8, hn=1, hkv=1, d=64),     # combos of 8 (32 queries per workgroup), ragged
    dict(B=2, N=300, hs=8, hn=2, hkv=4, d=64),    # 4:1 GDA on 2:1 GQA: two combos of 2 per noise group
    dict(B=1, N=520, hs=8, hn=2, hkv=2, d=64),    # combos of 4, three map-2 blocks, ragged
    dict(B=1, N=700, hs=16, hn=2, hkv=2, d=64),   # combos of 8, 22 query blocks
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{B}N{N}hs{hs}hn{hn}hkv{hkv}".format(**s))
@pytest.mark.parametrize("causal", [True, False])
def test_every_output(shape, causal):
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=61)
    out = fwd(inp, 0.7, 0.7, causal=causal)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.7, 0.7, causal=causal)
    ma, rel = assert_parity(as64(out), want, "bf16", f"shared {shape} causal={causal}")
    print(f"shared {shape} causal={causal}: max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)


def test_explicit_maps_and_weight():
    # noise group 0 = heads {1, 2, 5, 7} on key/value heads {0, 1, 1, 0}: combos {1, 7}, {2, 5};
    # noise group 1 = heads {0, 3, 4, 6} on {3, 2, 3, 2}: combos {0, 4}, {3, 6}
    shape = dict(B=1, N=230, hs=8, hn=2, hkv=4, d=64)
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=62)
    nz = [1, 0, 0, 1, 1, 0, 1, 0]
    kv = [3, 0, 1, 2, 3, 1, 2, 0]
    w = torch.linspace(-1.0, 2.0, 128, device="cuda")
    out = fwd(inp, 0.9, 0.6, noise_of_signal=nz, kv_of_signal=kv, norm_weight=w)
    # the general kernel on the same call (non-nested output rows)
    gen = torch.empty(1, 8, 230, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    fwd(inp, 0.9, 0.6, noise_of_signal=nz, kv_of_signal=kv, norm_weight=w, out=gen)
    assert torch.equal(out, gen.contiguous())
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.9, 0.6,
                            noise_of_signal=nz, kv_of_signal=kv, norm_weight=as64(w))
    # the weight multiplies each channel after the norm, so the unit-weight bar
    # applies to the outputs divided by max |w| = 2 (both kernels: max-abs 2.03e-2
    # before the division, on rows where o1 - lambda o2 nearly cancels)
    assert_parity(as64(out) / 2.0, want / 2.0, "bf16", "shared explicit maps")


@pytest.mark.parametrize("shape", [dict(B=2, N=160, hs=4, hn=1, hkv=2, d=64),
                                   dict(B=1, N=290, hs=8, hn=2, hkv=2, d=64)],
                         ids=["combos2", "combos4"])
@pytest.mark.parametrize("causal", [True, False])
def test_raw_output_maps_and_lse(shape, causal):
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=63)
    B, N, H = shape["B"], shape["N"], shape["hs"]
    lse = torch.full((2, B, H, N), -7.0, device="cuda")
    om = torch.full((2, B, N, H, 128), float("nan"), device="cuda")
    raw = fwd(inp, 0.8, 0.8, normalize=False, causal=causal, lse=lse, o_maps=om)
    want_raw = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.8, 0.8,
                                normalize=False, causal=causal)
    sc = norm_scale(want_raw, 0.8)
    assert_parity(as64(raw) * sc, want_raw * sc, "bf16", "shared raw output")
    maps = O.diff_attention_maps(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], causal=causal)
    got = as64(om)
    for i in range(2):  # each map's own output in fp32: its bf16 weights, <= 2^-9 relative each
        err = np.max(np.abs(got[i] - maps[i]))
        assert err <= 2.0 ** -7 * max(1.0, np.max(np.abs(maps[i]))), f"map {i + 1}: {err:.3e}"
    want_lse = O.diff_attention_lse(inp["q1"], inp["q2"], inp["k1"], inp["k2"], rows=np.arange(N), causal=causal)
    got_lse = as64(lse).transpose(0, 1, 3, 2)
    assert np.max(np.abs(got_lse - want_lse)) <= 2.0 ** -8


def test_identical_maps_cancel_exactly():
    # two noise heads, each over two signal heads on the noise head's own key/value
    # head; every signal head's Q1/K1 equals its noise head's Q2/K2 and lambda = 1,
    # so A1 = A2 and o = 0 exactly, though the map-1 and map-2 outputs come from
    # different launches
    inp = rand_inputs(B=2, N=300, hs=4, hn=2, hkv=2, d=64, dtype=torch.bfloat16, seed=64)
    inp["q1"] = inp["q2"].repeat_interleave(2, dim=2).contiguous()
    inp["k1"] = inp["k2"].clone()
    for normalize in (True, False):
        out = fwd(inp, 1.0, 0.8, normalize=normalize)
        assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("causal", [True, False])
def test_bitwise_equal_to_general_kernel(causal):
    # an output view whose head rows are not nested row-major ([B, H, N, dv]
    # storage seen as [B, N, H, dv]) sends the same call to the general kernel;
    # outputs, LSE and per-map outputs agree bit for bit
    shape = dict(B=2, N=333, hs=8, hn=2, hkv=4, d=64)
    B, N, H = shape["B"], shape["N"], shape["hs"]
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=65)
    w = torch.linspace(0.5, 1.5, 128, device="cuda")
    res = []
    for nested in (True, False):
        out = (torch.empty(B, N, H, 128, dtype=torch.bfloat16, device="cuda") if nested
               else torch.empty(B, H, N, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2))
        lse = torch.empty(2, B, H, N, device="cuda")
        om = torch.empty(2, B, N, H, 128, device="cuda")
        fwd(inp, 0.75, 0.6, causal=causal, out=out, lse=lse, o_maps=om, norm_weight=w)
        res.append((out.contiguous(), lse, om))
    for a, b, what in zip(res[0], res[1], ("out", "lse", "o_maps")):
        assert torch.equal(a, b), what
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.75, 0.6, causal=causal,
                            norm_weight=as64(w))
    assert_parity(as64(res[0][0]), want, "bf16", "shared vs oracle")


def test_climbing_scores():
    # scores of both maps climb along the keys, so the lazy references of both
    # launches move again and again
    B, N, d = 1, 600, 64
    g = torch.Generator().manual_seed(66)
    e = torch.full((d,), 0.125)
    ramp = (torch.arange(N, dtype=torch.float32) / 2.0)[None, :, None, None] * e
    inp = {"q1": (torch.randn(B, N, 4, d, generator=g) + e).bfloat16(),
           "q2": (torch.randn(B, N, 1, d, generator=g) + e).bfloat16(),
           "k1": (torch.randn(B, N, 2, d, generator=g) + ramp).bfloat16(),
           "k2": (torch.randn(B, N, 1, d, generator=g) + 0.8 * ramp).bfloat16(),
           "v": torch.randn(B, N, 2, 2 * d, generator=g).bfloat16()}
    lse = O.diff_attention_lse(inp["q1"], inp["q2"], inp["k1"], inp["k2"], rows=np.arange(N), causal=True)
    assert np.min(lse[1][:, -1, :]) - np.max(lse[1][:, :32, :]) > 20.0  # the noise map climbs too
    for causal in (True, False):
        got = fwd(inp, 0.6, 0.6, causal=causal)
        want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.6, 0.6, causal=causal)
        assert_parity(as64(got), want, "bf16", f"shared climbing causal={causal}")


def test_full_gqa_workload_bitwise_equal_to_general_kernel():
    # the 32k-token 4:1 GDA layer on 2:1 GQA key/value heads (the benchmark's
    # launch): every output element of the two-launch path equals the general
    # kernel's.  The parked A2 V rows are finite numbers when read as bf16, so a
    # NaN sentinel alone could not show that every output row was rewritten; the
    # general kernel's output is sentinel-checked and the two must agree bit for bit
    # (sampled rows of both against the oracle: tests/test_gpu_prefill.py).
    from differential_attention_diff_amd import workloads as W
    w = W.WORKLOADS["gda4to1_gqa_bf16_n32768"]
    inp = W.make_prefill_inputs(w)
    shared = fwd(inp, w.lam, w.lam_init)
    gen = torch.full((w.B, w.H_s, w.N, w.dv), float("nan"), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    fwd(inp, w.lam, w.lam_init, out=gen)
    assert bool(torch.isfinite(gen).all()), "general kernel: some outputs were not written"
    assert torch.equal(shared, gen.contiguous())

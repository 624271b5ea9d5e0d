"""GPU parity of the per-noise-group bf16 prefill (three signal heads per noise
head, each on its own key/value head: the 3:1 GDA layout), through gda_fwd,
against the fp64 oracle.  (Packed sequences of that layout run the general
kernel: tests/test_gpu_varlen.py.)

This kernel computes each noise map once per group and hands its weights to
the signal wavefronts through LDS, so the tests aim at what that hand-off can
get wrong: ragged query blocks (64 queries) and key tiles (32 keys), several
groups and explicit head maps, the reference moves of the noise map (published
with the weights and applied by the other wavefronts), the exact cancellation
of identical maps (which needs both maps to take identical arithmetic), the
per-map outputs and LSE the backward reads.

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
    dict(B=2, N=1, hs=3, hn=1, hkv=3, d=64),      # one token
    dict(B=1, N=33, hs=3, hn=1, hkv=3, d=64),     # one key past a tile
    dict(B=2, N=95, hs=6, hn=2, hkv=6, d=64),     # ragged second query group
    dict(B=1, N=257, hs=9, hn=3, hkv=9, d=64),    # three groups, ragged tail
    dict(B=1, N=640, hs=3, hn=1, hkv=3, d=64),    # ten query blocks, twenty key tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{B}N{N}hs{hs}".format(**s))
@pytest.mark.parametrize("causal", [True, False])
def test_every_output(shape, causal):
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=51)
    out = fwd(inp, 0.7, 0.7, causal=causal)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.7, 0.7, causal=causal)
    ma, rel = assert_parity(as64(out), want, "bf16", f"gda3 {shape} causal={causal}")
    print(f"gda3 {shape} causal={causal}: max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)


def test_explicit_maps_and_weight():
    # groups {4, 0, 7}, {2, 8, 5}, {1, 6, 3} on permuted key/value heads
    shape = dict(B=1, N=190, hs=9, hn=3, hkv=9, d=64)
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=52)
    nz = [0, 2, 1, 2, 0, 1, 2, 0, 1]
    kv = [3, 8, 0, 5, 1, 7, 2, 6, 4]
    w = torch.linspace(-1.0, 2.0, 128, device="cuda")
    out = fwd(inp, 0.9, 0.6, noise_of_signal=nz, kv_of_signal=kv, norm_weight=w)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.9, 0.6,
                            noise_of_signal=nz, kv_of_signal=kv, norm_weight=as64(w))
    assert_parity(as64(out), want, "bf16", "gda3 explicit maps")


@pytest.mark.parametrize("causal", [True, False])
def test_raw_output_maps_and_lse(causal):
    shape = dict(B=2, N=160, hs=6, hn=2, hkv=6, d=64)
    inp = rand_inputs(**shape, dtype=torch.bfloat16, seed=53)
    B, N, H = 2, 160, 6
    lse = torch.full((2, B, H, N), -7.0, device="cuda")
    om = torch.full((2, B, N, H, 128), float("nan"), device="cuda")
    raw = fwd(inp, 0.8, 0.8, normalize=False, causal=causal, lse=lse, o_maps=om)
    want_raw = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.8, 0.8,
                                normalize=False, causal=causal)
    sc = norm_scale(want_raw, 0.8)
    assert_parity(as64(raw) * sc, want_raw * sc, "bf16", "gda3 raw output")
    maps = O.diff_attention_maps(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], causal=causal)
    got = as64(om)
    for i in range(2):  # each map's own output in fp32: its bf16 weights, <= 2^-9 relative each
        err = np.max(np.abs(got[i] - maps[i]))
        assert err <= 2.0 ** -7 * max(1.0, np.max(np.abs(maps[i]))), f"map {i + 1}: {err:.3e}"
    want_lse = O.diff_attention_lse(inp["q1"], inp["q2"], inp["k1"], inp["k2"], rows=np.arange(N), causal=causal)
    got_lse = as64(lse).transpose(0, 1, 3, 2)
    assert np.max(np.abs(got_lse - want_lse)) <= 2.0 ** -8


def test_identical_maps_cancel_exactly():
    # every signal head's Q1/K1 equals its noise head's Q2/K2 and lambda = 1: A1 = A2
    # for all three heads of a group, so o = 0 exactly (distinct V per head)
    inp = rand_inputs(B=2, N=300, hs=6, hn=2, hkv=6, d=64, dtype=torch.bfloat16, seed=54)
    inp["q1"] = inp["q2"].repeat_interleave(3, dim=2).contiguous()
    inp["k1"] = inp["k2"].repeat_interleave(3, dim=2).contiguous()
    for normalize in (True, False):
        out = fwd(inp, 1.0, 0.8, normalize=normalize)
        assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("causal", [True, False])
def test_both_maps_climbing(causal):
    # Scores of both maps climb along the keys, so the lazy references of the
    # signal maps and of the shared noise map move again and again; each move of
    # the noise map must reach the two signal wavefronts' share of A2 V.
    B, N, H, d = 1, 600, 3, 64
    g = torch.Generator().manual_seed(55)
    e = torch.full((d,), 0.125)
    ramp = (torch.arange(N, dtype=torch.float32) / 2.0)[None, :, None, None] * e
    inp = {"q1": (torch.randn(B, N, H, d, generator=g) + e).bfloat16(),
           "q2": (torch.randn(B, N, 1, d, generator=g) + e).bfloat16(),
           "k1": (torch.randn(B, N, H, d, generator=g) + ramp).bfloat16(),
           "k2": (torch.randn(B, N, 1, d, generator=g) + 0.8 * ramp).bfloat16(),
           "v": torch.randn(B, N, H, 2 * d, generator=g).bfloat16()}
    lse = O.diff_attention_lse(inp["q1"], inp["q2"], inp["k1"], inp["k2"], rows=np.arange(N), causal=True)
    assert np.min(lse[1][:, -1, :]) - np.max(lse[1][:, :32, :]) > 20.0  # the noise map climbs too
    got = fwd(inp, 0.6, 0.6, causal=causal)
    want = O.diff_attention(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], 0.6, 0.6, causal=causal)
    assert_parity(as64(got), want, "bf16", f"gda3 climbing causal={causal}")

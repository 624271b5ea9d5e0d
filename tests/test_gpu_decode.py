"""GPU parity of gda_decode (split-K partial + combine) against the fp64
oracle, through the C ABI: the full serving workload (every output), ragged
and edge-case lengths, split-count independence, general head maps, and the
decode = last-prefill-row property."""

import numpy as np
import pytest
import torch

from differential_attention_diff_amd import ops
from differential_attention_diff_amd import workloads as W
from oracle import diffattn_oracle as O
from tests.helpers import as64, assert_parity, err_stats, norm_scale, to_dev

pytestmark = pytest.mark.gpu


def decode_inputs(B, L, hs, hn, hkv, lens, seed, d=64):
    g = torch.Generator("cpu").manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g).bfloat16()
    return {"q1": mk(B, hs, d), "q2": mk(B, hn, d), "k1_cache": mk(B, hkv, L, d), "k2_cache": mk(B, hn, L, d),
            "v_cache": mk(B, hkv, L, 2 * d), "seq_lens": torch.tensor(lens, dtype=torch.int32)}


def run(inp, lam, li, **kw):
    d = to_dev(inp)
    out = ops.gda_decode(d["q1"], d["q2"], d["k1_cache"], d["k2_cache"], d["v_cache"], d["seq_lens"], lam, li, **kw)
    torch.cuda.synchronize()
    return out


def oracle(inp, lam, li, **kw):
    return O.gda_decode(inp["q1"], inp["q2"], inp["k1_cache"], inp["k2_cache"], inp["v_cache"], inp["seq_lens"],
                        lam, li, **kw)


def test_small_ragged_lengths():
    lens = [1, 2, 63, 64, 65, 511, 512, 513, 700, 1000]
    inp = decode_inputs(len(lens), 1000, 6, 2, 2, lens, seed=21)
    out = run(inp, 0.75, 0.75)
    ma, rel = assert_parity(as64(out), oracle(inp, 0.75, 0.75), "bf16", "ragged decode")
    print(f"ragged decode max-abs {ma:.3e} rel {rel:.3e}")


@pytest.mark.parametrize("chunk", [128, 256, 1024, 2048])
def test_split_count_independence(chunk):
    lens = [4096, 3001, 1, 2048]
    inp = decode_inputs(4, 4096, 6, 2, 2, lens, seed=22)
    want = oracle(inp, 0.6, 0.5)
    out = run(inp, 0.6, 0.5, chunk=chunk)
    assert_parity(as64(out), want, "bf16", f"chunk={chunk}")
    ref = run(inp, 0.6, 0.5, chunk=256)
    ma, _ = err_stats(as64(out), as64(ref))
    assert ma <= 2 * 2.0 ** -8  # differs from the default split by bf16 rounding only


def test_zero_length_rows_are_zero():
    inp = decode_inputs(3, 256, 4, 2, 2, [0, 256, 0], seed=23)
    out = run(inp, 0.7, 0.7)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    assert_parity(as64(out), oracle(inp, 0.7, 0.7), "bf16", "zero-length")


def test_general_maps_and_no_norm_and_weight():
    # 8 signal heads, 2 noise heads, 4 kv heads; a group spans two kv heads (u = 2)
    inp = decode_inputs(3, 700, 8, 2, 4, [700, 333, 64], seed=24)
    out = run(inp, 0.8, 0.6)
    assert_parity(as64(out), oracle(inp, 0.8, 0.6), "bf16", "GDA 4:1 + GQA decode")
    nz, kv = [1, 1, 0, 0, 1, 0, 0, 1], [3, 0, 2, 1, 1, 3, 0, 2]
    out = run(inp, 0.8, 0.6, noise_of_signal=nz, kv_of_signal=kv)
    assert_parity(as64(out), oracle(inp, 0.8, 0.6, noise_of_signal=nz, kv_of_signal=kv), "bf16", "explicit maps")
    raw = run(inp, 0.8, 0.6, normalize=False)
    want = oracle(inp, 0.8, 0.6, normalize=False)
    sc = norm_scale(want, 0.6)
    assert_parity(as64(raw) * sc, want * sc, "bf16", "raw decode")
    w = torch.linspace(-0.5, 1.5, 128, device="cuda")
    out = run(inp, 0.8, 0.6, norm_weight=w)
    assert_parity(as64(out), oracle(inp, 0.8, 0.6, norm_weight=as64(w)), "bf16", "norm weight")


def test_decode_is_last_prefill_row():
    B, N, hs, hn, hkv = 2, 300, 6, 2, 2
    g = torch.Generator("cpu").manual_seed(25)
    mk = lambda *s: torch.randn(*s, generator=g).bfloat16()
    q1, q2, k1, k2, v = mk(B, N, hs, 64), mk(B, N, hn, 64), mk(B, N, hkv, 64), mk(B, N, hn, 64), mk(B, N, hkv, 128)
    pre = ops.gda_fwd(q1.cuda(), q2.cuda(), k1.cuda(), k2.cuda(), v.cuda(), 0.7, 0.7)
    t = lambda x: x.transpose(1, 2).contiguous()  # BSHD -> [B,H,L,D]
    dec = ops.gda_decode(q1[:, -1].cuda(), q2[:, -1].cuda(), t(k1).cuda(), t(k2).cuda(), t(v).cuda(),
                         torch.full((B,), N, dtype=torch.int32, device="cuda"), 0.7, 0.7)
    torch.cuda.synchronize()
    ma, _ = err_stats(as64(dec), as64(pre[:, -1]))
    assert ma <= 2 * 2.0 ** -7


def test_full_serving_workload_every_output():
    w = W.WORKLOADS["gda_decode_bf16_b64_l8192"]
    inp = W.make_decode_inputs(w)
    print("[decode] inputs ready", flush=True)
    out = run(inp, w.lam, w.lam_init)
    want = oracle(inp, w.lam, w.lam_init)
    ma, rel = assert_parity(as64(out), want, "bf16", "serving decode")
    print(f"[decode] {w.B}x{w.H_s} outputs: max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)


# --- fp8 (OCP e4m3) caches -------------------------------------------------------------------

def fp8_inputs(B, L, hs, hn, hkv, lens, seed, d=64):
    """bf16 queries; caches drawn in fp32, stored as e4m3 codes of x / scale (scale = max|x| / 448)."""
    g = torch.Generator("cpu").manual_seed(seed)
    out = {"q1": torch.randn(B, hs, d, generator=g).bfloat16(), "q2": torch.randn(B, hn, d, generator=g).bfloat16(),
           "seq_lens": torch.tensor(lens, dtype=torch.int32)}
    scales = []
    for k, h, w in (("k1_cache", hkv, d), ("k2_cache", hn, d), ("v_cache", hkv, 2 * d)):
        x = torch.randn(B, h, L, w, generator=g)
        sc = float(x.abs().max()) / 448.0
        out[k] = (x / sc).to(torch.float8_e4m3fn).view(torch.uint8)
        scales.append(sc)
    return out, tuple(scales)


def fp8_oracle(inp, scales, lam, li, **kw):
    return O.gda_decode_fp8(inp["q1"], inp["q2"], inp["k1_cache"], inp["k2_cache"], inp["v_cache"], scales,
                            inp["seq_lens"], lam, li, **kw)


@pytest.mark.parametrize("hs,hn,hkv", [(6, 2, 2), (8, 2, 4), (4, 4, 4)])
def test_fp8_cache_ragged_lengths(hs, hn, hkv):
    lens = [0, 1, 2, 127, 128, 129, 511, 700]
    inp, scales = fp8_inputs(len(lens), 700, hs, hn, hkv, lens, seed=24)
    out = run(inp, 0.75, 0.4, cache_scales=scales)
    want = fp8_oracle(inp, scales, 0.75, 0.4)
    ma, rel = assert_parity(as64(out), want, "bf16", f"fp8 decode {hs}/{hn}/{hkv}")
    print(f"fp8 decode {hs}/{hn}/{hkv} max-abs {ma:.3e} rel {rel:.3e}")
    assert torch.all(out[0] == 0)


def test_fp8_cache_raw_output_and_split_independence():
    lens = [2048, 1500, 3]
    inp, scales = fp8_inputs(3, 2048, 6, 2, 2, lens, seed=25)
    raw = run(inp, 0.6, 0.3, cache_scales=scales, normalize=False, chunk=256)
    want = fp8_oracle(inp, scales, 0.6, 0.3, normalize=False)
    sc = norm_scale(want, 0.3)
    assert_parity(as64(raw) * sc, want * sc, "bf16", "fp8 raw decode")
    # another split: the weights are rounded to bf16 against other running maxima
    # (each within 2^-9 relative); both splits stay within the bar of the oracle
    a = run(inp, 0.6, 0.5, cache_scales=scales, chunk=256)
    b = run(inp, 0.6, 0.5, cache_scales=scales, chunk=1024)
    want = fp8_oracle(inp, scales, 0.6, 0.5)
    assert_parity(as64(b), want, "bf16", "fp8 decode, chunk 1024")
    ma, _ = err_stats(as64(b), as64(a))
    assert ma <= 4 * 2.0 ** -8


def test_fp8_full_serving_workload_every_output():
    w = W.WORKLOADS["gda_decode_fp8_b64_l8192"]
    inp = W.make_decode_inputs(w)
    scales = inp.pop("cache_scales")
    print(f"[{w.name}] inputs ready, scales {scales}", flush=True)
    out = run(inp, w.lam, w.lam_init, cache_scales=scales, eps=w.eps)
    want = fp8_oracle(inp, scales, w.lam, w.lam_init, eps=w.eps)
    ma, rel = assert_parity(as64(out), want, "bf16", w.name)
    print(f"[{w.name}] max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)


# --- paged caches (block tables) -------------------------------------------------------------

def to_pages(cache, block_size, perm):
    """[B, H, L, D] -> pool [B * L / block_size, H, block_size, D] with sequence b's block j at
    pool index perm[b * nb + j]."""
    B, H, L, D = cache.shape
    nb = L // block_size
    blocks = cache.reshape(B, H, nb, block_size, D).permute(0, 2, 1, 3, 4).reshape(B * nb, H, block_size, D)
    pool = torch.empty_like(blocks)
    pool[perm] = blocks
    return pool.contiguous(), perm.reshape(B, nb).to(torch.int32)


@pytest.mark.parametrize("fp8,block_size", [(False, 128), (False, 512), (True, 256)])
def test_paged_caches_equal_contiguous(fp8, block_size):
    lens = [1, 129, 700, 1024, 0, 513]
    L = 1024
    if fp8:
        inp, scales = fp8_inputs(len(lens), L, 6, 2, 2, lens, seed=26)
        kw = dict(cache_scales=scales)
    else:
        inp, kw = decode_inputs(len(lens), L, 6, 2, 2, lens, seed=26), {}
    ref = run(inp, 0.7, 0.4, **kw)
    g = torch.Generator("cpu").manual_seed(27)
    perm = torch.randperm(len(lens) * (L // block_size), generator=g)
    paged = dict(inp)
    for k in ("k1_cache", "k2_cache", "v_cache"):
        paged[k], table = to_pages(inp[k], block_size, perm)
    d = to_dev(paged)
    out = ops.gda_decode(d["q1"], d["q2"], d["k1_cache"], d["k2_cache"], d["v_cache"], d["seq_lens"], 0.7, 0.4,
                         block_table=table.cuda(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)  # same products in the same order
    want = fp8_oracle(inp, scales, 0.7, 0.4) if fp8 else oracle(inp, 0.7, 0.4)
    assert_parity(as64(out), want, "bf16", f"paged decode fp8={fp8} block {block_size}")


def test_read_probe_reads_and_writes_nothing():
    # the benchmark's streaming-read probe behind the decode lines' measured reference
    import bench
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")  # 1 MiB, words never hit the sink value
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    bench.hbm_read_probe(buf, sink)
    bench.hbm_read_probe(buf[: (1 << 18) - 4], sink)  # a length that is not a multiple of the grid
    torch.cuda.synchronize()
    assert torch.all(sink == 0)


@pytest.mark.parametrize("fp8", [False, True])
def test_single_long_sequence_automatic_split(fp8):
    # one sequence of 16384 cached positions: the automatic split takes the smallest
    # partials (128 positions; 256 for e4m3), so the combine merges 128 or 64 of them
    L = 16384
    if fp8:
        inp, scales = fp8_inputs(1, L, 6, 2, 2, [L - 5], seed=27)
        out = run(inp, 0.7, 0.7, cache_scales=scales)
        want = fp8_oracle(inp, scales, 0.7, 0.7)
    else:
        inp = decode_inputs(1, L, 6, 2, 2, [L - 5], seed=27)
        out = run(inp, 0.7, 0.7)
        want = oracle(inp, 0.7, 0.7)
    ma, rel = assert_parity(as64(out), want, "bf16", f"one {L}-position sequence, fp8={fp8}")
    print(f"long single decode fp8={fp8}: max-abs {ma:.3e} rel {rel:.3e}")

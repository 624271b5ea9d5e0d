"""gda_decode_noalloc: the decode with its partials in the library's fixed
per-GPU scratch array instead of a caller workspace (for callers that cannot
allocate).  Host-side: sizes beyond the array are rejected before any HIP
call.  GPU: its output equals gda_decode's on the same inputs, on two calls in
a row (the second smaller, so it runs over what the first left in the array),
and both match the fp64 oracle to the bf16 bar."""

import ctypes
import os

import pytest
import torch

from differential_attention_diff_amd import ops
from oracle import diffattn_oracle as O
from tests.helpers import as64, assert_parity

FAKE = 0x7F0000000000
GIB = 1 << 30


def _lib():
    if not os.path.exists(ops.LIB_PATH):
        from differential_attention_diff_amd import build
        build.build()
    return ops.lib()


def test_noalloc_rejects_partials_beyond_the_scratch():
    L = _lib()
    a = ops.DecodeArgs()
    B, Lmax, hs, hn, hkv, d = 4096, 8192, 18, 6, 6, 64
    a.q1, a.q2, a.k1_cache, a.k2_cache, a.v_cache, a.seq_lens, a.out = (FAKE + i * 512 * GIB for i in range(7))
    a.B, a.Lmax, a.H_s, a.H_n, a.H_kv, a.d, a.dv, a.chunk = B, Lmax, hs, hn, hkv, d, 2 * d, 0
    a.s_q1[:], a.s_q2[:], a.s_out[:] = [hs * d, d], [hn * d, d], [hs * 2 * d, 2 * d]
    a.s_k1[:] = [hkv * Lmax * d, Lmax * d, d]
    a.s_k2[:] = [hn * Lmax * d, Lmax * d, d]
    a.s_v[:] = [hkv * Lmax * 2 * d, Lmax * 2 * d, 2 * d]
    a.lambda_, a.lambda_init, a.eps = 0.75, 0.75, 1e-5
    a.dtype = ops.DA_BF16
    need = L.gda_decode_workspace_bytes(ctypes.byref(a))
    assert need > (32 << 20)
    st = L.gda_decode_noalloc(ctypes.byref(a), None)
    assert st == ops.DA_EUNSUPPORTED and "fixed scratch" in ops.last_error()


def _inputs(B, Lmax, hs, hn, hkv, lens, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g).bfloat16()
    return {"q1": mk(B, hs, 64), "q2": mk(B, hn, 64), "k1": mk(B, hkv, Lmax, 64), "k2": mk(B, hn, Lmax, 64),
            "v": mk(B, hkv, Lmax, 128), "lens": torch.tensor(lens, dtype=torch.int32)}


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_twice():
    cases = [(16, 4096, 18, 6, 6, [4096 - 37 * i for i in range(16)], 41),   # larger first
             (3, 700, 6, 2, 2, [700, 1, 333], 42)]                          # then smaller
    for B, Lmax, hs, hn, hkv, lens, seed in cases:
        x = _inputs(B, Lmax, hs, hn, hkv, lens, seed)
        d = {k: v.cuda() for k, v in x.items()}
        print(f"[noalloc] B={B} Lmax={Lmax} H_s={hs} H_n={hn}", flush=True)
        ref = ops.gda_decode(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], d["lens"], 0.75, 0.75)
        out = torch.full_like(ref, float("nan"))
        ops.gda_decode_noalloc(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], d["lens"], 0.75, 0.75, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)  # same kernels, same split, same order
        want = O.gda_decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lens"], 0.75, 0.75)
        ma, rel = assert_parity(as64(out), want, "bf16", f"noalloc decode B={B}")
        print(f"[noalloc] B={B}: bitwise equal to gda_decode; max-abs {ma:.3e} rel-L2 {rel:.3e}", flush=True)

"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/diffattn.h declares, and rejects invalid arguments on the
host before any HIP call.  Pointers here are fake 16-byte-aligned addresses:
validation never dereferences them, and no valid argument set is passed (that
would reach a launch)."""

import ctypes
import os

import pytest

from differential_attention_diff_amd import ops

FAKE = 0x7F0000000000  # aligned fake device addresses, 1 GiB apart
GIB = 1 << 30


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        from differential_attention_diff_amd import build
        build.build()
    return ops.lib()


def test_exports_every_declared_symbol(L):
    names = ops.header_functions()
    assert set(names) >= {"diffattn_fwd", "gda_fwd", "gda_fwd_varlen", "gda_bwd", "gda_bwd_workspace_bytes",
                          "gda_decode", "gda_decode_workspace_bytes", "da_lambda_reparam", "da_lambda_reparam_bwd",
                          "da_status_str", "da_last_error", "da_abi_version"}
    for n in names:
        assert hasattr(L, n), f"libdiffattn.so does not export {n}"
    # the streaming-read probe is bench tooling, built into its own library
    assert not hasattr(L, "da_hbm_read_probe")


def test_version_and_status_strings(L):
    assert L.da_abi_version() == 3
    for s in range(5):
        assert ops.status_str(s).startswith("DA_")
    assert ops.status_str(99) == "unknown status"


def base_fwd(B=2, N=64, hs=6, hn=2, hkv=6, d=64, dtype=ops.DA_BF16):
    a = ops.FwdArgs()
    dv = 2 * d
    a.q1, a.q2, a.k1, a.k2, a.v, a.out = (FAKE + i * GIB for i in range(6))
    a.B, a.N, a.H_s, a.H_n, a.H_kv, a.d, a.dv = B, N, hs, hn, hkv, d, dv
    a.s_q1[:] = [N * hs * d, hs * d, d]
    a.s_q2[:] = [N * hn * d, hn * d, d]
    a.s_k1[:] = [N * hkv * d, hkv * d, d]
    a.s_k2[:] = [N * hn * d, hn * d, d]
    a.s_v[:] = [N * hkv * dv, hkv * dv, dv]
    a.s_out[:] = [N * hs * dv, hs * dv, dv]
    a.lambda_, a.lambda_init, a.eps = 0.7, 0.7, 1e-5
    a.dtype = dtype
    a.flags = ops.DA_CAUSAL
    return a


def call(L, a, entry="gda_fwd"):
    st = getattr(L, entry)(ctypes.byref(a), None)
    return st, ops.last_error()


@pytest.mark.parametrize("mutate,status,msg", [
    (lambda a: setattr(a, "q1", None), ops.DA_EINVAL, "q1 is NULL"),
    (lambda a: setattr(a, "out", None), ops.DA_EINVAL, "out is NULL"),
    (lambda a: setattr(a, "k2", FAKE + 3 * GIB + 8), ops.DA_EINVAL, "16-byte aligned"),
    (lambda a: setattr(a, "dv", 100), ops.DA_EINVAL, "2*d"),
    (lambda a: (setattr(a, "d", 48), setattr(a, "dv", 96)), ops.DA_EUNSUPPORTED, "d in {32, 64}"),
    (lambda a: setattr(a, "H_n", 4), ops.DA_EINVAL, "multiple of H_n"),
    (lambda a: setattr(a, "H_kv", 4), ops.DA_EINVAL, "multiple of H_kv"),
    (lambda a: setattr(a, "H_s", 512), ops.DA_EINVAL, "exceeds"),
    (lambda a: setattr(a, "N", -1), ops.DA_EINVAL, "negative"),
    (lambda a: a.s_v.__setitem__(1, 129), ops.DA_EINVAL, "multiple of 16 bytes"),
    (lambda a: a.s_q1.__setitem__(0, -8), ops.DA_EINVAL, "negative stride"),
    (lambda a: setattr(a, "flags", 8), ops.DA_EINVAL, "flag"),
    (lambda a: setattr(a, "eps", -1.0), ops.DA_EINVAL, "eps"),
    (lambda a: setattr(a, "eps", 0.0), ops.DA_EINVAL, "eps must be finite and > 0"),
    # 32-bit per-lane offsets inside a 128-row block: token strides above (2^32 - 256) / 256
    (lambda a: a.s_k1.__setitem__(1, 16777216), ops.DA_EUNSUPPORTED, "k1 token stride"),
    (lambda a: a.s_q2.__setitem__(1, 16777216), ops.DA_EUNSUPPORTED, "q2 token stride"),
    (lambda a: setattr(a, "lambda_", float("nan")), ops.DA_EINVAL, "finite"),
    (lambda a: setattr(a, "dtype", 7), ops.DA_EINVAL, "dtype"),
    (lambda a: setattr(a, "out", a.v), ops.DA_EINVAL, "overlaps v"),
    (lambda a: setattr(a, "out", FAKE + 4 * GIB + 1024), ops.DA_EINVAL, "overlaps v"),
    (lambda a: setattr(a, "o_maps", FAKE + 6 * GIB + 8), ops.DA_EINVAL, "o_maps is not 16-byte aligned"),
    (lambda a: setattr(a, "o_maps", FAKE + 5 * GIB - 64), ops.DA_EINVAL, "o_maps overlaps out"),
])
def test_fwd_validation(L, mutate, status, msg):
    a = base_fwd()
    mutate(a)
    st, err = call(L, a)
    assert st == status, err
    assert msg in err


def test_maps_validation(L):
    a = base_fwd()
    bad = (ctypes.c_int32 * 6)(0, 0, 0, 0, 1, 1)  # noise head 0 serves 4, expected 3
    a.noise_of_signal = ctypes.cast(bad, ctypes.POINTER(ctypes.c_int32))
    st, err = call(L, a)
    assert st == ops.DA_EINVAL and "serves 4" in err
    oob = (ctypes.c_int32 * 6)(0, 0, 0, 1, 1, 2)
    a.noise_of_signal = ctypes.cast(oob, ctypes.POINTER(ctypes.c_int32))
    st, err = call(L, a)
    assert st == ops.DA_EINVAL and "out of" in err


def test_plain_entry_requires_equal_heads(L):
    st, err = call(L, base_fwd(), "diffattn_fwd")
    assert st == ops.DA_EINVAL and "gda_fwd" in err
    a = base_fwd(hs=4, hn=4, hkv=4)
    keep = (ctypes.c_int32 * 4)(0, 1, 2, 3)
    a.kv_of_signal = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    st, err = call(L, a, "diffattn_fwd")
    assert st == ops.DA_EINVAL and "head maps" in err


@pytest.mark.parametrize("B,N", [(0, 64), (2, 0)])
def test_empty_is_noop(L, B, N):
    a = base_fwd(B=B, N=N)
    st, err = call(L, a)
    assert st == ops.DA_OK, err


CU = FAKE + 40 * GIB  # fake device address of cu_seqlens


def call_varlen(L, a, cu=CU, nseq=3, max_seqlen=40):
    st = L.gda_fwd_varlen(ctypes.byref(a), None if cu is None else ctypes.c_void_p(cu), nseq, max_seqlen, None)
    return st, ops.last_error()


@pytest.mark.parametrize("kw,batch,status,msg", [
    (dict(), 2, ops.DA_EINVAL, "B == 1"),
    (dict(cu=None), 1, ops.DA_EINVAL, "cu_seqlens is NULL"),
    (dict(cu=CU + 2), 1, ops.DA_EINVAL, "4-byte aligned"),
    (dict(nseq=-1), 1, ops.DA_EINVAL, "nseq"),
    (dict(max_seqlen=65), 1, ops.DA_EINVAL, "max_seqlen"),
    (dict(max_seqlen=-1), 1, ops.DA_EINVAL, "max_seqlen"),
])
def test_varlen_validation(L, kw, batch, status, msg):
    a = base_fwd(B=batch)
    st, err = call_varlen(L, a, **kw)
    assert st == status, err
    assert msg in err


def test_varlen_shared_checks_and_limits(L):
    a = base_fwd(B=1)
    a.s_k1[1] = 65  # the checks gda_fwd makes still apply
    st, err = call_varlen(L, a)
    assert st == ops.DA_EINVAL and "multiple of 16 bytes" in err
    a = base_fwd(B=1, dtype=ops.DA_F32)
    st, err = call_varlen(L, a, nseq=70000)
    assert st == ops.DA_EUNSUPPORTED and "sequences" in err


@pytest.mark.parametrize("kw", [dict(nseq=0, cu=None), dict(max_seqlen=0)])
def test_varlen_empty_is_noop(L, kw):
    st, err = call_varlen(L, base_fwd(B=1), **kw)
    assert st == ops.DA_OK, err


def base_bwd(B=2, N=64, hs=6, hn=2, hkv=6, d=64, dtype=ops.DA_BF16):
    a = ops.BwdArgs()
    dv = 2 * d
    (a.q1, a.q2, a.k1, a.k2, a.v, a.o_maps, a.lse, a.dout, a.grad_q1, a.grad_q2, a.grad_k1, a.grad_k2,
     a.grad_v, a.dlambda) = (FAKE + i * GIB for i in range(14))
    a.B, a.N, a.H_s, a.H_n, a.H_kv, a.d, a.dv = B, N, hs, hn, hkv, d, dv
    lead = lambda h, w: [N * h * w, h * w, w]
    a.s_q1[:], a.s_gq1[:] = lead(hs, d), lead(hs, d)
    a.s_q2[:], a.s_gq2[:] = lead(hn, d), lead(hn, d)
    a.s_k1[:], a.s_gk1[:] = lead(hkv, d), lead(hkv, d)
    a.s_k2[:], a.s_gk2[:] = lead(hn, d), lead(hn, d)
    a.s_v[:], a.s_gv[:] = lead(hkv, dv), lead(hkv, dv)
    a.s_dout[:] = lead(hs, dv)
    a.lambda_, a.lambda_init, a.eps = 0.7, 0.7, 1e-5
    a.dtype = dtype
    a.flags = ops.DA_CAUSAL
    return a


def test_bwd_workspace_bytes(L):
    a = base_bwd()
    rows = 2 * 64 * 6
    r256 = lambda x: (x + 255) // 256 * 256
    want = r256(rows * 128 * 2) + r256(rows * 16) + r256(((rows + 3) // 4) * 129 * 8)
    assert L.gda_bwd_workspace_bytes(ctypes.byref(a)) == want
    a = base_bwd(dtype=ops.DA_F32)
    assert L.gda_bwd_workspace_bytes(ctypes.byref(a)) == r256(rows * 128 * 4) + r256(rows * 16) + r256(
        ((rows + 3) // 4) * 129 * 8)
    assert L.gda_bwd_workspace_bytes(ctypes.byref(base_bwd(B=0))) == 0


@pytest.mark.parametrize("mutate,status,msg", [
    (lambda a: setattr(a, "dlambda", None), ops.DA_EINVAL, "dlambda is NULL"),
    (lambda a: setattr(a, "o_maps", None), ops.DA_EINVAL, "o_maps is NULL"),
    (lambda a: setattr(a, "lse", None), ops.DA_EINVAL, "lse is NULL"),
    (lambda a: setattr(a, "dnorm_w", FAKE + 20 * GIB), ops.DA_EINVAL, "dnorm_w needs norm_w"),
    (lambda a: setattr(a, "grad_v", None), ops.DA_EINVAL, "grad_v is NULL"),
    (lambda a: setattr(a, "grad_k1", a.q1), ops.DA_EINVAL, "grad_k1 overlaps q1"),
    (lambda a: setattr(a, "grad_k2", a.grad_q2), ops.DA_EINVAL, "grad_k2 overlaps grad_q2"),
    (lambda a: setattr(a, "grad_q1", FAKE + 6 * GIB), ops.DA_EINVAL, "grad_q1 overlaps lse"),
    (lambda a: a.s_gv.__setitem__(1, 100), ops.DA_EINVAL, "multiple of 16 bytes"),
    (lambda a: setattr(a, "flags", 4), ops.DA_EINVAL, "flag"),
    (lambda a: (setattr(a, "H_kv", 1)), ops.DA_EUNSUPPORTED, "not one run"),
    # 32-bit per-lane offsets inside a streamed block (bf16)
    (lambda a: a.s_v.__setitem__(1, 16777216), ops.DA_EUNSUPPORTED, "v token stride"),
    (lambda a: a.s_q1.__setitem__(1, 16777216), ops.DA_EUNSUPPORTED, "q1 token stride"),
])
def test_bwd_validation(L, mutate, status, msg):
    a = base_bwd()
    mutate(a)
    st = L.gda_bwd(ctypes.byref(a), None, 0, None)
    assert st == status, ops.last_error()
    assert msg in ops.last_error()


def test_bwd_workspace_required(L):
    a = base_bwd()
    assert L.gda_bwd(ctypes.byref(a), None, 0, None) == ops.DA_EWORKSPACE
    assert L.gda_bwd(ctypes.byref(a), ctypes.c_void_p(FAKE + 30 * GIB), 1024, None) == ops.DA_EWORKSPACE
    a = base_bwd(hs=8, hn=2, hkv=4, dtype=ops.DA_BF16)  # consecutive GQA inside each group: supported
    a.s_q1[:], a.s_gq1[:] = [64 * 8 * 64, 8 * 64, 64], [64 * 8 * 64, 8 * 64, 64]
    a.s_dout[:] = [64 * 8 * 128, 8 * 128, 128]
    a.s_k1[:], a.s_gk1[:] = [64 * 4 * 64, 4 * 64, 64], [64 * 4 * 64, 4 * 64, 64]
    a.s_v[:], a.s_gv[:] = [64 * 4 * 128, 4 * 128, 128], [64 * 4 * 128, 4 * 128, 128]
    assert L.gda_bwd(ctypes.byref(a), None, 0, None) == ops.DA_EWORKSPACE, ops.last_error()


def packed_grads(a, shift_q2=0):
    """Gradient views into one packed buffer laid out per token as [dq1 | dq2 | dk1 | dk2 | dv]
    (the layout of a fused projection's gradient); shift_q2 moves dq2 back by that many elements."""
    d, dv = a.d, a.dv
    heads = (a.H_s, a.H_n, a.H_kv, a.H_n, a.H_kv)
    widths = [h * w for h, w in zip(heads, (d, d, d, d, dv))]
    total = sum(widths)
    base, off = FAKE + 40 * GIB, 0
    for i, (ptr, strides, w, h) in enumerate(zip(("grad_q1", "grad_q2", "grad_k1", "grad_k2", "grad_v"),
                                                 ("s_gq1", "s_gq2", "s_gk1", "s_gk2", "s_gv"), widths, heads)):
        start = off - (shift_q2 if i == 1 else 0)
        setattr(a, ptr, base + 2 * start)
        getattr(a, strides)[:] = [a.N * total, total, w // h]
        off += w


def test_bwd_gradients_into_one_packed_buffer(L):
    # interleaved views whose per-token columns are disjoint are accepted ...
    a = base_bwd(hs=8, hn=2, hkv=4)
    a.s_q1[:], a.s_dout[:] = [64 * 8 * 64, 8 * 64, 64], [64 * 8 * 128, 8 * 128, 128]
    a.s_k1[:], a.s_v[:] = [64 * 4 * 64, 4 * 64, 64], [64 * 4 * 128, 4 * 128, 128]
    packed_grads(a)
    assert L.gda_bwd(ctypes.byref(a), None, 0, None) == ops.DA_EWORKSPACE, ops.last_error()
    # ... columns shared by two of them are not
    packed_grads(a, shift_q2=8)
    assert L.gda_bwd(ctypes.byref(a), None, 0, None) == ops.DA_EINVAL
    assert "grad_q2 overlaps grad_q1" in ops.last_error()


def test_fwd_out_sharing_columns_with_an_input_is_rejected(L):
    a = base_fwd()
    # out interleaved with q1 in one buffer, its first 8 channels on q1's last 8
    total = 6 * 64 + 6 * 128
    a.q1, a.out = FAKE + 40 * GIB, FAKE + 40 * GIB + 2 * (6 * 64 - 8)
    a.s_q1[:] = [64 * total, total, 64]
    a.s_out[:] = [64 * total, total, 128]
    st, err = call(L, a)
    assert st == ops.DA_EINVAL and "out overlaps q1" in err


def test_lambda_entry_validation(L):
    f = lambda i: ctypes.c_void_p(FAKE + i * GIB)
    st = L.da_lambda_reparam(f(0), f(1), f(2), f(3), 0, ctypes.c_float(0.5), f(4), None)
    assert st == ops.DA_EINVAL and "dim" in ops.last_error()
    st = L.da_lambda_reparam(f(0), None, f(2), f(3), 64, ctypes.c_float(0.5), f(4), None)
    assert st == ops.DA_EINVAL and "lk1 is NULL" in ops.last_error()
    st = L.da_lambda_reparam(f(0), f(1), f(2), f(3), 64, ctypes.c_float(float("inf")), f(4), None)
    assert st == ops.DA_EINVAL and "finite" in ops.last_error()
    st = L.da_lambda_reparam(f(0), f(1), f(2), f(3), 64, ctypes.c_float(0.5), ctypes.c_void_p(FAKE + 8), None)
    assert st == ops.DA_EINVAL and "overlaps lq1" in ops.last_error()
    st = L.da_lambda_reparam_bwd(f(0), f(1), f(2), f(3), 64, f(4), f(5), f(6), f(7), ctypes.c_void_p(FAKE + 7 * GIB + 2),
                                 None)
    assert st == ops.DA_EINVAL and "aligned" in ops.last_error()
    st = L.da_lambda_reparam_bwd(f(0), f(1), f(2), f(3), 64, f(4), f(5), f(6), f(7), f(5), None)
    assert st == ops.DA_EINVAL and "dlk2 overlaps dlq1" in ops.last_error()


def base_dec(B=64, L_=8192, hs=18, hn=6, hkv=6, d=64, chunk=0):
    a = ops.DecodeArgs()
    dv = 2 * d
    a.q1, a.q2, a.k1_cache, a.k2_cache, a.v_cache, a.seq_lens, a.out = (FAKE + i * 64 * GIB for i in range(7))
    a.B, a.Lmax, a.H_s, a.H_n, a.H_kv, a.d, a.dv, a.chunk = B, L_, hs, hn, hkv, d, dv, chunk
    a.s_q1[:] = [hs * d, d]
    a.s_q2[:] = [hn * d, d]
    a.s_out[:] = [hs * dv, dv]
    a.s_k1[:] = [hkv * L_ * d, L_ * d, d]
    a.s_k2[:] = [hn * L_ * d, L_ * d, d]
    a.s_v[:] = [hkv * L_ * dv, L_ * dv, dv]
    a.lambda_, a.lambda_init, a.eps = 0.75, 0.75, 1e-5
    a.dtype = ops.DA_BF16
    return a


def test_decode_workspace_bytes(L):
    a = base_dec()
    # automatic split: 64 x 6 x 8192 positions / 2560 partials -> chunks of 1280, 7 per
    # sequence; per (b, group, chunk): g + u = 3 + 1 slots of (dv + 2) floats
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 64 * 6 * 7 * 4 * 130 * 4
    a = base_dec(chunk=512)
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 64 * 6 * 16 * 4 * 130 * 4
    a = base_dec(B=2)  # 2 x 6 x 8192 / 2560 = 38 -> one sub-chunk, 128 positions
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 2 * 6 * 64 * 4 * 130 * 4
    a = base_dec(chunk=1024)
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 64 * 6 * 8 * 4 * 130 * 4
    a = base_dec(chunk=192)
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 0 and "multiple of 128" in ops.last_error()
    # the largest batch and cache the decode accepts still give a representable size
    a = base_dec(B=65535, L_=2**31 - 1, hs=256, hn=128, hkv=128)
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 65535 * 128 * ((2**31 - 1 + 2047) // 2048) * 3 * 130 * 4
    a = base_dec(chunk=4096)
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 0 and "exceeds" in ops.last_error()


def test_decode_fp8_validation(L):
    a = base_dec()
    a.cache_dtype = ops.DA_FP8_E4M3
    a.k1_scale, a.k2_scale, a.v_scale = 0.01, 0.0, 0.01
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EINVAL and "scales" in ops.last_error()
    a.k2_scale = float("nan")
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 0 and "scales" in ops.last_error()
    a.k2_scale = 0.02
    L_, hkv = 8192, 6
    a.s_k1[:] = [hkv * L_ * 64, L_ * 64, 64]   # 64-byte e4m3 rows: strides in bytes pass the 16-byte rule
    a.s_v[:] = [hkv * L_ * 128, L_ * 128, 128]
    a.s_k2[:] = [6 * L_ * 64, L_ * 64, 64]
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EWORKSPACE, ops.last_error()
    a.s_k1[2] = 56  # 56 bytes: not a multiple of 16
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EINVAL and "16 bytes" in ops.last_error()


def test_decode_paged_validation(L):
    a = base_dec()
    a.block_table = FAKE + 50 * GIB
    a.block_size, a.max_blocks, a.num_blocks = 64, 128, 8192
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EUNSUPPORTED and "block_size" in ops.last_error()
    a.block_size, a.max_blocks = 256, 16  # 4096 positions < Lmax 8192
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EINVAL and "Lmax" in ops.last_error()
    a.max_blocks, a.num_blocks = 32, 0
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EINVAL and "num_blocks" in ops.last_error()
    a.num_blocks = 2048
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EWORKSPACE, ops.last_error()
    a.cache_dtype = ops.DA_FP8_E4M3
    a.k1_scale = a.k2_scale = a.v_scale = 0.01
    a.block_size, a.max_blocks = 128, 64  # e4m3 caches need blocks of 256 positions
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EUNSUPPORTED and "256" in ops.last_error()


def test_decode_validation(L):
    a = base_dec()
    st = L.gda_decode(ctypes.byref(a), None, 0, None)
    assert st == ops.DA_EWORKSPACE, ops.last_error()
    st = L.gda_decode(ctypes.byref(a), ctypes.c_void_p(FAKE + 63 * GIB), 1024, None)
    assert st == ops.DA_EWORKSPACE and "needs" in ops.last_error()
    a = base_dec(d=32)
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EUNSUPPORTED
    a = base_dec()
    a.dtype = ops.DA_F32
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EUNSUPPORTED
    a = base_dec(hs=18, hn=2, hkv=2)  # 9 signal heads per noise head
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EUNSUPPORTED
    # 5 signal heads per noise head on 5 distinct key/value heads: g + u = 10 outputs
    a = base_dec(hs=10, hn=2, hkv=10)
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EUNSUPPORTED and "outputs" in ops.last_error()
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 0
    a = base_dec(hs=12, hn=2, hkv=4)  # g = 6 on u = 2 key/value heads: 8 outputs, accepted
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EWORKSPACE, ops.last_error()
    a = base_dec()
    a.seq_lens = None
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_EINVAL
    a = base_dec(B=0)
    assert L.gda_decode(ctypes.byref(a), None, 0, None) == ops.DA_OK


def test_empty_with_null_pointers_is_noop(L):
    # torch hands out NULL data pointers for empty tensors
    for B, N in ((0, 64), (2, 0)):
        a = base_fwd(B=B, N=N)
        a.q1 = a.q2 = a.k1 = a.k2 = a.v = a.out = None
        st, err = call(L, a)
        assert st == ops.DA_OK, err
    d = base_dec(B=0)
    d.q1 = d.q2 = d.k1_cache = d.k2_cache = d.v_cache = d.seq_lens = d.out = None
    assert L.gda_decode_workspace_bytes(ctypes.byref(d)) == 0
    assert L.gda_decode(ctypes.byref(d), None, 0, None) == ops.DA_OK


def test_decode_workspace_query_ignores_pointers(L):
    a = base_dec()
    a.q1 = a.q2 = a.k1_cache = a.k2_cache = a.v_cache = a.seq_lens = a.out = None
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 64 * 6 * 7 * 4 * 130 * 4  # automatic split: 1280 positions


def test_decode_batch_limit_and_overlap(L):
    a = base_dec(B=70000)  # the batch is a grid dimension of the decode kernels
    st = L.gda_decode(ctypes.byref(a), None, 0, None)
    assert st == ops.DA_EUNSUPPORTED and "65535" in ops.last_error()
    assert L.gda_decode_workspace_bytes(ctypes.byref(a)) == 0
    a = base_dec()
    need = L.gda_decode_workspace_bytes(ctypes.byref(a))
    ws = ctypes.c_void_p(FAKE + 7 * 64 * GIB)
    assert need > 0
    for field, msg in (("q1", "out overlaps q1"), ("v_cache", "out overlaps v_cache"),
                       ("seq_lens", "out overlaps seq_lens")):
        a = base_dec()
        a.out = getattr(a, field)
        assert L.gda_decode(ctypes.byref(a), ws, need, None) == ops.DA_EINVAL and msg in ops.last_error()
    a = base_dec()
    st = L.gda_decode(ctypes.byref(a), ctypes.c_void_p(a.k2_cache + 4096), need, None)
    assert st == ops.DA_EINVAL and "workspace overlaps k2_cache" in ops.last_error()
    st = L.gda_decode(ctypes.byref(a), ctypes.c_void_p(a.out - 256), need, None)
    assert st == ops.DA_EINVAL and "workspace overlaps out" in ops.last_error()


def test_bench_probe_validation():
    # the benchmark's streaming-read probe (bench_probe.so, not part of libdiffattn.so)
    import bench
    if not os.path.exists(bench.PROBE_LIB):
        bench.build_probe()
    P = bench.probe_lib()
    f = lambda i: ctypes.c_void_p(FAKE + i * GIB)
    assert P.bench_hbm_read_probe(None, 0, None, None) == 0  # nothing to read: no launch
    assert P.bench_hbm_read_probe(None, 1024, f(1), None) == 1
    assert P.bench_hbm_read_probe(ctypes.c_void_p(FAKE + 8), 1024, f(1), None) == 1
    assert P.bench_hbm_read_probe(f(0), 1000, f(1), None) == 1
    assert P.bench_hbm_read_probe(f(0), 1024, ctypes.c_void_p(FAKE + 512), None) == 1
    assert P.bench_hbm_read_probe(f(0), (1 << 40) + 16, f(2000), None) == 1

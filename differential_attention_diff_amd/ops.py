"""Python binding of libdiffattn.so (ctypes): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into device pointers, element strides and the current HIP
stream, and raises if the library is missing or returns an error.  Entry
points mirror the C ABI: ``diffattn_fwd``, ``gda_fwd``, ``gda_fwd_varlen``,
``gda_bwd`` (plus ``gda_bwd_workspace_bytes``), ``gda_decode`` (plus
``gda_decode_workspace_bytes``), ``lambda_reparam`` / ``lambda_reparam_bwd``;
``diff_attention`` wraps the forward and the backward as a torch autograd
function and ``lambda_from_params`` the lambda re-parameterisation.  lambda may
be a float or a device fp32 tensor (read by the kernels, no host round trip).
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdiffattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "diffattn.h")

DA_OK, DA_EINVAL, DA_EUNSUPPORTED, DA_EHIP, DA_EWORKSPACE = range(5)
DA_F32, DA_BF16, DA_FP8_E4M3 = 0, 1, 2
DA_CAUSAL, DA_NO_NORM = 1, 2

_i64x3 = ctypes.c_int64 * 3
_i64x2 = ctypes.c_int64 * 2


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("q1", ctypes.c_void_p), ("q2", ctypes.c_void_p), ("k1", ctypes.c_void_p), ("k2", ctypes.c_void_p),
        ("v", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H_s", ctypes.c_int64), ("H_n", ctypes.c_int64),
        ("H_kv", ctypes.c_int64), ("d", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("s_q1", _i64x3), ("s_q2", _i64x3), ("s_k1", _i64x3), ("s_k2", _i64x3), ("s_v", _i64x3),
        ("s_out", _i64x3),
        ("noise_of_signal", ctypes.POINTER(ctypes.c_int32)), ("kv_of_signal", ctypes.POINTER(ctypes.c_int32)),
        ("lambda_", ctypes.c_float), ("lambda_init", ctypes.c_float), ("eps", ctypes.c_float),
        ("norm_w", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("o_maps", ctypes.c_void_p), ("lambda_dev", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("q1", ctypes.c_void_p), ("q2", ctypes.c_void_p), ("k1", ctypes.c_void_p), ("k2", ctypes.c_void_p),
        ("v", ctypes.c_void_p), ("o_maps", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dout", ctypes.c_void_p),
        ("grad_q1", ctypes.c_void_p), ("grad_q2", ctypes.c_void_p), ("grad_k1", ctypes.c_void_p),
        ("grad_k2", ctypes.c_void_p), ("grad_v", ctypes.c_void_p),
        ("dlambda", ctypes.c_void_p), ("dnorm_w", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H_s", ctypes.c_int64), ("H_n", ctypes.c_int64),
        ("H_kv", ctypes.c_int64), ("d", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("s_q1", _i64x3), ("s_q2", _i64x3), ("s_k1", _i64x3), ("s_k2", _i64x3), ("s_v", _i64x3),
        ("s_dout", _i64x3),
        ("s_gq1", _i64x3), ("s_gq2", _i64x3), ("s_gk1", _i64x3), ("s_gk2", _i64x3), ("s_gv", _i64x3),
        ("noise_of_signal", ctypes.POINTER(ctypes.c_int32)), ("kv_of_signal", ctypes.POINTER(ctypes.c_int32)),
        ("lambda_", ctypes.c_float), ("lambda_init", ctypes.c_float), ("eps", ctypes.c_float),
        ("norm_w", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("lambda_dev", ctypes.c_void_p),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q1", ctypes.c_void_p), ("q2", ctypes.c_void_p), ("k1_cache", ctypes.c_void_p),
        ("k2_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("Lmax", ctypes.c_int64), ("H_s", ctypes.c_int64), ("H_n", ctypes.c_int64),
        ("H_kv", ctypes.c_int64), ("d", ctypes.c_int64), ("dv", ctypes.c_int64), ("chunk", ctypes.c_int64),
        ("s_q1", _i64x2), ("s_q2", _i64x2), ("s_out", _i64x2),
        ("s_k1", _i64x3), ("s_k2", _i64x3), ("s_v", _i64x3),
        ("noise_of_signal", ctypes.POINTER(ctypes.c_int32)), ("kv_of_signal", ctypes.POINTER(ctypes.c_int32)),
        ("lambda_", ctypes.c_float), ("lambda_init", ctypes.c_float), ("eps", ctypes.c_float),
        ("norm_w", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("lambda_dev", ctypes.c_void_p),
        ("cache_dtype", ctypes.c_int32), ("k1_scale", ctypes.c_float), ("k2_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int64), ("max_blocks", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
    ]


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)} -- {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdiffattn.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m differential_attention_diff_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.diffattn_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.gda_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.diffattn_fwd.restype = L.gda_fwd.restype = ctypes.c_int
        L.gda_fwd_varlen.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
        L.gda_fwd_varlen.restype = ctypes.c_int
        L.gda_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdArgs)]
        L.gda_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.gda_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gda_bwd.restype = ctypes.c_int
        L.gda_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
        L.gda_decode_workspace_bytes.restype = ctypes.c_size_t
        L.gda_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gda_decode.restype = ctypes.c_int
        L.gda_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
        L.gda_decode_noalloc.restype = ctypes.c_int
        _fp = ctypes.c_void_p
        L.da_lambda_reparam.argtypes = [_fp, _fp, _fp, _fp, ctypes.c_int64, ctypes.c_float, _fp, _fp]
        L.da_lambda_reparam.restype = ctypes.c_int
        L.da_lambda_reparam_bwd.argtypes = [_fp, _fp, _fp, _fp, ctypes.c_int64, _fp, _fp, _fp, _fp, _fp, _fp]
        L.da_lambda_reparam_bwd.restype = ctypes.c_int
        L.da_status_str.argtypes = [ctypes.c_int]
        L.da_status_str.restype = ctypes.c_char_p
        L.da_last_error.argtypes = []
        L.da_last_error.restype = ctypes.c_char_p
        L.da_abi_version.argtypes = []
        L.da_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/diffattn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)


def status_str(status: int) -> str:
    return lib().da_status_str(status).decode()


def last_error() -> str:
    return lib().da_last_error().decode()


def _check(status: int):
    if status != DA_OK:
        raise DiffAttnError(status, last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DA_BF16
    if t.dtype == torch.float32:
        return DA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _map(m, hs):
    if m is None:
        return None, None
    arr = (ctypes.c_int32 * hs)(*[int(x) for x in m])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), arr


def _set_lambda(a, lam):
    """A float goes by value; a device tensor (one fp32 element) by pointer, read when the kernels run."""
    if torch.is_tensor(lam):
        if lam.dtype != torch.float32 or lam.numel() != 1 or not lam.is_cuda:
            raise ValueError("a lambda tensor must be one fp32 element on the device")
        a.lambda_, a.lambda_dev = 0.0, lam.data_ptr()
    else:
        a.lambda_, a.lambda_dev = float(lam), None


def _lead(t: torch.Tensor, k: int):
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return [int(s) for s in t.stride()[:k]]


def fwd_args(q1, q2, k1, k2, v, out, lam, lam_init, *, eps=1e-5, norm_weight=None, causal=True, normalize=True,
             noise_of_signal=None, kv_of_signal=None, lse=None, o_maps=None):
    """Fill the C argument struct from BSHD tensors (returns (args, keepalive))."""
    B, N, hs, d = q1.shape
    a = FwdArgs()
    a.q1, a.q2, a.k1, a.k2, a.v, a.out = (t.data_ptr() for t in (q1, q2, k1, k2, v, out))
    a.B, a.N, a.H_s, a.H_n, a.H_kv, a.d, a.dv = B, N, hs, q2.shape[2], k1.shape[2], d, v.shape[3]
    a.s_q1[:], a.s_q2[:], a.s_k1[:] = _lead(q1, 3), _lead(q2, 3), _lead(k1, 3)
    a.s_k2[:], a.s_v[:], a.s_out[:] = _lead(k2, 3), _lead(v, 3), _lead(out, 3)
    nz, nz_keep = _map(noise_of_signal, hs)
    kv, kv_keep = _map(kv_of_signal, hs)
    a.noise_of_signal, a.kv_of_signal = nz, kv
    _set_lambda(a, lam)
    a.lambda_init, a.eps = float(lam_init), float(eps)
    a.norm_w = None if norm_weight is None else norm_weight.data_ptr()
    a.lse = None if lse is None else lse.data_ptr()
    a.o_maps = None if o_maps is None else o_maps.data_ptr()
    a.dtype = _dtype_code(q1)
    a.flags = (DA_CAUSAL if causal else 0) | (0 if normalize else DA_NO_NORM)
    return a, (nz_keep, kv_keep)


def _fwd(entry, q1, q2, k1, k2, v, lam, lam_init, out=None, stream=None, **kw):
    if out is None:
        out = torch.empty(q1.shape[:3] + (v.shape[3],), dtype=q1.dtype, device=q1.device)
    a, keep = fwd_args(q1, q2, k1, k2, v, out, lam, lam_init, **kw)
    _check(entry(ctypes.byref(a), _stream(stream)))
    del keep
    return out


def diffattn_fwd(q1, q2, k1, k2, v, lam, lam_init, *, out=None, stream=None, **kw):
    """Plain differential attention forward (H_n = H_kv = H_s); see include/diffattn.h."""
    return _fwd(lib().diffattn_fwd, q1, q2, k1, k2, v, lam, lam_init, out=out, stream=stream, **kw)


def gda_fwd(q1, q2, k1, k2, v, lam, lam_init, *, out=None, stream=None, **kw):
    """Grouped differential attention forward; see include/diffattn.h."""
    return _fwd(lib().gda_fwd, q1, q2, k1, k2, v, lam, lam_init, out=out, stream=stream, **kw)


def gda_fwd_varlen(q1, q2, k1, k2, v, cu_seqlens, max_seqlen, lam, lam_init, *, out=None, lse=None, stream=None,
                   **kw):
    """Packed variable-length GDA prefill; see include/diffattn.h.

    q1 [T,H_s,d], q2/k2 [T,H_n,d], k1 [T,H_kv,d], v [T,H_kv,dv] hold the
    sequences one after another; cu_seqlens is a device int32 tensor [nseq+1]
    and max_seqlen a host int bounding the lengths.  lse, when given, is fp32
    [2,H_s,T].  Tokens outside every sequence keep the value `out` held.
    """
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of nseq + 1 offsets")
    if cu_seqlens.device != q1.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous tensor on the device of q1")
    if out is None:
        out = torch.empty(q1.shape[:2] + (v.shape[2],), dtype=q1.dtype, device=q1.device)
    t4 = [x.unsqueeze(0) for x in (q1, q2, k1, k2, v, out)]
    a, keep = fwd_args(*t4[:5], t4[5], lam, lam_init, lse=lse, **kw)
    _check(lib().gda_fwd_varlen(ctypes.byref(a), ctypes.c_void_p(cu_seqlens.data_ptr()),
                                cu_seqlens.numel() - 1, int(max_seqlen), _stream(stream)))
    del keep
    return out


def bwd_args(q1, q2, k1, k2, v, o_maps, lse, dout, grads, dlambda, lam, lam_init, *, eps=1e-5, norm_weight=None,
             dnorm_weight=None, causal=True, normalize=True, noise_of_signal=None, kv_of_signal=None):
    """Fill the backward struct; grads = (dq1, dq2, dk1, dk2, dv) shaped like the inputs."""
    B, N, hs, d = q1.shape
    a = BwdArgs()
    a.q1, a.q2, a.k1, a.k2, a.v = (t.data_ptr() for t in (q1, q2, k1, k2, v))
    a.o_maps, a.lse, a.dout = o_maps.data_ptr(), lse.data_ptr(), dout.data_ptr()
    a.grad_q1, a.grad_q2, a.grad_k1, a.grad_k2, a.grad_v = (t.data_ptr() for t in grads)
    a.dlambda = dlambda.data_ptr()
    a.dnorm_w = None if dnorm_weight is None else dnorm_weight.data_ptr()
    a.B, a.N, a.H_s, a.H_n, a.H_kv, a.d, a.dv = B, N, hs, q2.shape[2], k1.shape[2], d, v.shape[3]
    a.s_q1[:], a.s_q2[:], a.s_k1[:] = _lead(q1, 3), _lead(q2, 3), _lead(k1, 3)
    a.s_k2[:], a.s_v[:], a.s_dout[:] = _lead(k2, 3), _lead(v, 3), _lead(dout, 3)
    a.s_gq1[:], a.s_gq2[:], a.s_gk1[:], a.s_gk2[:], a.s_gv[:] = (_lead(t, 3) for t in grads)
    nz, nz_keep = _map(noise_of_signal, hs)
    kv, kv_keep = _map(kv_of_signal, hs)
    a.noise_of_signal, a.kv_of_signal = nz, kv
    _set_lambda(a, lam)
    a.lambda_init, a.eps = float(lam_init), float(eps)
    a.norm_w = None if norm_weight is None else norm_weight.data_ptr()
    a.dtype = _dtype_code(q1)
    a.flags = (DA_CAUSAL if causal else 0) | (0 if normalize else DA_NO_NORM)
    return a, (nz_keep, kv_keep)


def gda_bwd_workspace_bytes(q1, q2, k1, k2, v, o_maps, lse, dout, **kw) -> int:
    """Workspace bytes gda_bwd needs for these tensors (shapes and dtype only)."""
    grads = (q1, q2, k1, k2, v)  # shapes and strides only: nothing is written
    a, keep = bwd_args(q1, q2, k1, k2, v, o_maps, lse, dout, grads, lse, 0.0, 0.0,
                       **{k: x for k, x in kw.items() if k not in ("lam", "lam_init")})
    return int(lib().gda_bwd_workspace_bytes(ctypes.byref(a)))


def gda_bwd(q1, q2, k1, k2, v, o_maps, lse, dout, lam, lam_init, *, grads=None, dnorm_weight=None, workspace=None,
            stream=None, **kw):
    """Backward of gda_fwd; o_maps and lse as stored by the forward; see include/diffattn.h.
    Returns (dq1, dq2, dk1, dk2, dv, dlambda [1] fp32)."""
    if grads is None:
        grads = tuple(torch.empty_like(t, memory_format=torch.contiguous_format) for t in (q1, q2, k1, k2, v))
    dlambda = torch.empty(1, dtype=torch.float32, device=q1.device)
    a, keep = bwd_args(q1, q2, k1, k2, v, o_maps, lse, dout, grads, dlambda, lam, lam_init,
                       dnorm_weight=dnorm_weight, **kw)
    need = int(lib().gda_bwd_workspace_bytes(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    _check(lib().gda_bwd(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                         _stream(stream)))
    del keep
    return tuple(grads) + (dlambda,)


class _DiffAttnFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q1, q2, k1, k2, v, lam, norm_weight, lam_init, eps, causal, normalize, nz, kvm):
        # a tensor lambda stays on the device (read by the kernels): no host round trip
        lam_f = lam.detach().reshape(1).float().contiguous() if torch.is_tensor(lam) else float(lam)
        B, N, hs, _ = q1.shape
        lse = torch.empty(2, B, hs, N, dtype=torch.float32, device=q1.device)
        o_maps = torch.empty(2, B, N, hs, v.shape[3], dtype=torch.float32, device=q1.device)
        out = gda_fwd(q1, q2, k1, k2, v, lam_f, lam_init, eps=eps, norm_weight=norm_weight, causal=causal,
                      normalize=normalize, noise_of_signal=nz, kv_of_signal=kvm, lse=lse, o_maps=o_maps)
        ctx.save_for_backward(q1, q2, k1, k2, v, o_maps, lse, norm_weight)
        ctx.cfg = (lam_f, lam.shape if torch.is_tensor(lam) else None, lam_init, eps, causal, normalize, nz, kvm)
        return out

    @staticmethod
    def backward(ctx, dout):
        q1, q2, k1, k2, v, o_maps, lse, w = ctx.saved_tensors
        lam_f, lam_shape, lam_init, eps, causal, normalize, nz, kvm = ctx.cfg
        want_w = w is not None and ctx.needs_input_grad[6] and normalize
        dw = torch.empty(v.shape[3], dtype=torch.float32, device=q1.device) if want_w else None
        dq1, dq2, dk1, dk2, dvv, dlam = gda_bwd(q1, q2, k1, k2, v, o_maps, lse, dout.contiguous(), lam_f, lam_init,
                                                dnorm_weight=dw, eps=eps, norm_weight=w, causal=causal,
                                                normalize=normalize, noise_of_signal=nz, kv_of_signal=kvm)
        return (dq1, dq2, dk1, dk2, dvv, None if lam_shape is None else dlam.reshape(lam_shape), dw,
                None, None, None, None, None, None)


def diff_attention(q1, q2, k1, k2, v, lam, lam_init, *, norm_weight=None, eps=1e-5, causal=True, normalize=True,
                   noise_of_signal=None, kv_of_signal=None):
    """Differentiable (grouped) differential attention: gda_fwd forward, gda_bwd backward.
    lam may be a float or a 0-d tensor (then it receives dL/dlambda); norm_weight an fp32
    [dv] tensor (receives dL/dw when it requires grad)."""
    return _DiffAttnFn.apply(q1, q2, k1, k2, v, lam, norm_weight, lam_init, eps, causal, normalize,
                             noise_of_signal, kv_of_signal)


def lambda_reparam(lq1, lk1, lq2, lk2, lambda_init, *, out=None, stream=None):
    """lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init on the device (fp32 [1])."""
    vs = [x.contiguous() for x in (lq1, lk1, lq2, lk2)]
    if any(x.dtype != torch.float32 or not x.is_cuda for x in vs):
        raise ValueError("the lambda vectors must be fp32 device tensors")
    out = torch.empty(1, dtype=torch.float32, device=lq1.device) if out is None else out
    _check(lib().da_lambda_reparam(*(ctypes.c_void_p(x.data_ptr()) for x in vs), vs[0].numel(), float(lambda_init),
                                   ctypes.c_void_p(out.data_ptr()), _stream(stream)))
    return out


def lambda_reparam_bwd(lq1, lk1, lq2, lk2, dlambda, *, stream=None):
    """Gradients (dlq1, dlk1, dlq2, dlk2) of lambda_reparam for the device scalar dlambda."""
    vs = [x.contiguous() for x in (lq1, lk1, lq2, lk2)]
    outs = [torch.empty_like(x) for x in vs]
    dl = dlambda.reshape(1).float().contiguous()
    _check(lib().da_lambda_reparam_bwd(*(ctypes.c_void_p(x.data_ptr()) for x in vs), vs[0].numel(),
                                       ctypes.c_void_p(dl.data_ptr()), *(ctypes.c_void_p(x.data_ptr()) for x in outs),
                                       _stream(stream)))
    return tuple(outs)


class _LambdaFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, lq1, lk1, lq2, lk2, lambda_init):
        ctx.save_for_backward(lq1, lk1, lq2, lk2)
        return lambda_reparam(lq1, lk1, lq2, lk2, lambda_init).reshape(())

    @staticmethod
    def backward(ctx, dlam):
        return lambda_reparam_bwd(*ctx.saved_tensors, dlam) + (None,)


def lambda_from_params(lq1, lk1, lq2, lk2, lambda_init):
    """Differentiable lambda from the four learnable vectors, computed on the device
    ([DA-blog] "Learnable Lambda Re-parameterization"); pass it to diff_attention."""
    return _LambdaFn.apply(lq1, lk1, lq2, lk2, lambda_init)


def decode_args(q1, q2, k1c, k2c, vc, seq_lens, out, lam, lam_init, *, eps=1e-5, norm_weight=None, normalize=True,
                chunk=0, noise_of_signal=None, kv_of_signal=None, cache_scales=None, block_table=None):
    B, hs, d = q1.shape
    a = DecodeArgs()
    a.q1, a.q2, a.k1_cache, a.k2_cache, a.v_cache = (t.data_ptr() for t in (q1, q2, k1c, k2c, vc))
    a.seq_lens = seq_lens.data_ptr()
    a.out = 0 if out is None else out.data_ptr()
    a.B, a.Lmax, a.H_s, a.H_n, a.H_kv, a.d, a.dv = B, k1c.shape[2], hs, q2.shape[1], k1c.shape[1], d, vc.shape[3]
    a.chunk = int(chunk)
    a.s_q1[:], a.s_q2[:] = _lead(q1, 2), _lead(q2, 2)
    a.s_out[:] = [hs * vc.shape[3], vc.shape[3]] if out is None else _lead(out, 2)
    a.s_k1[:], a.s_k2[:], a.s_v[:] = _lead(k1c, 3), _lead(k2c, 3), _lead(vc, 3)
    nz, nz_keep = _map(noise_of_signal, hs)
    kv, kv_keep = _map(kv_of_signal, hs)
    a.noise_of_signal, a.kv_of_signal = nz, kv
    _set_lambda(a, lam)
    a.lambda_init, a.eps = float(lam_init), float(eps)
    a.norm_w = None if norm_weight is None else norm_weight.data_ptr()
    a.dtype = _dtype_code(q1)
    a.flags = 0 if normalize else DA_NO_NORM
    if k1c.dtype in (torch.uint8, torch.float8_e4m3fn):  # e4m3 codes, read as value * scale
        if cache_scales is None:
            raise ValueError("fp8 caches need cache_scales = (k1_scale, k2_scale, v_scale)")
        a.cache_dtype = DA_FP8_E4M3
        a.k1_scale, a.k2_scale, a.v_scale = (float(x) for x in cache_scales)
    if block_table is not None:  # paged: caches are pools [num_blocks, H, block_size, D]
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be an int32 [B, max_blocks] tensor")
        if not block_table.is_contiguous() or block_table.device != q1.device:
            raise ValueError("block_table must be contiguous and on the device of q1")
        a.block_table = block_table.data_ptr()
        a.block_size, a.max_blocks, a.num_blocks = k1c.shape[2], block_table.shape[1], k1c.shape[0]
        a.Lmax = a.max_blocks * a.block_size
    return a, (nz_keep, kv_keep)


def gda_decode_workspace_bytes(q1, q2, k1c, k2c, vc, seq_lens, **kw) -> int:
    a, keep = decode_args(q1, q2, k1c, k2c, vc, seq_lens, None, 0.0, 0.0,
                          **{k: v for k, v in kw.items() if k not in ("lam", "lam_init")})
    return int(lib().gda_decode_workspace_bytes(ctypes.byref(a)))


def gda_decode(q1, q2, k1c, k2c, vc, seq_lens, lam, lam_init, *, out=None, workspace=None, stream=None, **kw):
    """Split-K GDA decode; caches [B,H,Lmax,D]; see include/diffattn.h."""
    if out is None:
        out = torch.empty((q1.shape[0], q1.shape[1], vc.shape[3]), dtype=q1.dtype, device=q1.device)
    a, keep = decode_args(q1, q2, k1c, k2c, vc, seq_lens, out, lam, lam_init, **kw)
    need = int(lib().gda_decode_workspace_bytes(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    _check(lib().gda_decode(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                            _stream(stream)))
    del keep
    return out


def gda_decode_noalloc(q1, q2, k1c, k2c, vc, seq_lens, lam, lam_init, *, out, stream=None, **kw):
    """gda_decode with the partials in the library's fixed per-GPU scratch (no
    workspace, nothing allocated by the call); `out` must be given.  See
    include/diffattn.h for the size limit and the one-call-at-a-time rule."""
    a, keep = decode_args(q1, q2, k1c, k2c, vc, seq_lens, out, lam, lam_init, **kw)
    _check(lib().gda_decode_noalloc(ctypes.byref(a), _stream(stream)))
    del keep
    return out

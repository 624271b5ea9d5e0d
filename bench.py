#!/usr/bin/env python3
"""Benchmark of the fused causal differential-attention forward on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-extra] [--no-cpu-baseline] [--out FILE] [--copy-calibration]

A step is one call of the hot path on one batch of synthetic, seeded input
already resident in HBM: for the headline workload (the 3B-like Diff
Transformer layer, 4 x 4096 tokens, 24 heads, d = 64, bf16) one gda_fwd /
diffattn_fwd launch.  W untimed steps, then exactly K steps bracketed by
torch.cuda.synchronize(), timed with HIP events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes to
the C ABI).  One JSON line is printed; `value` is F_alg TFLOP/s (each product
of the DiffAttn equation counted once, causal pairs only).  The same line
carries the roofline of the kernel (against the 2.5 PFLOP/s dense bf16 MFMA
peak), the F_exec view (F_alg plus the second P.V an exact one-pass kernel
must issue), the grouped (3:1) prefill, the packed variable-length prefill
(8 sequences of 256..4096 tokens in one call), the split-K decode with bf16
and with e4m3 caches (HBM GB/s against 8 TB/s) and the backward of the two 4096-token layers (gda_bwd) measured
the same way, and the fp64 CPU oracle timed on a
bounded sample of the same workload on the host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from differential_attention_diff_amd import workloads as W  # noqa: E402

METRIC = "diff-attn fwd TFLOP/s (% bf16 MFMA peak) at seq 4096; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

# HBM bytes per launch of the dominant kernel (per step of the multi-kernel decode and
# backward), from rocprofv3 FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch, mean of
# the workload's calls) scaled by what the same counters read for a plain 1 GiB device
# copy in the same run (FETCH x 2.0, WRITE x 1.0); see the HBM counter summaries under
# profiles/.  Each entry is valid only for the kernel sources its counters were taken on
# (sha256 of each file) and is reported as null otherwise.
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "differential_attention_diff_amd", "csrc")
_PREFILL_SRC = {"fwd_bf16.hip": "d47272efd7ac7857523abeaf9b939ef93dd82175fb2d6133f5627b7e5cc5aa5e",
           "fwd_gda3_bf16.hip": "6e12ddf0799d1e53927c36c30a0c36bafc4e32723051557589df3d36876b2a43",
           "fwd_common.h": "bb6ae20a6225278b019d48ff544959515d34ac3ce94bf0133686525236becee1",
           "abi.cpp": "213b8ef6083a5b9334b57809f4192c9222f65971fceab68ed81c6f4b47a26142"}
_DECODE_SRC = {"decode_bf16.hip": "e6011a5ce752106b4036e40c96a967168254d9825c8f60702d4a8c6f597c5e98",
           "abi.cpp": "213b8ef6083a5b9334b57809f4192c9222f65971fceab68ed81c6f4b47a26142"}
_BACKWARD_SRC = {"bwd_ring_bf16.hip": "c14ac302d2cfd9c2eda99c4e2fdb2af7d1be86f3ff0f64e97a0f023919466fa7",
           "bwd_rows.hip": "5fcb2e7c9d1de27467041285c83fc0866eda7e55c9463d69e2401f8423138335",
           "fwd_common.h": "bb6ae20a6225278b019d48ff544959515d34ac3ce94bf0133686525236becee1"}
_KIB = 1024


def _hbm(fetch_kib, write_kib):
    """Calibrated bytes from counter KiB: FETCH x 2.0, WRITE x 1.0."""
    return (fetch_kib * 2.0 + write_kib) * _KIB


MEASURED_TRAFFIC = {
    # prefill: the step's kernel (the map-2 and map-1 launches for shared combos)
    ("prefill", "diff3b_bf16_n4096"): {"sha256": _PREFILL_SRC, "bytes": _hbm(147774.7, 98304.4)},
    ("prefill", "gda3to1_bf16_n4096"): {"sha256": _PREFILL_SRC, "bytes": _hbm(114755.4, 73728.2)},
    ("prefill", "gda4to1_gqa_bf16_n32768"): {"sha256": _PREFILL_SRC,
                                            "bytes": _hbm(143368.4 + 317272.3, 131153.0 + 131072.0)},
    ("prefill", "gda3to1_varlen_bf16_8x4096"): {"sha256": _PREFILL_SRC, "bytes": _hbm(152185.5, 101299.5)},
    # decode: decode_partial_kernel + decode_combine_kernel
    ("decode", "gda_decode_bf16_b64_l8192"): {"sha256": _DECODE_SRC,
                                              "bytes": _hbm(594999.0 + 2114.4, 4119.4 + 288.0)},
    ("decode", "gda_decode_fp8_b64_l8192"): {"sha256": _DECODE_SRC,
                                             "bytes": _hbm(294355.2 + 2114.4, 4119.4 + 288.0)},
    # backward: bwd_prep + bwd_dq_ring + bwd_dkv_ring + bwd_finalize
    ("backward", "diff3b_bf16_n4096"): {"sha256": _BACKWARD_SRC,
                                        "bytes": _hbm(258293.8 + 393794.8 + 290292.9 + 110.6,
                                                      112542.5 + 147455.5 + 196754.6)},
    ("backward", "gda3to1_bf16_n4096"): {"sha256": _BACKWARD_SRC,
                                         "bytes": _hbm(193937.8 + 450707.0 + 456022.9 + 110.6,
                                                      84649.0 + 61441.6 + 123085.2)},
}


def shared_combo_size(w) -> int:
    """Heads per (noise head, key/value head) combo under the default head maps (0: not uniform)."""
    g, gk = w.H_s // w.H_n, w.H_s // w.H_kv
    combos = {}
    for h in range(w.H_s):
        combos[(h // g, h // gk)] = combos.get((h // g, h // gk), 0) + 1
    sizes = set(combos.values())
    return sizes.pop() if len(sizes) == 1 else 0


def prefill_kernel(w) -> str:
    """The prefill kernels gda_fwd runs for a fixed-length workload at d = 64: the map-2 and
    map-1 launches for combos of 2, 4 or 8 signal heads on one noise and one key/value head,
    the per-noise-group kernel for three signal heads per noise head on distinct key/value
    heads, else the general kernel (always for packed sequences and d = 32)."""
    if w.d == 64 and w.kind != "varlen":
        if shared_combo_size(w) in (2, 4, 8):
            return "fwd_shared_kernel<64, false> + fwd_shared_kernel<64, true> (step time)"
        if w.H_s == 3 * w.H_n and w.H_kv == w.H_s:
            return "fwd_gda3_kernel"
    return f"fwd_bf16_kernel<{w.d}>"


def measured_traffic(path: str, workload: str):
    """Counter-derived HBM bytes per launch (or step), or None if absent or a kernel source changed."""
    entry = MEASURED_TRAFFIC.get((path, workload))
    if entry is None:
        return None
    for source, sha in entry["sha256"].items():
        try:
            with open(os.path.join(CSRC, source), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != sha:
                    return None
        except OSError:
            return None
    return entry["bytes"]


# The pages' own throughput figures, carried as context (not a target): model-level
# tokens/s of a Diff Transformer against a standard Transformer of the same size.
PAGES_CONTEXT = {
    "diff_vs_transformer_throughput": [
        {"source": "Differential Transformer (atlas.scime.ai), Measured effects / Limitations",
         "figure": "6-12% (elsewhere on the same page 5-12%) lower throughput at 3B scale",
         "hardware": "not stated"},
        {"source": "llms.blog, Hardware Implementations and Serving Considerations",
         "figure": "3B at 4K tokens, forward+backward training: 6,718 vs 7,491 tokens/s (12%); "
                   "forward prefill: 44,521 vs 48,762 tokens/s (10%); 13B at 2K prefill: 5%",
         "hardware": "NVIDIA H100"},
    ],
    "note": "model-level figures on other hardware; this line measures the attention kernel alone",
}


# ---------------------------------------------------------------------------
# work accounting (algorithmic; independent of how the kernels execute it)
# ---------------------------------------------------------------------------

def pairs(w):
    return w.B * w.N * (w.N + 1) // 2 if w.causal else w.B * w.N * w.N


def f_alg(w):
    """QK1 per signal head + QK2 per noise head (2d each) + one PV per signal head (2dv), per causal pair."""
    return pairs(w) * (w.H_s * 2 * w.d + w.H_n * 2 * w.d + w.H_s * 2 * w.dv)


def f_exec(w):
    """f_alg + one more PV (2dv) per distinct (noise head, kv head) combination (consecutive maps)."""
    g, gk = w.H_s // w.H_n, w.H_s // w.H_kv
    distinct = len({(h // g, h // gk) for h in range(w.H_s)})
    return f_alg(w) + pairs(w) * distinct * 2 * w.dv


def f_alg_bwd(w):
    """Products the gradient of the DiffAttn equation needs, each counted once per causal pair:
    per signal head the recomputed Q1K1^T (2d), dP = dO V^T (2dv), dV (2dv), dQ1 and dK1 (2d each);
    per noise head the recomputed Q2K2^T, dQ2 and dK2 (2d each; dS2 summed over the group first)."""
    return pairs(w) * (w.H_s * (3 * 2 * w.d + 2 * 2 * w.dv) + w.H_n * 3 * 2 * w.d)


def prefill_bytes(w):
    e = 2 if w.dtype == "bf16" else 4
    return e * w.B * w.N * ((w.H_s + w.H_n) * w.d + (w.H_kv + w.H_n) * w.d + w.H_kv * w.dv + w.H_s * w.dv)


def decode_bytes(w, seq_lens):
    """Each cached K1/V byte of every kv head and K2 byte of every noise head for positions < L_b,
    plus the queries and the output."""
    L = int(np.sum(seq_lens))
    ce = 1 if w.cache == "fp8" else 2  # cache bytes per element
    per_pos = ce * (w.H_kv * w.d + w.H_n * w.d + w.H_kv * w.dv)
    return L * per_pos + 2 * w.B * ((w.H_s + w.H_n) * w.d + w.H_s * w.dv)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands, on a bounded sample
# ---------------------------------------------------------------------------

_CPU = {}


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_unit(unit):
    from oracle import diffattn_oracle as O
    b, h = unit
    a = _CPU
    O.diff_attention_rows(a["q1"][b:b + 1], a["q2"][b:b + 1], a["k1"][b:b + 1], a["k2"][b:b + 1],
                          a["v"][b:b + 1], a["lam"], a["lam_init"], rows=a["rows"], heads=[h], eps=a["eps"])
    return 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, nrows: int):
    """Time the oracle on `nrows` query rows (spread over the sequence) for every (batch, signal head)
    of the workload, one process per core; report F_alg TFLOP/s of that sample."""
    import multiprocessing as mp
    visible = len(os.sched_getaffinity(0))
    # one process per core of the host share one GPU gets (16 cores per GPU on the
    # MI355X boxes this runs on, whatever the affinity mask shows)
    cores = max(1, min(visible, 16))
    rows = np.unique(np.linspace(0, w.N - 1, nrows).round().astype(np.int64))
    _CPU.clear()
    _CPU.update({k: inp[k].float().double().numpy() for k in ("q1", "q2", "k1", "k2", "v")})
    _CPU.update(rows=rows, lam=w.lam, lam_init=w.lam_init, eps=w.eps)
    units = [(b, h) for b in range(w.B) for h in range(w.H_s)]
    ctx = mp.get_context("fork")   # fork before any GPU initialisation in this process
    with ctx.Pool(cores, initializer=_limit_blas) as pool:
        pool.map(_oracle_unit, units[:cores])   # warm the workers (imports)
        t0 = time.perf_counter()
        pool.map(_oracle_unit, units, chunksize=1)
        dt = time.perf_counter() - t0
    vis = int(np.sum(rows + 1)) if w.causal else len(rows) * w.N
    flops = w.B * vis * (w.H_s * 2 * w.d + w.H_n * 2 * w.d + w.H_s * 2 * w.dv)
    _CPU.clear()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3), "cores_visible": visible, "cpu_model": cpu_model(),
            "sample": f"{len(rows)} query rows evenly spaced over [0, {w.N}) x {w.B} batches x {w.H_s} signal heads "
                      f"of {w.name} (fp64 NumPy oracle, one process per core, BLAS 1 thread each); "
                      f"F_alg of the sampled causal pairs / wall time"}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per step


def bench_prefill(w, steps, warmup, inp=None):
    import torch
    from differential_attention_diff_amd import ops
    inp = W.make_prefill_inputs(w) if inp is None else inp
    d = {k: v.cuda() for k, v in inp.items()}
    out = torch.empty(w.B, w.N, w.H_s, w.dv, dtype=w.torch_dtype, device="cuda")
    plain = w.H_n == w.H_s and w.H_kv == w.H_s
    entry = ops.diffattn_fwd if plain else ops.gda_fwd
    fn = lambda: entry(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], w.lam, w.lam_init, out=out, eps=w.eps)
    ms = time_steps(fn, steps, warmup)
    fa, fe = f_alg(w), f_exec(w)
    ach, ache = fa / (ms * 1e-3) / 1e12, fe / (ms * 1e-3) / 1e12
    return {
        "workload": w.name, "value": ach, "unit": "TFLOP/s", "ms_per_step": ms,
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H_s": w.H_s, "H_n": w.H_n, "H_kv": w.H_kv, "d": w.d,
                   "dv": w.dv, "causal": w.causal, "entry": "diffattn_fwd" if plain else "gda_fwd",
                   "flop_convention": "F_alg"},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill", w.name),
                     "flops_per_launch": fa, "kernel": prefill_kernel(w)},
        "roofline_exec": {"achieved": ache, "frac": ache / PEAK_BF16_TFLOPS, "flops_per_launch": fe},
        "algorithmic_bytes": prefill_bytes(w),
    }


def bench_varlen(w, steps, warmup):
    """Packed prefill: F_alg summed over the sequences' own causal pairs."""
    import torch
    from differential_attention_diff_amd import ops
    inp = W.make_varlen_inputs(w)
    d = {k: (v.cuda() if hasattr(v, "cuda") else v) for k, v in inp.items()}
    T = d["q1"].shape[0]
    out = torch.empty(T, w.H_s, w.dv, dtype=w.torch_dtype, device="cuda")
    fn = lambda: ops.gda_fwd_varlen(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], d["cu_seqlens"], d["max_seqlen"],
                                    w.lam, w.lam_init, out=out, eps=w.eps)
    ms = time_steps(fn, steps, warmup)
    lengths = np.diff(inp["cu_seqlens"].numpy().astype(np.int64))
    per_pair = w.H_s * 2 * w.d + w.H_n * 2 * w.d + w.H_s * 2 * w.dv
    fa = int(np.sum(lengths * (lengths + 1) // 2)) * per_pair
    ach = fa / (ms * 1e-3) / 1e12
    return {
        "workload": w.name, "value": ach, "unit": "TFLOP/s", "ms_per_step": ms,
        "config": {"workload": w.name, "nseq": w.B, "lengths": lengths.tolist(), "tokens": T,
                   "max_seqlen": d["max_seqlen"], "H_s": w.H_s, "H_n": w.H_n, "H_kv": w.H_kv, "d": w.d, "dv": w.dv,
                   "causal": True, "entry": "gda_fwd_varlen", "flop_convention": "F_alg"},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill", w.name),
                     "flops_per_launch": fa, "kernel": prefill_kernel(w)},
    }


def bench_backward(w, steps, warmup):
    """gda_bwd on the prefill workload (row pass, dQ pass, dK/dV pass, reduction), with the forward's
    lse and per-map outputs and a seeded dout resident in HBM."""
    import torch
    from differential_attention_diff_amd import ops
    d = {k: v.cuda() for k, v in W.make_prefill_inputs(w).items()}
    g = torch.Generator("cpu").manual_seed(w.seed + 100)
    dout = torch.randn(w.B, w.N, w.H_s, w.dv, generator=g).to(w.torch_dtype).cuda()
    lse = torch.empty(2, w.B, w.H_s, w.N, device="cuda")
    om = torch.empty(2, w.B, w.N, w.H_s, w.dv, device="cuda")
    ops.gda_fwd(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], w.lam, w.lam_init, eps=w.eps, lse=lse, o_maps=om)
    grads = tuple(torch.empty_like(d[k]) for k in ("q1", "q2", "k1", "k2", "v"))
    nbytes = ops.gda_bwd_workspace_bytes(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], om, lse, dout)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fn = lambda: ops.gda_bwd(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], om, lse, dout, w.lam, w.lam_init,
                             grads=grads, workspace=ws, eps=w.eps)
    ms = time_steps(fn, steps, warmup)
    fb = f_alg_bwd(w)
    ach = fb / (ms * 1e-3) / 1e12
    return {
        "workload": w.name + " backward", "value": ach, "unit": "TFLOP/s", "ms_per_step": ms,
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H_s": w.H_s, "H_n": w.H_n, "H_kv": w.H_kv, "d": w.d,
                   "dv": w.dv, "causal": w.causal, "entry": "gda_bwd", "flop_convention": "F_alg backward"},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic("backward", w.name),
                     "flops_per_launch": fb,
                     "kernel": "bwd_prep + bwd_dq_ring_kernel + bwd_dkv_ring_kernel + bwd_finalize (step time)"},
    }


def bench_decode(w, steps, warmup):
    import torch
    from differential_attention_diff_amd import ops
    inp = W.make_decode_inputs(w)
    scales = inp.pop("cache_scales", None)
    d = {k: v.cuda() for k, v in inp.items()}
    out = torch.empty(w.B, w.H_s, w.dv, dtype=w.torch_dtype, device="cuda")
    nbytes = ops.gda_decode_workspace_bytes(d["q1"], d["q2"], d["k1_cache"], d["k2_cache"], d["v_cache"],
                                            d["seq_lens"], cache_scales=scales)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fn = lambda: ops.gda_decode(d["q1"], d["q2"], d["k1_cache"], d["k2_cache"], d["v_cache"], d["seq_lens"],
                                w.lam, w.lam_init, out=out, workspace=ws, eps=w.eps, cache_scales=scales)
    ms = time_steps(fn, steps, warmup)
    nb = decode_bytes(w, inp["seq_lens"].numpy())
    gbs = nb / (ms * 1e-3) / 1e9
    probe = stream_read_probe(nb, steps, warmup)
    return {
        "workload": w.name, "metric": "decode HBM GB/s", "value": gbs, "unit": "GB/s", "ms_per_step": ms,
        "config": {"workload": w.name, "B": w.B, "Lmax": w.N, "len_range": list(w.len_range),
                   "sum_seq_lens": int(inp["seq_lens"].sum()), "H_s": w.H_s, "H_n": w.H_n, "H_kv": w.H_kv,
                   "d": w.d, "dv": w.dv, "cache": "e4m3 + per-cache scale" if w.cache == "fp8" else "bf16",
                   "entry": "gda_decode"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("decode", w.name),
                     "bytes_per_launch": nb,
                     "kernel": "decode_partial_kernel + decode_combine_kernel (step time)",
                     "stream_read_probe": probe, "frac_of_probe": gbs / probe["value"]},
    }


PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")
_probe = None


def build_probe(verbose: bool = False) -> str:
    """Compile bench_probe.hip (the streaming-read probe; not part of libdiffattn.so)."""
    from differential_attention_diff_amd import build as B
    return B.build_shared(PROBE_SRC, PROBE_LIB, verbose)


def probe_lib():
    global _probe
    if _probe is None:
        import ctypes
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(PROBE_LIB)
        L.bench_hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.bench_hbm_read_probe.restype = ctypes.c_int
        L.bench_issue_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.bench_issue_probe.restype = ctypes.c_int
        _probe = L
    return _probe


def hbm_read_probe(buf, sink, stream=None):
    """Read every byte of the device tensor `buf` once with the streaming-read probe;
    `sink` is a device fp32 tensor (written only with negligible probability)."""
    import ctypes
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    st = probe_lib().bench_hbm_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                          ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise RuntimeError(f"bench_hbm_read_probe returned {st}")


def stream_read_probe(nbytes, steps, warmup):
    """Read rate of a plain streaming-read kernel (bench_probe.hip) over a buffer of
    `nbytes`, the size of one decode step's reads: the measured reference beside the
    published 8 TB/s."""
    import torch
    nb = (int(nbytes) + 15) // 16 * 16
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    ms = time_steps(lambda: hbm_read_probe(buf, sink), steps, warmup)
    del buf
    return {"value": nb / (ms * 1e-3) / 1e9, "unit": "GB/s", "bytes": nb,
            "kernel": "hbm_read_probe_kernel (non-temporal 16-B loads, 4 in flight per thread, 16384 x 256 threads)"}


ISSUE_PROBE_OPS = ["v_fma_f32 v,v,const", "v_fma_f32 v,s,v", "v_fma_f32 v,v,v", "v_mul_f32 v,v", "v_add_u32 v,v",
                   "v_cvt_pk_bf16_f32", "v_dot2c_f32_bf16", "v_exp_f32", "v_mov_b32", "v_exp_f32 (8 per 4 MFMAs)"]
ISSUE_PROBE_PER_ITER = [32] * 9 + [8]  # VALU instructions per wavefront and iteration


def issue_probe(iters=2048, reps=2):
    """What runs beside the matrix pipe (bench_probe.hip, bench_issue_probe): per VALU
    type, the time of its wavefronts alone (mode 1, two per SIMD), of the MFMA
    wavefronts alone (mode 0, one per SIMD) and of both sharing the SIMDs (mode 2).
    `ns_per_instr` is the SIMD's issue time per wavefront instruction with two
    wavefronts issuing that type; `overlap` is the share of the shorter part hidden
    under the longer: (mfma + valu/2 - both) / min(mfma, valu/2), 1 = fully hidden,
    0 = serialised (valu/2: one of the two VALU wavefronts, as in mode 2)."""
    import ctypes
    import torch
    L = probe_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * 4  # four rounds of one workgroup per CU
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()

    def launch(op, mode):
        st = L.bench_issue_probe(op, mode, iters, blocks, ctypes.c_void_p(out.data_ptr()), out.numel(),
                                 ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError(f"bench_issue_probe returned {st}")

    rows = []
    for rep in range(reps):
        t_m = time_steps(lambda: launch(0, 0), 2, 1)
        for op, name in enumerate(ISSUE_PROBE_OPS):
            per_simd = blocks / cus * 2 * iters * ISSUE_PROBE_PER_ITER[op]  # VALU instructions per SIMD, mode 1
            t_v = time_steps(lambda: launch(op, 1), 2, 1)
            t_b = time_steps(lambda: launch(op, 2), 2, 1)
            half = t_v / 2
            rows.append({"rep": rep, "op": name, "ns_per_instr": t_v * 1e6 / per_simd, "valu_ms": half,
                         "mfma_ms": t_m, "both_ms": t_b, "overlap": (t_m + half - t_b) / min(t_m, half)})
    mfma_ns = min(r["mfma_ms"] for r in rows) * 1e6 / (blocks / cus * iters * 4)  # MFMAs per SIMD in mode 0
    return {"probe": "issue", "mfma": "v_mfma_f32_32x32x16_bf16", "ns_per_mfma_per_simd": mfma_ns, "rows": rows}


def device_info():
    """The device the line was measured on, and the dense bf16 peak its CU count implies at
    the published 2.4 GHz (4 SIMDs x 1024 FLOP per clock per CU); the clock the matrix cores
    hold under load is lower (about 2.0 GHz in the counter profiles)."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    cus = int(getattr(pr, "multi_processor_count", 0))
    info = {"name": torch.cuda.get_device_name(0), "arch": getattr(pr, "gcnArchName", None), "cus": cus,
            "bf16_peak_at_2p4ghz_tflops": cus * 4 * 1024 * 2.4e9 / 1e12 if cus else None}
    clk = getattr(pr, "clock_rate", None)  # kHz, where torch exposes it
    if clk:
        info["max_sclk_mhz"] = clk / 1000.0
    return info


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """Plain device-to-device copies of a known size: a profiler's FETCH_SIZE / WRITE_SIZE for
    these dispatches should read nbytes each; the ratio scales the counters of the kernels."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes, "copies": reps}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="diff3b_bf16_n4096",
                    choices=[k for k in W.ORDER if k != "tiny_diff_f32"] + ["gda3to1_varlen_bf16_8x4096",
                                                                             "gda_decode_fp8_b64_l8192"])
    ap.add_argument("--no-extra", action="store_true", help="skip the grouped, packed and decode lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed work, run 3 plain device copies of 1 GiB (reference dispatches that "
                         "scale the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows in the CPU-baseline sample (default: every row of the 4096-token workload)")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--issue-probe", action="store_true",
                    help="instead of the benchmark: which VALU instruction types run beside the matrix pipe "
                         "(bench_probe.hip), one JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is described in the design "
              "notes but not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.issue_probe:
        line = json.dumps(issue_probe())
        print(line, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(line + "\n")
        return

    w = W.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = W.make_prefill_inputs(w) if w.kind == "prefill" else None

    cpu = None
    if not args.no_cpu_baseline and w.kind == "prefill":
        print(f"[bench] CPU oracle baseline ({args.cpu_rows} rows sample)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, args.cpu_rows)
        print(f"[bench] CPU oracle: {cpu['seconds']} s on {cpu['cores']} cores", file=sys.stderr, flush=True)

    import torch
    print(f"[bench] GPU {torch.cuda.get_device_name(0)}: timing {w.name}", file=sys.stderr, flush=True)
    if w.kind == "prefill":
        head = bench_prefill(w, args.steps, args.warmup, inp)
    else:
        head = (bench_varlen if w.kind == "varlen" else bench_decode)(w, args.steps, args.warmup)
    extra = []
    if not args.no_extra:
        for name in ("gda3to1_bf16_n4096", "gda4to1_gqa_bf16_n32768", "gda_decode_bf16_b64_l8192",
                     "gda_decode_fp8_b64_l8192", "gda3to1_varlen_bf16_8x4096"):
            if name == w.name:
                continue
            ew = W.WORKLOADS[name]
            print(f"[bench] timing {name}", file=sys.stderr, flush=True)
            run = {"prefill": bench_prefill, "decode": bench_decode, "varlen": bench_varlen}[ew.kind]
            extra.append(run(ew, args.steps, args.warmup))
        for name in ("diff3b_bf16_n4096", "gda3to1_bf16_n4096"):
            print(f"[bench] timing {name} backward", file=sys.stderr, flush=True)
            extra.append(bench_backward(W.WORKLOADS[name], args.steps, args.warmup))

    line = {
        "metric": METRIC,
        "value": round(head["value"], 3),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    if "roofline_exec" in head:
        line["roofline_exec"] = head["roofline_exec"]
    line["cpu_baseline"] = cpu
    line["context"] = PAGES_CONTEXT
    line["device"] = device_info()
    line["extra"] = extra
    if args.copy_calibration:
        line["copy_calibration"] = copy_calibration()
    text = json.dumps(line)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()

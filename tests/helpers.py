"""Shared helpers for the GPU tests: device copies, the parity bar, input
builders.  Inputs come from the seeded generators; expected values from the
fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

# parity bar: fp32 max-abs 1e-5; bf16 max-abs 2e-2 and relative L2 5e-3
F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_REL_L2 = 5e-3


def to_dev(d: dict) -> dict:
    return {k: v.to("cuda") for k, v in d.items()}


def as64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def err_stats(got: np.ndarray, want: np.ndarray):
    diff = got - want
    maxabs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    return maxabs, rel


def assert_parity(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    maxabs, rel = err_stats(got, want)
    if dtype == "f32":
        assert maxabs <= F32_ATOL, f"{what}: fp32 max-abs {maxabs:.3e} > {F32_ATOL}"
    else:
        assert maxabs <= BF16_ATOL and rel <= BF16_REL_L2, \
            f"{what}: bf16 max-abs {maxabs:.3e} (bar {BF16_ATOL}), rel-L2 {rel:.3e} (bar {BF16_REL_L2})"
    return maxabs, rel


def sample_rows(N: int, extra: int, seed: int):
    """Rows at tile and block edges plus seeded random rows."""
    fixed = {0, 1, 31, 32, 63, 64, 65, 127, 128, 129, N // 2, N - 129, N - 128, N - 65, N - 64, N - 33, N - 2, N - 1}
    rng = np.random.default_rng(seed)
    rand = set(rng.integers(0, N, extra).tolist())
    return sorted(r for r in fixed | rand if 0 <= r < N)


def rand_inputs(B, N, hs, hn, hkv, d, dtype, seed, v_std=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g).to(dtype)
    return {"q1": mk(B, N, hs, d), "q2": mk(B, N, hn, d), "k1": mk(B, N, hkv, d), "k2": mk(B, N, hn, d),
            "v": (torch.randn(B, N, hkv, 2 * d, generator=g) * v_std).to(dtype)}


def norm_scale(want_raw: np.ndarray, lam_init: float, eps: float = 1e-5) -> np.ndarray:
    """Per-row factor the head norm applies to the oracle's raw output,
    (1 - lambda_init) / sqrt(mean(o^2) + eps): the bf16 bar is stated for the
    normalised output, so a raw (DA_NO_NORM) result is held to it after the
    same per-row scaling."""
    return (1.0 - lam_init) / np.sqrt(np.mean(want_raw ** 2, axis=-1, keepdims=True) + eps)

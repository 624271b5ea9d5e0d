"""GPU checks of lambda on the device: the re-parameterisation and its
gradient against the oracle, and the prefill / decode / backward reading
lambda from a device scalar (bitwise equal to passing the same value by
host), end to end through autograd."""

import numpy as np
import pytest
import torch

from differential_attention_diff_amd import ops
from differential_attention_diff_amd import workloads as W
from oracle import diffattn_oracle as O
from tests.helpers import as64, rand_inputs

pytestmark = pytest.mark.gpu


def vecs(dim, seed, scale=0.1):
    g = torch.Generator("cpu").manual_seed(seed)
    return [(torch.randn(dim, generator=g) * scale).cuda() for _ in range(4)]


@pytest.mark.parametrize("dim", [1, 64, 1000])
def test_reparam_and_gradient_match_the_oracle(dim):
    v = vecs(dim, 90 + dim)
    lam = ops.lambda_reparam(*v, 0.35)
    torch.cuda.synchronize()
    want = O.lambda_reparam(*[x.cpu() for x in v], 0.35)
    assert abs(float(lam.cpu()[0]) - want) <= 1e-6 * max(1.0, abs(want))
    dl = torch.tensor([1.3], device="cuda")
    got = ops.lambda_reparam_bwd(*v, dl)
    torch.cuda.synchronize()
    for g, w in zip(got, O.lambda_reparam_grad(*[x.cpu() for x in v], 1.3)):
        np.testing.assert_allclose(as64(g), w, rtol=1e-5, atol=1e-7)


def test_device_lambda_equals_host_lambda():
    inp = {k: x.cuda() for k, x in rand_inputs(B=1, N=200, hs=6, hn=2, hkv=2, d=64, dtype=torch.bfloat16,
                                              seed=91).items()}
    lam_h = 0.7125
    lam_d = torch.tensor([lam_h], device="cuda")
    lse = [torch.empty(2, 1, 6, 200, device="cuda") for _ in range(2)]
    om = [torch.empty(2, 1, 200, 6, 128, device="cuda") for _ in range(2)]
    a = ops.gda_fwd(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], lam_h, 0.3, lse=lse[0], o_maps=om[0])
    b = ops.gda_fwd(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], lam_d, 0.3, lse=lse[1], o_maps=om[1])
    assert torch.equal(a, b)
    dout = torch.randn(1, 200, 6, 128, generator=torch.Generator("cpu").manual_seed(92)).to(torch.bfloat16).cuda()
    ga = ops.gda_bwd(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], om[0], lse[0], dout, lam_h, 0.3)
    gb = ops.gda_bwd(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], om[1], lse[1], dout, lam_d, 0.3)
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)
    w = W.WORKLOADS["gda_decode_bf16_b64_l8192"]
    d = {k: x.cuda() for k, x in W.make_decode_inputs(w, B=3, Lmax=512, len_range=(1, 512)).items()}
    da = ops.gda_decode(d["q1"], d["q2"], d["k1_cache"], d["k2_cache"], d["v_cache"], d["seq_lens"], lam_h, 0.3)
    db = ops.gda_decode(d["q1"], d["q2"], d["k1_cache"], d["k2_cache"], d["v_cache"], d["seq_lens"], lam_d, 0.3)
    torch.cuda.synchronize()
    assert torch.equal(da, db)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_autograd_through_the_reparameterisation(dtype):
    inp = rand_inputs(B=1, N=80, hs=4, hn=2, hkv=2, d=64, dtype=dtype, seed=93)
    d = {k: x.cuda().requires_grad_(True) for k, x in inp.items()}
    v = [x.requires_grad_(True) for x in vecs(64, 94)]
    lam = ops.lambda_from_params(*v, 0.2)
    out = ops.diff_attention(d["q1"], d["q2"], d["k1"], d["k2"], d["v"], lam, 0.2)
    dout = torch.randn(1, 80, 4, 128, generator=torch.Generator("cpu").manual_seed(95)).to(dtype)
    (out.float() * dout.cuda().float()).sum().backward()
    lam_o = O.lambda_reparam(*[x.detach().cpu() for x in v], 0.2)
    want = O.diff_attention_backward(inp["q1"], inp["q2"], inp["k1"], inp["k2"], inp["v"], dout, lam_o, 0.2)
    wl = O.lambda_reparam_grad(*[x.detach().cpu() for x in v], want["dlambda"])
    if dtype == torch.float32:
        for g, w_ in zip(v, wl):
            np.testing.assert_allclose(as64(g.grad), w_, rtol=1e-4, atol=1e-4 * np.max(np.abs(w_)))
    else:
        # each vector's gradient is dlambda times its Jacobian; bf16 dlambda is held
        # to 2^-7 of the L2 norm of the terms it sums (see the backward tests)
        jac = O.lambda_reparam_grad(*[x.detach().cpu() for x in v], 1.0)
        for g, w_, j in zip(v, wl, jac):
            err = np.abs(as64(g.grad) - w_)
            bar = 2.0 ** -7 * want["dlambda_scale"] * np.abs(j) + 1e-5 * np.abs(w_)  # + the fp32 chain's rounding
            assert np.all(err <= bar), f"max error / bar {np.max(err / bar):.3f}"

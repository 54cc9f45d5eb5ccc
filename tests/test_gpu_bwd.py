"""GPU parity of the backward kernels (dq, dk, dv) against the fp64 oracle.

Tolerance (bf16 inputs).  The kernels round P and dS to bf16 as MFMA operands
(relative error up to 2^-9 each, independent from element to element) and the
gradients to bf16 on output (2^-9); accumulation is fp32.  Random-signed
rounding errors of relative size u add in quadrature, each contributing about
u / sqrt(3) ~ 1.1e-3 to the relative L2 error: two to three such terms give
~2-3e-3 (dq and dk pass through dS and the output rounding, dv through P and
the output rounding).  The bound is the forward's, rel-L2 <= 5e-3 per gradient
tensor, with its max-abs bound (2e-2) taken relative to the largest reference
magnitude.  Padded key slots must be
exactly zero, and the results must be bitwise deterministic and bitwise
independent of what the padded slots hold.
"""

import math

import numpy as np
import pytest
import torch

from long_context_prefix_amd import _lib, prefix_attention
from long_context_prefix_amd.workloads import make_inputs
from oracle import ref_prefix_bwd
from tests.parity import assert_grad_parity, log, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _grads(q, k, v, kv, scale, seed):
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, scale)
    g = torch.Generator(device="cpu").manual_seed(seed)
    dout = torch.randn(q.shape, generator=g).to(q.dtype).to(DEV)
    dq, dk, dv = _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, scale)
    torch.cuda.synchronize()
    return dout, dq, dk, dv


def _check(name, got, ref, what):
    assert_grad_parity(name, got, ref, what)


def _compare(q, k, v, kv, scale, seed, what):
    dout, dq, dk, dv = _grads(q, k, v, kv, scale, seed)
    lens = kv.cpu().numpy()
    rq, rk, rv = ref_prefix_bwd(to64(q), to64(k), to64(v), lens, scale, to64(dout))
    _check("dq", dq, rq, what)
    _check("dk", dk, rk, what)
    _check("dv", dv, rv, what)
    S = k.shape[2]
    for b, n in enumerate(lens):
        if n < S:
            assert torch.all(dk[b, :, n:] == 0) and torch.all(dv[b, :, n:] == 0), f"{what}: padded gradient"
    return dq, dk, dv


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Tq", [1, 17, 64, 150])
def test_bwd_edge_matrix(D, Tq):
    S = 300
    lens = [0, 1, 63, 64, 65, 129, S]
    log(f"bwd edge D={D} Tq={Tq} lens={lens}")
    q, k, v, kv = make_inputs(len(lens), 2, Tq, S, D, lens, "bf16", 1.0, seed=900 + D + Tq, device=DEV)
    _compare(q, k, v, kv, 1.0 / math.sqrt(D), 77 + Tq, f"bwd D={D} Tq={Tq}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bwd_multi_tile_sharp(D):
    """Several query and key tiles in both kernels, ragged tails, peaky attention (q x 3)."""
    B, H, Tq, S = 2, 3, 333, 777
    lens = [700, 777]
    log(f"bwd sharp D={D}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=950 + D, device=DEV)
    q.mul_(3.0)
    _compare(q, k, v, kv, 1.0 / math.sqrt(D), 5, f"bwd sharp D={D}")


def test_bwd_padding_invariance_and_determinism():
    B, H, Tq, S, D = 3, 2, 200, 400, 128
    lens = [400, 213, 1]
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=960, device=DEV)
    k2, v2 = k.clone(), v.clone()
    for b, n in enumerate(lens):
        k2[b, :, n:] = float("nan")
        v2[b, :, n:] = float("nan")
    a = _grads(q, k, v, kv, 0.1, 3)
    b_ = _grads(q, k2, v2, kv, 0.1, 3)
    c = _grads(q, k, v, kv, 0.1, 3)
    for x, y, z in zip(a[1:], b_[1:], c[1:]):
        assert torch.equal(x, y), "padded slot contents changed a gradient"
        assert torch.equal(x, z), "two runs differ"


def test_bwd_empty_sizes():
    D = 64
    # Tq = 0: dk and dv are zero (no query depends on the keys)
    q, k, v, kv = make_inputs(2, 1, 0, 100, D, [100, 50], "bf16", 1.0, seed=970, device=DEV)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    e = torch.empty_like(q)
    lse = torch.empty((2, 1, 0), dtype=torch.float32, device=DEV)
    _lib.attn_prefix_bwd(q, k, v, kv, e, e, lse, 0.125, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    # S = 0: dq is zero
    q, k, v, kv = make_inputs(2, 1, 10, 0, D, [0, 0], "bf16", 1.0, seed=971, device=DEV)
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, 0.125)
    dq = torch.full_like(q, 7.0)
    _lib.attn_prefix_bwd(q, k, v, kv, out, torch.ones_like(q), lse, 0.125, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_bwd_unsupported_is_an_error():
    """The backward takes bf16 only: fp32 inputs are refused, not rerouted."""
    q, k, v, kv = make_inputs(1, 1, 8, 8, 64, [8], "f32", 1.0, seed=972, device=DEV)
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, 0.125)
    with pytest.raises(_lib.AttnError):
        _lib.attn_prefix_bwd(q, k, v, kv, out, out, lse, 0.125)


def test_autograd_wrapper_matches_oracle():
    B, H, Tq, S, D = 2, 2, 96, 160, 64
    lens = [160, 37]
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=980, device=DEV)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = prefix_attention(qq, kk, vv, kv)
    g = torch.Generator(device="cpu").manual_seed(81)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    out.backward(dout)
    torch.cuda.synchronize()
    rq, rk, rv = ref_prefix_bwd(to64(q), to64(k), to64(v), np.array(lens), 1.0 / math.sqrt(D), to64(dout))
    _check("dq", qq.grad, rq, "autograd")
    _check("dk", kk.grad, rk, "autograd")
    _check("dv", vv.grad, rv, "autograd")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_bwd_scale_sign_and_zero(D, scale):
    """Negative scales (the dq kernel negates Q internally), scale 0 (uniform weights: every
    gradient path still runs) and a large scale, on ragged lengths whose last key tiles are
    partly masked."""
    B, H, Tq, S = 2, 2, 130, 300
    lens = [300, 77]
    log(f"bwd scale={scale} D={D}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=990 + D, device=DEV)
    _compare(q, k, v, kv, scale, 11, f"bwd scale={scale} D={D}")

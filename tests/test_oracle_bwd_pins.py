"""Pins of the fp64 backward oracle (``ref_prefix_bwd``) to facts outside it.

The backward is the exact derivative of the forward, so it is pinned by:
* central finite differences of the (separately pinned) forward oracle;
* torch's own CPU float64 autograd through ``scaled_dot_product_attention``, on
  truncated keys and with a boolean prefix mask (a library routine, not shared
  code);
* closed forms: n = 1 makes the output independent of q and k (zero dq, dk) and
  dv[0] the sum of dout over the queries; n = 0 gives zero gradients;
* invariants: the key gradients sum to zero over the valid keys, the value
  gradients sum to the summed dout, padded slots get exactly zero even when
  they hold NaN, gradients are linear in dout, a ragged batch equals
  per-element calls.

The identity that carries the prefix mask over to the gradients is the
truncation identity of page "Rewrite prefix key-padding masks as k/v truncation
to keep SDPA on the flash path (PyTorch)" (section Fix); ragged batches are the
per-element form of its section Tests.  Each check is a plain function of the
backward callable so that planted mistakes (on the CPU, below) can be run
through the same checks.
"""

import numpy as np
import pytest
import torch

import oracle.attn_oracle as O
from oracle import ref_prefix_bwd, ref_prefix_fwd

SCALE = 0.625  # exact in fp32, so the fp32 rounding of the scale plays no part


def _case(seed, B=2, H=2, T=5, S=9, D=4, lens=(9, 4), pad=1e4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, D))
    k = rng.standard_normal((B, H, S, D))
    v = rng.standard_normal((B, H, S, D))
    for b, n in enumerate(lens):
        k[b, :, n:] = pad * np.sign(rng.standard_normal(k[b, :, n:].shape))
        v[b, :, n:] = pad * np.sign(rng.standard_normal(v[b, :, n:].shape))
    dout = rng.standard_normal((B, H, T, D))
    return q, k, v, np.array(lens), dout, rng


# --------------------------------------------------------------------------- checks


def check_finite_differences(bwd):
    """<grad, delta> equals the central difference of sum(dout * out) along delta."""
    q, k, v, lens, dout, rng = _case(31)
    dq, dk, dv = bwd(q, k, v, lens, SCALE, dout)

    def loss(qq, kk, vv):
        return float((ref_prefix_fwd(qq, kk, vv, lens, SCALE)[0] * dout).sum())

    eps = 1e-5
    for which, g in (("q", dq), ("k", dk), ("v", dv)):
        d = rng.standard_normal(g.shape)
        args_p = [q, k, v]
        args_m = [q, k, v]
        i = "qkv".index(which)
        args_p[i] = args_p[i] + eps * d
        args_m[i] = args_m[i] - eps * d
        fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        dot = float((g * d).sum())
        assert abs(fd - dot) <= 1e-7 * max(1.0, abs(dot)), (which, fd, dot)


def check_library_autograd(bwd):
    """torch float64 autograd: truncated keys, and the [B,1,1,S] bool prefix mask."""
    q, k, v, lens, dout, _ = _case(32)
    dq, dk, dv = bwd(q, k, v, lens, SCALE, dout)
    B, H, T, D = q.shape
    S = k.shape[2]
    for b in range(B):
        n = int(lens[b])
        tq = torch.tensor(q[b:b + 1], requires_grad=True)
        tk = torch.tensor(k[b:b + 1, :, :n], requires_grad=True)
        tv = torch.tensor(v[b:b + 1, :, :n], requires_grad=True)
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=SCALE)
        out.backward(torch.tensor(dout[b:b + 1]))
        np.testing.assert_allclose(dq[b], tq.grad[0].numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[b, :, :n], tk.grad[0].numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[b, :, :n], tv.grad[0].numpy(), rtol=0, atol=1e-11)
    # masked form over all S slots with finite pads: same gradients, zero on the pads
    mask = torch.from_numpy(np.arange(S)[None, :] < lens[:, None])[:, None, None, :]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=SCALE)
    out.backward(torch.tensor(dout))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def check_n_one_and_zero(bwd):
    """n = 1: out = v_0 for every query, so dq = dk = 0 exactly and dv_0 = sum_i dout_i.
    n = 0: the output is the constant 0 and every gradient is 0."""
    q, k, v, _, dout, _ = _case(33, lens=(1, 0))
    dq, dk, dv = bwd(q, k, v, np.array([1, 0]), SCALE, dout)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(dv[0, :, 0], dout[0].sum(axis=1), rtol=0, atol=1e-13)
    assert np.all(dv[0, :, 1:] == 0.0)
    assert np.all(dv[1] == 0.0)


def check_sums_and_pads(bwd):
    """sum_j dk_j = 0 (softmax gradients sum to zero over the keys); sum_j dv_j = sum_i dout_i;
    NaN in padded slots changes nothing and the padded gradient is exactly zero."""
    q, k, v, lens, dout, _ = _case(34, lens=(9, 3))
    dq, dk, dv = bwd(q, k, v, lens, SCALE, dout)
    for b, n in enumerate(lens):
        scale_ref = np.abs(dk[b]).max() + 1.0
        assert np.abs(dk[b, :, :n].sum(axis=1)).max() <= 1e-12 * scale_ref
        np.testing.assert_allclose(dv[b, :, :n].sum(axis=1), dout[b].sum(axis=1), rtol=0, atol=1e-12)
        assert np.all(dk[b, :, n:] == 0.0) and np.all(dv[b, :, n:] == 0.0)
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k2[b, :, n:] = np.nan
        v2[b, :, n:] = np.nan
    g2 = bwd(q, k2, v2, lens, SCALE, dout)
    for a, b2 in zip((dq, dk, dv), g2):
        assert np.array_equal(a, b2)


def check_ragged_and_linearity(bwd):
    """One ragged call equals per-element calls bit for bit; gradients are linear in dout."""
    q, k, v, lens, dout, rng = _case(35, B=3, lens=(9, 2, 6))
    full = bwd(q, k, v, lens, SCALE, dout)
    for b in range(3):
        one = bwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], SCALE, dout[b:b + 1])
        for a, c in zip(full, one):
            assert np.array_equal(a[b:b + 1], c)
    d2 = rng.standard_normal(dout.shape)
    g1 = bwd(q, k, v, lens, SCALE, dout)
    g2 = bwd(q, k, v, lens, SCALE, d2)
    g3 = bwd(q, k, v, lens, SCALE, dout + 2.0 * d2)
    for a, b2, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, a + 2.0 * b2, rtol=0, atol=1e-11)


ALL_CHECKS = [check_finite_differences, check_library_autograd, check_n_one_and_zero, check_sums_and_pads,
              check_ragged_and_linearity]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_bwd_oracle_pin(check):
    check(ref_prefix_bwd)


# ------------------------------------------------------- planted mistakes, on the CPU


def _mutant_grad(kind):
    def grad(q, k, v, dout, s64):
        t, n = q.shape[0], k.shape[0]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        if n == 0 or t == 0:
            return dq, dk, dv
        sc = s64 * (q @ k.T)
        e = np.exp(sc - sc.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dv = (e if kind == "dv_unnormalised" else p).T @ dout
        dp = dout @ v.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        if kind == "no_delta":
            delta = 0.0
        if kind == "delta_from_dp_only":
            delta = dp.sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        if kind == "flipped_ds":
            ds = -ds
        dq = s64 * (ds @ (v if kind == "dq_uses_v" else k))
        dk = (1.0 if kind == "dk_no_scale" else s64) * (ds.T @ (dout if kind == "dk_uses_dout" else q))
        return dq, dk, dv

    return grad


def _mutant_bwd_unsliced(q, k, v, kv_len, scale, dout):
    """Forgets the prefix: attends over every slot."""
    return ref_prefix_bwd(q, k, v, np.full_like(np.asarray(kv_len), k.shape[2]), scale, dout)


@pytest.mark.parametrize("mutant", ["dv_unnormalised", "no_delta", "delta_from_dp_only", "flipped_ds", "dq_uses_v",
                                    "dk_no_scale", "dk_uses_dout", "unsliced_keys"])
def test_bwd_planted_mistakes_are_caught(mutant, monkeypatch):
    if mutant == "unsliced_keys":
        bwd = _mutant_bwd_unsliced
    else:
        monkeypatch.setattr(O, "_grad_one", _mutant_grad(mutant))
        bwd = O.ref_prefix_bwd
    failures = 0
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(bwd)
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1, f"planted mistake {mutant!r} passed every pin"

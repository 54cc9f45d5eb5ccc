"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each check is a plain function taking the oracle's three entry points, so the
same checks run against the real oracle and against deliberately broken copies
(planted on the CPU, in ``test_planted_mistakes_are_caught``): a plausible slip
-- a dropped scale, an off-by-one prefix, a swapped operand, a wrong sign, a
bad merge weight -- must fail at least one pin.

Sources of the facts:
* masking a key prefix equals truncating k/v to it; a ragged mask equals
  per-element truncated forwards; an all-False mask is legal (page "Rewrite
  prefix key-padding masks as k/v truncation to keep SDPA on the flash path
  (PyTorch)", sections Fix and Tests);
* an LSE-weighted merge of partials over unequal key sets equals the single
  pass (page "Add sequence-parallel multi-GPU inference (PyTorch and JAX) and a
  cuDNN flash attention option", section Sequence-parallel inference);
* closed forms (n = 1, uniform scores, hand-derived weight ratios), softmax
  invariants, brute force, and torch's own CPU attention as a library routine.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.attn_oracle as O
from oracle import brute_force, ref_lse_combine, ref_prefix_fwd, ref_splitkv_partial

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class Oracle:
    """The three oracle entry points, swappable for the planted-mistake test."""

    def __init__(self, fwd=ref_prefix_fwd, split=ref_splitkv_partial, combine=ref_lse_combine):
        self.fwd, self.split, self.combine = fwd, split, combine


REAL = Oracle()


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _pads(rng, k, v, lens, value=1e4):
    k = k.copy()
    v = v.copy()
    for b, n in enumerate(lens):
        k[b, :, n:] = value * np.sign(rng.standard_normal(k[b, :, n:].shape))
        v[b, :, n:] = value * np.sign(rng.standard_normal(v[b, :, n:].shape))
    return k, v


# --------------------------------------------------------------------------- checks


def check_brute_force(o: Oracle):
    """P1: pure-Python loops agree with the oracle on every tiny shape and every n."""
    rng = np.random.default_rng(11)
    for s_slots in range(0, 8):
        for d in (1, 2, 4, 8):
            for tq in (1, 3, 5):
                for n in range(0, s_slots + 1):
                    lens = np.array([n, s_slots - n])
                    q = _rand(rng, 2, 2, tq, d)
                    k = _rand(rng, 2, 2, s_slots, d)
                    v = _rand(rng, 2, 2, s_slots, d)
                    k, v = _pads(rng, k, v, lens, 3.0)
                    scale = 1.0 / math.sqrt(d)
                    ob, lb = brute_force(q, k, v, lens, scale)
                    out, lse = o.fwd(q, k, v, lens, scale)
                    np.testing.assert_allclose(out, np.array(ob).reshape(out.shape), rtol=0, atol=1e-12)
                    lb = np.array(lb).reshape(lse.shape)
                    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
                    fin = np.isfinite(lb)
                    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def _masked_reference(q, k, v, lens, scale):
    """Attention over all S slots with an additive -inf mask on j >= n_b (n_b >= 1)."""
    s64 = float(np.float64(np.float32(scale)))
    out = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        valid = np.arange(k.shape[2]) < lens[b]
        for h in range(q.shape[1]):
            sc = s64 * (q[b, h] @ k[b, h].T)
            sc = np.where(valid[None, :], sc, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            z = e.sum(axis=1, keepdims=True)
            out[b, h] = (e @ np.where(valid[:, None], v[b, h], 0.0)) / z
            lse[b, h] = (m + np.log(z))[:, 0]
    return out, lse


def check_masked_equals_truncated(o: Oracle):
    """P2: an explicit -inf mask over all S slots equals the truncated oracle."""
    rng = np.random.default_rng(12)
    for (b_, h_, tq, s_slots, d) in [(1, 2, 7, 33, 16), (3, 1, 5, 64, 8), (2, 2, 9, 40, 32)]:
        lens = rng.integers(1, s_slots + 1, size=b_)
        q = _rand(rng, b_, h_, tq, d)
        k = _rand(rng, b_, h_, s_slots, d)
        v = _rand(rng, b_, h_, s_slots, d)
        k, v = _pads(rng, k, v, lens)
        out, lse = o.fwd(q, k, v, lens, 0.3)
        mo, ml = _masked_reference(q, k, v, lens, 0.3)
        np.testing.assert_allclose(out, mo, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ml, rtol=0, atol=1e-13)


def check_ragged_equals_per_element(o: Oracle):
    """P3: one ragged call equals B separate single-element calls, bit for bit."""
    rng = np.random.default_rng(13)
    b_, h_, tq, s_slots, d = 4, 2, 6, 30, 8
    lens = np.array([0, 1, 17, 30])
    q = _rand(rng, b_, h_, tq, d)
    k = _rand(rng, b_, h_, s_slots, d)
    v = _rand(rng, b_, h_, s_slots, d)
    k, v = _pads(rng, k, v, lens)
    out, lse = o.fwd(q, k, v, lens, 0.25)
    for b in range(b_):
        ob, lb = o.fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], 0.25)
        assert np.array_equal(out[b:b + 1], ob)
        assert np.array_equal(lse[b:b + 1], lb)
        # ... and with the pads cut away entirely (S = n_b)
        n = lens[b]
        oc, lc = o.fwd(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], [n], 0.25)
        np.testing.assert_allclose(out[b:b + 1], oc, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b:b + 1], lc, rtol=0, atol=1e-13)


def check_rows_are_distributions(o: Oracle):
    """P4: with V = identity the output rows are the softmax rows themselves.

    They are non-negative, sum to 1, vanish on padded slots, and each entry
    equals exp(scale * q.k_j - lse), which ties lse to out.
    """
    rng = np.random.default_rng(14)
    s_slots, d, tq = 12, 5, 4
    lens = np.array([9, 1, 12])
    q = _rand(rng, 3, 2, tq, d, scale=2.0)
    k = _rand(rng, 3, 2, s_slots, d)
    k, _ = _pads(rng, k, k, lens)
    v = np.broadcast_to(np.eye(s_slots), (3, 2, s_slots, s_slots)).copy()
    out, lse = o.fwd(q, k, v, lens, 0.7)
    s64 = float(np.float64(np.float32(0.7)))
    for b, n in enumerate(lens):
        p = out[b]
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-13)
        assert np.all(p[..., n:] == 0.0)
        expect = np.exp(s64 * np.einsum("htd,hjd->htj", q[b], k[b, :, :n]) - lse[b][..., None])
        np.testing.assert_allclose(p[..., :n], expect, rtol=1e-12, atol=1e-15)


def _random_partition(rng, n, parts):
    cuts = np.sort(rng.integers(0, n + 1, size=parts - 1))
    return np.concatenate([[0], cuts, [n]])


def check_lse_merge(o: Oracle):
    """P5: merging partials over any contiguous partition equals the single pass.

    Covers unequal parts, empty parts and single-key parts, and the fixed-size
    chunking of ``ref_splitkv_partial`` (chunk = 1, 3, 64), with n_b < S.
    """
    rng = np.random.default_rng(15)
    b_, h_, tq, s_slots, d = 2, 2, 5, 70, 8
    lens = np.array([61, 70])
    q = _rand(rng, b_, h_, tq, d, scale=1.5)
    k = _rand(rng, b_, h_, s_slots, d)
    v = _rand(rng, b_, h_, s_slots, d)
    k, v = _pads(rng, k, v, lens)
    full_o, full_l = o.fwd(q, k, v, lens, 0.4)
    for trial in range(6):
        parts = 2 + trial
        for b in range(b_):
            n = lens[b]
            edges = _random_partition(rng, n, parts)
            po, pl = [], []
            for a, e in zip(edges[:-1], edges[1:]):
                pa, la = o.fwd(q[b:b + 1], k[b:b + 1, :, a:e], v[b:b + 1, :, a:e], [e - a], 0.4)
                po.append(pa)
                pl.append(la)
            mo, ml = o.combine(np.stack(po, 0), np.stack(pl, 0), axis=0)
            np.testing.assert_allclose(mo, full_o[b:b + 1], rtol=0, atol=1e-12)
            np.testing.assert_allclose(ml, full_l[b:b + 1], rtol=0, atol=1e-12)
    for chunk in (1, 3, 64):
        po, pl = o.split(q, k, v, lens, 0.4, chunk)
        c_ = -(-s_slots // chunk)
        assert po.shape == (b_, h_, c_, tq, d) and pl.shape == (b_, h_, c_, tq)
        for b in range(b_):
            for c in range(c_):
                lo, hi = c * chunk, min((c + 1) * chunk, lens[b])
                if hi <= lo:
                    assert np.all(po[b, :, c] == 0) and np.all(np.isneginf(pl[b, :, c]))
                else:
                    ob, lb = brute_force(q[b:b + 1], k[b:b + 1, :, lo:hi], v[b:b + 1, :, lo:hi], [hi - lo], 0.4)
                    np.testing.assert_allclose(po[b, :, c], np.array(ob)[0], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(pl[b, :, c], np.array(lb)[0], rtol=0, atol=1e-12)
        mo, ml = o.combine(po, pl, axis=2)
        np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
    # every part empty -> (0, -inf)
    eo, el = o.combine(np.zeros((3, 1, 2, 4)), np.full((3, 1, 2), -np.inf), axis=0)
    assert np.all(eo == 0) and np.all(np.isneginf(el))


def check_special_cases(o: Oracle):
    """P6: n = 0 gives (0, -inf); n = 1 gives v_0 exactly and lse = scale * q.k_0."""
    rng = np.random.default_rng(16)
    q = _rand(rng, 2, 3, 4, 8)
    k = _rand(rng, 2, 3, 6, 8)
    v = _rand(rng, 2, 3, 6, 8)
    out, lse = o.fwd(q, k, v, [0, 1], 0.125)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.array_equal(out[1], np.broadcast_to(v[1, :, :1], out[1].shape))
    np.testing.assert_allclose(lse[1], 0.125 * np.einsum("htd,hd->ht", q[1], k[1, :, 0]), rtol=0, atol=1e-14)
    # S = 0 slots at all
    out0, lse0 = o.fwd(q, k[:, :, :0], v[:, :, :0], [0, 0], 0.125)
    assert np.all(out0 == 0.0) and np.all(np.isneginf(lse0))


def check_closed_forms(o: Oracle):
    """P7 and hand-derived weights.

    * Equal keys (or q = 0): out = mean(v[:n]), lse = s + ln n.
    * D = 1, q = 1, scale = 1, keys 0, ln 2, ln 4 (one pad): weights 1 : 2 : 4, so
      out = (v0 + 2 v1 + 4 v2) / 7 and lse = ln 7.  With v = 1, 2, 4 -> out = 3.
    * keys 0 and ln 3 with v = 2, 6 -> weights 1 : 3 -> out = 5, lse = ln 4.
    """
    rng = np.random.default_rng(17)
    q = _rand(rng, 1, 2, 3, 6)
    kvec = _rand(rng, 6)
    k = np.broadcast_to(kvec, (1, 2, 10, 6)).copy()
    v = _rand(rng, 1, 2, 10, 6)
    k, v = _pads(rng, k, v, [7])
    out, lse = o.fwd(q, k, v, [7], 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, :, :7].mean(2, keepdims=True), out.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bhtd,d->bht", q, kvec) + math.log(7), rtol=0, atol=1e-13)
    out, lse = o.fwd(np.zeros((1, 1, 2, 6)), _rand(rng, 1, 1, 5, 6), v[:, :1, :5], [5], 0.5)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0, :5].mean(0), (2, 6)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(5), rtol=0, atol=1e-14)

    qa = np.ones((1, 1, 1, 1))
    ka = np.array([0.0, math.log(2.0), math.log(4.0), 9.0]).reshape(1, 1, 4, 1)
    va = np.array([1.0, 2.0, 4.0, -1e4]).reshape(1, 1, 4, 1)
    out, lse = o.fwd(qa, ka, va, [3], 1.0)
    assert abs(out.item() - 3.0) < 1e-13 and abs(lse.item() - math.log(7.0)) < 1e-13
    kb = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    vb = np.array([2.0, 6.0]).reshape(1, 1, 2, 1)
    out, lse = o.fwd(qa, kb, vb, [2], 1.0)
    assert abs(out.item() - 5.0) < 1e-13 and abs(lse.item() - math.log(4.0)) < 1e-13
    # The same split into single-key chunks: L_c = score, O_c = v_c.
    po, pl = o.split(qa, ka, va, [3], 1.0, 1)
    np.testing.assert_allclose(pl[0, 0, :3, 0], [0.0, math.log(2.0), math.log(4.0)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(po[0, 0, :3, 0, 0], [1.0, 2.0, 4.0], rtol=0, atol=0)
    assert np.isneginf(pl[0, 0, 3, 0]) and po[0, 0, 3, 0, 0] == 0.0


def check_invariants(o: Oracle):
    """P8: key permutation, key shift, convex hull, linearity in V."""
    rng = np.random.default_rng(18)
    b_, h_, tq, s_slots, d = 2, 2, 6, 20, 8
    lens = np.array([13, 20])
    q = _rand(rng, b_, h_, tq, d)
    k = _rand(rng, b_, h_, s_slots, d)
    v = _rand(rng, b_, h_, s_slots, d)
    k, v = _pads(rng, k, v, lens)
    out, lse = o.fwd(q, k, v, lens, 0.35)
    s64 = float(np.float64(np.float32(0.35)))
    kp, vp = k.copy(), v.copy()
    for b, n in enumerate(lens):
        perm = rng.permutation(n)
        kp[b, :, :n] = k[b][:, perm]
        vp[b, :, :n] = v[b][:, perm]
    o2, l2 = o.fwd(q, kp, vp, lens, 0.35)
    np.testing.assert_allclose(o2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-13)
    u = _rand(rng, d)
    o3, l3 = o.fwd(q, k + u, v, lens, 0.35)
    np.testing.assert_allclose(o3, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, lse + s64 * np.einsum("bhtd,d->bht", q, u), rtol=0, atol=1e-12)
    for b, n in enumerate(lens):
        lo = v[b, :, :n].min(axis=1)[:, None, :]
        hi = v[b, :, :n].max(axis=1)[:, None, :]
        assert np.all(out[b] >= lo - 1e-14) and np.all(out[b] <= hi + 1e-14)
    w = _rand(rng, b_, h_, s_slots, d)
    o4, _ = o.fwd(q, k, 2.0 * v - 3.0 * w, lens, 0.35)
    o5, _ = o.fwd(q, k, w, lens, 0.35)
    np.testing.assert_allclose(o4, 2.0 * out - 3.0 * o5, rtol=0, atol=1e-12)


def check_library_attention(o: Oracle):
    """P9: torch's CPU float64 attention, truncated and with a [B,1,1,S] bool mask."""
    rng = np.random.default_rng(19)
    b_, h_, tq, s_slots, d = 3, 2, 9, 40, 16
    lens = np.array([1, 23, 40])
    q = _rand(rng, b_, h_, tq, d)
    k = _rand(rng, b_, h_, s_slots, d)
    v = _rand(rng, b_, h_, s_slots, d)
    k, v = _pads(rng, k, v, lens)
    out, lse = o.fwd(q, k, v, lens, 1.0 / math.sqrt(d))
    tq_, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = torch.arange(s_slots)[None, None, None, :] < torch.from_numpy(lens)[:, None, None, None]
    masked = torch.nn.functional.scaled_dot_product_attention(tq_, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(out, masked.numpy(), rtol=0, atol=1e-12)
    for b, n in enumerate(lens):
        ref = torch.nn.functional.scaled_dot_product_attention(tq_[b:b + 1], tk[b:b + 1, :, :n], tv[b:b + 1, :, :n])
        np.testing.assert_allclose(out[b:b + 1], ref.numpy(), rtol=0, atol=1e-12)
        s64 = float(np.float64(np.float32(1.0 / math.sqrt(d))))
        ref_lse = torch.logsumexp(s64 * tq_[b] @ tk[b, :, :n].transpose(-1, -2), dim=-1)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), rtol=0, atol=1e-12)


ALL_CHECKS = [
    check_brute_force,
    check_masked_equals_truncated,
    check_ragged_equals_per_element,
    check_rows_are_distributions,
    check_lse_merge,
    check_special_cases,
    check_closed_forms,
    check_invariants,
    check_library_attention,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(REAL)


# --------------------------------------------------------------- the pages' numbers


def test_fp32_masked_vs_truncated_roundoff():
    """P10: torch fp32 masked vs truncated differ by round-off of the size the pages report."""
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["masked_vs_truncated_fp32"]
    g = torch.Generator().manual_seed(20)
    q = torch.randn(1, 2, 256, 64, generator=g)
    k = torch.randn(1, 2, 256, 64, generator=g)
    v = torch.randn(1, 2, 256, 64, generator=g)
    n = 200
    mask = (torch.arange(256) < n)[None, None, None, :]
    masked = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    trunc = torch.nn.functional.scaled_dot_product_attention(q, k[:, :, :n], v[:, :, :n])
    diff = (masked - trunc).abs().max().item()
    # Same order as the observed figure; both are far inside the fp32 parity bound.
    assert diff < 50 * fig["observed_max_abs_diff"]


def test_unfused_score_bytes_match_pages():
    from long_context_prefix_amd.footprint import mask_copy_bytes, unfused_score_bytes

    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    for row in fig["score_matrix_bytes"]:
        gb = unfused_score_bytes(row["context_rows"], row["context_rows"], row["heads"], row["elem_bytes"]) / 1e9
        assert abs(gb - row["printed_gb"]) / row["printed_gb"] < row["rel_tol"]
    mc = fig["mask_copy_gib"][0]
    for views, tokens, gib in mc["rows"]:
        assert views * mc["tokens_per_view"] == tokens
        got = mask_copy_bytes(tokens, mc["heads"], mc["elem_bytes"]) / 2**30
        assert abs(got - gib) < 0.05


# ------------------------------------------------------- planted mistakes, on the CPU


def _mutant_attend(kind):
    real = O._attend_one

    def attend(q, k, v, s64):
        if kind == "dropped_scale":
            return real(q, k, v, 1.0)
        if kind == "wrong_sign":
            return real(q, k, v, -s64)
        if kind == "k_as_v":
            return real(q, k, k, s64)
        if kind == "no_normalisation":
            out, lse = real(q, k, v, s64)
            return out * math.exp(0.5), lse
        if kind == "lse_log2":
            out, lse = real(q, k, v, s64)
            return out, lse / math.log(2.0)
        if kind == "transposed_q":
            if q.shape[0] == q.shape[1]:
                return real(q.T.copy(), k, v, s64)
            return real(q[::-1].copy(), k, v, s64)
        raise AssertionError(kind)

    return attend


def _mutant_fwd_off_by_one(q, k, v, kv_len, scale):
    lens = np.minimum(np.asarray(kv_len) + 1, k.shape[2])
    return ref_prefix_fwd(q, k, v, lens, scale)


def _mutant_combine_uniform(part_out, part_lse, axis=2):
    po = np.moveaxis(np.asarray(part_out, np.float64), axis, 0)
    pl = np.moveaxis(np.asarray(part_lse, np.float64), axis, 0)
    m = pl.max(0)
    w = np.where(np.isneginf(pl), 0.0, 1.0)
    ws = w.sum(0)
    out = (w[..., None] * po).sum(0) / np.where(ws == 0, 1, ws)[..., None]
    return out, np.where(np.isneginf(m), -np.inf, m + np.log(np.where(ws == 0, 1, ws)))


def _mutant_split_shift(q, k, v, kv_len, scale, chunk):
    po, pl = ref_splitkv_partial(q, k, v, np.maximum(np.asarray(kv_len) - 1, 0), scale, chunk)
    return po, pl


@pytest.mark.parametrize(
    "mutant",
    ["dropped_scale", "wrong_sign", "k_as_v", "no_normalisation", "lse_log2", "transposed_q",
     "off_by_one_prefix", "uniform_merge", "split_drops_last_key"],
)
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    if mutant == "off_by_one_prefix":
        o = Oracle(fwd=_mutant_fwd_off_by_one)
    elif mutant == "uniform_merge":
        o = Oracle(combine=_mutant_combine_uniform)
    elif mutant == "split_drops_last_key":
        o = Oracle(split=_mutant_split_shift)
    else:
        monkeypatch.setattr(O, "_attend_one", _mutant_attend(mutant))
        o = Oracle()
    failures = 0
    for check in ALL_CHECKS:
        try:
            check(o)
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1, f"planted mistake {mutant!r} passed every pin"


# ------------------------------------------------------------- mask -> lengths


def test_mask_to_kv_len_hand_cases():
    from oracle import ref_prefix_mask_to_kv_len as f

    T, F = True, False
    cases = [
        ([T, T, T, T], 4),  # all valid
        ([F, F, F, F], 0),  # all-False mask: a legal prefix of length 0 (PR #80, Tests)
        ([T, T, F, F], 2),
        ([T, F, F, F], 1),
        ([T, F, T, F], -1),  # a hole: not a prefix mask
        ([F, T, T, T], -1),  # suffix mask
        ([T, T, T, F, T], -1),
    ]
    for row, n in cases:
        assert f(np.array([row]))[0] == n, (row, n)
    # [B,1,1,S] layout, ragged lengths, and S = 0
    m = np.zeros((3, 1, 1, 6), dtype=bool)
    m[0, ..., :6] = True
    m[1, ..., :1] = True
    assert f(m).tolist() == [6, 1, 0]
    assert f(np.zeros((2, 0), dtype=bool)).tolist() == [0, 0]


def test_mask_lengths_feed_the_truncation_identity():
    """For prefix masks, masked attention (torch, float64) equals the oracle at the derived lengths."""
    from oracle import ref_prefix_mask_to_kv_len

    rng = np.random.default_rng(21)
    B, H, tq, S, d = 4, 2, 5, 30, 8
    lens = np.array([30, 1, 17, 9])
    mask = np.arange(S)[None, :] < lens[:, None]
    got = ref_prefix_mask_to_kv_len(mask[:, None, None, :])
    assert got.tolist() == lens.tolist()
    q, k, v = (rng.standard_normal((B, H, n, d)) for n in (tq, S, S))
    out, _ = ref_prefix_fwd(q, k, v, got, 0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask[:, None, None, :]), scale=float(np.float32(0.3)))
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)

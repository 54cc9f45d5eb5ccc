"""Full-size workloads on the GPU, in the launch configurations the benchmark times.

The oracle cannot afford every output at these sizes, so it checks seeded
samples of query rows (always including the first and the last row) and, for
the split-KV workload, whole sequences (the first, the last and seeded ones).
"""

import numpy as np
import pytest
import torch

from long_context_prefix_amd import _lib
from long_context_prefix_amd.workloads import WORKLOADS, make_workload, sample_rows
from oracle import ref_prefix_bwd, ref_prefix_fwd, ref_splitkv_partial
from tests.parity import assert_grad_parity, assert_parity, gather_rows, log, to64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,rows", [("icl_16k", 256), ("ragged_32k", 128), ("icl_121k", 128)])
def test_fused_workload_sampled_rows(name, rows):
    w = WORKLOADS[name]
    lens = w.lens()
    log(f"workload {name}: B={w.B} H={w.H} D={w.D} Tq={w.Tq} S={w.S} kv_len={lens.tolist()}")
    q, k, v, kv = make_workload(w, device=DEV)
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    torch.cuda.synchronize()
    sel = sample_rows(w.seed, w.Tq, rows, w.B * w.H)
    q_s = to64(gather_rows(q, sel))
    nmax = int(lens.max())
    ro, rl = ref_prefix_fwd(q_s, to64(k[:, :, :nmax]), to64(v[:, :, :nmax]), lens, w.scale)
    assert_parity(gather_rows(out, sel), gather_rows(lse, sel), ro, rl, "bf16", name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,rows", [("icl_16k", 128), ("icl_121k", 32)])
def test_fused_workload_sharp_sampled_rows(name, rows):
    """The ICL workloads at full size with q scaled by 4 (exact in bf16): scores spread 4x
    wider, so attention concentrates on a few hundred to a few thousand keys and the outputs
    grow from ~2e-3 rms (where the 2e-2 max-abs bound says nothing) to 1-4e-2; the scores also
    spread further from each row's first-tile reference max.  Same launch as the benchmark."""
    w = WORKLOADS[name]
    lens = w.lens()
    log(f"workload {name} (q x 4): B={w.B} H={w.H} D={w.D} Tq={w.Tq} S={w.S} kv_len={lens.tolist()}")
    q, k, v, kv = make_workload(w, device=DEV)
    q.mul_(4.0)
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    torch.cuda.synchronize()
    sel = sample_rows(w.seed + 3, w.Tq, rows, w.B * w.H)
    nmax = int(lens.max())
    ro, rl = ref_prefix_fwd(to64(gather_rows(q, sel)), to64(k[:, :, :nmax]), to64(v[:, :, :nmax]), lens, w.scale)
    rms = float(np.sqrt(np.mean(ro * ro)))
    log(f"{name} sharp: reference output rms {rms:.3e}")
    assert rms > 1e-2  # peaked attention: five times the plain draw's output
    assert_parity(gather_rows(out, sel), gather_rows(lse, sel), ro, rl, "bf16", f"{name} sharp")


@pytest.mark.timeout(900)
def test_inducing_splitkv_workload():
    w = WORKLOADS["inducing_splitkv"]
    lens = w.lens()
    log(f"workload {w.name}: B={w.B} H={w.H} D={w.D} Tq={w.Tq} S={w.S} n={lens[0]} chunk={w.chunk}")
    q, k, v, kv = make_workload(w, device=DEV)
    po, pl = _lib.attn_splitkv_partial(q, k, v, kv, w.chunk, w.scale)
    out, lse = _lib.attn_lse_combine(po, pl, torch.bfloat16)
    fo, fl = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    torch.cuda.synchronize()
    assert po.shape[2] == 25
    rng = np.random.default_rng(w.seed)
    seqs = sorted(set([0, w.B - 1] + rng.choice(np.arange(1, w.B - 1), size=16, replace=False).tolist()))
    assert len(seqs) == 18  # 16 seeded sequences plus the first and the last
    for b in seqs:
        n = int(lens[b])
        qb, kb, vb = to64(q[b:b + 1]), to64(k[b:b + 1, :, :n]), to64(v[b:b + 1, :, :n])
        ro, rl = ref_prefix_fwd(qb, kb, vb, [n], w.scale)
        assert_parity(out[b:b + 1], lse[b:b + 1], ro, rl, "bf16", f"split-KV seq {b}")
        assert_parity(fo[b:b + 1], fl[b:b + 1], ro, rl, "bf16", f"fused seq {b}")
        if b == w.B - 1:
            # the last valid chunk holds 1,696 keys; compare it on its own
            rpo, rpl = ref_splitkv_partial(qb, to64(k[b:b + 1]), to64(v[b:b + 1]), [n], w.scale, w.chunk)
            assert_parity(po[b:b + 1, :, 24], pl[b:b + 1, :, 24], rpo[:, :, 24], rpl[:, :, 24], "bf16",
                          f"partial chunk 24 seq {b}")


@pytest.mark.timeout(900)
def test_backward_ragged_32k():
    """The backward at its full size: dq on seeded query rows of every (b, h); dk and dv
    over every key of one head of the n = 6153 element (all 32768 queries feed them);
    zero gradients on every padded slot."""
    w = WORKLOADS["ragged_32k"]
    lens = w.lens()
    log(f"backward workload {w.name}: kv_len={lens.tolist()}")
    q, k, v, kv = make_workload(w, device=DEV)
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    g = torch.Generator(device="cpu").manual_seed(w.seed + 77)
    dout = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    dq, dk, dv = _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, w.scale)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        assert torch.all(dk[b, :, n:] == 0) and torch.all(dv[b, :, n:] == 0), f"padded gradient, element {b}"
    sel = sample_rows(w.seed + 1, w.Tq, 32, w.B * w.H)
    nmax = int(lens.max())
    rq, _, _ = ref_prefix_bwd(to64(gather_rows(q, sel)), to64(k[:, :, :nmax]), to64(v[:, :, :nmax]), lens, w.scale,
                              to64(gather_rows(dout, sel)))
    assert_grad_parity("dq (sampled rows)", gather_rows(dq, sel), rq, w.name)
    b, h = 1, 0
    n = int(lens[b])
    sl = (slice(b, b + 1), slice(h, h + 1))
    _, rk, rv = ref_prefix_bwd(to64(q[sl]), to64(k[sl][:, :, :n]), to64(v[sl][:, :, :n]), [n], w.scale,
                               to64(dout[sl]))
    assert_grad_parity("dk (one head)", dk[sl][:, :, :n], rk, w.name)
    assert_grad_parity("dv (one head)", dv[sl][:, :, :n], rv, w.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["icl_121k", "ragged_32k"])
def test_full_size_determinism_and_padding_invariance(name):
    """At full size: two runs give the same bits, and NaN in every padded key slot changes no bit."""
    w = WORKLOADS[name]
    lens = w.lens()
    log(f"workload {name}: determinism and NaN-pad invariance, kv_len={lens.tolist()}")
    q, k, v, kv = make_workload(w, device=DEV)
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    out2, lse2 = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "two runs differ"
    del out2, lse2
    for b, n in enumerate(lens):
        k[b, :, int(n):] = float("nan")
        v[b, :, int(n):] = float("nan")
    out3, lse3 = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out3) and torch.equal(lse, lse3), "padded slots changed the result"


@pytest.mark.timeout(900)
def test_ragged_32k_wave_forms_same_bits(monkeypatch):
    """At the ragged 32k shape the host takes the eight-wave form of the 32-row kernel; the
    four-wave form, forced, must give the same output and LSE bits (the same per-row
    arithmetic), and the default launch must be one of the two."""
    w = WORKLOADS["ragged_32k"]
    log(f"workload ragged_32k: four- against eight-wave form, kv_len={w.lens().tolist()}")
    q, k, v, kv = make_workload(w, device=DEV)
    res = {}
    for form in ("128", "128x8", None):
        if form is None:
            monkeypatch.delenv("ATTN_PREFIX_FWD_ROWS", raising=False)
        else:
            monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", form)
        res[form] = _lib.attn_prefix_fwd(q, k, v, kv, w.scale)
    torch.cuda.synchronize()
    for form in ("128x8", None):
        assert torch.equal(res["128"][0], res[form][0]) and torch.equal(res["128"][1], res[form][1]), form

"""GPU parity of the HIP kernels against the fp64 oracle, through the C ABI.

Small cases span several 128-row query tiles and 64-key tiles with ragged
tails; the edge matrix covers n in {0, 1, 63, 64, 65, S}, T_q in {1, 17, 128,
129} and D in {64, 128, 256}.  Bitwise properties (padding invariance,
determinism, n = 1) and guard-byte checks follow.  Full-size workloads are in
``test_gpu_workloads.py``.
"""

import math

import numpy as np
import pytest
import torch

from long_context_prefix_amd import _lib
from long_context_prefix_amd.workloads import WORKLOADS, make_inputs, make_workload
from oracle import ref_lse_combine, ref_prefix_fwd, ref_splitkv_partial
from tests.parity import assert_parity, log, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np(t):
    return to64(t)


def _run_fused(q, k, v, kv, scale):
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, scale)
    torch.cuda.synchronize()
    return out, lse


def _oracle(q, k, v, kv, scale):
    return ref_prefix_fwd(_np(q), _np(k), _np(v), kv.cpu().numpy(), scale)


@pytest.fixture(params=[128, "128x8", 256, "mixed"])
def fwd_rows(request, monkeypatch):
    """Force the bf16 forward path: 32 query rows per wave (128 per workgroup of four waves, or
    256 per workgroup of eight at D <= 128), 64 (256 per workgroup), or, at D = 256, both in
    one grid (every full 256-row tile on the 64-row path, the remaining rows on the 32-row
    one).  D = 64 has no 64-row kernel, D = 128 no mixed grid, D = 256 no eight-wave form:
    those cases are skipped, as is mixed where no 256-row tile is full or none is left over."""
    monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", str(request.param))
    return request.param


def _skip_dup(D, rows, Tq=None):
    if rows == "128x8" and D == 256:
        pytest.skip("no eight-wave form at this head dim")
    if D == 64 and rows not in (128, "128x8"):
        pytest.skip("no 64-row kernel at this head dim")
    if D == 128 and rows == "mixed":
        pytest.skip("no mixed grid at this head dim")
    if rows == "mixed" and (Tq is None or Tq < 256 or Tq % 256 == 0):
        pytest.skip("mixed is one of the two kernels at this T_q")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Tq", [1, 17, 128, 129])
def test_edge_matrix_bf16(D, Tq, fwd_rows):
    _skip_dup(D, fwd_rows, Tq)
    S = 200
    lens = [0, 1, 63, 64, 65, S]
    log(f"edge bf16 D={D} Tq={Tq} S={S} lens={lens} rows={fwd_rows}")
    q, k, v, kv = make_inputs(len(lens), 2, Tq, S, D, lens, "bf16", 1.0, seed=100 + D + Tq, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"edge D={D} Tq={Tq}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_multi_tile_bf16_sharp(D, fwd_rows):
    """Several query and key tiles, ragged tails, peaky attention (q scaled x4)."""
    _skip_dup(D, fwd_rows, 300)
    B, H, Tq, S = 2, 3, 300, 777
    lens = [700, 777]
    log(f"sharp bf16 D={D}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=200 + D, device=DEV)
    q.mul_(4.0)
    scale = 1.0 / math.sqrt(D)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"sharp D={D}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_fp32_inputs(D):
    B, H, Tq, S = 2, 2, 150, 300
    lens = [0 if D == 64 else 1, 257]
    log(f"fp32 D={D}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "f32", 1.0, seed=300 + D, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "f32", f"fp32 D={D}")


def test_tiny_prefix_mask_workload():
    w = WORKLOADS["tiny_prefix_mask"]
    log("tiny_prefix_mask workload")
    q, k, v, kv = make_workload(w, device=DEV)
    out, lse = _run_fused(q, k, v, kv, w.scale)
    ro, rl = _oracle(q, k, v, kv, w.scale)
    assert_parity(out, lse, ro, rl, "f32", "tiny_prefix_mask")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [64, 128, 192])
@pytest.mark.parametrize("Tq", [130, 100])  # 100: one query tile per head (the streaming launch)
def test_splitkv_partial_and_combine(dtype, chunk, Tq):
    D = 128
    B, H, S = 3, 2, 450
    lens = [0, 129, 450]
    log(f"splitkv dtype={dtype} chunk={chunk} Tq={Tq}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, dtype, 1.0, seed=400 + chunk, device=DEV)
    scale = 1.0 / math.sqrt(D)
    po, pl = _lib.attn_splitkv_partial(q, k, v, kv, chunk, scale)
    torch.cuda.synchronize()
    rpo, rpl = ref_splitkv_partial(_np(q), _np(k), _np(v), np.array(lens), scale, chunk)
    assert po.shape == rpo.shape
    assert_parity(po, pl, rpo, rpl, dtype, f"partials {dtype} chunk={chunk}")
    # the merge kernel alone, on the GPU's own partials, fp32 output
    mo, ml = _lib.attn_lse_combine(po, pl, torch.float32)
    torch.cuda.synchronize()
    eo, el = ref_lse_combine(_np(po), _np(pl), axis=2)
    o, lg = _np(mo), _np(ml)
    assert np.array_equal(np.isneginf(lg), np.isneginf(el))
    fin = ~np.isneginf(el)
    assert np.abs(o - eo).max() <= 1e-5
    assert np.abs(lg[fin] - el[fin]).max() <= 1e-5
    # end to end against the single-pass oracle
    out, lse = _lib.splitkv_fwd(q, k, v, kv, chunk, scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, dtype, f"split end-to-end {dtype} chunk={chunk}")
    if dtype == "f32":
        # fp32 inputs: exact products on both paths, so split and fused agree to fp32 round-off
        fo, fl = _run_fused(q, k, v, kv, scale)
        assert np.abs(_np(fo) - _np(out)).max() <= 2e-6
        a, b = _np(fl), _np(lse)
        assert np.array_equal(np.isneginf(a), np.isneginf(b))
        m = np.isfinite(a)
        assert np.abs(a[m] - b[m]).max() <= 2e-6


def test_combine_edge_cases():
    D = 64
    # every partial -inf -> (0, -inf); C = 0 -> (0, -inf)
    po = torch.randn(1, 2, 3, 5, D, device=DEV)
    pl = torch.full((1, 2, 3, 5), -math.inf, device=DEV)
    pl[0, 1, 1, 2] = 0.5
    out, lse = _lib.attn_lse_combine(po, pl, torch.float32)
    torch.cuda.synchronize()
    o, l = _np(out), _np(lse)
    assert np.all(o[0, 0] == 0) and np.all(np.isneginf(l[0, 0]))
    np.testing.assert_allclose(o[0, 1, 2], _np(po)[0, 1, 1, 2], rtol=0, atol=1e-6)
    assert abs(l[0, 1, 2] - 0.5) < 1e-6
    empty_o = torch.empty(1, 2, 0, 5, D, device=DEV)
    empty_l = torch.empty(1, 2, 0, 5, device=DEV)
    out, lse = _lib.attn_lse_combine(empty_o, empty_l, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("D", [128, 256])
def test_padding_invariance_bitwise(D, fwd_rows):
    """Pads never read: no pads, +-1e4 pads and NaN pads give identical bits."""
    _skip_dup(D, fwd_rows, 70)
    B, H, Tq, n = 2, 2, 70, 333
    log(f"padding invariance D={D}")
    q, k, v, kv = make_inputs(B, H, Tq, n, D, [n, 129], "bf16", 1.0, seed=500 + D, device=DEV)
    base_o, base_l = _run_fused(q, k, v, kv, 0.1)
    for pad, S in ((1e4, n + 77), (float("nan"), n + 200)):
        kp = torch.empty(B, H, S, D, dtype=k.dtype, device=DEV).fill_(pad)
        vp = torch.empty_like(kp).fill_(pad)
        kp[:, :, :n] = k
        vp[:, :, :n] = v
        # element 1 has n = 129, so k[:, :, 129:n] are pads already in the base call
        o, l = _run_fused(q, kp, vp, kv, 0.1)
        assert torch.equal(o, base_o), f"pad={pad}"
        assert torch.equal(l, base_l), f"pad={pad}"
        po1, pl1 = _lib.attn_splitkv_partial(q, k, v, kv, 128, 0.1)
        po2, pl2 = _lib.attn_splitkv_partial(q, kp, vp, kv, 128, 0.1)
        torch.cuda.synchronize()
        C1 = po1.shape[2]
        assert torch.equal(po1, po2[:, :, :C1]) and torch.equal(pl1, pl2[:, :, :C1])
        assert torch.all(po2[:, :, C1:] == 0) and torch.all(torch.isneginf(pl2[:, :, C1:]))


def test_determinism_bitwise(fwd_rows):
    _skip_dup(256, fwd_rows, 300)
    q, k, v, kv = make_inputs(2, 4, 300, 1000, 256, [1000, 517], "bf16", 0.7, seed=600, device=DEV)
    o1, l1 = _run_fused(q, k, v, kv, 0.0625)
    o2, l2 = _run_fused(q, k, v, kv, 0.0625)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_n_equals_one_is_exact(dtype):
    D = 128
    q, k, v, kv = make_inputs(2, 2, 40, 90, D, [1, 1], dtype, 1.0, seed=700, device=DEV)
    out, lse = _run_fused(q, k, v, kv, 0.2)
    assert torch.equal(out, v[:, :, :1].expand_as(out))
    expect = 0.2 * torch.einsum("bhtd,bhd->bht", q.double().cpu(), k[:, :, 0].double().cpu())
    assert (lse.double().cpu() - expect).abs().max().item() <= 1e-4


def test_n_zero_and_empty_slots():
    q, k, v, kv = make_inputs(2, 2, 40, 64, 64, [0, 0], "bf16", 1.0, seed=800, device=DEV, pad=float("nan"))
    out, lse = _run_fused(q, k, v, kv, 0.125)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    k0 = torch.empty(2, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    out, lse = _run_fused(q, k0, k0, kv, 0.125)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_kv_len_out_of_range_is_clamped():
    q, k, v, kv = make_inputs(2, 1, 20, 100, 64, [100, 5], "bf16", 1.0, seed=900, device=DEV)
    bad = torch.tensor([1000, -7], dtype=torch.int32, device=DEV)
    out, lse = _run_fused(q, k, v, bad, 0.125)
    ro, rl = _oracle(q, k, v, torch.tensor([100, 0], dtype=torch.int32), 0.125)
    assert_parity(out, lse, ro, rl, "bf16", "clamped kv_len")


@pytest.mark.parametrize("Tq,D", [(130, 128), (17, 128), (45, 64), (100, 256)])
def test_guard_bytes_untouched(Tq, D):
    """Nothing is written past any output, also when a wave's 32 rows run past T_q
    (one query tile per head: partial rows are then written whole rows at a time)."""
    B, H, S = 2, 2, 300
    log(f"guard bytes Tq={Tq} D={D}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, [300, 65], "bf16", 1.0, seed=1000, device=DEV)
    G = 4096
    n_out, n_lse = B * H * Tq * D, B * H * Tq
    out_buf = torch.full((n_out + G,), 7.0, dtype=torch.bfloat16, device=DEV)
    lse_buf = torch.full((n_lse + G,), 7.0, dtype=torch.float32, device=DEV)
    _lib.attn_prefix_fwd(q, k, v, kv, 0.1, out=out_buf[:n_out].view(B, H, Tq, D), lse=lse_buf[:n_lse].view(B, H, Tq))
    C = -(-S // 64)
    n_po, n_pl = B * H * C * Tq * D, B * H * C * Tq
    po_buf = torch.full((n_po + G,), 7.0, dtype=torch.float32, device=DEV)
    pl_buf = torch.full((n_pl + G,), 7.0, dtype=torch.float32, device=DEV)
    _lib.attn_splitkv_partial(q, k, v, kv, 64, 0.1, part_out=po_buf[:n_po].view(B, H, C, Tq, D),
                              part_lse=pl_buf[:n_pl].view(B, H, C, Tq))
    torch.cuda.synchronize()
    for buf, n in ((out_buf, n_out), (lse_buf, n_lse), (po_buf, n_po), (pl_buf, n_pl)):
        assert torch.all(buf[n:] == 7.0)
        assert not torch.any(torch.isnan(buf[:n]))


def test_no_device_allocation():
    """The library allocates nothing: free device memory is unchanged by a call."""
    q, k, v, kv = make_inputs(1, 8, 1024, 4096, 256, [4000], "bf16", 1.0, seed=1100, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(1, 8, 1024, dtype=torch.float32, device=DEV)
    po = torch.empty(1, 8, 2, 1024, 256, dtype=torch.float32, device=DEV)
    pl = torch.empty(1, 8, 2, 1024, dtype=torch.float32, device=DEV)
    for _ in range(2):  # the first launches load the code objects; measure after them
        _lib.attn_prefix_fwd(q, k, v, kv, 0.1, out=out, lse=lse)
        _lib.attn_splitkv_partial(q, k, v, kv, 2048, 0.1, part_out=po, part_lse=pl)
        _lib.attn_lse_combine(po, pl, torch.bfloat16, out=out, lse=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    _lib.attn_prefix_fwd(q, k, v, kv, 0.1, out=out, lse=lse)
    _lib.attn_splitkv_partial(q, k, v, kv, 2048, 0.1, part_out=po, part_lse=pl)
    _lib.attn_lse_combine(po, pl, torch.bfloat16, out=out, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("Tq", [140, 100])  # 100: one query tile per head (the streaming launch)
def test_splitkv_other_head_dims(D, Tq):
    B, H, S = 2, 2, 700
    lens = [650, 0]
    log(f"splitkv D={D} Tq={Tq}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=1200 + D, device=DEV)
    scale = 1.0 / math.sqrt(D)
    po, pl = _lib.attn_splitkv_partial(q, k, v, kv, 256, scale)
    torch.cuda.synchronize()
    rpo, rpl = ref_splitkv_partial(_np(q), _np(k), _np(v), np.array(lens), scale, 256)
    assert_parity(po, pl, rpo, rpl, "bf16", f"partials D={D}")
    out, lse = _lib.splitkv_fwd(q, k, v, kv, 256, scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"split end-to-end D={D}")


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.9])
def test_scale_sign_and_zero(scale, fwd_rows):
    """Negative scales (Q is negated internally), scale 0 (uniform weights) and a large scale."""
    _skip_dup(256, fwd_rows, 130)
    D, B, H, Tq, S = 256, 2, 2, 130, 300
    lens = [300, 77]
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=1300, device=DEV)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"scale={scale}")
    po, pl = _lib.attn_splitkv_partial(q, k, v, kv, 64, scale)
    so, sl = _lib.attn_lse_combine(po, pl, torch.float32)
    torch.cuda.synchronize()
    assert_parity(so, sl, ro, rl, "bf16", f"split scale={scale}")


@pytest.mark.parametrize("D", [128, 256])
def test_growing_scores_exercise_rescale(D):
    """Key norms grow along the sequence, so every row's scores climb far past the max of its
    first key tile, the reference its probabilities are first taken against."""
    B, H, Tq, S = 1, 2, 64, 2048
    g = torch.Generator(device=DEV).manual_seed(1400 + D)
    q = torch.randn(B, H, Tq, D, device=DEV, generator=g).abs().to(torch.bfloat16)
    ramp = torch.linspace(0.0, 6.0, S, device=DEV).view(1, 1, S, 1)
    k = (torch.rand(B, H, S, D, device=DEV, generator=g) * ramp).to(torch.bfloat16)
    v = torch.randn(B, H, S, D, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.tensor([S], dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert np.isfinite(rl).all() and rl.max() > 20.0  # scores grow far past the first tile's
    assert_parity(out, lse, ro, rl, "bf16", f"growing D={D}")


@pytest.mark.parametrize("D", [128, 256])
def test_score_jump_past_exp_overflow(D, fwd_rows):
    """One late key block scores more than 128 log2 units above everything before it, so a
    probability taken against an earlier reference overflows fp32 (2^128): either kernel
    must redo its pass against a reference at or above the jump."""
    _skip_dup(D, fwd_rows, 300)
    B, H, Tq, S = 1, 2, 300, 1500
    q, k, v, kv = make_inputs(B, H, Tq, S, D, [S], "bf16", 1.0, seed=1900 + D, device=DEV)
    scale = 1.0 / math.sqrt(D)
    # keys 1200..1263 become a large multiple of the mean query direction
    qm = q.float().mean(dim=2, keepdim=True)
    k[:, :, 1200:1264] = (qm / qm.norm(dim=-1, keepdim=True) * 40.0 * math.sqrt(D)).to(torch.bfloat16)
    s = torch.einsum("bhtd,bhsd->bhts", q.double().cpu(), k.double().cpu()) * scale / math.log(2.0)
    jump = (s[..., 1200:1264].amax(-1) - s[..., :64].amax(-1)).max().item()
    assert jump > 128.0, jump
    log(f"score jump D={D} rows={fwd_rows}: {jump:.0f} log2 units")
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert_parity(out, lse, ro, rl, "bf16", f"score jump D={D}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Tq", [100, 300])
def test_splitkv_score_jump_redoes_the_chunk(D, Tq):
    """A key block 128+ log2 units above everything before it sits inside a later chunk, past
    that chunk's first tile: the partial kernel must redo that chunk's pass (a probability taken
    against the chunk's first-tile max would overflow fp32), in the partial launch, its
    streaming form (T_q <= 128) and the single launch, and the merge must still give the
    oracle's result."""
    B, H, S, chunk = 2, 2, 2000, 512
    lens = [2000, 1500]
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=1950 + D + Tq, device=DEV)
    scale = 1.0 / math.sqrt(D)
    qm = q.float().mean(dim=2, keepdim=True)
    k[:, :, 1300:1364] = (qm / qm.norm(dim=-1, keepdim=True) * 40.0 * math.sqrt(D)).to(torch.bfloat16)
    s = torch.einsum("bhtd,bhsd->bhts", q.double().cpu(), k.double().cpu()) * scale / math.log(2.0)
    # the largest climb of any row of each (b, h), the smallest of those over (b, h)
    jump = (s[..., 1300:1364].amax(-1) - s[..., 1024:1088].amax(-1)).amax(-1).min().item()
    log(f"split score jump D={D} Tq={Tq}: {jump:.0f} log2 units over the chunk's first tile")
    assert jump > 128.0, jump
    ro, rl = ref_prefix_fwd(_np(q), _np(k), _np(v), np.array(lens), scale)
    po, pl = _lib.attn_splitkv_partial(q, k, v, kv, chunk, scale)
    out, lse = _lib.attn_lse_combine(po, pl, q.dtype)
    torch.cuda.synchronize()
    assert torch.isfinite(po).all() and torch.isfinite(out.float()).all()
    assert_parity(out, lse, ro, rl, "bf16", f"split score jump D={D} Tq={Tq}")
    _, rpl = ref_splitkv_partial(_np(q), _np(k), _np(v), np.array(lens), scale, chunk)
    gpl = pl.cpu().double().numpy()
    fin = np.isfinite(rpl)
    assert np.array_equal(np.isfinite(gpl), fin)  # the empty chunk is -inf on both
    assert np.abs(gpl[fin] - rpl[fin]).max() < 1e-3  # chunk 2 of both elements took the redo
    o1, l1 = _lib.attn_splitkv_fwd(q, k, v, kv, chunk, scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, out) and torch.equal(l1, lse), "single launch differs from partial + combine"


@pytest.mark.timeout(900)
def test_largest_key_slice(fwd_rows):
    """One (b, h) key slice just under the 2^31-byte limit (D=256 bf16, S = 2^22 - 64):
    offsets near the top of the range stay correct (both D = 256 kernels; with the 64-row
    one, the dominant last key of the second case also sends the workgroup through its
    second pass)."""
    _skip_dup(256, fwd_rows, 64)
    D, S = 256, (1 << 22) - 64
    n = S - 5
    Tq = 64
    g = torch.Generator(device=DEV).manual_seed(1500)
    k = torch.empty(1, 1, S, D, dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    k.normal_(generator=g)
    v.normal_(generator=g)
    q = torch.randn(1, 1, Tq, D, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.tensor([n], dtype=torch.int32, device=DEV)
    out, lse = _run_fused(q, k, v, kv, 0.0625)
    # the oracle over all n keys, on 16 query rows
    rows = torch.arange(0, Tq, 4, device=DEV)
    ro, rl = ref_prefix_fwd(_np(q[:, :, rows]), _np(k[:, :, :n]), _np(v[:, :, :n]), [n], 0.0625)
    assert_parity(out[:, :, rows], lse[:, :, rows], ro, rl, "bf16", "largest slice")
    # the tail keys matter: a query aligned with the last valid key sees it dominate
    q2 = (k[:, :, n - 1:n] * 8).contiguous()
    o2, l2 = _run_fused(q2, k, v, kv, 0.0625)
    r2o, r2l = ref_prefix_fwd(_np(q2), _np(k[:, :, :n]), _np(v[:, :, :n]), [n], 0.0625)
    assert_parity(o2, l2, r2o, r2l, "bf16", "largest slice, last key")


@pytest.mark.parametrize("D,Tq,chunk,dtype", [(64, 1, 64, "bf16"), (128, 129, 128, "bf16"), (256, 300, 192, "bf16"),
                                              (128, 200, 64, "f32"), (128, 150, 4096, "bf16"), (128, 100, 64, "bf16"),
                                              (256, 64, 128, "bf16")])
def test_splitkv_single_launch(D, Tq, chunk, dtype):
    """One launch (partials, then the last chunk per query tile merges) gives the same bits as
    partial + combine, and the oracle's result; partial buffers start as NaN so a merge that
    read a partial before it was written would show; the counters come back zero.  The calls
    alternate between two query sets, so a merge that read the previous call's partials would
    show too.  T_q <= 128 takes the streaming launch, whose hand-off is at device scope."""
    B, H, S = 3, 2, 700
    lens = [700, 0, 333]
    log(f"single-launch split D={D} Tq={Tq} chunk={chunk} {dtype}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, dtype, 1.0, seed=4000 + D + Tq, device=DEV)
    scale = 1.0 / math.sqrt(D)
    C = -(-S // chunk)
    po = torch.full((B, H, C, Tq, D), float("nan"), device=DEV)
    pl = torch.full((B, H, C, Tq), float("nan"), device=DEV)
    counters = torch.zeros((B, H, -(-Tq // 128)), dtype=torch.int32, device=DEV)
    q_alt = (q.float() * -0.75).to(q.dtype)
    for rep in range(4):  # later calls reuse the counters the earlier ones reset
        qq = q if rep % 2 == 0 else q_alt
        if rep < 2:
            po.fill_(float("nan"))
            pl.fill_(float("nan"))
        out, lse = _lib.attn_splitkv_fwd(qq, k, v, kv, chunk, scale, part_out=po, part_lse=pl, counters=counters)
        torch.cuda.synchronize()
        assert int(counters.abs().sum()) == 0, "counters not reset"
        rpo, rpl = _lib.attn_splitkv_partial(qq, k, v, kv, chunk, scale)
        rout, rlse = _lib.attn_lse_combine(rpo, rpl, q.dtype)
        torch.cuda.synchronize()
        assert torch.equal(out, rout) and torch.equal(lse, rlse), f"call {rep}: differs from partial + combine"
    ro, rl = ref_prefix_fwd(to64(qq), to64(k), to64(v), np.array(lens), scale)  # the last call's queries
    assert_parity(out, lse, ro, rl, dtype, f"single-launch split D={D}")


# ---- the 64-rows-per-wave kernel, forced (the library takes it for large D = 256 launches)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("Tq", [129, 256, 257, 511])
def test_wide_edge_matrix(Tq, D, monkeypatch):
    """256-row query tiles with ragged tails, 32-key tiles (at D = 128 two per 64-key DMA
    tile): n on both sides of every tile boundary up to 129, and S."""
    monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", "256")
    S = 200
    lens = [0, 1, 31, 32, 33, 63, 64, 65, 96, 127, 129, S]
    log(f"wide edge D={D} Tq={Tq} lens={lens}")
    q, k, v, kv = make_inputs(len(lens), 2, Tq, S, D, lens, "bf16", 1.0, seed=1500 + Tq + D, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"wide edge D={D} Tq={Tq}")


def _first_tile_margins_log2(q, k, n, scale):
    """Per row, the amount by which its max scaled score climbs above its max over the first
    64 keys, in log2 units (the first tile of the 32-row kernel; the 64-row kernel's is the
    first 32, from which the climb is at least as large).  Both kernels redo a pass past a
    slack of 20.  Past 128, a probability taken against the first tile's max overflows fp32
    (2^128), so a kernel that skipped the second pass would return inf or NaN for that row."""
    s = torch.einsum("bhtd,bhsd->bhts", q.double().cpu(), k[:, :, :n].double().cpu()) * scale / math.log(2.0)
    return s.amax(-1) - s[..., :64].amax(-1)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_growing_scores_take_second_pass(D, fwd_rows):
    """Key norms grow along the sequence, so every row climbs more than 128 log2 units past its
    first tile's max (one pass against that reference would overflow fp32): the workgroups
    must redo their pass against a reference no score of the row exceeds."""
    _skip_dup(D, fwd_rows, 300)
    B, H, Tq, S = 1, 2, 300, 2048
    g = torch.Generator(device=DEV).manual_seed(1600)
    q = torch.randn(B, H, Tq, D, device=DEV, generator=g).abs().to(torch.bfloat16)
    ramp = torch.linspace(0.0, 30.0 * math.sqrt(256 / D), S, device=DEV).view(1, 1, S, 1)
    k = (torch.rand(B, H, S, D, device=DEV, generator=g) * ramp).to(torch.bfloat16)
    v = torch.randn(B, H, S, D, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.tensor([S], dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(D)
    margins = _first_tile_margins_log2(q, k, S, scale)
    log(f"growing D={D} rows={fwd_rows}: first-tile margins {margins.min().item():.0f}..{margins.max().item():.0f} log2 units")
    assert margins.min().item() > 128.0  # every row needs the second pass
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"growing D={D} rows={fwd_rows}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_one_row_takes_second_pass(D, fwd_rows):
    """One query row meets one late key more than 128 log2 units above everything before it
    (fp32 overflow against the first tile's max); the other rows of its workgroup do not,
    and every row must come out right after the redo."""
    _skip_dup(D, fwd_rows, 512)
    B, H, Tq, S = 1, 1, 512, 1000
    q, k, v, kv = make_inputs(B, H, Tq, S, D, [S], "bf16", 1.0, seed=1700, device=DEV)
    scale = 1.0 / math.sqrt(D)
    k[0, 0, 900] = (q[0, 0, 37].float() * 10.0 * math.sqrt(256 / D)).to(torch.bfloat16)  # row 37 meets key 900
    margin = _first_tile_margins_log2(q[:, :, 37:38], k, S, scale).max().item()
    log(f"one row D={D} rows={fwd_rows}: first-tile margin {margin:.0f} log2 units")
    assert margin > 128.0
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"one bad row D={D} rows={fwd_rows}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Tq", [1, 200, 256, 257, 700, 1024])
def test_eight_waves_same_bits(D, Tq, monkeypatch):
    """The 32-row kernel with eight waves per workgroup (256 rows, four LDS buffers of K and
    V, a barrier every other tile) runs the same per-row arithmetic as the four-wave form, so
    its output and LSE bits must be identical, on both sides of every tile boundary and with
    rows past T_q in the last workgroup."""
    S = 700
    lens = [0, 1, 63, 64, 65, 129, 300, S]
    log(f"eight waves D={D} Tq={Tq} lens={lens}")
    q, k, v, kv = make_inputs(len(lens), 2, Tq, S, D, lens, "bf16", 1.0, seed=2100 + Tq + D, device=DEV,
                              pad=float("nan"))
    scale = 1.0 / math.sqrt(D)
    monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", "128")
    o4, l4 = _run_fused(q, k, v, kv, scale)
    monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", "128x8")
    o8, l8 = _run_fused(q, k, v, kv, scale)
    assert torch.equal(o4, o8) and torch.equal(l4, l8), "eight waves differ from four"
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(o8, l8, ro, rl, "bf16", f"eight waves D={D} Tq={Tq}")


@pytest.mark.parametrize("Tq", [257, 300, 511, 700])
def test_mixed_edge_matrix(Tq, monkeypatch):
    """Both D = 256 paths in one grid: full 256-row tiles on the 64-row path, the rows after
    them on the 32-row path (row bases past 0, workgroup bases past 0)."""
    monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", "mixed")
    D, S = 256, 200
    lens = [0, 1, 31, 32, 33, 64, 65, S]
    log(f"mixed edge Tq={Tq} lens={lens}")
    q, k, v, kv = make_inputs(len(lens), 2, Tq, S, D, lens, "bf16", 1.0, seed=1800 + Tq, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out, lse = _run_fused(q, k, v, kv, scale)
    ro, rl = _oracle(q, k, v, kv, scale)
    assert_parity(out, lse, ro, rl, "bf16", f"mixed edge Tq={Tq}")

"""Shared helpers of the GPU parity tests: tolerances and the comparison.

Tolerances (fp64 oracle on the exact stored input values):
  * fp32 inputs: max |out - ref| <= 1e-4 (the fp32 bound of the sharded-vs-
    single-device checks on tabfm PR #81, section Tests); lse max-abs <= 1e-4.
  * bf16 inputs: max |out - ref| <= 2e-2 AND ||out - ref||_2 / ||ref||_2 <= 5e-3;
    lse max-abs <= 1e-3.
  * -inf LSE entries (n = 0, empty chunks) must match exactly and the matching
    outputs must be exactly 0.
"""

import math
import sys

import numpy as np
import torch

TOL = {
    "f32": dict(out_abs=1e-4, out_rel=None, lse_abs=1e-4),
    "bf16": dict(out_abs=2e-2, out_rel=5e-3, lse_abs=1e-3),
}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def assert_parity(out_gpu, lse_gpu, out_ref, lse_ref, dtype: str, what: str = ""):
    """Element-wise comparison against the oracle at the tolerance of ``dtype``."""
    tol = TOL[dtype]
    o = to64(out_gpu) if isinstance(out_gpu, torch.Tensor) else np.asarray(out_gpu, np.float64)
    r = np.asarray(out_ref, np.float64)
    assert o.shape == r.shape, (o.shape, r.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    diff = np.abs(o - r)
    max_abs = float(diff.max()) if diff.size else 0.0
    rn = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(o - r) / rn) if rn > 0 else float(np.linalg.norm(o - r))
    msg = f"{what}: out max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    if lse_gpu is not None:
        lg = to64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else np.asarray(lse_gpu, np.float64)
        lr = np.asarray(lse_ref, np.float64)
        assert lg.shape == lr.shape
        ninf_g, ninf_r = np.isneginf(lg), np.isneginf(lr)
        assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf LSE pattern differs"
        fin = ~ninf_r
        assert np.isfinite(lg[fin]).all(), f"{what}: non-finite LSE"
        lse_abs = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
        msg += f" lse_max_abs={lse_abs:.3e}"
        # rows without any valid key are exactly zero
        if ninf_r.any():
            assert np.all(o[ninf_r] == 0.0), f"{what}: rows with no valid key are not zero"
        assert lse_abs <= tol["lse_abs"], msg
    log(msg)
    assert max_abs <= tol["out_abs"], msg
    if tol["out_rel"] is not None:
        assert rel <= tol["out_rel"], msg
    return max_abs, rel


def gather_rows(x: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    """x [B, H, T, ...] and rows [B*H, R] -> x[b, h, rows[b*H + h]] as [B, H, R, ...]."""
    B, H = x.shape[:2]
    idx = torch.as_tensor(rows, device=x.device).view(B, H, -1)
    shape = list(idx.shape) + [1] * (x.dim() - 3)
    idx = idx.view(shape).expand(*idx.shape, *x.shape[3:])
    return torch.gather(x, 2, idx)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# Backward (bf16 inputs): rel-L2 per gradient tensor, and max-abs relative to the
# largest reference magnitude; the derivation is in tests/test_gpu_bwd.py.
GRAD_REL_L2 = 5e-3
GRAD_MAX_ABS_REL = 2e-2


def assert_grad_parity(name: str, got, ref, what: str = ""):
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what} {name}: non-finite"
    rn = float(np.linalg.norm(r))
    err = float(np.linalg.norm(g - r))
    rel = err / rn if rn > 0 else err
    mx = float(np.abs(g - r).max()) if g.size else 0.0
    top = float(np.abs(r).max()) if r.size else 0.0
    log(f"{what} {name}: rel_l2={rel:.3e} max_abs={mx:.3e} (ref max {top:.3e})")
    assert rel <= GRAD_REL_L2, f"{what} {name}: rel_l2 {rel:.3e}"
    assert mx <= GRAD_MAX_ABS_REL * max(top, 1e-6), f"{what} {name}: max_abs {mx:.3e}"
    return rel, mx

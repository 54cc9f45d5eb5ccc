"""Seeded random shapes through the backward kernels, against the fp64 oracle.

Each case draws B (up to 5, so that batches of distinct lengths take the
longest-first workgroup order), H, T_q, S, the per-element lengths (0 and S
included at random), the head dim and a scale of either sign; padded key slots
hold NaN.  dq, dk and dv are compared with the oracle's gradients at the
backward tolerance, padded slots must be exactly zero, and the allocation-free
entry point must give the same bits.
"""

import math
import os

import numpy as np
import pytest
import torch

from long_context_prefix_amd import _lib
from long_context_prefix_amd.workloads import make_inputs
from oracle import ref_prefix_bwd
from tests.parity import assert_grad_parity, log, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
# more cases, or another seed range, on demand: ATTN_TEST_RANDOM_CASES, ATTN_TEST_RANDOM_SEED
N_CASES = int(os.environ.get("ATTN_TEST_RANDOM_CASES", "24"))
SEED = int(os.environ.get("ATTN_TEST_RANDOM_SEED", "0"))


def _case(i):
    rng = np.random.default_rng(9500 + SEED + i)
    D = int(rng.choice([64, 128, 128, 256]))
    B = int(rng.integers(1, 6))
    H = int(rng.integers(1, 3))
    Tq = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 400))]))
    S = int(rng.integers(1, 400))
    lens = rng.integers(0, S + 1, size=B)
    if B > 1:
        lens[rng.integers(0, B)] = S
    scale = float((1.0 / math.sqrt(D)) * rng.choice([1.0, 1.5, -1.0]))
    return D, B, H, Tq, S, [int(x) for x in lens], scale


@pytest.mark.parametrize("i", range(N_CASES))
def test_bwd_random_shape(i):
    D, B, H, Tq, S, lens, scale = _case(i)
    log(f"bwd random case {i}: D={D} B={B} H={H} Tq={Tq} S={S} lens={lens} scale={scale:.4f}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=9600 + SEED + i, device=DEV,
                              pad=float("nan"))
    out, lse = _lib.attn_prefix_fwd(q, k, v, kv, scale)
    g = torch.Generator(device="cpu").manual_seed(9700 + SEED + i)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    dq, dk, dv = _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, scale)
    torch.cuda.synchronize()
    # the oracle slices the keys to each prefix before any arithmetic (the NaN pads never enter)
    # and returns exact zeros on padded slots
    rq, rk, rv = ref_prefix_bwd(to64(q), to64(k), to64(v), np.array(lens), scale, to64(dout))
    for b, n in enumerate(lens):
        assert torch.all(dk[b, :, n:] == 0) and torch.all(dv[b, :, n:] == 0), f"case {i}: padded gradient"
    what = f"bwd random case {i}"
    if np.abs(rq).max() > 0:
        assert_grad_parity("dq", dq, rq, what)
    else:
        assert torch.all(dq == 0), f"{what}: dq of a batch with no valid key"
    if np.abs(rk).max() > 0:
        assert_grad_parity("dk", dk, rk, what)
        assert_grad_parity("dv", dv, rv, what)
    nq, nk, nv = (torch.full_like(t, float("nan")) for t in (dq, dk, dv))
    _lib.attn_prefix_bwd_noalloc(q, k, v, kv, out, dout, lse, nq, nk, nv, scale)
    torch.cuda.synchronize()
    for name, x, y in (("dq", nq, dq), ("dk", nk, dk), ("dv", nv, dv)):
        assert torch.equal(x, y), f"{what}: the allocation-free entry point differs in {name}"

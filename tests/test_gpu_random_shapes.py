"""Seeded random shapes through every forward path, against the fp64 oracle.

Each case draws B, H, T_q, S, the per-element lengths (0 and S included at
random), the head dim, the dtype and a scale of either sign, and runs the
fused forward with each bf16 path forced (32 query rows per wave with four or
eight waves per workgroup at D <= 128, 64 rows per wave at D = 128 and 256, and
both in one grid at D = 256), plus split-KV partials and their merge.
"""

import math
import os

import numpy as np
import pytest
import torch

from long_context_prefix_amd import _lib
from long_context_prefix_amd.workloads import make_inputs
from oracle import ref_prefix_fwd
from tests.parity import assert_parity, log, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
# more cases, or another seed range, on demand: ATTN_TEST_RANDOM_CASES, ATTN_TEST_RANDOM_SEED
N_CASES = int(os.environ.get("ATTN_TEST_RANDOM_CASES", "96"))
SEED = int(os.environ.get("ATTN_TEST_RANDOM_SEED", "0"))


def _case(i):
    rng = np.random.default_rng(9000 + SEED + i)
    D = int(rng.choice([64, 128, 256, 256]))
    dtype = "f32" if (D != 256 and rng.random() < 0.25) else "bf16"
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 3))
    Tq = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 800))]))
    S = int(rng.integers(1, 400))
    lens = rng.integers(0, S + 1, size=B)
    if B > 1:
        lens[rng.integers(0, B)] = S
    scale = float((1.0 / math.sqrt(D)) * rng.choice([1.0, 2.0, -1.0]))
    return D, dtype, B, H, Tq, S, [int(x) for x in lens], scale


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i, monkeypatch):
    D, dtype, B, H, Tq, S, lens, scale = _case(i)
    log(f"random case {i}: D={D} {dtype} B={B} H={H} Tq={Tq} S={S} lens={lens} scale={scale:.4f}")
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, dtype, 1.0, seed=9100 + SEED + i, device=DEV,
                              pad=float("nan"))
    ro, rl = ref_prefix_fwd(to64(q), to64(k), to64(v), np.array(lens), scale)
    paths = ["128"]
    if dtype == "bf16" and D == 256:
        paths = ["128", "256", "mixed"]
    elif dtype == "bf16" and D == 128:
        paths = ["128", "128x8", "256"]
    elif dtype == "bf16":
        paths = ["128", "128x8"]
    for rows in paths:
        monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", rows)
        out, lse = _lib.attn_prefix_fwd(q, k, v, kv, scale)
        torch.cuda.synchronize()
        assert_parity(out, lse, ro, rl, dtype, f"random case {i}, rows {rows}")
    chunk = 64 * int(np.random.default_rng(9200 + SEED + i).integers(1, 4))
    so, sl = _lib.splitkv_fwd(q, k, v, kv, chunk, scale)
    torch.cuda.synchronize()
    assert_parity(so, sl, ro, rl, dtype, f"random case {i}, split-KV chunk {chunk}")

"""The allocation-free backward entry point (attn_prefix_bwd_noalloc), through the C ABI.

It must give the bits of attn_prefix_bwd (same kernels, delta in the library's own
device array instead of a workspace argument) on consecutive calls, the second one
smaller than the first, so that nothing of the first call's scratch contents leaks
into the second; and it must allocate nothing through torch.
"""

import ctypes
import math

import pytest
import torch

from long_context_prefix_amd import _lib
from long_context_prefix_amd.workloads import make_inputs
from tests.parity import log

DEV = "cuda"
MAX_ROWS = 1 << 22


@pytest.mark.gpu
def test_noalloc_backward_matches_the_workspace_entry_point():
    cases = [  # (B, H, Tq, S, D, lens): the second call is smaller than the first
        (3, 4, 700, 900, 128, [900, 1, 517]),
        (2, 2, 150, 320, 256, [300, 0]),
        (1, 2, 65, 64, 64, [64]),
    ]
    for i, (B, H, Tq, S, D, lens) in enumerate(cases):
        log(f"noalloc backward call {i}: B={B} H={H} Tq={Tq} S={S} D={D} lens={lens}")
        q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=5100 + i, device=DEV)
        scale = 1.0 / math.sqrt(D)
        out, lse = _lib.attn_prefix_fwd(q, k, v, kv, scale)
        g = torch.Generator(device="cpu").manual_seed(5200 + i)
        dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
        want = _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, scale)
        got = tuple(torch.full_like(t, float("nan")) for t in want)
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0)
        _lib.attn_prefix_bwd_noalloc(q, k, v, kv, out, dout, lse, *got, scale)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0) == before, "torch allocated"
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(a, b), f"call {i}: {name} differs from attn_prefix_bwd"


@pytest.mark.gpu
def test_noalloc_backward_rejects_more_rows_than_its_scratch():
    L = _lib.load()
    P = ctypes.c_void_p(4096)

    def call(B, H, Tq, kv=P):
        return L.attn_prefix_bwd_noalloc(P, P, P, kv, P, P, P, B, H, Tq, 64, 64, 0.125, 0, P, P, P, None)

    assert call(1, 8, MAX_ROWS // 8, kv=None) == 1  # within the limit: the NULL kv_len is what fails
    assert call(1, 8, MAX_ROWS // 8 + 1) == 2  # one row past it: ATTN_ERR_SHAPE, nothing launched

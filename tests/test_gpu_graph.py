"""The library's calls inside a captured HIP graph.

Every entry point only enqueues kernels on the caller's stream (no allocation,
no host synchronization, no memset), so a training or serving loop can capture
them.  The graph is replayed several times with eager work in between, and
every replay must reproduce the eager results bit for bit.
"""

import math

import pytest
import torch

from long_context_prefix_amd import _lib
from long_context_prefix_amd.workloads import make_inputs
from tests.parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_graph_replays_match_eager():
    B, H, Tq, S, D = 2, 2, 200, 500, 128
    lens = [500, 123]
    q, k, v, _ = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=5150, device=DEV)
    mask = (torch.arange(S, device=DEV)[None, :] < torch.tensor(lens, device=DEV)[:, None])[:, None, None, :]
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(DEV)
    scale = 1.0 / math.sqrt(D)
    chunk = 128
    C = -(-S // chunk)
    # every buffer is allocated before capture
    kv = torch.empty(B, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), device=DEV)
    po = torch.empty((B, H, C, Tq, D), device=DEV)
    pl = torch.empty((B, H, C, Tq), device=DEV)
    sout = torch.empty_like(q)
    slse = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)

    def step():
        _lib.attn_prefix_mask_to_kv_len(mask, kv)
        _lib.attn_prefix_fwd(q, k, v, kv, scale, out=out, lse=lse)
        _lib.attn_splitkv_partial(q, k, v, kv, chunk, scale, part_out=po, part_lse=pl)
        _lib.attn_lse_combine(po, pl, torch.bfloat16, out=sout, lse=slse)
        _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, scale, dq=dq, dk=dk, dv=dv, delta=delta)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (kv, out, lse, sout, slse, dq, dk, dv)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (kv, out, lse, sout, slse, dq, dk, dv):  # scribble between replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("kv_len", "out", "lse", "split out", "split lse", "dq", "dk", "dv"),
                                   (kv, out, lse, sout, slse, dq, dk, dv), eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
        log(f"graph replay {rep}: identical to eager")


def test_graph_with_the_allocation_free_backward():
    """The allocation-free backward in a captured graph: nothing is allocated at capture or
    replay (its delta lives in the library's device array), and eager calls of another shape
    between the replays, which overwrite that array, do not change what a replay computes."""
    B, H, Tq, S, D = 2, 2, 150, 300, 128
    lens = [300, 77]
    q, k, v, kv = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=5160, device=DEV)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(10)).to(torch.bfloat16).to(DEV)
    scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # another shape whose eager calls run between the replays
    q2, k2, v2, kv2 = make_inputs(3, 1, 400, 200, 64, [200, 5, 150], "bf16", 1.0, seed=5161, device=DEV)
    out2, lse2 = _lib.attn_prefix_fwd(q2, k2, v2, kv2, 0.125)
    g2 = tuple(torch.empty_like(t) for t in (q2, k2, v2))

    def step():
        _lib.attn_prefix_fwd(q, k, v, kv, scale, out=out, lse=lse)
        _lib.attn_prefix_bwd_noalloc(q, k, v, kv, out, dout, lse, dq, dk, dv, scale)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, dq, dk, dv)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        _lib.attn_prefix_bwd_noalloc(q2, k2, v2, kv2, out2, out2, lse2, *g2, 0.125)  # overwrites the scratch
        for t in (out, lse, dq, dk, dv):
            t.zero_()
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0) == before
        for name, got, want in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
        log(f"graph replay {rep} with the allocation-free backward: identical to eager")

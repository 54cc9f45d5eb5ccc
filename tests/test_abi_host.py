"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function ``include/attn_prefix.h``
declares, and reject every bad argument with its documented status code before
any HIP call (the ABI calls below pass fake, never-dereferenced addresses).
"""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from long_context_prefix_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_prefix.h")

OK, NULLPTR, SHAPE, DTYPE, UNSUP, ALIGN, CHUNK, HIP, ARG = range(9)
BF16, F32 = 0, 1
P = ctypes.c_void_p(4096)  # aligned fake device address; never dereferenced on these paths
PM = ctypes.c_void_p(4096 + 8)  # misaligned for 16-byte tensors


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(_lib.EXPORTED), names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = set(line.split()[-1] for line in nm.stdout.splitlines() if " T " in line)
        for name in declared_functions():
            assert name in exported, name


def test_version_and_chunks(L):
    assert L.attn_version() == (0 << 16) | (2 << 8)
    assert L.attn_splitkv_num_chunks(102400, 4096) == 25
    assert L.attn_splitkv_num_chunks(4096, 4096) == 1
    assert L.attn_splitkv_num_chunks(4097, 4096) == 2
    assert L.attn_splitkv_num_chunks(0, 64) == 0
    assert L.attn_splitkv_num_chunks(10, 0) == -1
    assert L.attn_splitkv_num_chunks(-1, 64) == -1


def test_status_strings(L):
    for code in range(9):
        s = _lib.status_string(code)
        assert s and s != "unknown status"
    assert _lib.status_string(99) == "unknown status"


def fwd(L, q=P, k=P, v=P, kv=P, B=1, H=1, Tq=1, S=1, D=64, scale=0.125, dt=BF16, out=P, lse=None):
    return L.attn_prefix_fwd(q, k, v, kv, B, H, Tq, S, D, scale, dt, out, lse, None)


def split(L, q=P, k=P, v=P, kv=P, B=1, H=1, Tq=1, S=64, D=64, scale=0.125, dt=BF16, chunk=64, po=P, pl=P):
    return L.attn_splitkv_partial(q, k, v, kv, B, H, Tq, S, D, scale, dt, chunk, po, pl, None)


def combine(L, po=P, pl=P, B=1, H=1, C=2, Tq=1, D=64, dt=BF16, out=P, lse=None):
    return L.attn_lse_combine(po, pl, B, H, C, Tq, D, dt, out, lse, None)


def test_prefix_fwd_argument_errors(L):
    assert fwd(L, dt=2) == DTYPE
    assert fwd(L, dt=-1) == DTYPE
    for bad in (dict(B=-1), dict(H=-1), dict(Tq=-1), dict(S=-1), dict(D=-64)):
        assert fwd(L, **bad) == SHAPE, bad
    for d in (0, 32, 96, 100, 512):
        assert fwd(L, D=d) == UNSUP, d
    assert fwd(L, scale=float("nan")) == ARG
    assert fwd(L, scale=float("inf")) == ARG
    # precedence: dtype before shape before head dim before scale
    assert fwd(L, dt=5, B=-1, D=7) == DTYPE
    assert fwd(L, B=-1, D=7) == SHAPE
    assert fwd(L, D=7, scale=float("nan")) == UNSUP
    for name in ("q", "kv", "out"):
        assert fwd(L, **{name: None}) == NULLPTR, name
    assert fwd(L, k=None) == NULLPTR
    assert fwd(L, v=None) == NULLPTR
    for name in ("q", "k", "v", "out"):
        assert fwd(L, **{name: PM}) == ALIGN, name
    assert fwd(L, kv=ctypes.c_void_p(4098)) == ALIGN
    assert fwd(L, lse=ctypes.c_void_p(4097)) == ALIGN
    # limits: per-(b,h) K/V slice beyond 2^31 bytes, or too many workgroups
    assert fwd(L, S=2**22, D=256) == SHAPE
    assert fwd(L, S=2**22, D=256, dt=F32) == SHAPE
    assert fwd(L, B=2**16, H=2**16, Tq=128) == SHAPE


def test_prefix_fwd_empty_calls_are_noops(L):
    # zero-sized batches, heads or queries: no work, pointers may be NULL
    for z in (dict(B=0), dict(H=0), dict(Tq=0)):
        assert fwd(L, q=None, k=None, v=None, kv=None, out=None, **z) == OK, z
    # S = 0 with nothing to read: k and v may be NULL (not launched here: B = 0)
    assert fwd(L, B=0, S=0, k=None, v=None) == OK


def test_splitkv_argument_errors(L):
    assert split(L, chunk=0) == CHUNK
    assert split(L, chunk=-64) == CHUNK
    assert split(L, chunk=96) == CHUNK
    assert split(L, chunk=100) == CHUNK
    assert split(L, dt=3) == DTYPE
    assert split(L, D=48) == UNSUP
    assert split(L, po=None) == NULLPTR
    assert split(L, pl=None) == NULLPTR
    assert split(L, po=PM) == ALIGN
    assert split(L, pl=ctypes.c_void_p(4098)) == ALIGN
    assert split(L, B=0, po=None, pl=None) == OK
    assert split(L, S=2**20, chunk=64, B=2**14, H=8) == SHAPE  # 2^31 workgroups


def test_combine_argument_errors(L):
    assert combine(L, dt=7) == DTYPE
    assert combine(L, C=-1) == SHAPE
    assert combine(L, D=32) == UNSUP
    assert combine(L, out=None) == NULLPTR
    assert combine(L, po=None) == NULLPTR
    assert combine(L, pl=None) == NULLPTR
    assert combine(L, out=PM) == ALIGN
    assert combine(L, po=PM) == ALIGN
    assert combine(L, lse=ctypes.c_void_p(4097)) == ALIGN
    assert combine(L, B=0, out=None) == OK


def test_binding_rejects_bad_tensors_before_the_abi():
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    kv = torch.tensor([4], dtype=torch.int32)
    with pytest.raises(ValueError):
        _lib.attn_prefix_fwd(q, q, q, kv)  # CPU tensors
    with pytest.raises(ValueError):
        _lib.attn_prefix_fwd(q, q[..., :32], q, kv)
    with pytest.raises(ValueError):
        _lib.attn_prefix_fwd(q, q, q, kv.to(torch.int64))
    with pytest.raises(ValueError):
        _lib.attn_prefix_fwd(q.half(), q.half(), q.half(), kv)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_mask_to_kv_len_argument_errors(L):
    def call(mask=P, B=2, S=8, stride=8, kv=P):
        return L.attn_prefix_mask_to_kv_len(mask, B, S, stride, kv, None)

    assert call(B=-1) == SHAPE
    assert call(S=-1) == SHAPE
    assert call(stride=-8) == SHAPE
    assert call(mask=None) == NULLPTR
    assert call(kv=None) == NULLPTR
    assert call(kv=ctypes.c_void_p(4098)) == ALIGN
    assert call(B=0, mask=None, kv=None) == OK  # empty batch: nothing launched


def test_mask_binding_rejects_bad_masks():
    m = torch.ones(2, 1, 1, 8, dtype=torch.bool)
    with pytest.raises(ValueError):
        _lib.attn_prefix_mask_to_kv_len(m)  # CPU tensor
    with pytest.raises(ValueError):
        _lib.attn_prefix_mask_to_kv_len(torch.ones(2, 2, 1, 8, dtype=torch.bool))  # per-head mask
    with pytest.raises(ValueError):
        _lib.attn_prefix_mask_to_kv_len(torch.zeros(2, 8, dtype=torch.float32))  # additive bias
    with pytest.raises(ValueError):
        _lib.attn_prefix_mask_to_kv_len(torch.ones(8, dtype=torch.bool))


def test_bwd_argument_errors(L):
    def call(q=P, k=P, v=P, kv=P, out=P, dout=P, lse=P, B=1, H=1, Tq=8, S=8, D=64, scale=0.125, dt=BF16,
             delta=P, dq=P, dk=P, dv=P):
        return L.attn_prefix_bwd(q, k, v, kv, out, dout, lse, B, H, Tq, S, D, scale, dt, delta, dq, dk, dv, None)

    assert call(dt=9) == DTYPE
    assert call(B=-1) == SHAPE
    assert call(dt=F32) == UNSUP  # the backward is bf16 only
    assert call(D=512) == UNSUP
    assert call(D=32) == UNSUP
    assert call(scale=float("nan")) == ARG
    for name in ("q", "kv", "out", "dout", "lse", "delta", "dq", "dk", "dv", "k", "v"):
        assert call(**{name: None}) == NULLPTR, name
    for name in ("q", "out", "dout", "dq", "dk", "dv", "k", "v"):
        assert call(**{name: PM}) == ALIGN, name
    assert call(lse=ctypes.c_void_p(4097)) == ALIGN
    assert call(delta=ctypes.c_void_p(4098)) == ALIGN
    assert call(B=0, q=None, k=None, v=None, kv=None, out=None, dout=None, lse=None, delta=None, dq=None, dk=None,
                dv=None) == OK
    assert call(S=2**23, D=128) == SHAPE  # 2^31 bytes per (b, h) slice


def test_single_launch_split_argument_errors(L):
    def call(counters=P, out=P, lse=None, chunk=64, **kw):
        a = dict(q=P, k=P, v=P, kv=P, B=1, H=1, Tq=1, S=64, D=64, scale=0.125, dt=BF16, po=P, pl=P)
        a.update(kw)
        return L.attn_splitkv_fwd(a["q"], a["k"], a["v"], a["kv"], a["B"], a["H"], a["Tq"], a["S"], a["D"],
                                  a["scale"], a["dt"], chunk, a["po"], a["pl"], counters, out, lse, None)

    assert call(chunk=96) == CHUNK
    assert call(counters=None) == NULLPTR
    assert call(out=None) == NULLPTR
    assert call(counters=ctypes.c_void_p(4098)) == ALIGN
    assert call(out=PM) == ALIGN
    assert call(lse=ctypes.c_void_p(4097)) == ALIGN
    assert call(B=0, counters=None, out=None) == OK


# A 1-D dispatch counts work-items (workgroups x threads) in 32 bits: 256-thread launches hold
# at most 2^24 - 1 workgroups, the 512-thread mask launch 2^23 - 1.  Sizes are checked before
# pointers, so a call just inside the limit with a NULL pointer returns ATTN_ERR_NULLPTR (and
# launches nothing), the same call one workgroup past it ATTN_ERR_SHAPE.
MAX_WG = (2**32 - 1) // 256


def test_launch_limits_forward_and_split(L):
    assert MAX_WG == 2**24 - 1
    # fused forward: B * H * ceil(Tq / 128) workgroups
    assert fwd(L, q=None, Tq=128 * MAX_WG) == NULLPTR
    assert fwd(L, q=None, Tq=128 * MAX_WG + 1) == SHAPE
    assert fwd(L, q=None, B=2**8, H=2**8, Tq=128 * 255) == NULLPTR  # 2^24 - 2^16 workgroups
    assert fwd(L, q=None, B=2**8, H=2**8, Tq=128 * 256) == SHAPE  # exactly 2^24
    assert fwd(L, q=None, B=2**8, H=2**8, Tq=128 * 4096) == SHAPE  # between 2^24 and 2^31 workgroups
    # split partial: B * H * ceil(Tq / 128) * C
    assert split(L, po=None, B=MAX_WG) == NULLPTR
    assert split(L, po=None, B=MAX_WG + 1) == SHAPE
    assert split(L, po=None, B=MAX_WG // 3, S=192) == NULLPTR  # C = 3
    assert split(L, po=None, B=MAX_WG // 3 + 1, S=192) == SHAPE


def test_launch_limit_eight_wave_forward(L, monkeypatch):
    """The eight-wave forward launches 512-thread workgroups, half as many as the size check
    of the four-wave grid counted: its own grid is checked too (here B * H = 2^23 workgroups of
    512 threads, 2^32 work-items, which the four-wave check lets through).  Only the failing
    side is probed: a grid that fit would be launched."""
    monkeypatch.setenv("ATTN_PREFIX_FWD_ROWS", "128x8")
    assert fwd(L, B=2**23, D=128) == SHAPE
    assert fwd(L, B=2**22, H=2, D=64) == SHAPE


def test_launch_limits_single_launch_split(L):
    def call(**kw):
        a = dict(B=1, H=1, Tq=1, S=64)
        a.update(kw)
        return L.attn_splitkv_fwd(P, P, P, P, a["B"], a["H"], a["Tq"], a["S"], 64, 0.125, BF16, 64, P, P,
                                  None, P, None, None)

    assert call(B=MAX_WG) == NULLPTR  # counters NULL: the size check passed
    assert call(B=MAX_WG + 1) == SHAPE


def test_launch_limits_combine_mask_and_backward(L):
    # merge: 1024 / D rows per workgroup
    assert combine(L, out=None, Tq=16 * MAX_WG, D=64) == NULLPTR
    assert combine(L, out=None, Tq=16 * MAX_WG + 1, D=64) == SHAPE
    assert combine(L, out=None, Tq=4 * MAX_WG, D=256) == NULLPTR
    assert combine(L, out=None, Tq=4 * MAX_WG + 1, D=256) == SHAPE
    # mask detector: one 512-thread workgroup per row
    mask_max = (2**32 - 1) // 512
    assert L.attn_prefix_mask_to_kv_len(P, mask_max, 8, 8, None, None) == NULLPTR
    assert L.attn_prefix_mask_to_kv_len(P, mask_max + 1, 8, 8, None, None) == SHAPE

    def bwd(B=1, H=1, Tq=8, S=8, D=256, kv=None):
        return L.attn_prefix_bwd(P, P, P, kv, P, P, P, B, H, Tq, S, D, 0.125, BF16, P, P, P, P, None)

    # delta: 2048 / D rows per workgroup (8 at D = 256)
    assert bwd(Tq=8 * MAX_WG) == NULLPTR
    assert bwd(Tq=8 * MAX_WG + 1) == SHAPE
    # dk/dv: B * H * ceil(S / 128) workgroups
    assert bwd(B=MAX_WG, Tq=0, S=128, D=64) == NULLPTR
    assert bwd(B=MAX_WG + 1, Tq=0, S=128, D=64) == SHAPE

"""ctypes binding of libattnprefix.so (argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
``include/attn_prefix.h``; torch supplies device memory and the current
stream.  There is no fallback: if the library is missing, or a call returns a
non-OK status, these functions raise.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnprefix.so")

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULLPTR", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_DTYPE", 4: "ATTN_ERR_UNSUPPORTED",
    5: "ATTN_ERR_ALIGN", 6: "ATTN_ERR_CHUNK", 7: "ATTN_ERR_HIP", 8: "ATTN_ERR_ARG",
}
ATTN_BF16, ATTN_F32 = 0, 1
EXPORTED = ("attn_version", "attn_prefix_fwd", "attn_splitkv_partial", "attn_lse_combine", "attn_splitkv_fwd",
            "attn_prefix_mask_to_kv_len", "attn_prefix_bwd", "attn_prefix_bwd_noalloc", "attn_splitkv_num_chunks",
            "attn_status_string")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(code, code)} ({text})")
        self.code = code


def load() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_prefix_amd.build` "
                          "(the attention path has no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_version.restype = i32
    L.attn_version.argtypes = []
    L.attn_prefix_fwd.restype = i32
    L.attn_prefix_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp]
    L.attn_splitkv_partial.restype = i32
    L.attn_splitkv_partial.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp]
    L.attn_lse_combine.restype = i32
    L.attn_lse_combine.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    L.attn_prefix_mask_to_kv_len.restype = i32
    L.attn_prefix_mask_to_kv_len.argtypes = [vp, i32, i32, ctypes.c_int64, vp, vp]
    L.attn_splitkv_fwd.restype = i32
    L.attn_splitkv_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.attn_prefix_bwd.restype = i32
    L.attn_prefix_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp]
    L.attn_prefix_bwd_noalloc.restype = i32
    L.attn_prefix_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp]
    L.attn_splitkv_num_chunks.restype = i32
    L.attn_splitkv_num_chunks.argtypes = [i32, i32]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_status_string.argtypes = [i32]
    _lib = L
    return L


def status_string(code: int) -> str:
    return load().attn_status_string(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != ATTN_OK:
        raise AttnError(fn, code, status_string(code))


def _call(fn: str, dev: torch.device, *args) -> None:
    """Call a library entry point with `dev` as the current HIP device (the library launches
    on the current device, which must be the one that holds the tensors) and raise on error."""
    with torch.cuda.device(dev):
        code = getattr(load(), fn)(*args)
    _check(fn, code)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t: torch.Tensor, name: str, device: torch.device) -> None:
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_splitkv_num_chunks(S: int, chunk: int) -> int:
    return int(load().attn_splitkv_num_chunks(int(S), int(chunk)))


def _fwd_shapes(q, k, v, kv_len):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    B, H, Tq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    if kv_len.dtype != torch.int32 or kv_len.shape != (B,):
        raise ValueError("kv_len must be int32 [B]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (kv_len, "kv_len")):
        _require(t, name, dev)
    return B, H, Tq, k.shape[2], D, dev


def attn_prefix_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_len: torch.Tensor,
                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused prefix-masked attention; returns (out [B,H,Tq,D], lse [B,H,Tq] fp32 or None)."""
    B, H, Tq, S, D, dev = _fwd_shapes(q, k, v, kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    _require(out, "out", dev)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if lse is not None:
        _require(lse, "lse", dev)
        if lse.shape != (B, H, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, H, Tq]")
    _call("attn_prefix_fwd", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), B, H, Tq, S, D, scale,
          _dtype_code(q), _ptr(out), _ptr(lse), _stream(dev))
    return out, lse


def attn_splitkv_partial(q, k, v, kv_len, chunk: int, scale: Optional[float] = None,
                         part_out: Optional[torch.Tensor] = None, part_lse: Optional[torch.Tensor] = None):
    """Per-chunk fp32 partials; returns (part_out [B,H,C,Tq,D], part_lse [B,H,C,Tq])."""
    B, H, Tq, S, D, dev = _fwd_shapes(q, k, v, kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    C = -(-S // chunk)
    if part_out is None:
        part_out = torch.empty((B, H, C, Tq, D), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((B, H, C, Tq), dtype=torch.float32, device=dev)
    _require(part_out, "part_out", dev)
    _require(part_lse, "part_lse", dev)
    if part_out.shape != (B, H, C, Tq, D) or part_lse.shape != (B, H, C, Tq):
        raise ValueError("partial buffers have the wrong shape")
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise ValueError("partial buffers must be fp32")
    _call("attn_splitkv_partial", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), B, H, Tq, S, D, scale,
          _dtype_code(q), int(chunk), _ptr(part_out), _ptr(part_lse), _stream(dev))
    return part_out, part_lse


def attn_lse_combine(part_out: torch.Tensor, part_lse: torch.Tensor, out_dtype=torch.bfloat16,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = True):
    """Exact LSE merge of partials [B,H,C,Tq,D]; returns (out [B,H,Tq,D], lse [B,H,Tq])."""
    if part_out.dim() != 5 or part_lse.dim() != 4 or part_out.shape[:4] != part_lse.shape:
        raise ValueError("part_out must be [B,H,C,Tq,D] and part_lse [B,H,C,Tq]")
    B, H, C, Tq, D = part_out.shape
    dev = part_out.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    _require(part_out, "part_out", dev)
    _require(part_lse, "part_lse", dev)
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise ValueError("partial buffers must be fp32")
    if out is None:
        out = torch.empty((B, H, Tq, D), dtype=out_dtype, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    _require(out, "out", dev)
    if out.shape != (B, H, Tq, D):
        raise ValueError("out must be [B, H, Tq, D]")
    if lse is not None:
        _require(lse, "lse", dev)
        if lse.shape != (B, H, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, H, Tq]")
    _call("attn_lse_combine", dev, _ptr(part_out), _ptr(part_lse), B, H, C, Tq, D, _dtype_code(out), _ptr(out),
          _ptr(lse), _stream(dev))
    return out, lse


def splitkv_fwd(q, k, v, kv_len, chunk: int, scale: Optional[float] = None, return_lse: bool = True):
    """Split-KV attention: per-chunk partials, then the exact merge (two launches, one stream)."""
    po, pl = attn_splitkv_partial(q, k, v, kv_len, chunk, scale)
    return attn_lse_combine(po, pl, q.dtype, return_lse=return_lse)


def attn_prefix_mask_to_kv_len(mask: torch.Tensor, kv_len: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device-side conversion of a key mask ([B, S] or [B, 1, 1, S], bool or uint8,
    True = attend) into int32 lengths; a row that is not a prefix mask gives -1."""
    if mask.dim() == 4:
        if mask.shape[1] != 1 or mask.shape[2] != 1:
            raise ValueError("a 4-D key mask must be [B, 1, 1, S] (broadcast over heads and queries)")
        B, S = mask.shape[0], mask.shape[3]
        row_stride = mask.stride(0)
    elif mask.dim() == 2:
        B, S = mask.shape
        row_stride = mask.stride(0)
    else:
        raise ValueError("key mask must be [B, S] or [B, 1, 1, S]")
    if mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("key mask must be bool or uint8 (a float bias is not a padding mask)")
    if mask.device.type != "cuda":
        raise ValueError("mask must live on a GPU")
    if row_stride < 0:
        raise ValueError("negative batch stride")
    if S > 1 and mask.stride(-1) != 1:
        raise ValueError("the key axis of the mask must be contiguous")
    if kv_len is None:
        kv_len = torch.empty(B, dtype=torch.int32, device=mask.device)
    elif kv_len.dtype != torch.int32 or kv_len.shape != (B,) or kv_len.device != mask.device:
        raise ValueError("kv_len must be int32 [B] on the mask's device")
    _call("attn_prefix_mask_to_kv_len", mask.device, _ptr(mask), B, S, int(row_stride), _ptr(kv_len),
          _stream(mask.device))
    return kv_len


def kv_len_from_prefix_mask(mask: torch.Tensor) -> torch.Tensor:
    """Lengths of a prefix key-padding mask; raises ValueError (after one sync) for any
    row that is not True...True False...False.  There is no fallback to a dense mask."""
    kv_len = attn_prefix_mask_to_kv_len(mask)
    bad = torch.nonzero(kv_len < 0).flatten()
    if bad.numel():
        raise ValueError(f"attention mask rows {bad.tolist()[:8]} are not prefix key-padding masks")
    return kv_len


def sdpa_prefix(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, attn_mask: torch.Tensor,
                scale: Optional[float] = None) -> torch.Tensor:
    """Scaled-dot-product attention with a [B, 1, 1, S] (or [B, S]) boolean prefix key mask,
    ragged lengths included, on the fused kernel.  Non-prefix masks raise."""
    kv_len = kv_len_from_prefix_mask(attn_mask)
    out, _ = attn_prefix_fwd(q, k, v, kv_len, scale, return_lse=False)
    return out


def attn_prefix_bwd(q, k, v, kv_len, out, dout, lse, scale: Optional[float] = None,
                    dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                    dv: Optional[torch.Tensor] = None, delta: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of the prefix-masked forward, bf16, D in {64, 128, 256}.

    ``out`` and ``lse`` are the forward's results; ``delta`` is an optional fp32
    [B, H, Tq] workspace (rowsum(dout * out)).  dk and dv are zero on padded slots.
    """
    B, H, Tq, S, D, dev = _fwd_shapes(q, k, v, kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    for t, name in ((out, "out"), (dout, "dout")):
        _require(t, name, dev)
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    _require(lse, "lse", dev)
    if lse.shape != (B, H, Tq) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, H, Tq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, Tq), dtype=torch.float32, device=dev) if delta is None else delta
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _require(t, name, dev)
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} has the wrong shape or dtype")
    _require(delta, "delta", dev)
    if delta.shape != (B, H, Tq) or delta.dtype != torch.float32:
        raise ValueError("delta must be fp32 [B, H, Tq]")
    _call("attn_prefix_bwd", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), _ptr(out), _ptr(dout), _ptr(lse),
          B, H, Tq, S, D, scale, _dtype_code(q), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
          _stream(dev))
    return dq, dk, dv


def attn_prefix_bwd_noalloc(q, k, v, kv_len, out, dout, lse, dq, dk, dv, scale: Optional[float] = None):
    """attn_prefix_bwd into caller-provided dq, dk, dv, with no workspace argument: the
    library keeps delta in a device array of its own (at most 4,194,304 rows of
    B * H * Tq), so the call allocates nothing.  Calls that overlap in time on one GPU race
    on that array."""
    B, H, Tq, S, D, dev = _fwd_shapes(q, k, v, kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    for t, ref, name in ((out, q, "out"), (dout, q, "dout"), (dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _require(t, name, dev)
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} has the wrong shape or dtype")
    _require(lse, "lse", dev)
    if lse.shape != (B, H, Tq) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, H, Tq]")
    _call("attn_prefix_bwd_noalloc", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), _ptr(out), _ptr(dout), _ptr(lse),
          B, H, Tq, S, D, scale, _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv),
          _stream(dev))
    return dq, dk, dv


class _PrefixAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, kv_len, scale):
        out, lse = attn_prefix_fwd(q, k, v, kv_len, scale)
        ctx.save_for_backward(q, k, v, kv_len, out, lse)
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, kv_len, out, lse = ctx.saved_tensors
        dq, dk, dv = attn_prefix_bwd(q, k, v, kv_len, out, dout.contiguous(), lse, ctx.scale)
        return dq, dk, dv, None, None


def prefix_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_len: torch.Tensor,
                     scale: Optional[float] = None) -> torch.Tensor:
    """Differentiable prefix-masked attention (forward and backward on the HIP kernels)."""
    return _PrefixAttention.apply(q, k, v, kv_len, scale)


def attn_splitkv_fwd(q, k, v, kv_len, chunk: int, scale: Optional[float] = None,
                     part_out: Optional[torch.Tensor] = None, part_lse: Optional[torch.Tensor] = None,
                     counters: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Split-KV partials and their merge in one launch; returns (out, lse).

    ``counters`` (int32 [B, H, ceil(Tq/128)]) must be zero before the call and is
    zero again after it; it is allocated when not given.
    """
    B, H, Tq, S, D, dev = _fwd_shapes(q, k, v, kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    C = -(-S // chunk)
    if part_out is None:
        part_out = torch.empty((B, H, C, Tq, D), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((B, H, C, Tq), dtype=torch.float32, device=dev)
    nqt = -(-Tq // 128)
    if counters is None:
        counters = torch.zeros((B, H, nqt), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    for t, name in ((part_out, "part_out"), (part_lse, "part_lse"), (counters, "counters"), (out, "out")):
        _require(t, name, dev)
    if part_out.shape != (B, H, C, Tq, D) or part_lse.shape != (B, H, C, Tq):
        raise ValueError("partial buffers have the wrong shape")
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise ValueError("partial buffers must be fp32")
    if counters.dtype != torch.int32 or counters.shape != (B, H, nqt):
        raise ValueError("counters must be int32 [B, H, ceil(Tq / 128)]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if lse is not None:
        _require(lse, "lse", dev)
        if lse.shape != (B, H, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, H, Tq]")
    _call("attn_splitkv_fwd", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), B, H, Tq, S, D, scale, _dtype_code(q),
          int(chunk), _ptr(part_out), _ptr(part_lse), _ptr(counters), _ptr(out), _ptr(lse),
          _stream(dev))
    return out, lse

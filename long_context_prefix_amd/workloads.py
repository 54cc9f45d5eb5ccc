"""Seeded synthetic inputs shaped like the pages' attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it without sharing any of the method's code.

Recipe (same for every workload):
  * ``kv_len`` is drawn first, on the host, with ``numpy.random.default_rng(seed)``;
  * then q, k, v are drawn as fp32 standard normals from a torch generator seeded
    with ``seed`` on the target device, multiplied by ``sigma`` in fp32 and
    rounded to the storage dtype (round-to-nearest-even for bf16);
  * then every padded key slot j >= kv_len[b] of k and v is overwritten with
    +-``pad`` (random sign, magnitude 1e4 by default; stored in bf16 as +-9984),
    or with NaN when ``pad`` is NaN.  The pads exist to show that they are never
    read: they must not change any result.
Large workloads are drawn one batch element at a time with seed ``seed + 1 + b``
so that one sequence can be regenerated alone.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "sample_rows", "ragged_kv_len"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    Tq: int
    S: int
    kv_len: tuple  # one entry per batch element, or () for the ragged draw
    dtype: str  # "bf16" or "f32"
    sigma: float
    seed: int
    chunk: int = 0  # split-KV chunk (keys); 0 when the workload uses the fused call
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def lens(self) -> np.ndarray:
        if self.kv_len:
            return np.asarray(self.kv_len, dtype=np.int32)
        return ragged_kv_len(self.seed, self.B, self.S)


def ragged_kv_len(seed: int, batch: int, s_slots: int) -> np.ndarray:
    """Per-element prefix lengths drawn uniformly in [1, S], forcing 1 and S in."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, s_slots + 1, size=batch).astype(np.int32)
    lens[0] = 1
    lens[-1] = s_slots
    return lens


_R2 = 1.0 / math.sqrt(2.0)

# The five workloads: a tiny fp32 prefix-mask check, ICL blocks at 16k and 121k
# context rows (head dim 256), a ragged packed batch, and the column
# set-transformer's inducing attention split into 4,096-key chunks.
WORKLOADS = {
    "tiny_prefix_mask": Workload("tiny_prefix_mask", 1, 2, 64, 256, 256, (200,), "f32", 1.0, 1001,
                                 note="fp32, n=200 of S=256"),
    "icl_16k": Workload("icl_16k", 1, 8, 256, 20480, 16384, (16384,), "bf16", _R2, 1002,
                        note="16,384 context keys, 20,480 query rows"),
    "ragged_32k": Workload("ragged_32k", 8, 8, 128, 32768, 32768, (), "bf16", 1.0, 1003,
                           note="n_b ~ U[1, 32768] with 1 and S forced"),
    "inducing_splitkv": Workload("inducing_splitkv", 160, 4, 128, 128, 102400, (100000,) * 160, "bf16",
                                 1.0, 1004, chunk=4096, note="160 sequences, 4,096-key chunks"),
    "icl_121k": Workload("icl_121k", 1, 8, 256, 131072, 131072, (121000,), "bf16", _R2, 1005,
                         note="121,000 valid keys of 131,072 slots"),
}


def _torch_dtype(dtype: str):
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _fill_normal(t: torch.Tensor, gen: torch.Generator, sigma: float) -> None:
    tmp = torch.empty(t.shape, dtype=torch.float32, device=t.device)
    tmp.normal_(0.0, 1.0, generator=gen)
    if sigma != 1.0:
        tmp.mul_(np.float32(sigma).item())
    t.copy_(tmp)  # fp32 -> storage dtype, round to nearest even


def _fill_pads(k: torch.Tensor, v: torch.Tensor, lens, gen: torch.Generator, pad: float) -> None:
    s_slots = k.shape[2]
    for b, n in enumerate(lens):
        n = int(n)
        if n >= s_slots:
            continue
        for t in (k, v):
            region = t[b, :, n:, :]
            if math.isnan(pad):
                region.fill_(float("nan"))
            else:
                sign = torch.randint(0, 2, region.shape, generator=gen, device=t.device, dtype=torch.int8)
                region.copy_((sign.to(torch.float32) * 2.0 - 1.0) * pad)


def make_inputs(B: int, H: int, Tq: int, S: int, D: int, kv_len, dtype: str = "bf16", sigma: float = 1.0,
                seed: int = 0, device="cpu", pad: float = 1e4, per_sequence: bool = False):
    """Draw (q, k, v, kv_len) for one case; see the module docstring for the recipe.

    Returns q [B,H,Tq,D], k/v [B,H,S,D] in ``dtype`` and kv_len int32 [B], all on
    ``device``.  ``per_sequence`` draws each batch element from its own generator
    (seed + 1 + b) so huge batches never need an fp32 copy of the whole tensor.
    """
    lens = np.asarray(kv_len, dtype=np.int32).reshape(-1)
    assert lens.shape[0] == B
    tdt = _torch_dtype(dtype)
    dev = torch.device(device)
    q = torch.empty((B, H, Tq, D), dtype=tdt, device=dev)
    k = torch.empty((B, H, S, D), dtype=tdt, device=dev)
    v = torch.empty((B, H, S, D), dtype=tdt, device=dev)
    if per_sequence:
        for b in range(B):
            gen = torch.Generator(device=dev)
            gen.manual_seed(seed + 1 + b)
            for t in (q, k, v):
                _fill_normal(t[b], gen, sigma)
            _fill_pads(k[b:b + 1], v[b:b + 1], lens[b:b + 1], gen, pad)
    else:
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        for t in (q, k, v):
            _fill_normal(t, gen, sigma)
        _fill_pads(k, v, lens, gen, pad)
    return q, k, v, torch.from_numpy(lens.copy()).to(dev)


def make_workload(w: Workload, device="cpu", pad: float = 1e4):
    """Inputs of a named workload (per-sequence drawing for batches above 8)."""
    return make_inputs(w.B, w.H, w.Tq, w.S, w.D, w.lens(), w.dtype, w.sigma, w.seed, device, pad,
                       per_sequence=w.B > 8)


def sample_rows(seed: int, Tq: int, count: int, groups: int) -> np.ndarray:
    """Sorted query-row samples, one set per (b, h) group, always holding 0 and Tq-1."""
    rng = np.random.default_rng(seed + 7919)
    count = min(count, Tq)
    rows = np.empty((groups, count), dtype=np.int64)
    for g in range(groups):
        if count == Tq:
            rows[g] = np.arange(Tq)
            continue
        pick = rng.choice(np.arange(1, Tq - 1), size=count - 2, replace=False) if count > 2 else np.array([], np.int64)
        rows[g] = np.sort(np.concatenate([[0, Tq - 1], pick]))[:count]
    return rows

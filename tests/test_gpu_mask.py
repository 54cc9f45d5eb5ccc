"""Device-side prefix-mask detection and the SDPA-style entry, against the oracle.

``attn_prefix_mask_to_kv_len`` must agree bit for bit with
``oracle.ref_prefix_mask_to_kv_len`` (lengths, and -1 for rows that are not
prefix masks) over row lengths that exercise the aligned 16-byte body, the
unaligned head and the tail, strided and broadcast row layouts, and uint8 masks
with values other than 1.  ``sdpa_prefix`` must match the fp64 attention oracle
on the lengths the mask implies and refuse any mask that is not a prefix.
"""

import math

import numpy as np
import pytest
import torch

from long_context_prefix_amd import _lib, kv_len_from_prefix_mask, sdpa_prefix
from long_context_prefix_amd.workloads import make_inputs
from oracle import ref_prefix_fwd, ref_prefix_mask_to_kv_len
from tests.parity import assert_parity, log, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _mask_rows(S, rng):
    """Row patterns: prefixes of every interesting length, holes, late Trues."""
    rows = []
    for n in sorted({0, 1, 15, 16, 17, S // 2, S - 1, S} & set(range(S + 1))):
        r = np.zeros(S, dtype=bool)
        r[:n] = True
        rows.append(r)
    for _ in range(4):
        n = int(rng.integers(0, S + 1))
        r = np.zeros(S, dtype=bool)
        r[:n] = True
        rows.append(r)
        if n >= 2:  # a hole inside the prefix
            h = r.copy()
            h[int(rng.integers(0, n - 1))] = False
            rows.append(h)
        if n < S:  # a True after the first False
            t = r.copy()
            t[int(rng.integers(n, S))] = True
            rows.append(t)
    if S >= 1:
        last = np.zeros(S, dtype=bool)
        last[-1] = True
        rows.append(last)
        first_off = np.ones(S, dtype=bool)
        first_off[0] = False
        rows.append(first_off)
    return np.stack(rows) if rows else np.zeros((1, 0), dtype=bool)


@pytest.mark.parametrize("S", [0, 1, 7, 15, 16, 17, 31, 64, 255, 4097, 121_000])
def test_mask_lengths_match_oracle(S):
    rng = np.random.default_rng(7000 + S)
    rows = _mask_rows(S, rng)
    log(f"mask S={S} rows={rows.shape[0]}")
    want = ref_prefix_mask_to_kv_len(rows)
    m = torch.from_numpy(rows).to(DEV)
    got = _lib.attn_prefix_mask_to_kv_len(m.view(rows.shape[0], 1, 1, S))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("offset", [0, 1, 5, 13])
def test_mask_strided_and_misaligned_rows(offset):
    """Rows taken from a wider buffer at odd offsets: every row has its own alignment."""
    rng = np.random.default_rng(7100 + offset)
    S, B, width = 1000, 24, 1037
    rows = _mask_rows(S, rng)[:B]
    B = rows.shape[0]
    buf = torch.zeros(B, width, dtype=torch.uint8, device=DEV)
    buf[:, offset:offset + S] = torch.from_numpy(rows.astype(np.uint8) * 9).to(DEV)  # nonzero != 1
    view = buf[:, offset:offset + S]
    log(f"mask strided offset={offset} stride={view.stride(0)}")
    got = _lib.attn_prefix_mask_to_kv_len(view)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy().astype(np.int64), ref_prefix_mask_to_kv_len(rows))


def test_mask_broadcast_row():
    """A batch stride of 0 (one row expanded over the batch) repeats that row's answer."""
    row = torch.zeros(1, 1, 1, 300, dtype=torch.bool, device=DEV)
    row[..., :123] = True
    m = row.expand(5, 1, 1, 300)
    assert m.stride(0) == 0
    got = _lib.attn_prefix_mask_to_kv_len(m)
    torch.cuda.synchronize()
    assert got.cpu().tolist() == [123] * 5


def test_sdpa_prefix_matches_oracle():
    B, H, Tq, S, D = 4, 2, 150, 700, 128
    lens = [0, 1, 333, 700]
    log("sdpa_prefix ragged")
    q, k, v, _ = make_inputs(B, H, Tq, S, D, lens, "bf16", 1.0, seed=7200, device=DEV)
    mask = torch.zeros(B, 1, 1, S, dtype=torch.bool, device=DEV)
    for b, n in enumerate(lens):
        mask[b, ..., :n] = True
    out = sdpa_prefix(q, k, v, mask)
    torch.cuda.synchronize()
    ro, rl = ref_prefix_fwd(to64(q), to64(k), to64(v), np.array(lens), 1.0 / math.sqrt(D))
    assert_parity(out, None, ro, None, "bf16", "sdpa_prefix")
    assert kv_len_from_prefix_mask(mask).cpu().tolist() == lens


def test_sdpa_prefix_refuses_non_prefix_masks():
    B, H, Tq, S, D = 2, 1, 4, 64, 64
    q = torch.zeros(B, H, Tq, D, dtype=torch.bfloat16, device=DEV)
    mask = torch.ones(B, 1, 1, S, dtype=torch.bool, device=DEV)
    mask[1, ..., 10] = False  # a hole
    with pytest.raises(ValueError, match=r"\[1\]"):
        sdpa_prefix(q, q.new_zeros(B, H, S, D), q.new_zeros(B, H, S, D), mask)

"""Closed-form memory footprints that the fused kernels avoid (host logic).

* ``unfused_score_bytes``: the [T_q, T_src] score matrix per head that an
  unfused (math-backend) attention would hold for one layer, as the page
  "Rewrite prefix key-padding masks as k/v truncation to keep SDPA on the flash
  path (PyTorch)" computes it in its sections Problem and Measured.
* ``mask_copy_bytes``: a dense per-head [N, N] mask copy, as tabulated on the
  page "Broadcast SDPA attn_mask instead of materializing a per-head copy"
  (section Why).  The kernels here take one length per batch element instead.
"""


def unfused_score_bytes(t_q: int, t_src: int, heads: int, elem_bytes: int) -> int:
    return t_q * t_src * heads * elem_bytes


def mask_copy_bytes(n_tokens: int, heads: int, elem_bytes: int) -> int:
    return n_tokens * n_tokens * heads * elem_bytes


def splitkv_partial_bytes(batch: int, heads: int, chunks: int, t_q: int, d: int) -> int:
    """fp32 partial outputs plus fp32 LSE statistics for the split-KV path."""
    return batch * heads * chunks * t_q * (d + 1) * 4

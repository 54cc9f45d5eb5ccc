"""Prefix-masked and split-KV attention for MI355X (gfx950).

The public calls mirror the C ABI of ``libattnprefix.so``:

* ``attn_prefix_fwd(q, k, v, kv_len, scale)`` -- fused attention where batch
  element b attends only to its first ``kv_len[b]`` keys;
* ``attn_splitkv_partial(q, k, v, kv_len, chunk, scale)`` -- fp32 partials
  over fixed key chunks;
* ``attn_lse_combine(part_out, part_lse)`` -- their exact log-sum-exp merge;
* ``attn_splitkv_fwd(q, k, v, kv_len, chunk)`` -- both in one launch (the last
  chunk to finish merges);
* ``attn_prefix_mask_to_kv_len(mask)`` / ``sdpa_prefix(q, k, v, attn_mask)`` --
  a [B, 1, 1, S] boolean prefix mask turned into lengths on the device, and an
  SDPA-style entry that raises on any other mask;
* ``attn_prefix_bwd(...)`` / ``prefix_attention(q, k, v, kv_len)`` -- the
  gradients, and a differentiable wrapper for training on ragged batches;
  ``attn_prefix_bwd_noalloc(...)`` computes them with no workspace argument and
  no allocation, for callers that cannot allocate.

The library is loaded on first use; a missing build raises instead of falling
back to anything else.
"""

from ._lib import (  # noqa: F401
    AttnError,
    attn_lse_combine,
    attn_prefix_bwd,
    attn_prefix_bwd_noalloc,
    attn_prefix_fwd,
    attn_prefix_mask_to_kv_len,
    attn_splitkv_fwd,
    attn_splitkv_num_chunks,
    attn_splitkv_partial,
    kv_len_from_prefix_mask,
    load,
    prefix_attention,
    sdpa_prefix,
    splitkv_fwd,
    status_string,
)

__version__ = "0.2.0"

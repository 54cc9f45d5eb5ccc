"""Prefix-masked and split-KV attention for MI355X (gfx950).

The public calls mirror the C ABI of ``libattnprefix.so``:

* ``attn_prefix_fwd(q, k, v, kv_len, scale)`` -- fused attention where batch
  element b attends only to its first ``kv_len[b]`` keys;
* ``attn_splitkv_partial(q, k, v, kv_len, chunk, scale)`` -- fp32 partials
  over fixed key chunks;
* ``attn_lse_combine(part_out, part_lse)`` -- their exact log-sum-exp merge.

The library is loaded on first use; a missing build raises instead of falling
back to anything else.
"""

from ._lib import (  # noqa: F401
    AttnError,
    attn_lse_combine,
    attn_prefix_fwd,
    attn_splitkv_num_chunks,
    attn_splitkv_partial,
    load,
    splitkv_fwd,
    status_string,
)

__version__ = "0.1.0"

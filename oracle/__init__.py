"""fp64 CPU oracle for prefix-masked and split-KV attention.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import it.  The product library never does.
"""

from .attn_oracle import (  # noqa: F401
    brute_force,
    num_chunks,
    ref_lse_combine,
    ref_prefix_bwd,
    ref_prefix_mask_to_kv_len,
    ref_prefix_fwd,
    ref_splitkv_partial,
    scale64,
)

"""fp64 CPU oracle for sparse self-speculative decode attention.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  The HIP library never calls into it.
"""
from .sss_oracle import (  # noqa: F401
    attention_partial,
    block_mass_unit,
    block_topk,
    draft,
    draft_token_set,
    gather_unit,
    kv_commit,
    kv_write,
    layout_union,
    merge,
    sparse_verify,
    sparse_verify_token_set,
    topk_unit,
    verify,
    verify_unit,
    verify_with_scores,
    window_start,
)

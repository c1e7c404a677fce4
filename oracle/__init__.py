"""CPU oracle for the H-Spec drafter layer — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 NumPy statement of what the drafter
layer computes.  It exists to check the HIP path, and nothing else may use it:
only tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py
import it.  The product path (the C-ABI library and its Python binding) never
imports, calls or falls back to anything here, and this package never imports
the product package.

Sources:
  * "H-Spec: Parallel Speculative Decoding Without a Drafter-Side KV Cache",
    Abstract, and the review page's Summary: Mamba modules start from a
    projection of the target's last-token hidden state; attention modules read
    the target's KV cache in place with no drafter-side cache; Mamba's parallel
    scan keeps drafting block-parallel.
  * Mamba-2 (Dao & Gu, 2024, "Transformers are SSMs"), the SSD recurrence and
    its chunked form, for the scan arithmetic the pages name but do not print,
    and the Mamba-2 block around the scan (projections, short convolution,
    gated normalisation).

Every function below is pinned by tests/test_oracle_*.py against closed forms,
brute force, library routines or hand-derived golden values.  The layer's
end-to-end quality figures on the pages need trained weights and stay
"parity unpinned" (nothing here claims them).
"""
from .numerics import decode, BF16, F32
from .init_state import init_state
from .ssd import ssd_recurrence, ssd_chunked
from .attention import (PoisonedRead, gather_context, block_attention,
                        block_attention_ranges, split_partials, merge_partials, key_index)
from .plan import (range_plan, plan_len, range_count, request_granules, request_pieces, segment_granules,
                   granule_slabs)
from .layer import draft_layer
from .mamba_block import (mamba_block, causal_conv, gated_rmsnorm, silu, softplus,
                          in_proj_sizes)
from .kv_inject import kv_project, kv_inject, extra_kv_bytes_per_token
from .stack import stack_forward, rmsnorm

__all__ = [
    "decode", "BF16", "F32", "init_state", "ssd_recurrence", "ssd_chunked",
    "PoisonedRead", "gather_context", "block_attention", "block_attention_ranges",
    "split_partials", "merge_partials", "key_index", "range_plan", "plan_len", "range_count", "segment_granules",
    "request_granules", "request_pieces", "granule_slabs",
    "draft_layer", "mamba_block", "causal_conv", "gated_rmsnorm", "silu", "softplus",
    "in_proj_sizes", "kv_project", "kv_inject", "extra_kv_bytes_per_token", "stack_forward",
    "rmsnorm",
]

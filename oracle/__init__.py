"""fp64 CPU oracle for exact attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never does, and the oracle imports
nothing from the library.
"""
from .attention import (  # noqa: F401
    MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT,
    MOD_NONE, MOD_ALIBI, MOD_SOFTCAP, MOD_LOCAL_BOOST, MOD_REL_BIAS,
    TILE_EMPTY, TILE_PARTIAL, TILE_FULL,
    Variant, default_alibi_slopes, kv_head, allowed, modify, modify_grad,
    forward, probabilities, backward_head, backward, loss, rel_index, rel_bias_grad,
    count_pairs, tile_states, logsumexp_row_fsum,
)

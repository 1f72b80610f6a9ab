"""CPU oracle for the Skip-Softmax (BLASST) FlashAttention forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may use this package; the library and its Python binding never do.
It is plain numpy in float64 (the skip vote in float32, the kernel's
precision), plus the same method in plain C (c_oracle: softmax attention in
double precision and the tiled recurrence in single precision, built with
gcc on first use).  Neither shares code with the HIP path.
"""
from . import c_oracle  # noqa: F401
from . import fp8  # noqa: F401
from .skip_attention import (  # noqa: F401
    BLOCK_K,
    BLOCK_Q,
    HeadResult,
    SkipResult,
    dense_attention,
    dense_head,
    from_bf16,
    lambda_for_skip_fraction,
    ln_lambda_f32,
    masked_dense_head,
    prefix_max_margins_head,
    resolve_lambda,
    skip_attention,
    skip_attention_varlen,
    skip_head,
    skip_mask_from_row_maxima,
    skipped_mass_head,
    tile_row_maxima_head,
    max_prob_head,
    virtual_tile_head,
)

"""CPU oracle of the block-draft readout hot path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
CPU-baseline leg of the benchmark may import this package.  The product (the HIP
library and its Python binding) never imports, calls or links it, and this
package imports nothing from the product.

See ``oracle.reference`` for the definitions and the pages each one follows.
"""
from .reference import (  # noqa: F401
    widen, round_to_f32, f32_to_bf16_bits, fuse_fc, lm_head, markov_bias,
    semi_ar_argmax, score_draft, first_argmax, top2_gap, target_argmax, truncate_by_confidence,
    verify_greedy, mean_acceptance_length, drafted_token_rate, block_step,
)

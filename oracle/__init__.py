"""CPU oracle for the activation-sparse ReLU FFN decode step (test infrastructure).

This package is test infrastructure.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it.  The GPU library never calls it;
the two share no code.  Everything here is plain numpy in float64, written to
be read against the PowerInfer pages, not to be fast.

Parity status: every function is pinned by CPU tests against values fixed
independently of this code (hand-derived worked examples, exact rational
brute force on tiny layers, special cases that reduce to a textbook routine,
invariants of the definition, and the floating-point error bound).
"""

from .ffn import (  # noqa: F401
    GUARD_SAFETY,
    activations,
    certain_union,
    compact,
    dense_weights,
    dequant_q4g32,
    down_projection,
    exact_mask,
    forward,
    forward_masked,
    gamma,
    guard_band_exact,
    guard_band_predictor,
    hot_mask,
    pre_activations,
    prob_band_exact,
    prob_band_predictor,
    PROB_LAMBDA,
    predictor_hidden,
    predictor_logits,
    predicted_mask,
    round_to_act,
    threshold_logit,
    union_mask,
)

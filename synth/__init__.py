"""Seeded synthetic inputs for the activation-sparse ReLU FFN decode step.

This package only *produces data*: layer weights, predictor weights, biases,
token inputs and the int4 packed encoding of weights.  It computes no part of
the FFN, the predictor, the mask or the down projection.  Both the CPU oracle
(through the tests) and the GPU library (through the tests and the benchmark)
are fed from here; neither side imports the other.
"""

from .configs import CONFIGS, LayerConfig, config_by_name  # noqa: F401
from .layers import (  # noqa: F401
    Layer,
    firing_probs,
    make_layer,
    make_tokens,
    make_lattice_layer,
    make_lattice_tokens,
    quantize_q4g32,
    pack_nibbles,
)

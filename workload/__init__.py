"""Seeded synthetic inputs for the predictor-gated sparse FFN.

This module only *draws* inputs: weights, biases chosen so that neurons fire
with a Zipf-shaped probability profile, decode tokens and Bernoulli masks.  It
holds none of the method's arithmetic (no predictor, threshold, compaction,
gather or reduction), so both the HIP path and the CPU oracle may be fed from
it without sharing any computation.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    layer_seed,
    zipf_profile,
    make_layer,
    make_tokens,
    bernoulli_mask,
    q4_0_pack,
    q4_0_quantize,
)

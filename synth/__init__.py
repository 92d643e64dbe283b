"""Seeded synthetic inputs shared by the oracle side and the HIP side of every test.

This package holds workload generation only (shapes, random weights, calibrated biases,
tokens, integer fixtures). It contains none of the decode method's arithmetic: no
prediction, thresholding, compaction or FFN evaluation happens here. Both sides of a parity
test receive the exact bytes produced here.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    Layer, integer_layer, layer_activity_target, make_layer, make_tokens, zipf_targets,
    seed_for,
)

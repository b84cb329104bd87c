"""Seeded synthetic inputs for the LatentMoE layer.

This package is shared by the oracle (``oracle/``) and by the GPU-side tests
and benchmark.  It draws random numbers and nothing else: it holds none of the
layer's arithmetic (no quantisation, no routing, no matmul).
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    config,
    gen_hidden,
    gen_logit_bias,
    gen_router,
    gen_selection_bias,
    gen_weight,
    n_matrices,
    weight_shape,
    WEIGHT_NAMES,
)

"""Seeded synthetic inputs and workload shapes, shared by tests and benchmark.

This package holds no part of the method's arithmetic: it only names the
workload shapes and draws Gaussian inputs from seeded generators.  Both the
oracle side and the HIP side of a parity test receive the same arrays from it.
"""

from .configs import LayerConfig, CONFIGS, config  # noqa: F401
from .generators import (  # noqa: F401
    layer_weights, chunk_x, chunk_q, dense_weights, block_weights, to_storage_tensor,
)

"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package holds input generators and the workload registry only: it contains none of the
quantization arithmetic, and it imports neither the oracle nor the HIP package.
"""

from .layers import (  # noqa: F401
    CONFIGS,
    MatrixSpec,
    QuantConfig,
    activation_chunks,
    config,
    make_activations,
    make_weight,
    seed_for,
)

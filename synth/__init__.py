"""Seeded synthetic workloads (inputs only) shared by the oracle tests, the GPU
tests and the benchmark."""
from .configs import CONFIGS, BY_NAME, HEADLINE, LayerConfig, HEAD_TYPES  # noqa: F401
from .workload import LayerGen, head_types  # noqa: F401

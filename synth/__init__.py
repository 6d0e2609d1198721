"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark."""
from .configs import WORKLOADS, SparsePRConfig, get_config, with_overrides  # noqa: F401
from .generate import make_qkv, as_f64, planted_clusters  # noqa: F401

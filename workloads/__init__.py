"""Seeded synthetic inputs shared by the tests and the benchmark (random draws only)."""
from .gen import CONFIGS, Config, routing, activations, weights, expert_counts, bf16_to_f32  # noqa: F401

"""Seeded synthetic workloads for the speculative-decoding verification step.

This package only draws inputs (queries, KV caches, draft trees, logits, draft
distributions, uniforms).  It holds none of the verification arithmetic and is
the one piece shared by the fp64 oracle tests, the GPU parity tests and the
benchmark.
"""
from .configs import CONFIGS, config, scaled
from .gen import Workload, generate, bf16_bits, bf16_to_f32

__all__ = ["CONFIGS", "config", "scaled", "Workload", "generate", "bf16_bits", "bf16_to_f32"]

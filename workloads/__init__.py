"""Seeded synthetic inputs for one draft-tree step.

This module stands in for the models and datasets of the pages (the drafter, the
target model, the benchmark prompts), which do not exist here. It produces plain
arrays only: logit tables, query/key/value tensors, random tree shapes, spine tokens
and the uniforms a sampler consumes. It holds none of the method's arithmetic (no
tree building, no scoring, no attention, no verification); both the CPU oracle and
the GPU path receive the same arrays from here.

Every array is drawn from ``np.random.default_rng(SeedSequence([seed, stream, idx]))``
so that any single row can be regenerated on its own. Normals are drawn in float32,
scaled, and stored as bf16 (round to nearest even) for the bf16 configurations.
"""
from .configs import (CONFIGS, config_by_name, Workload, make_workload, make_step_inputs, step_seed,
                      bf16_bits_to_f32, f32_to_bf16_bits)

__all__ = ["CONFIGS", "config_by_name", "Workload", "make_workload", "make_step_inputs", "step_seed",
           "bf16_bits_to_f32", "f32_to_bf16_bits"]

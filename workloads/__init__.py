"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .synth import (CONFIGS, Workload, WorkloadSpec, bf16_bits_to_f32, f32_to_bf16_bits, gen_group,
                    make_workload, spec, to_f32)

__all__ = ["CONFIGS", "Workload", "WorkloadSpec", "bf16_bits_to_f32", "f32_to_bf16_bits", "gen_group",
           "make_workload", "spec", "to_f32"]

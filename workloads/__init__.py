"""Seeded synthetic workloads (random draws and dtype rounding only)."""

from .inputs import (CONFIGS, DECODE_CONFIG, PRECOND_ETA, DecodeWorkload, Workload, bf16_round, chunk_inputs,
                     decode_inputs, decode_slice, grad_inputs, grad_slice, precond_factors, precond_inputs, precond_slice, round_to_io,
                     slice_inputs)

__all__ = ["CONFIGS", "DECODE_CONFIG", "DecodeWorkload", "Workload", "bf16_round", "chunk_inputs",
           "decode_inputs", "decode_slice", "grad_inputs", "grad_slice", "PRECOND_ETA", "precond_factors", "precond_inputs", "precond_slice", "round_to_io",
           "slice_inputs"]

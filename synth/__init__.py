"""Seeded synthetic inputs shaped like the Muon workloads.

This module holds no arithmetic of the method: it only draws random numbers
(NumPy PCG64 streams keyed by (workload, layer, kind, step)) and rounds them
to the stored dtype.  Both the HIP path's tests/benchmark and the CPU oracle
take their inputs from here, so they see identical bytes.

bfloat16 tensors are returned as uint16 bit patterns; float32 tensors as
float32 arrays.  N(0, s) means standard deviation s.
"""

from synth.workloads import (  # noqa: F401
    TensorSpec, Workload, rng_for, to_bf16_bits, bf16_bits_to_f32,
    workload, WORKLOADS, gradient, momentum0, weight, activations,
)

"""Seeded synthetic inputs for the RMA hot path.

This package draws every input that the tests, the benchmark and the smoke
check feed to both the HIP library and the float64 oracle.  It holds no step
of the method itself: no normalisation, rotation, attention, scoring or
selection.  It only produces bytes.

Two generators are used:

* A counter-based generator for the large BF16 tensors (K/V state, hidden
  states, queries).  Element ``i`` of a tensor with stream key ``(k1, k2)`` is
  ``TABLE[mix32(mix32(i + k1) ^ k2) >> 16]``, where ``mix32`` is a 32-bit
  integer mixer (the "lowbias32" finaliser: xor-shift 16, multiply
  0x7feb352d, xor-shift 15, multiply 0x846ca68b, xor-shift 16) and ``TABLE``
  holds the BF16 bit patterns of the 65536 standard-normal quantiles
  ``Phi^-1((j + 0.5) / 65536)``.  It is implemented twice, once with NumPy on
  the host and once with torch integer ops on any device; both compute the
  same integers, so any slice can be regenerated bit-identically on the host
  while the full tensor is drawn directly in device memory.
* NumPy ``Generator(PCG64)`` streams for the small FP32 tensors (scorer
  weights, norm gains, anchor scores) and for the distinct source positions.
  These are drawn on the host and copied to the device.

Stream keys come from ``blake2b`` over the master seed and a tuple of names,
so every (workload, layer, tensor) has its own independent stream.
"""

from .core import (  # noqa: F401
    MASTER_SEED,
    StreamKey,
    stream_key,
    normal_bf16_table,
    normal_bf16_np,
    normal_bf16_at_np,
    normal_bf16_torch_,
    normal_f32_np,
    distinct_ints_np,
    rng_np,
    bf16_bits_to_f32_np,
)
from . import workloads  # noqa: F401

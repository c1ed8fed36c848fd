"""Seeded synthetic inputs shared by the GPU path's callers and the oracle's.

This module holds no attention, RoPE or ring arithmetic: it only draws
numbers and rounds them to the run dtype.  Both sides of a parity check read
the same arrays from here.

Recipe: every (workload, layer, kind, request) has its own stream,
numpy.random.default_rng([seed, workload_id, layer, kind, request]).  Values
are standard normals drawn in float64, multiplied by the workload's standard
deviation, cast to float32 (round to nearest even) and, for bf16 workloads,
rounded again to bf16 (round to nearest even).  The returned float32 arrays
hold exactly the bf16 values, so upcasting them to float64 is exact.
"""

from __future__ import annotations

import numpy as np

# stream kinds
Q_PREFILL, K_PREFILL, V_PREFILL, Q_DECODE, K_DECODE, V_DECODE = range(6)


def round_to_bf16(x) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw(seed: int, workload_id: int, layer: int, kind: int, request: int,
         shape, std: float, dtype: str) -> np.ndarray:
    """One seeded block of inputs, rounded to the run dtype (float32 array)."""
    rng = np.random.default_rng([seed, workload_id, layer, kind, request])
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")

"""Fixed Hadamard rotation of Q and K along the head dimension (CPU oracle; test infrastructure).

Sources: Pith review of MXAttention, Axiom & Free-Parameter Ledger (a fixed
orthogonal Hadamard rotation on Q/K is a calibration-free outlier suppressor,
section 4.3 / 5.4) and Figure 1 caption (the rotation is applied to Q/K);
10100.com explainer (the full scheme adds a Hadamard rotation on Q/K).

Readings (the pages give neither the normalisation nor the arithmetic):
  * H_d is the Sylvester matrix, H[i, j] = (-1)**popcount(i & j), and the
    rotation is orthonormal: y = x @ H_d / sqrt(d).
  * Because the quantiser's codes are integers decided from y, y is *defined*
    in fp32 so that a GPU can reproduce it bit for bit: convert to fp32
    (exact for bf16/fp32 inputs), run the fast Walsh-Hadamard butterflies for
    h = 1, 2, 4, ..., d/2 in that order, each pair (i, i + h) with i & h == 0
    becoming (a + b, a - b) in IEEE fp32 round-to-nearest-even, then multiply
    once by c = fl32(1 / sqrt(d)).  The plain definition x @ H / sqrt(d) in
    float64 pins this to within fp32 rounding (tests/test_oracle_hadamard.py).
"""
from __future__ import annotations

import math

import numpy as np


def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), integer entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    bits = np.bitwise_and.outer(i, i)
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(bits)
    return np.where(pop % 2 == 0, 1, -1).astype(np.int64)


def inv_sqrt_f32(d: int) -> np.float32:
    """c = fl32(1/sqrt(d)): the float64 value rounded once to fp32."""
    return np.float32(1.0 / math.sqrt(d))


def fwht_fp32(x) -> np.ndarray:
    """Orthonormal Hadamard rotation of the last axis, defined in fp32 (see module docstring)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("last axis must be a power of two")
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b          # float32 + float32 -> float32, one IEEE rounding
        v[..., 1, :] = a - b
        h *= 2
    return (y * inv_sqrt_f32(d)).astype(np.float32)


def rotate_f64(x) -> np.ndarray:
    """The plain definition y = x @ H / sqrt(d) in float64 (for pinning fwht_fp32)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return x @ sylvester(d).astype(np.float64) / math.sqrt(d)

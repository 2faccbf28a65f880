"""Oracle dequantisation of 4-bit group-64 substitute weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"SubSpec" summary (jjl357.github.io), section 4.1.1: the substitute draft
replaces each linear weight with a 4-bit group-64 affine code, weight =
(code - zero) * scale with per-group half-precision scale and zero.  The
group runs over 64 consecutive inputs of one output row; two codes share a
byte, the even input in the low nibble.
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> codes uint8 [N, K] (even index = low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    N, Kh = p.shape
    q = np.empty((N, 2 * Kh), dtype=np.uint8)
    q[:, 0::2] = p & 0x0F
    q[:, 1::2] = p >> 4
    return q


def dequantize(packed: np.ndarray, scale_f16: np.ndarray, zero_f16: np.ndarray) -> np.ndarray:
    """float64 [N, K] weights (code - zero) * scale."""
    q = unpack_codes(packed).astype(np.float64)
    N, K = q.shape
    s = np.asarray(scale_f16, dtype=np.float16).astype(np.float64)
    z = np.asarray(zero_f16, dtype=np.float16).astype(np.float64)
    q = q.reshape(N, K // GROUP, GROUP)
    return ((q - z[..., None]) * s[..., None]).reshape(N, K)

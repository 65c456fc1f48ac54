"""fp64 oracle of the 8-bit forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never touches it.

The pages name FP8 as FlashAttention-3's next step ("FlashAttention: Move
Less, Not Compute Less", section "FA1 to FA3") without fixing a format or a
quantisation.  The reading taken: each of q, k, v is stored as OCP FP8 E4M3
codes with one dequantisation factor per tensor, and the result is the
exact attention of the dequantised tensors (so the 8-bit path is checked
against the same definition as the 16-bit ones).

E4M3 as defined by the Open Compute Project 8-bit floating point
specification (OFP8): bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0
mantissa; exponent 0 encodes subnormals m/8 * 2^-6; exponent 15 with
mantissa 7 is NaN (there is no infinity); the largest finite value is
0x7E = 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

from .attention import naive_attention


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode E4M3 codes (uint8) to the exactly equal float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, out)


def attention_fp8(q_codes, k_codes, v_codes, q_descale, k_descale, v_descale, causal, scale, rows=None):
    """(O, L) of one head from E4M3 codes q [n, d], k, v [n, d]: the exact
    attention of q_descale * decode(q), k_descale * decode(k),
    v_descale * decode(v)."""
    q = e4m3_to_f64(q_codes) * float(q_descale)
    k = e4m3_to_f64(k_codes) * float(k_descale)
    v = e4m3_to_f64(v_codes) * float(v_descale)
    return naive_attention(q, k, v, causal, scale, rows=rows)

"""Bit-level decoders for the storage formats the decode-attention path reads.

TEST INFRASTRUCTURE ONLY: this module is part of the CPU oracle.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does.

Both decoders are written from the published format definitions, not from
any library's conversion routine, so that the tests can pin them against an
independent implementation (PyTorch's dtype casts):

* bfloat16 is the upper half of an IEEE-754 binary32 word (1 sign bit, 8
  exponent bits with bias 127, 7 stored mantissa bits).  Widening is exact:
  put the 16 bits in the high half of a 32-bit word.
* float8 e4m3fn is the OCP 8-bit format with 1 sign bit, 4 exponent bits
  (bias 7) and 3 mantissa bits, no infinities, subnormals at exponent 0, and
  one NaN pattern per sign (exponent and mantissa all ones).  Largest finite
  magnitude 448, smallest subnormal 2^-9.

The pages name the KV-cache data types: "bf16" or "fp8" (ATOM configuration
guide, "Master configuration (Config)" table, ``kv_cache_dtype``), and note
that gfx942-era kernels needed e4m3fn values normalised to the e4m3fnuz
variant (ATOM model operations guide, "Weight processing"); gfx950 uses the
OCP e4m3fn encoding directly, which is the one decoded here.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_bits_to_f64", "e4m3fn_value", "e4m3fn_table", "e4m3fn_bytes_to_f64"]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode raw bfloat16 bit patterns (any integer dtype, 16 significant
    bits) to float64.  Exact for every pattern, NaN payloads included up to
    NaN-ness."""
    u = np.asarray(bits).astype(np.uint32) & np.uint32(0xFFFF)
    with np.errstate(invalid="ignore"):          # NaN patterns widen to NaN
        return (u << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, from the format definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")          # the only NaN encoding (one per sign)
    if exp_field == 0:
        # subnormal: 0.mmm * 2^(1 - bias) = m/8 * 2^-6 = m * 2^-9
        return sign * man_field * 2.0 ** -9
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


_E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
_E4M3FN_TABLE.setflags(write=False)


def e4m3fn_table() -> np.ndarray:
    """All 256 e4m3fn codes decoded to float64 (read-only array)."""
    return _E4M3FN_TABLE


def e4m3fn_bytes_to_f64(codes) -> np.ndarray:
    """Decode an array of e4m3fn bytes to float64 by table lookup."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.astype(np.int64) & 0xFF
    return _E4M3FN_TABLE[c]

"""Plain CPU oracle for the paged KV-cache write (new tokens' K/V into the
block layout), with per-token fp8 quantisation.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg may import this module; the product
path never does, and it shares no code with the HIP path.

What it computes
----------------
The decode step writes the new tokens' K and V into the paged cache before
attention runs (ATOM model operations guide, "Multi-head attention
(attention_mha.py)", forward flow: RoPE + KV-cache write, then dispatch).
The guide's "KV cache operations" table names the two writes this oracle
defines: the standard write for a bf16 cache and the fp8 write with
per-token quantisation; its source-file list has a slot mapping that says
which KV slot each token is written to (``token_layout/slots.py``), and the
ROCm blog "Optimizing ATOM and vLLM-ATOM for High-Interactivity Inference"
("Attention Input Fusion") describes the fused form that calculates the fp8
scales and writes K/V straight into the paged cache.

For every new token ``t`` with slot ``s = slot_mapping[t]``:

* ``s < 0`` (a padding token) or ``s >= num_blocks * BS``: nothing is
  written (``BS`` = the block size, the cache's second dimension);
* otherwise block ``s // BS``, position ``s % BS`` receives, for each kv
  head ``h``:
    - bf16 cache: the token's bf16 row, bit for bit;
    - fp8 cache: ``a = max_d |x_d|`` over the row (x widened exactly to
      float32), ``scale = a / 448`` (1 when ``a == 0``), codes
      ``e4m3fn(clamp(x_d / scale, -448, 448))`` rounded to nearest, ties to
      even; ``scale`` goes to ``k_scale`` / ``v_scale[block, pos, h]``.

The pages give no formula for the per-token scale.  The one taken is the
absmax rule that maps the row's largest magnitude onto the format's largest
finite value, 448: the scale is the row's absolute maximum over 448, and
every element is divided by that stored scale, so that dequantisation
(code times scale) inverts exactly the step the code was taken from.  Both
divisions are correctly rounded IEEE float32 divisions (gradual underflow
included), the precision in which the quantised code is decided.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_table

__all__ = ["FP8_MAX", "e4m3fn_encode", "quantize_rows_e4m3fn", "reshape_and_cache"]

FP8_MAX = 448.0

# The finite non-negative e4m3fn values in code order (codes 0x00 .. 0x7E):
# the encoding is monotone for non-negative codes, so neighbouring codes are
# neighbouring values.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3fn_table()[:0x7F].copy()


def e4m3fn_encode(y) -> np.ndarray:
    """Round float values (|y| <= 448, no NaN) to the nearest e4m3fn code,
    ties to the even code; the sign is kept (negative values that round to
    zero give -0, code 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(y).any() or (np.abs(y) > FP8_MAX).any():
        raise ValueError("e4m3fn_encode takes finite values within +-448")
    mag = np.abs(y)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")           # first value >= mag
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(mag == _POS_VALUES[hi], _POS_CODES[hi], code)  # exact hits
    sign = np.signbit(y).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_rows_e4m3fn(x) -> tuple:
    """Per-row absmax quantisation of float32 rows ``x[..., D]`` to e4m3fn:
    returns (codes uint8 [..., D], scales float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    nonzero = amax > 0
    scale = np.where(nonzero, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return e4m3fn_encode(y), scale


def reshape_and_cache(k_new_bits, v_new_bits, slot_mapping, k_cache, v_cache,
                      k_scale=None, v_scale=None, kv_dtype: str = "bf16"):
    """The cache write on host copies.

    ``k_new_bits`` / ``v_new_bits``: bf16 bit patterns ``[T, Hkv, D]``;
    ``slot_mapping``: ``[T]`` integers; ``k_cache`` / ``v_cache``: uint16
    (bf16 bits) or uint8 (e4m3fn) ``[NB, BS, Hkv, D]``; ``k_scale`` /
    ``v_scale``: float32 ``[NB, BS, Hkv]`` for an fp8 cache.  Returns new
    arrays ``(k_cache, v_cache, k_scale, v_scale)``; the inputs are not
    modified.
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, dtype=np.float32, copy=True)
    vs = None if v_scale is None else np.array(v_scale, dtype=np.float32, copy=True)
    nb, bs = kc.shape[0], kc.shape[1]
    fp8 = kv_dtype == "fp8_e4m3fn"
    slots = np.asarray(slot_mapping).astype(np.int64)
    for t, s in enumerate(slots):
        if s < 0 or s >= nb * bs:
            continue
        blk, pos = int(s // bs), int(s % bs)
        for src, cache, sc in ((k_new_bits, kc, ks), (v_new_bits, vc, vs)):
            row = np.asarray(src[t])                                   # [Hkv, D] bf16 bits
            if fp8:
                codes, scale = quantize_rows_e4m3fn(bf16_bits_to_f64(row).astype(np.float32))
                cache[blk, pos] = codes
                sc[blk, pos] = scale
            else:
                cache[blk, pos] = row.astype(cache.dtype)
    return kc, vc, ks, vs

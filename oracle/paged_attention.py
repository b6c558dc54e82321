"""Plain, slow, obviously correct CPU oracle for paged-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP path, and nothing on the product path calls it.

What it computes (float64 throughout)
-------------------------------------
For every sequence ``b`` with ``n = query_lens[b]`` new query tokens and
``L = context_lens[b]`` tokens in the cache (the ``n`` new tokens included,
because the cache write precedes the attention call: ATOM model operations
guide, "Multi-head attention (attention_mha.py)", forward flow: RoPE + KV
cache write, then dispatch), every query row ``t < n`` sits at sequence
position ``pos = L - n + t`` and every query head ``h`` reads KV head
``g = h // G`` with ``G = Hq // Hkv`` (contiguous grouping; the same
``q_heads / kv_heads`` ratio that the model operations guide's paged-kernel
envelope table multiplies into the query group):

    key j (lo <= j <= pos) lives in physical block  bt[b, j // BS],
                                    slot            j % BS
    k_j  = K[blk, slot, g, :] * (k_scale[blk, slot, g]  if fp8 else 1)
    v_j  = V[blk, slot, g, :] * (v_scale[blk, slot, g]  if fp8 else 1)
    x_j  = scale * <q[b, t, h, :], k_j>
    out[b, t, h, :] = sum_j exp(x_j) v_j / (sum_j exp(x_j) + exp(sink_h))

with ``lo = 0`` and no ``exp(sink_h)`` term by default.  Two options that
the model operations guide's decode dispatch names ("Attention
operations": the sliding-window condition of the Triton decode path) and
that the landing page's model table lists for GPT-OSS ("Sliding window +
attention sinks") change this; the pages give neither a formula, so the
readings taken are the common ones:

* sliding window ``w >= 1``: row ``t`` sees the ``w`` most recent
  positions up to its own, ``lo = max(0, pos - w + 1)``; ``w <= 0`` or
  ``None`` is no window (the dispatch's ``-1``);
* attention sinks: one logit ``sink_h`` per query head, in the units of
  ``x`` (after the softmax scale), that joins the softmax normaliser and
  carries no value; ``-inf`` turns a head's sink off.

This is the plain definition of softmax attention over a block-table
addressed cache; the split-context / log-sum-exp method that the ROCm blog
"Optimizing ATOM and vLLM-ATOM for High-Interactivity Inference" describes
("Attention Decode: Split Memory Work to Fill the Device") reaches the same
result up to rounding order, so the oracle is the definition itself, with a
library matmul as the only primitive.

Storage conventions (the pages fix the block size and the dtypes, not a byte
layout; these are the readings taken):

* block size ``BS`` = the cache's second dimension: 16 by default (ATOM
  configuration guide, "Master configuration (Config)",
  ``kv_cache_block_size``: a multiple of 16, or exactly 1); token j of a
  sequence is slot ``j % BS`` of physical block ``bt[b, j // BS]``;
* caches logically ``[num_blocks, BS, kv_heads, head_dim]``, bf16 bit
  patterns (uint16) or OCP e4m3fn bytes (uint8) ("bf16" / "fp8",
  ``kv_cache_dtype`` in the same table);
* fp8 caches carry one float32 scale per (block, slot, kv head), i.e. per
  token and head, logically ``[num_blocks, BS, kv_heads]`` (the k/v caches
  "and scales" of ``KVCacheConfig`` in the configuration guide's
  "Quick reference"; per-token quantised writes in the model operations
  guide, "KV cache operations");
* ``q`` is bf16 bits ``[B, Qmax, Hq, D]`` (the rectangular speculative
  decode step of the model operations guide's token-layout file list); rows
  ``t >= query_lens[b]`` are not produced and come back as NaN.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_bytes_to_f64

__all__ = ["BLOCK_SIZE", "paged_decode_attention", "gather_sequence_kv"]

BLOCK_SIZE = 16


def _decode_cache(cache, kv_dtype: str) -> callable:
    if kv_dtype == "bf16":
        return bf16_bits_to_f64
    if kv_dtype == "fp8_e4m3fn":
        return e4m3fn_bytes_to_f64
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def gather_sequence_kv(cache, block_table_row, length: int, kv_dtype: str,
                       scales=None) -> np.ndarray:
    """Gather the first ``length`` tokens of one sequence through its block
    table row and return them dequantised as float64 ``[length, Hkv, D]``.

    With block size ``bs = cache.shape[1]``, token j is slot ``j % bs`` of
    physical block ``block_table_row[j // bs]``.
    """
    decode = _decode_cache(cache, kv_dtype)
    bs = np.asarray(cache).shape[1]
    j = np.arange(length)
    blk = np.asarray(block_table_row)[j // bs].astype(np.int64)
    slot = j % bs
    raw = np.asarray(cache)[blk, slot]                   # [length, Hkv, D]
    vals = decode(raw)
    if kv_dtype == "fp8_e4m3fn":
        if scales is None:
            raise ValueError("fp8 cache needs its per-token scales")
        s = np.asarray(scales, dtype=np.float32)[blk, slot].astype(np.float64)
        vals = vals * s[:, :, None]                      # exact in float64
    elif scales is not None:
        raise ValueError("scales are only defined for the fp8 cache")
    return vals


def paged_decode_attention(q_bits, k_cache, v_cache, block_tables, context_lens,
                           query_lens, scale, k_scale=None, v_scale=None,
                           kv_dtype: str = "bf16", batch_subset=None,
                           sliding_window=None, sinks=None):
    """Reference output, float64 ``[B, Qmax, Hq, D]``.

    ``q_bits``: uint16 bf16 patterns ``[B, Qmax, Hq, D]``.
    ``k_cache``/``v_cache``: uint16 (bf16) or uint8 (e4m3fn)
    ``[NB, BS, Hkv, D]``.  ``block_tables``: ``[B, W]`` integers.
    ``context_lens``/``query_lens``: ``[B]`` integers (``query_lens=None``
    means every sequence has ``Qmax`` query rows).  ``scale``: the softmax
    scale as the float32 value the caller passes.  ``k_scale``/``v_scale``:
    float32 ``[NB, BS, Hkv]`` (fp8 only).  ``batch_subset``: optional list of
    sequence indices to compute (others stay NaN), for sampled checks of
    large workloads.  ``sliding_window``: ``None`` or an int (``<= 0``: no
    window).  ``sinks``: ``None`` or float32 ``[Hq]`` sink logits.
    """
    q_bits = np.asarray(q_bits)
    if q_bits.ndim == 3:
        q_bits = q_bits[:, None]
    B, Qmax, Hq, D = q_bits.shape
    NB, bs, Hkv, Dk = np.asarray(k_cache).shape
    if bs < 1 or Dk != D or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    G = Hq // Hkv
    window = None if sliding_window is None or int(sliding_window) <= 0 else int(sliding_window)
    sink = None
    if sinks is not None:
        sink = np.asarray(sinks, dtype=np.float32).astype(np.float64)
        if sink.shape != (Hq,) or np.isnan(sink).any() or (sink == np.inf).any():
            raise ValueError("sinks must be [Hq] values below +inf")
    ctx = np.asarray(context_lens).astype(np.int64)
    qlens = (np.full(B, Qmax, dtype=np.int64) if query_lens is None
             else np.asarray(query_lens).astype(np.int64))
    tables = np.asarray(block_tables).astype(np.int64)
    s = np.float64(np.float32(scale))

    out = np.full((B, Qmax, Hq, D), np.nan, dtype=np.float64)
    seqs = range(B) if batch_subset is None else batch_subset
    for b in seqs:
        L, n = int(ctx[b]), int(qlens[b])
        if n == 0:
            continue
        if not (1 <= n <= Qmax and n <= L <= bs * tables.shape[1]):
            raise ValueError(f"sequence {b}: query_len {n}, context_len {L} out of range")
        used = tables[b, : (L + bs - 1) // bs]
        if used.min() < 0 or used.max() >= NB:
            raise ValueError(f"sequence {b}: block id out of range")
        K = gather_sequence_kv(k_cache, tables[b], L, kv_dtype, k_scale)   # [L, Hkv, D]
        V = gather_sequence_kv(v_cache, tables[b], L, kv_dtype, v_scale)
        Q = bf16_bits_to_f64(q_bits[b, :n])                                 # [n, Hq, D]
        # causal limit of row t: keys 0 .. L - n + t (the window's start below)
        pos = L - n + np.arange(n)
        visible = np.arange(L)[None, :] <= pos[:, None]                     # [n, L]
        if window is not None:
            visible &= np.arange(L)[None, :] > (pos - window)[:, None]
        for g in range(Hkv):
            Qg = Q[:, g * G:(g + 1) * G, :]                                 # [n, G, D]
            x = s * np.matmul(Qg, K[:, g, :].T)                             # [n, G, L]
            x = np.where(visible[:, None, :], x, -np.inf)
            mx = x.max(axis=-1, keepdims=True)
            if sink is not None:
                sk = sink[g * G:(g + 1) * G][None, :, None]                 # [1, G, 1]
                mx = np.maximum(mx, sk)
                e = np.exp(x - mx)
                den = e.sum(axis=-1, keepdims=True) + np.exp(sk - mx)
            else:
                e = np.exp(x - mx)
                den = e.sum(axis=-1, keepdims=True)
            out[b, :n, g * G:(g + 1) * G, :] = np.matmul(e, V[:, g, :]) / den
    return out

"""Plain CPU oracle for paged prefill (chunked prefill) attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg may import this module; the product
path never does, and it shares no code with the HIP path.

What it computes
----------------
The model operations guide runs prefill attention through a variable-length
flash-attention call ("Attention operations": prefill always takes
``flash_attn_varlen_func``; the kernel table also lists a unified paged
prefill kernel), its attention builder prepares block tables and cumulative
sequence lengths for every prefill step ("Backend abstraction"), and its
source-file list places a ragged prefill chunk's tokens in their own
sequences (``token_layout/prefill.py``).  The reading taken here:

* the new tokens of all sequences are packed row after row: sequence ``b``
  owns rows ``cu[b] .. cu[b+1]-1`` of ``q`` and ``out`` (``n_b = cu[b+1] -
  cu[b]`` rows, ``cu[0] = 0``);
* they are the last ``n_b`` of its ``L_b = context_lens[b]`` tokens, whose
  K/V are already in the paged cache (the chunk's own rows were written
  before the call; earlier chunks or a cached prefix make up the rest);
* row ``t`` of sequence ``b`` sits at position ``L_b - n_b + t`` and attends
  causally to keys ``0 .. L_b - n_b + t`` through the block table — the same
  definition as decode attention with ``n_b`` query rows, so this oracle
  lays the packed rows out per sequence and evaluates that definition
  (``paged_decode_attention``), with the same sliding window and attention
  sinks as the decode call when they are given (the model operations
  guide's attention dispatch takes a sliding window; the README's model
  table gives GPT-OSS a sliding window and sinks): the row at position
  ``a`` sees keys ``max(0, a - w + 1) .. a``, and a head's sink logit joins
  the softmax normaliser only.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import paged_decode_attention

__all__ = ["paged_prefill_attention"]


def paged_prefill_attention(q_bits, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q,
                            scale, k_scale=None, v_scale=None, kv_dtype: str = "bf16",
                            batch_subset=None, row_subset=None, sliding_window=None, sinks=None):
    """Reference output, float64 ``[T, Hq, D]`` for packed bf16 bits ``q_bits``
    ``[T, Hq, D]``; rows of sequences left out by ``batch_subset`` are NaN.
    ``row_subset`` (optional, with one sequence in ``batch_subset``): only
    those rows of that sequence (indices into its chunk) are computed."""
    q_bits = np.asarray(q_bits)
    T, Hq, D = q_bits.shape
    cu = np.asarray(cu_seqlens_q).astype(np.int64)
    B = cu.shape[0] - 1
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens_q must rise from 0 to the packed row count")
    ctx = np.asarray(context_lens).astype(np.int64)
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    seqs = range(B) if batch_subset is None else batch_subset
    tables = np.asarray(block_tables)
    for b in seqs:
        n = int(cu[b + 1] - cu[b])
        if n == 0:
            continue
        if row_subset is None:
            # the sequence's n rows as the query rows of one decode call
            one = paged_decode_attention(q_bits[cu[b]:cu[b + 1]][None], k_cache, v_cache, tables[b:b + 1],
                                         [int(ctx[b])], [n], scale, k_scale, v_scale, kv_dtype,
                                         sliding_window=sliding_window, sinks=sinks)
            out[cu[b]:cu[b + 1]] = one[0]
            continue
        # a chosen row t alone: the one query row of a sequence whose cache
        # holds its first L - n + t + 1 tokens
        for t in np.asarray(row_subset, dtype=np.int64):
            Lt = int(ctx[b]) - n + int(t) + 1
            one = paged_decode_attention(q_bits[cu[b] + t][None, None], k_cache, v_cache, tables[b:b + 1],
                                         [Lt], [1], scale, k_scale, v_scale, kv_dtype,
                                         sliding_window=sliding_window, sinks=sinks)
            out[cu[b] + t] = one[0, 0]
    return out

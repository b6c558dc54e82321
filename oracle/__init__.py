"""CPU oracle for paged-KV decode attention and the paged KV-cache write.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain float64
definition that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it; the product path (the ``paged_attention_decode_attn_amd`` package
and its C-ABI library) never imports, links or calls anything here, and the
two share no code.

Modules
-------
formats          bf16 and OCP float8 e4m3fn bit-level decoders
paged_attention  dense softmax attention gathered through the block table
split_merge      split-context partial states and their log-sum-exp merge
cache_write      new tokens' K/V into the paged cache through a slot mapping,
                 bf16 bit copies or per-token absmax fp8 e4m3fn quantisation
prefill          packed variable-length prefill chunks over the paged cache

Every function is pinned by ``-m "not gpu"`` tests against closed forms,
invariants, brute force and independent library routines; no function here
is "parity unpinned".
"""
from .formats import bf16_bits_to_f64, e4m3fn_bytes_to_f64, e4m3fn_table, e4m3fn_value
from .paged_attention import BLOCK_SIZE, gather_sequence_kv, paged_decode_attention
from .split_merge import merge_states, partial_state
from .cache_write import e4m3fn_encode, quantize_rows_e4m3fn, reshape_and_cache
from .prefill import paged_prefill_attention

__all__ = [
    "BLOCK_SIZE", "bf16_bits_to_f64", "e4m3fn_bytes_to_f64", "e4m3fn_table",
    "e4m3fn_value", "gather_sequence_kv", "paged_decode_attention",
    "merge_states", "partial_state", "e4m3fn_encode", "quantize_rows_e4m3fn",
    "reshape_and_cache", "paged_prefill_attention",
]

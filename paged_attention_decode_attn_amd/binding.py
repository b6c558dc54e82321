"""ctypes binding of ``libpaged_attn.so`` (argument marshalling only).

Every entry point has the C name of ``include/paged_attn.h``.  Tensors are
PyTorch tensors, used for device memory and streams only: each call turns
them into ``pa_tensor`` descriptors (data pointer, dtype code, sizes,
element strides) and passes the current HIP stream.  All computation runs in
the library's HIP kernels; there is no fallback of any kind, and a missing
library raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

import torch

from .build import INCLUDE
from .build import LIB_PATH as _BUILT_LIB

# the in-tree build, and only it
LIB_PATH = _BUILT_LIB
HEADERS = ("paged_attn.h", "paged_attn_tuning.h")

PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3FN, PA_DTYPE_FP32, PA_DTYPE_INT32 = 1, 2, 3, 4
PA_OK = 0
STATUS_NAMES = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_DTYPE", -3: "PA_ERR_SHAPE",
                -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_LAYOUT", -6: "PA_ERR_CAPTURE",
                -7: "PA_ERR_HIP", -8: "PA_ERR_NOMEM", -9: "PA_ERR_ARG"}


class PaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class PaPlan(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("row_tiles", ctypes.c_int32),
                ("heads_per_group", ctypes.c_int32), ("min_share_chunks", ctypes.c_int32),
                ("reduce_rows", ctypes.c_int32), ("reduce_col4", ctypes.c_int32),
                ("reduce_lanes", ctypes.c_int32), ("expected_partials", ctypes.c_int32),
                ("whole_segments", ctypes.c_int32), ("row_waves", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("reduce_groups", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({status}): {detail}")


_lib = None
_lock = threading.Lock()
_P = ctypes.POINTER(PaTensor)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m paged_attention_decode_attn_amd.build` (no fallback exists)")
                L = ctypes.CDLL(LIB_PATH)
                args11 = [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]
                L.paged_attn_decode.argtypes = args11 + [_P, ctypes.c_void_p]
                L.paged_attn_decode_noalloc.argtypes = args11 + [_P, ctypes.c_void_p]
                L.paged_attn_check.argtypes = args11 + [_P]
                L.paged_attn_decode_ext.argtypes = args11 + [ctypes.c_int32, _P, _P, ctypes.c_void_p]
                L.paged_attn_check_ext.argtypes = args11 + [ctypes.c_int32, _P, _P]
                args_pf = [_P] * 6 + [ctypes.c_int32, ctypes.c_float, _P, _P, _P]
                L.paged_attn_prefill.argtypes = args_pf + [ctypes.c_void_p]
                L.paged_attn_check_prefill.argtypes = args_pf
                L.paged_attn_prefill_ext.argtypes = args_pf[:-1] + [ctypes.c_int32, _P, _P, ctypes.c_void_p]
                L.paged_attn_check_prefill_ext.argtypes = args_pf[:-1] + [ctypes.c_int32, _P, _P]
                L.paged_attn_reshape_and_cache.argtypes = [_P] * 7 + [ctypes.c_void_p]
                L.paged_attn_check_reshape_and_cache.argtypes = [_P] * 7
                L.paged_attn_plan.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int32, ctypes.c_int32,
                                                                     ctypes.POINTER(PaPlan)]
                L.paged_attn_set_workgroups.argtypes = [ctypes.c_int32]
                L.paged_attn_set_min_share.argtypes = [ctypes.c_int32]
                L.paged_attn_set_heads_per_group.argtypes = [ctypes.c_int32]
                L.paged_attn_set_write_pieces.argtypes = [ctypes.c_int32]
                L.paged_attn_reserve.argtypes = [ctypes.c_int64, ctypes.c_void_p]
                L.paged_attn_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_int32] * 4 + [
                    ctypes.c_void_p, ctypes.c_void_p]
                L.paged_attn_probe_gather_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                                                           ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p] + [
                    ctypes.c_int32] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
                i32p = ctypes.POINTER(ctypes.c_int32)
                L.paged_attn_check_metadata.argtypes = [i32p, i32p, i32p] + [ctypes.c_int64] * 6 + [ctypes.c_int32]
                L.paged_attn_profile_begin.argtypes = [ctypes.c_int32]
                L.paged_attn_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double),
                                                     ctypes.POINTER(ctypes.c_double),
                                                     ctypes.POINTER(ctypes.c_int32)]
                L.paged_attn_strerror.argtypes = [ctypes.c_int]
                L.paged_attn_strerror.restype = ctypes.c_char_p
                L.paged_attn_last_error.argtypes = []
                L.paged_attn_last_error.restype = ctypes.c_char_p
                for name in ("paged_attn_decode", "paged_attn_decode_noalloc", "paged_attn_check", "paged_attn_plan",
                             "paged_attn_decode_ext", "paged_attn_check_ext",
                             "paged_attn_prefill", "paged_attn_check_prefill",
                             "paged_attn_prefill_ext", "paged_attn_check_prefill_ext",
                             "paged_attn_reshape_and_cache", "paged_attn_check_reshape_and_cache",
                             "paged_attn_set_workgroups", "paged_attn_set_min_share",
                             "paged_attn_set_heads_per_group", "paged_attn_set_write_pieces",
                             "paged_attn_reserve", "paged_attn_probe_stream_read", "paged_attn_probe_gather_read",
                             "paged_attn_check_metadata", "paged_attn_profile_begin",
                             "paged_attn_profile_end"):
                    getattr(L, name).restype = ctypes.c_int
                _lib = L
    return _lib


def header_functions() -> list:
    """Names of every function that the headers under ``include/`` declare."""
    names = set()
    for h in HEADERS:
        text = open(os.path.join(INCLUDE, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(paged_attn_\w+)\s*\(", text))
    return sorted(names)


def _raise(status: int, where: str):
    if status != PA_OK:
        detail = (lib().paged_attn_last_error() or b"").decode(errors="replace")
        raise PagedAttnError(status, where, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_DTYPE_FP8_E4M3FN
    if t.dtype == torch.float32:
        return PA_DTYPE_FP32
    if t.dtype == torch.int32:
        return PA_DTYPE_INT32
    return 0                     # no pa_dtype: the library rejects it with PA_ERR_DTYPE


def describe(t: Optional[torch.Tensor], dtype_code: Optional[int] = None) -> Optional[PaTensor]:
    """A ``pa_tensor`` for ``t`` (None stays None)."""
    if t is None:
        return None
    if t.dim() > 4:
        raise ValueError("tensors of rank > 4 are not described")
    d = PaTensor()
    d.data = t.data_ptr() if t.numel() else (t.data_ptr() or None)
    d.dtype = _dtype_code(t) if dtype_code is None else dtype_code
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d: Optional[PaTensor]):
    return ctypes.byref(d) if d is not None else None


def _stream_handle(t: torch.Tensor, stream) -> ctypes.c_void_p:
    if stream is None:
        if t.is_cuda:
            stream = torch.cuda.current_stream(t.device)
        else:
            return ctypes.c_void_p(None)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale,
                      k_scale=None, v_scale=None, out=None, stream=None):
    """Run the library's decode attention; returns ``out`` (allocated with
    ``torch.empty_like(q)`` when not given).  Raises PagedAttnError on any
    non-zero status."""
    if out is None:
        out = torch.empty_like(q)
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, query_lens)]
    dks, dvs, dout = describe(k_scale), describe(v_scale), describe(out)
    st = lib().paged_attn_decode(*[_ref(d) for d in descs], ctypes.c_float(scale), _ref(dks),
                                 _ref(dvs), _ref(dout), _stream_handle(q, stream))
    _raise(st, "paged_attn_decode")
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale,
                              k_scale=None, v_scale=None, out=None, stream=None):
    """``paged_attn_decode`` through the entry point that allocates nothing
    (partial results in the library's static per-device scratch array);
    ``out`` must be given (this call allocates no tensor either)."""
    if out is None:
        raise ValueError("paged_attn_decode_noalloc takes a caller-allocated out")
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, query_lens)]
    st = lib().paged_attn_decode_noalloc(*[_ref(d) for d in descs], ctypes.c_float(scale),
                                         _ref(describe(k_scale)), _ref(describe(v_scale)),
                                         _ref(describe(out)), _stream_handle(q, stream))
    _raise(st, "paged_attn_decode_noalloc")
    return out


def paged_attn_check(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale,
                     k_scale=None, v_scale=None, out=None) -> int:
    """Status of the host-side validation (no GPU access, no data read)."""
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, query_lens)]
    return lib().paged_attn_check(*[_ref(d) for d in descs], ctypes.c_float(scale),
                                  _ref(describe(k_scale)), _ref(describe(v_scale)),
                                  _ref(describe(out)))


def paged_attn_decode_ext(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale,
                          k_scale=None, v_scale=None, sliding_window=0, sinks=None, out=None,
                          stream=None):
    """``paged_attn_decode`` with a sliding window (``<= 0``: none) and
    per-query-head sink logits (fp32 ``[Hq]`` or None)."""
    if out is None:
        out = torch.empty_like(q)
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, query_lens)]
    st = lib().paged_attn_decode_ext(*[_ref(d) for d in descs], ctypes.c_float(scale),
                                     _ref(describe(k_scale)), _ref(describe(v_scale)),
                                     ctypes.c_int32(int(sliding_window)), _ref(describe(sinks)),
                                     _ref(describe(out)), _stream_handle(q, stream))
    _raise(st, "paged_attn_decode_ext")
    return out


def paged_attn_check_ext(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale,
                         k_scale=None, v_scale=None, sliding_window=0, sinks=None, out=None) -> int:
    """Status of the host-side validation of ``paged_attn_decode_ext``."""
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, query_lens)]
    return lib().paged_attn_check_ext(*[_ref(d) for d in descs], ctypes.c_float(scale),
                                      _ref(describe(k_scale)), _ref(describe(v_scale)),
                                      ctypes.c_int32(int(sliding_window)), _ref(describe(sinks)),
                                      _ref(describe(out)))


def paged_attn_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len, scale,
                       out=None, stream=None, k_scale=None, v_scale=None):
    """Causal attention of packed prefill chunks (bf16 ``[T, Hq, D]``; sequence
    ``b`` owns rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1``, the last of
    its ``context_lens[b]`` cached tokens); an fp8 cache takes ``k_scale`` and
    ``v_scale``.  Returns ``out``."""
    if out is None:
        out = torch.empty_like(q)
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q)]
    st = lib().paged_attn_prefill(*[_ref(d) for d in descs], ctypes.c_int32(int(max_query_len)),
                                  ctypes.c_float(scale), _ref(describe(k_scale)), _ref(describe(v_scale)),
                                  _ref(describe(out)), _stream_handle(q, stream))
    _raise(st, "paged_attn_prefill")
    return out


def paged_attn_prefill_ext(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len, scale,
                           sliding_window=0, sinks=None, out=None, stream=None, k_scale=None, v_scale=None):
    """``paged_attn_prefill`` with a sliding window (``> 0``: a row sees its
    ``sliding_window`` most recent positions) and per-query-head sink logits
    (fp32 ``[Hq]`` or None); returns ``out``."""
    if out is None:
        out = torch.empty_like(q)
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q)]
    st = lib().paged_attn_prefill_ext(*[_ref(d) for d in descs], ctypes.c_int32(int(max_query_len)),
                                      ctypes.c_float(scale), _ref(describe(k_scale)), _ref(describe(v_scale)),
                                      ctypes.c_int32(int(sliding_window)),
                                      _ref(describe(sinks)), _ref(describe(out)), _stream_handle(q, stream))
    _raise(st, "paged_attn_prefill_ext")
    return out


def paged_attn_check_prefill_ext(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len,
                                 scale, k_scale=None, v_scale=None, sliding_window=0, sinks=None,
                                 out=None) -> int:
    """Status of the host-side validation of ``paged_attn_prefill_ext``."""
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q)]
    return lib().paged_attn_check_prefill_ext(*[_ref(d) for d in descs], ctypes.c_int32(int(max_query_len)),
                                              ctypes.c_float(scale), _ref(describe(k_scale)),
                                              _ref(describe(v_scale)), ctypes.c_int32(int(sliding_window)),
                                              _ref(describe(sinks)), _ref(describe(out)))


def paged_attn_check_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len, scale,
                             k_scale=None, v_scale=None, out=None) -> int:
    """Status of the host-side validation of ``paged_attn_prefill``."""
    descs = [describe(x) for x in (q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q)]
    return lib().paged_attn_check_prefill(*[_ref(d) for d in descs], ctypes.c_int32(int(max_query_len)),
                                          ctypes.c_float(scale), _ref(describe(k_scale)),
                                          _ref(describe(v_scale)), _ref(describe(out)))


def paged_attn_reshape_and_cache(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None,
                                 v_scale=None, stream=None) -> None:
    """Write the new tokens' K/V (bf16 ``[T, Hkv, D]``) into the paged cache
    at ``slot_mapping`` (int32 ``[T]``), quantising per token when the cache
    is fp8 (then ``k_scale`` / ``v_scale`` are written too).  Raises
    PagedAttnError on any non-zero status."""
    d = [describe(x) for x in (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)]
    st = lib().paged_attn_reshape_and_cache(*[_ref(x) for x in d], _stream_handle(k_new, stream))
    _raise(st, "paged_attn_reshape_and_cache")


def paged_attn_check_reshape_and_cache(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None,
                                       v_scale=None) -> int:
    """Status of the cache write's host-side validation (no GPU access)."""
    d = [describe(x) for x in (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)]
    return lib().paged_attn_check_reshape_and_cache(*[_ref(x) for x in d])


def paged_attn_check_descriptors(q, k_cache, v_cache, block_tables, context_lens, query_lens,
                                 scale, k_scale, v_scale, out) -> int:
    """``paged_attn_check`` on raw ``PaTensor`` descriptors (None = NULL)."""
    return lib().paged_attn_check(_ref(q), _ref(k_cache), _ref(v_cache), _ref(block_tables),
                                  _ref(context_lens), _ref(query_lens), ctypes.c_float(scale),
                                  _ref(k_scale), _ref(v_scale), _ref(out))


def paged_attn_plan(batch, q_heads, kv_heads, head_dim, query_len, max_context,
                    kv_dtype="bf16", num_cus=256) -> dict:
    """The split-context plan; ``max_context`` is the most cache tokens one
    sequence's rows can read (block size x table width)."""
    code = PA_DTYPE_FP8_E4M3FN if kv_dtype == "fp8_e4m3fn" else PA_DTYPE_BF16
    p = PaPlan()
    st = lib().paged_attn_plan(batch, q_heads, kv_heads, head_dim, query_len, max_context, code,
                               num_cus, ctypes.byref(p))
    _raise(st, "paged_attn_plan")
    return p.as_dict()


def paged_attn_set_workgroups(workgroups: int) -> None:
    _raise(lib().paged_attn_set_workgroups(int(workgroups)), "paged_attn_set_workgroups")


def paged_attn_set_min_share(chunks: int) -> None:
    _raise(lib().paged_attn_set_min_share(int(chunks)), "paged_attn_set_min_share")


def paged_attn_set_heads_per_group(heads: int) -> None:
    _raise(lib().paged_attn_set_heads_per_group(int(heads)), "paged_attn_set_heads_per_group")


def paged_attn_set_write_pieces(pieces: int) -> None:
    _raise(lib().paged_attn_set_write_pieces(int(pieces)), "paged_attn_set_write_pieces")


def paged_attn_reserve(nbytes: int, stream=None) -> None:
    s = ctypes.c_void_p(None) if stream is None else ctypes.c_void_p(
        stream if isinstance(stream, int) else stream.cuda_stream)
    _raise(lib().paged_attn_reserve(int(nbytes), s), "paged_attn_reserve")


def paged_attn_check_metadata(context_lens, query_lens, block_tables, query_len: int,
                              num_blocks: int, block_size: int = 16, sliding_window: int = 0) -> None:
    """Check the device-side preconditions on host copies (raises on violation)."""
    ctx = context_lens.detach().to("cpu", torch.int32).contiguous()
    tbl = block_tables.detach().to("cpu", torch.int32).contiguous()
    ql = None if query_lens is None else query_lens.detach().to("cpu", torch.int32).contiguous()
    i32p = ctypes.POINTER(ctypes.c_int32)
    st = lib().paged_attn_check_metadata(
        ctypes.cast(ctx.data_ptr(), i32p),
        None if ql is None else ctypes.cast(ql.data_ptr(), i32p),
        ctypes.cast(tbl.data_ptr(), i32p), ctx.numel(), tbl.shape[1], tbl.stride(0),
        query_len, num_blocks, block_size, ctypes.c_int32(int(sliding_window)))
    _raise(st, "paged_attn_check_metadata")


def paged_attn_profile_begin(max_calls: int) -> None:
    _raise(lib().paged_attn_profile_begin(int(max_calls)), "paged_attn_profile_begin")


def paged_attn_profile_end() -> dict:
    part, red, calls = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    _raise(lib().paged_attn_profile_end(ctypes.byref(part), ctypes.byref(red), ctypes.byref(calls)),
           "paged_attn_profile_end")
    return {"partition_ms": part.value, "reduce_ms": red.value, "calls": calls.value}


def paged_attn_probe_stream_read(src: torch.Tensor, workgroups: int, threads: int, unroll: int,
                                 grid_stride: bool, sink: torch.Tensor, stream=None) -> None:
    """The streaming-read probe over the whole of ``src`` (measurement only)."""
    st = lib().paged_attn_probe_stream_read(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                            int(workgroups), int(threads), int(unroll), int(bool(grid_stride)),
                                            ctypes.c_void_p(sink.data_ptr()), _stream_handle(src, stream))
    _raise(st, "paged_attn_probe_stream_read")


def paged_attn_probe_gather_read(arrays, block_ids: torch.Tensor, num_blocks: int, workgroups: int, threads: int,
                                 unroll: int, sink: torch.Tensor, stream=None) -> None:
    """The gather probe (measurement only): ``arrays`` is up to four
    (tensor, block stride in bytes, bytes read per block) triples."""
    arrays = list(arrays) + [(None, 0, 0)] * (4 - len(arrays))
    ptrs = (ctypes.c_void_p * 4)(*[None if t is None else t.data_ptr() for t, _, _ in arrays])
    strides = (ctypes.c_int64 * 4)(*[int(st) for _, st, _ in arrays])
    nbytes = (ctypes.c_int32 * 4)(*[int(nb) for _, _, nb in arrays])
    st = lib().paged_attn_probe_gather_read(ptrs, strides, nbytes, ctypes.c_void_p(block_ids.data_ptr()),
                                            int(block_ids.numel()), int(num_blocks), int(workgroups), int(threads),
                                            int(unroll), ctypes.c_void_p(sink.data_ptr()),
                                            _stream_handle(block_ids, stream))
    _raise(st, "paged_attn_probe_gather_read")


def paged_attn_strerror(status: int) -> str:
    return lib().paged_attn_strerror(status).decode()


def paged_attn_last_error() -> str:
    return lib().paged_attn_last_error().decode()

"""Paged-KV decode attention for MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``include/paged_attn.h`` (``libpaged_attn.so``, built in-tree by
``paged_attention_decode_attn_amd.build``); ``binding`` is a thin ctypes
layer with the same entry-point names, and ``workloads`` draws seeded
synthetic inputs.  Importing the package does not load the library; the
first call does, and raises if it has not been built.
"""
from . import workloads  # noqa: F401  (inputs only; no GPU, no library)

_BINDING_NAMES = (
    "paged_attn_decode", "paged_attn_check", "paged_attn_decode_ext", "paged_attn_check_ext",
    "paged_attn_prefill", "paged_attn_check_prefill", "paged_attn_prefill_ext", "paged_attn_check_prefill_ext",
    "paged_attn_check_descriptors", "paged_attn_plan",
    "paged_attn_reshape_and_cache", "paged_attn_check_reshape_and_cache",
    "paged_attn_set_workgroups", "paged_attn_set_min_share", "paged_attn_set_heads_per_group",
    "paged_attn_reserve", "paged_attn_check_metadata",
    "paged_attn_profile_begin", "paged_attn_profile_end", "paged_attn_strerror",
    "paged_attn_last_error", "PagedAttnError", "PaTensor", "describe", "lib",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_BINDING_NAMES) + ["workloads"]

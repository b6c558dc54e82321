"""Host-side checks of the seeded input generator (no GPU)."""
import numpy as np
import pytest
import torch

from paged_attention_decode_attn_amd.workloads import CONFIGS, CONFIG_ORDER, generate, kv_bytes


def _small(name, **kw):
    s = CONFIGS[name]
    base = dict(batch=min(s.batch, 3), ctx_hi=min(s.ctx_hi, 300), ctx_lo=min(s.ctx_lo, 300),
                pool_blocks=80)
    base.update(kw)
    return s.replace(**base)


def test_five_configs_have_the_stated_shapes():
    assert CONFIG_ORDER == ["tiny", "llama3_8b", "long_ctx", "fp8", "mtp_verify"]
    t = CONFIGS["tiny"]
    assert (t.batch, t.qlen, t.hq, t.hkv, t.head_dim, t.ctx_lo, t.ctx_hi, t.pool_blocks) == \
        (1, 1, 32, 8, 128, 512, 512, 64)
    assert abs(t.softmax_scale - 128 ** -0.5) < 1e-15
    assert CONFIGS["long_ctx"].ctx_hi == 131072 and CONFIGS["long_ctx"].hq == 64
    f = CONFIGS["fp8"]
    assert (f.kv_dtype, f.head_dim, f.batch, f.ctx_lo, f.ctx_hi) == ("fp8_e4m3fn", 64, 16, 512, 32768)
    m = CONFIGS["mtp_verify"]
    assert (m.batch, m.qlen, m.ctx_lo, m.ctx_hi) == (64, 2, 256, 16384)
    for s in CONFIGS.values():
        assert s.table_width * s.block_size >= s.ctx_hi and s.block_size % 16 == 0
        assert s.pool_blocks >= s.batch * s.table_width or s.name.startswith("tiny")


def test_tiny_config_is_deterministic_and_disjoint():
    a = generate(CONFIGS["tiny"])
    b = generate(CONFIGS["tiny"])
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache),
                 (a.block_tables, b.block_tables)]:
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
    assert a.block_tables.shape == (1, 32)
    used = a.block_tables[0].tolist()
    assert len(set(used)) == 32 and all(0 <= u < 64 for u in used)
    assert a.context_lens.tolist() == [512] and a.query_lens.tolist() == [1]
    assert kv_bytes(a.context_lens, 8, 128, "bf16") == 2 * 512 * 8 * 128 * 2


def test_ragged_contexts_in_range_and_tables_disjoint():
    w = generate(_small("llama3_8b", ctx_lo=20, ctx_hi=300))
    ctx = w.context_lens.tolist()
    assert all(20 <= c <= 300 for c in ctx)
    seen = set()
    for b, c in enumerate(ctx):
        ids = w.block_tables[b, : (c + 15) // 16].tolist()
        assert not (set(ids) & seen)
        seen |= set(ids)


def test_fp8_rows_use_absmax_over_448_scales():
    w = generate(_small("fp8"))
    k8 = w.k_cache.view(torch.float8_e4m3fn).to(torch.float32)
    b0 = int(w.block_tables[0, 0])
    rows = k8[b0]                                           # [16, Hkv, D]
    amax = rows.abs().amax(-1)
    assert torch.all(amax <= 448) and torch.all(amax >= 416)   # absmax maps to 448 up to rounding
    assert w.k_scale.shape == (80, 16, 8) and w.k_scale.stride() == (128, 1, 16)
    assert torch.all(w.k_scale[b0] > 0)


def test_poison_marks_unread_memory_nan():
    w = generate(_small("llama3_8b", batch=2, ctx_lo=17, ctx_hi=40), poison=True)
    L = w.context_lens.tolist()
    for b, c in enumerate(L):
        n = (c + 15) // 16
        last = int(w.block_tables[b, n - 1])
        tail = c - (n - 1) * 16
        if tail < 16:
            assert torch.isnan(w.k_cache[last, tail:].float()).all()
        assert not torch.isnan(w.k_cache[last, :tail].float()).any()
        pad = w.block_tables[b, n:]
        if pad.numel():
            assert torch.isnan(w.v_cache[int(pad[0])].float()).all()


def test_numpy_inputs_are_the_same_bytes():
    w = generate(_small("fp8", batch=2))
    d = w.numpy_inputs()
    assert d["q_bits"].dtype == np.uint16 and d["k_cache"].dtype == np.uint8
    assert np.array_equal(d["q_bits"], w.q.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(d["k_scale"], w.k_scale.numpy())


def test_rejects_pool_too_small():
    with pytest.raises(ValueError):
        generate(CONFIGS["tiny"].replace(pool_blocks=16))


def test_ragged_query_lengths_are_drawn_in_range_and_reproducibly():
    from paged_attention_decode_attn_amd.workloads import CONFIGS, generate
    spec = CONFIGS["mtp_verify_ragged"].replace(batch=40, ctx_lo=8, ctx_hi=300, pool_blocks=1000)
    a, b = generate(spec), generate(spec)
    ql = a.query_lens
    assert ql.dtype == torch.int32 and int(ql.min()) >= 1 and int(ql.max()) <= 4
    assert len(set(ql.tolist())) > 1                                # actually ragged
    assert torch.equal(ql, b.query_lens) and torch.equal(a.k_cache, b.k_cache)
    # specs without qlen_lo draw nothing extra: the five workloads are unchanged
    assert CONFIGS["mtp_verify"].qlen_lo is None


def test_block_size_window_and_sinks_in_the_generator():
    from paged_attention_decode_attn_amd.workloads import kv_bytes
    spec = CONFIGS["mtp_verify"].replace(batch=3, ctx_lo=2, ctx_hi=300, pool_blocks=20, block_size=64,
                                         sliding_window=50, sinks=True)
    w = generate(spec)
    assert w.k_cache.shape[1] == 64 and w.block_tables.shape[1] == 5
    assert w.sinks.shape == (spec.hq,) and float(w.sinks.min()) >= -2 and float(w.sinks.max()) <= 8
    # the draws before the sinks are those of the same spec without sinks
    w0 = generate(spec.replace(sinks=False))
    assert torch.equal(w.k_cache.view(torch.int16), w0.k_cache.view(torch.int16)) and w0.sinks is None
    ins = w.numpy_inputs()
    assert ins["sliding_window"] == 50 and ins["sinks"].shape == (spec.hq,)
    # a window bounds the attended tokens: min(L, window + n - 1) per sequence
    ctx, ql = torch.tensor([10, 100, 60]), torch.tensor([2, 2, 0])
    per = 2 * spec.hkv * spec.head_dim * 2
    assert kv_bytes(ctx, spec.hkv, spec.head_dim, "bf16", ql, 50) == (10 + 51 + 0) * per
    assert kv_bytes(ctx, spec.hkv, spec.head_dim, "bf16") == 170 * per

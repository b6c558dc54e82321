"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, validates descriptors, plans partitions and checks
metadata.  No compute entry point is called here."""
import ctypes

import pytest
import torch

from paged_attention_decode_attn_amd import binding as B

NB, HKV, D, BQ, QMAX, HQ, W = 10, 2, 128, 3, 2, 8, 4


def _tensors(kv="bf16", d=D, hq=HQ, hkv=HKV, qmax=QMAX, block=16):
    q = torch.zeros(BQ, qmax, hq, d, dtype=torch.bfloat16)
    cdt = torch.uint8 if kv == "fp8" else torch.bfloat16
    kc = torch.zeros(NB, block, hkv, d, dtype=cdt)
    vc = torch.zeros(NB, block, hkv, d, dtype=cdt)
    bt = torch.zeros(BQ, W, dtype=torch.int32)
    ctx = torch.ones(BQ, dtype=torch.int32)
    ql = torch.ones(BQ, dtype=torch.int32)
    ks = vs = None
    if kv == "fp8":
        ks = torch.ones(NB, hkv, block).permute(0, 2, 1)
        vs = torch.ones(NB, hkv, block).permute(0, 2, 1)
    out = torch.empty_like(q)
    return dict(q=q, k_cache=kc, v_cache=vc, block_tables=bt, context_lens=ctx, query_lens=ql,
                scale=0.125, k_scale=ks, v_scale=vs, out=out)


def _check(**kw):
    return B.paged_attn_check(**kw)


def test_library_exports_every_header_function():
    L = B.lib()
    names = B.header_functions()
    assert "paged_attn_decode" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"


def test_valid_descriptors_pass_bf16_and_fp8():
    assert _check(**_tensors()) == B.PA_OK
    assert _check(**_tensors("fp8")) == B.PA_OK
    t = _tensors(qmax=1)
    t["q"] = t["q"][:, 0]
    t["out"] = t["out"][:, 0]                      # rank-3 q: Qmax = 1
    assert _check(**t) == B.PA_OK
    t = _tensors()
    t["query_lens"] = None                         # NULL query_lens: all Qmax
    assert _check(**t) == B.PA_OK
    t = _tensors(d=64, hq=64, hkv=8, qmax=1)
    assert _check(**t) == B.PA_OK


def _status(name):
    return {v: k for k, v in B.STATUS_NAMES.items()}[name]


@pytest.mark.parametrize("mutate,expect", [
    (lambda t: t.update(q=None), "PA_ERR_NULL"),
    (lambda t: t.update(out=None), "PA_ERR_NULL"),
    (lambda t: t.update(k_cache=None), "PA_ERR_NULL"),
    (lambda t: t.update(q=t["q"].float()), "PA_ERR_DTYPE"),
    (lambda t: t.update(out=t["out"].half()), "PA_ERR_DTYPE"),
    (lambda t: t.update(block_tables=t["block_tables"].long()), "PA_ERR_DTYPE"),
    (lambda t: t.update(context_lens=t["context_lens"].long()), "PA_ERR_DTYPE"),
    (lambda t: t.update(v_cache=t["v_cache"].view(torch.int16).view(torch.uint8)[..., :D]), "PA_ERR_DTYPE"),
    (lambda t: t.update(out=t["out"][:2]), "PA_ERR_SHAPE"),
    (lambda t: t.update(block_tables=t["block_tables"][:2]), "PA_ERR_SHAPE"),
    (lambda t: t.update(context_lens=t["context_lens"][:1]), "PA_ERR_SHAPE"),
    (lambda t: t.update(query_lens=t["query_lens"][:2]), "PA_ERR_SHAPE"),
    (lambda t: t.update(v_cache=t["v_cache"][:5]), "PA_ERR_SHAPE"),
    (lambda t: t.update(k_scale=torch.ones(NB, HKV, 16).permute(0, 2, 1)), "PA_ERR_ARG"),
    (lambda t: t.update(scale=float("nan")), "PA_ERR_ARG"),
    (lambda t: t.update(scale=float("inf")), "PA_ERR_ARG"),
    (lambda t: t.update(q=t["q"].transpose(2, 3).contiguous().transpose(2, 3),
                        out=t["out"]), "PA_ERR_LAYOUT"),
    (lambda t: t.update(k_cache=torch.zeros(NB * 16 * HKV * D + 1, dtype=torch.bfloat16)[1:]
                        .view(NB, 16, HKV, D)), "PA_ERR_LAYOUT"),      # base off by 2 bytes
    (lambda t: t.update(v_cache=torch.zeros(NB, 16, HKV, D + 4, dtype=torch.bfloat16)[..., :D]),
     "PA_ERR_LAYOUT"),                                                  # token stride 264 B
    (lambda t: t.update(block_tables=torch.zeros(W, BQ, dtype=torch.int32).t()), "PA_ERR_LAYOUT"),
])
def test_validation_errors(mutate, expect):
    t = _tensors()
    mutate(t)
    assert _check(**t) == _status(expect)
    assert B.paged_attn_last_error() != ""
    assert B.paged_attn_strerror(_status(expect)) not in ("", "unknown status")


@pytest.mark.parametrize("kw,expect", [
    (dict(block=8), "PA_ERR_UNSUPPORTED"),
    (dict(d=96), "PA_ERR_UNSUPPORTED"),
    (dict(d=512), "PA_ERR_UNSUPPORTED"),
    (dict(d=256, hq=40, hkv=1, qmax=2), "PA_ERR_UNSUPPORTED"),  # 80 rows at head_dim 256
    (dict(hq=6, hkv=4), "PA_ERR_UNSUPPORTED"),
    (dict(hq=40, hkv=1, qmax=2), "PA_ERR_UNSUPPORTED"),      # 80 rows per kv head
])
def test_unsupported_configurations(kw, expect):
    assert _check(**_tensors(**kw)) == _status(expect)


@pytest.mark.parametrize("block", [32, 48, 64, 256, 4096])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_block_sizes_that_are_multiples_of_16_are_accepted(block, kv):
    assert _check(**_tensors(kv, block=block)) == B.PA_OK


@pytest.mark.parametrize("block", [1, 8, 24, 40, 4112, 8192])
def test_other_block_sizes_are_unsupported(block):
    assert _check(**_tensors(block=block)) == _status("PA_ERR_UNSUPPORTED")


def test_fp8_scales_follow_the_block_size():
    t = _tensors("fp8", block=64)
    t["k_scale"] = torch.ones(NB, HKV, 16).permute(0, 2, 1)          # 16 slots, blocks of 64
    assert _check(**t) == _status("PA_ERR_SHAPE")


def test_block_table_reach_limit():
    t = _tensors(block=4096)
    t["block_tables"] = torch.zeros(BQ, (1 << 30) // 4096 + 1, dtype=torch.int32)
    assert _check(**t) == _status("PA_ERR_UNSUPPORTED")
    t["block_tables"] = torch.zeros(BQ, (1 << 30) // 4096, dtype=torch.int32)
    assert _check(**t) == B.PA_OK


def test_check_ext_window_and_sinks():
    t = _tensors()
    sinks = torch.zeros(HQ, dtype=torch.float32)
    for window in (-1, 0, 1, 128, 1 << 30):
        assert B.paged_attn_check_ext(**t, sliding_window=window, sinks=sinks) == B.PA_OK
        assert B.paged_attn_check_ext(**t, sliding_window=window) == B.PA_OK
    assert B.paged_attn_check_ext(**t, sinks=torch.zeros(2 * HQ)[::2]) == B.PA_OK     # strided
    assert B.paged_attn_check_ext(**t, sinks=sinks[:-1]) == _status("PA_ERR_SHAPE")
    assert B.paged_attn_check_ext(**t, sinks=sinks[None]) == _status("PA_ERR_SHAPE")
    assert B.paged_attn_check_ext(**t, sinks=sinks.to(torch.bfloat16)) == _status("PA_ERR_DTYPE")
    t2 = _tensors()
    t2["scale"] = float("nan")                                     # the other rules still apply
    assert B.paged_attn_check_ext(**t2, sinks=sinks) == _status("PA_ERR_ARG")


def test_rows_limit_is_inclusive():
    assert _check(**_tensors(hq=32, hkv=1, qmax=2)) == B.PA_OK      # exactly 64 rows
    assert _check(**_tensors(d=256, hq=16, hkv=2, qmax=2)) == B.PA_OK          # 16 rows at head_dim 256
    assert _check(**_tensors(d=256, hq=32, hkv=1, qmax=2)) == B.PA_OK          # 64 rows at head_dim 256
    assert _check(**_tensors("fp8", d=256, hq=8, hkv=8, qmax=1)) == B.PA_OK


def test_head_dim_256_plans_one_wave_per_16_rows():
    # a head_dim-256 wave holds one 16-row tile: more rows take more waves
    # per kv head, and a workgroup stays at 4 waves
    p = B.paged_attn_plan(8, 16, 8, 256, 1, 8192)
    assert p["row_tiles"] == 1 and p["row_waves"] == 1 and p["heads_per_group"] <= 4
    for hq, hkv, qlen, tiles in ((32, 2, 2, 2), (16, 2, 3, 2), (48, 2, 2, 3), (64, 4, 4, 4), (32, 1, 2, 4)):
        p = B.paged_attn_plan(8, hq, hkv, 256, qlen, 8192)
        assert p["row_tiles"] == tiles and p["row_waves"] == tiles, (hq, hkv, qlen, p)
        assert p["heads_per_group"] * tiles <= 4 and hkv % p["heads_per_group"] == 0
        assert p["workspace_bytes"] == 2 * p["workgroups"] * p["heads_per_group"] * p["rows"] * 257 * 4 + 8 * 4
    for d in (64, 128):                                   # other head dims: one wave per kv head
        assert B.paged_attn_plan(8, 32, 2, d, 2, 8192)["row_waves"] == 1
    B.paged_attn_set_heads_per_group(2)
    try:
        assert B.paged_attn_plan(8, 32, 2, 256, 2, 8192)["heads_per_group"] == 2      # 2 x 2 waves
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_plan(8, 48, 2, 256, 2, 8192)                                  # 2 x 3 waves
    finally:
        B.paged_attn_set_heads_per_group(0)


def test_head_dim_256_plans_fit_one_cu_for_every_shape():
    # every head_dim-256 plan: one wave per 16-row tile, at most 4 waves per
    # workgroup, kv heads split evenly, at most 4 waves per CU in the split
    # schedule, and a workspace that holds every partial slot
    cus = 256
    for hkv in (1, 2, 3, 4, 8, 16):
        for g in (1, 2, 3, 8, 16, 17, 32, 64):
            for qlen in (1, 2, 3, 4):
                if g * qlen > 64:
                    continue
                for batch in (1, 4, 64):
                    for ctx in (128, 8192):
                        p = B.paged_attn_plan(batch, hkv * g, hkv, 256, qlen, ctx, "bf16", cus)
                        rows, tiles = g * qlen, -(-g * qlen // 16)
                        hg = p["heads_per_group"]
                        assert (p["rows"], p["row_tiles"], p["row_waves"]) == (rows, tiles, tiles)
                        assert hkv % hg == 0 and hg * tiles <= 4, p
                        if p["whole_segments"]:
                            assert p["workgroups"] == batch * (hkv // hg) and p["workspace_bytes"] == 0
                        else:
                            assert p["workgroups"] * hg * tiles <= 4 * cus, p
                            assert p["workspace_bytes"] == 2 * p["workgroups"] * hg * rows * 257 * 4 + batch * 4


def test_fp8_scale_rules():
    t = _tensors("fp8")
    t["k_scale"] = None
    assert _check(**t) == _status("PA_ERR_NULL")
    t = _tensors("fp8")
    t["v_scale"] = torch.ones(NB, 16, HKV)                            # slot dim not contiguous
    assert _check(**t) == _status("PA_ERR_LAYOUT")
    t = _tensors("fp8")
    t["k_scale"] = torch.ones(NB, 8, HKV).permute(0, 2, 1)            # wrong shape
    assert _check(**t) == _status("PA_ERR_SHAPE")
    t = _tensors("fp8")
    t["k_scale"] = t["k_scale"].double()
    assert _check(**t) == _status("PA_ERR_DTYPE")
    t = _tensors("fp8")
    t["v_cache"] = t["v_cache"].view(torch.int16).view(torch.bfloat16) if False else \
        torch.zeros(NB, 16, HKV, D, dtype=torch.bfloat16)            # mixed K/V dtypes
    assert _check(**t) == _status("PA_ERR_DTYPE")


def test_misaligned_base_pointer():
    t = _tensors()
    d = [B.describe(t[k]) for k in ("q", "k_cache", "v_cache", "block_tables", "context_lens",
                                    "query_lens", "out")]
    assert B.paged_attn_check_descriptors(d[0], d[1], d[2], d[3], d[4], d[5], 0.1, None, None, d[6]) == 0
    d[1].data = d[1].data + 2
    assert B.paged_attn_check_descriptors(d[0], d[1], d[2], d[3], d[4], d[5], 0.1, None, None,
                                          d[6]) == _status("PA_ERR_LAYOUT")
    d[1].data = None
    assert B.paged_attn_check_descriptors(d[0], d[1], d[2], d[3], d[4], d[5], 0.1, None, None,
                                          d[6]) == _status("PA_ERR_NULL")


def _check_descs(t, **edit):
    """paged_attn_check on descriptors of ``t`` with fields replaced:
    edit = {name: [(field, dim, value), ...]}."""
    d = {k: B.describe(v) for k, v in t.items() if k != "scale"}
    for name, changes in edit.items():
        for field, dim, value in changes:
            getattr(d[name], field)[dim] = value
    names = ("q", "k_cache", "v_cache", "block_tables", "context_lens", "query_lens")
    return B.lib().paged_attn_check(*[B._ref(d[n]) for n in names], ctypes.c_float(0.125),
                                    B._ref(d["k_scale"]), B._ref(d["v_scale"]), B._ref(d["out"]))


def test_descriptor_size_limits():
    t = _tensors(qmax=1)
    assert _check_descs(t) == B.PA_OK
    # a dim of size 1 may carry any stride: only its index 0 is used
    assert _check_descs(t, q=[("stride", 1, 1 << 62)], out=[("stride", 1, 1 << 62)]) == B.PA_OK
    # a tensor reaching 2^48 bytes or more, or a size of 2^48, is refused
    assert _check_descs(t, q=[("stride", 0, 1 << 62)]) == _status("PA_ERR_UNSUPPORTED")
    assert _check_descs(t, out=[("stride", 0, (1 << 47) // 2)]) == _status("PA_ERR_UNSUPPORTED")
    assert _check_descs(t, k_cache=[("shape", 0, 1 << 48), ("stride", 0, 0)]) == _status("PA_ERR_UNSUPPORTED")
    # pools of 2^31 blocks (int32 block ids) and more than 65536 kv heads
    many = [("shape", 0, 1 << 31), ("stride", 0, 0)]
    assert _check_descs(t, k_cache=many, v_cache=many) == _status("PA_ERR_UNSUPPORTED")
    heads = [("shape", 2, 70000), ("stride", 2, 0)]
    assert _check_descs(t, k_cache=heads, v_cache=heads, q=heads, out=heads) == _status("PA_ERR_UNSUPPORTED")


def test_empty_batch_is_valid():
    t = _tensors()
    for k in ("q", "out", "block_tables", "context_lens", "query_lens"):
        t[k] = t[k][:0]
    assert _check(**t) == B.PA_OK


@pytest.mark.parametrize("shape", [
    (1, 32, 8, 128, 1, 32), (4, 32, 8, 128, 1, 512), (1, 64, 8, 128, 1, 8192),
    (16, 64, 8, 64, 1, 2048), (64, 64, 8, 128, 2, 1024), (3, 8, 8, 64, 4, 1),
    (1, 4, 1, 128, 1, 1 << 16), (0, 8, 2, 128, 1, 4), (64, 64, 8, 64, 1, 10), (256, 32, 8, 128, 2, 32),
])
def test_plan_properties(shape):
    b, hq, hkv, d, ql, w = shape
    p = B.paged_attn_plan(b, hq, hkv, d, ql, 16 * w)
    assert p["rows"] == hq // hkv * ql and p["row_tiles"] == (p["rows"] + 15) // 16
    hg = p["heads_per_group"]
    assert hkv % hg == 0 and 1 <= hg <= (8 if p["row_tiles"] == 1 else 4)
    seq_chunks = (16 * w + 31) // 32
    max_chunks = b * (hkv // hg) * seq_chunks
    n = p["workgroups"]
    assert n >= 1 and p["min_share_chunks"] >= 1
    assert n == 1 or n * p["min_share_chunks"] <= max_chunks          # no share below the minimum
    rg, cb, pl = p["reduce_rows"], p["reduce_col4"], p["reduce_lanes"]
    assert rg * cb * pl <= 256 and (hq // hkv) % rg == 0 and (d // 4) % cb == 0
    assert pl * 8 >= min(p["expected_partials"], 256)      # one round of loads (up to 32 lanes)
    if p["whole_segments"]:
        # one workgroup per short segment: no partials, no merge
        assert n == b * (hkv // hg) and n >= 256 and 16 * w <= 512
        assert p["reduce_groups"] == 0 and p["workspace_bytes"] == 0
    elif n > 1:
        assert p["reduce_groups"] == b * ql * hkv * (hq // hkv // rg) * (d // 4 // cb)
        assert p["workspace_bytes"] == 2 * n * hg * p["rows"] * (d + 1) * 4 + 4 * b
    else:
        assert p["reduce_groups"] == 0 and p["workspace_bytes"] == 0
    assert p == B.paged_attn_plan(b, hq, hkv, d, ql, 16 * w)      # deterministic


def test_plan_fills_the_device_for_long_single_sequence():
    p = B.paged_attn_plan(1, 64, 8, 128, 1, 16 * 8192, num_cus=256)
    assert p["workgroups"] * p["heads_per_group"] >= 1024          # at least one wave per SIMD
    small = B.paged_attn_plan(1, 64, 8, 128, 1, 16 * 8192, num_cus=8)
    assert small["workgroups"] < p["workgroups"]


def test_workgroup_and_share_overrides_and_reset():
    try:
        B.paged_attn_set_workgroups(5)
        p = B.paged_attn_plan(4, 32, 8, 128, 1, 16 * 512)
        assert p["workgroups"] == 5
        B.paged_attn_set_workgroups(1)
        p = B.paged_attn_plan(4, 32, 8, 128, 1, 16 * 512)
        assert p["workgroups"] == 1 and p["reduce_groups"] == 0 and p["workspace_bytes"] == 0
        B.paged_attn_set_workgroups(1 << 30)                      # capped by the chunk count
        p = B.paged_attn_plan(1, 32, 8, 128, 1, 16 * 32)
        assert p["workgroups"] == 16 // p["min_share_chunks"] * (8 // p["heads_per_group"])
        B.paged_attn_set_workgroups(0)
        B.paged_attn_set_min_share(4)
        p = B.paged_attn_plan(1, 32, 8, 128, 1, 16 * 32)
        assert p["min_share_chunks"] == 4 and p["workgroups"] * 4 <= 16 * (8 // p["heads_per_group"])
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_set_workgroups(-1)
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_set_min_share(-3)
    finally:
        B.paged_attn_set_workgroups(0)
        B.paged_attn_set_min_share(0)
    assert B.paged_attn_plan(1, 32, 8, 128, 1, 16 * 32)["min_share_chunks"] == 1


def test_heads_per_group_override():
    try:
        B.paged_attn_set_heads_per_group(2)
        assert B.paged_attn_plan(1, 64, 8, 128, 1, 16 * 8192)["heads_per_group"] == 2
        B.paged_attn_set_heads_per_group(3)                     # does not divide 8 kv heads
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_plan(1, 64, 8, 128, 1, 16 * 8192)
        B.paged_attn_set_heads_per_group(8)                     # 64 rows: at most 4 heads
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_plan(1, 64, 1, 128, 1, 16 * 8192)
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_set_heads_per_group(9)
    finally:
        B.paged_attn_set_heads_per_group(0)


def test_plan_grids():
    # about 8 chunks per wave, at least a quarter of the CUs, at most the
    # chip; the largest head group that still gives every CU a workgroup
    p = B.paged_attn_plan(1, 32, 8, 128, 1, 16 * 32)                  # one 512-token sequence
    assert p["heads_per_group"] == 1 and p["workgroups"] == 64    # latency bound: spread out
    p = B.paged_attn_plan(4, 32, 8, 128, 1, 16 * 512)                 # 4 x <= 8192 tokens
    assert p["heads_per_group"] == 2 and p["workgroups"] == 256
    p = B.paged_attn_plan(1, 64, 8, 128, 1, 16 * 8192)                # 131072 tokens, batch 1
    assert p["heads_per_group"] == 4 and p["workgroups"] == 256   # 256-byte rows: one wave per SIMD
    p = B.paged_attn_plan(16, 64, 8, 64, 1, 16 * 2048)                # fp8-sized rows, bf16 cache
    assert p["heads_per_group"] == 8 and p["workgroups"] == 256
    p = B.paged_attn_plan(16, 64, 8, 64, 1, 16 * 2048, kv_dtype="fp8_e4m3fn")
    assert p["heads_per_group"] == 8 and p["workgroups"] == 256   # whole token rows per workgroup
    p = B.paged_attn_plan(64, 64, 8, 128, 2, 16 * 1024)               # MTP verify
    assert p["heads_per_group"] == 4 and p["workgroups"] == 256
    p = B.paged_attn_plan(1, 64, 8, 128, 1, 16 * 8192, num_cus=8)     # a small device
    assert p["workgroups"] == 8


def test_plan_takes_whole_segments_when_short_and_many():
    # a 128-token window (at most 160 tokens read): 64 x 8 segments
    p = B.paged_attn_plan(64, 64, 8, 64, 1, 160)
    assert p["whole_segments"] == 1 and p["heads_per_group"] == 2 and p["workgroups"] == 256
    assert p["reduce_groups"] == 0 and p["workspace_bytes"] == 0
    # too few segments for the device, or segments too long: shares
    assert B.paged_attn_plan(64, 64, 8, 64, 1, 160, num_cus=1024)["whole_segments"] == 0
    assert B.paged_attn_plan(4, 64, 8, 64, 1, 160)["whole_segments"] == 0
    assert B.paged_attn_plan(64, 64, 8, 64, 1, 16 * 33)["whole_segments"] == 0
    assert B.paged_attn_plan(64, 64, 8, 64, 1, 16 * 32)["whole_segments"] == 1
    # a grid or share override keeps the split
    try:
        B.paged_attn_set_workgroups(7)
        assert B.paged_attn_plan(64, 64, 8, 64, 1, 160)["whole_segments"] == 0
    finally:
        B.paged_attn_set_workgroups(0)


def test_plan_rejects_chunk_index_overflow():
    with pytest.raises(B.PagedAttnError):
        B.paged_attn_plan(16384, 8, 8, 128, 1, 16 * 1 << 20)


def test_plan_keeps_whole_rows_when_halving_would_overflow_the_chunk_index():
    # 16384 sequences x 100000 chunks fit the 31-bit chunk index with one
    # head group but not with two, so the heads per workgroup stay whole;
    # a quarter of that context takes one wave per SIMD as usual
    p = B.paged_attn_plan(16384, 64, 8, 128, 1, 32 * 100000)
    assert p["heads_per_group"] == 8 and p["workgroups"] == 256
    p = B.paged_attn_plan(16384, 64, 8, 128, 1, 32 * 25000)
    assert p["heads_per_group"] == 4 and p["workgroups"] == 256


def test_plan_rejects_bad_sizes():
    with pytest.raises(B.PagedAttnError):
        B.paged_attn_plan(1, 6, 4, 128, 1, 16 * 4)
    with pytest.raises(B.PagedAttnError):
        B.paged_attn_plan(1, 8, 8, 128, 1, 16 * 0)


def test_check_metadata():
    ctx = torch.tensor([5, 33], dtype=torch.int32)
    ql = torch.tensor([1, 2], dtype=torch.int32)
    bt = torch.tensor([[3, 9, 9], [0, 1, 2]], dtype=torch.int32)
    B.paged_attn_check_metadata(ctx, ql, bt, 2, 10)
    B.paged_attn_check_metadata(ctx, None, bt, 2, 10)
    bad = [
        (torch.tensor([5, 49], dtype=torch.int32), ql, bt),              # L > 16 W
        (ctx, torch.tensor([1, 3], dtype=torch.int32), bt),              # n > Qmax
        (torch.tensor([0, 33], dtype=torch.int32), ql, bt),              # n > L
        (ctx, ql, torch.tensor([[3, 9, 9], [0, 10, 2]], dtype=torch.int32)),   # id >= NB
        (ctx, ql, torch.tensor([[-1, 9, 9], [0, 1, 2]], dtype=torch.int32)),   # id < 0
    ]
    for c, q, t in bad:
        with pytest.raises(B.PagedAttnError):
            B.paged_attn_check_metadata(c, q, t, 2, 10)
    # entries past ceil(L / 16) are never read, so anything goes there
    B.paged_attn_check_metadata(ctx, ql, torch.tensor([[3, -7, 99], [0, 1, 2]], dtype=torch.int32), 2, 10)


def test_check_metadata_block_size_and_window():
    ctx = torch.tensor([100, 64], dtype=torch.int32)
    ql = torch.tensor([1, 1], dtype=torch.int32)
    bt = torch.tensor([[-5, 3], [1, -1]], dtype=torch.int32)
    with pytest.raises(B.PagedAttnError):                          # entry 0 of row 0 holds keys
        B.paged_attn_check_metadata(ctx, ql, bt, 1, 4, block_size=64)
    # a 30-token window: row 0 sees keys 70..99 (entry 1 only), row 1 keys
    # 34..63 (entry 0 only)
    B.paged_attn_check_metadata(ctx, ql, bt, 1, 4, block_size=64, sliding_window=30)
    with pytest.raises(B.PagedAttnError):                          # row 1 sees entry 0 = -1
        B.paged_attn_check_metadata(ctx, ql, torch.tensor([[-5, 3], [-1, 2]], dtype=torch.int32), 1, 4,
                                    block_size=64, sliding_window=30)
    with pytest.raises(B.PagedAttnError):                          # L > block_size * W
        B.paged_attn_check_metadata(torch.tensor([129, 1], dtype=torch.int32), ql, bt, 1, 4, block_size=64,
                                    sliding_window=30)


def test_strerror_covers_every_status():
    for code in B.STATUS_NAMES:
        assert B.paged_attn_strerror(code) != "unknown status"
    assert B.paged_attn_strerror(12345) == "unknown status"


def _write_tensors(kv="bf16", T=5, hkv=HKV, d=D, block=16):
    kn = torch.zeros(T, hkv, d, dtype=torch.bfloat16)
    vn = torch.zeros(T, hkv, d, dtype=torch.bfloat16)
    sm = torch.zeros(T, dtype=torch.int32)
    cdt = torch.uint8 if kv == "fp8" else torch.bfloat16
    kc = torch.zeros(NB, block, hkv, d, dtype=cdt)
    vc = torch.zeros(NB, block, hkv, d, dtype=cdt)
    ks = vs = None
    if kv == "fp8":
        ks = torch.ones(NB, hkv, block).permute(0, 2, 1)
        vs = torch.ones(NB, hkv, block).permute(0, 2, 1)
    return dict(k_new=kn, v_new=vn, slot_mapping=sm, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_cache_write_validation_accepts_good_arguments(kv):
    assert B.paged_attn_check_reshape_and_cache(**_write_tensors(kv)) == B.PA_OK
    t = _write_tensors(kv, T=0)                                   # nothing to write
    assert B.paged_attn_check_reshape_and_cache(**t) == B.PA_OK
    for block in (32, 64, 256, 4096):
        assert B.paged_attn_check_reshape_and_cache(**_write_tensors(kv, block=block)) == B.PA_OK
    for block in (8, 24, 8192):
        assert B.paged_attn_check_reshape_and_cache(**_write_tensors(kv, block=block)) == \
            _status("PA_ERR_UNSUPPORTED")


def test_cache_write_validation_rejects_bad_arguments():
    def status(**over):
        t = _write_tensors(over.pop("kv", "bf16"))
        t.update(over)
        return B.STATUS_NAMES[B.paged_attn_check_reshape_and_cache(**t)]
    assert status(k_new=torch.zeros(5, HKV, D)) == "PA_ERR_DTYPE"                      # fp32 rows
    assert status(slot_mapping=torch.zeros(5, dtype=torch.int64)) == "PA_ERR_DTYPE"
    assert status(slot_mapping=torch.zeros(4, dtype=torch.int32)) == "PA_ERR_SHAPE"
    assert status(v_new=torch.zeros(5, HKV, 64, dtype=torch.bfloat16)) == "PA_ERR_SHAPE"
    assert status(k_cache=torch.zeros(NB, 8, HKV, D, dtype=torch.bfloat16),
                  v_cache=torch.zeros(NB, 8, HKV, D, dtype=torch.bfloat16)) == "PA_ERR_UNSUPPORTED"
    assert status(kv="fp8", k_scale=None) == "PA_ERR_NULL"
    assert status(k_scale=torch.ones(NB, 16, HKV)) == "PA_ERR_ARG"                    # scales with bf16
    assert status(kv="fp8", k_scale=torch.ones(NB, 16, HKV)) == "PA_ERR_LAYOUT"       # slot dim not contiguous
    assert status(k_new=torch.zeros(5, HKV, 2 * D, dtype=torch.bfloat16)[:, :, 1:D + 1]) == "PA_ERR_LAYOUT"
    assert status(k_new=None) == "PA_ERR_NULL"


def _prefill_tensors(T=20, hq=8, hkv=2, d=128, block=16, B_=3):
    q = torch.zeros(T, hq, d, dtype=torch.bfloat16)
    kc = torch.zeros(NB, block, hkv, d, dtype=torch.bfloat16)
    vc = torch.zeros(NB, block, hkv, d, dtype=torch.bfloat16)
    bt = torch.zeros(B_, W, dtype=torch.int32)
    ctx = torch.full((B_,), 30, dtype=torch.int32)
    cu = torch.tensor([0, 5, 12, T][:B_ + 1], dtype=torch.int32)
    return dict(q=q, k_cache=kc, v_cache=vc, block_tables=bt, context_lens=ctx, cu_seqlens_q=cu,
                max_query_len=8, scale=0.1, out=torch.empty_like(q))


def test_prefill_validation():
    def status(**over):
        t = _prefill_tensors()
        t.update(over)
        return B.STATUS_NAMES[B.paged_attn_check_prefill(**t)]
    assert status() == "PA_OK"
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**_prefill_tensors(d=64, hq=64, hkv=1))] == "PA_OK"
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**_prefill_tensors(block=64))] == "PA_OK"
    assert status(cu_seqlens_q=torch.tensor([0, 5, 20], dtype=torch.int32)) == "PA_ERR_SHAPE"     # B + 1 entries
    assert status(cu_seqlens_q=torch.tensor([0, 5, 12, 20], dtype=torch.int64)) == "PA_ERR_DTYPE"
    assert status(max_query_len=-1) == "PA_ERR_ARG"
    assert status(scale=float("nan")) == "PA_ERR_ARG"
    assert status(out=torch.zeros(19, 8, 128, dtype=torch.bfloat16)) == "PA_ERR_SHAPE"
    # fp8: both caches e4m3fn, with fp32 scales [NB, 16, Hkv] whose slot dimension is contiguous
    k8, v8 = (torch.zeros(NB, 16, 2, 128, dtype=torch.uint8) for _ in range(2))
    sc = torch.ones(NB, 2, 16).permute(0, 2, 1)
    assert status(k_cache=k8) == "PA_ERR_DTYPE"                                  # v_cache still bf16
    assert status(k_cache=k8, v_cache=v8) == "PA_ERR_NULL"                       # no scales
    assert status(k_cache=k8, v_cache=v8, k_scale=sc, v_scale=sc) == "PA_OK"
    assert status(k_cache=k8, v_cache=v8, k_scale=sc[:, :8], v_scale=sc) == "PA_ERR_SHAPE"
    assert status(k_cache=k8, v_cache=v8, k_scale=torch.ones(NB, 16, 2), v_scale=sc) == "PA_ERR_LAYOUT"   # slots strided
    assert status(k_scale=torch.ones(NB, 16, 2)) == "PA_ERR_ARG"
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**_prefill_tensors(d=256))] == "PA_OK"
    t = _prefill_tensors(d=256, hq=64, hkv=2)                                         # ratio 32 > 16 at head_dim 256
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**t)] == "PA_ERR_UNSUPPORTED"
    t = _prefill_tensors(d=96)
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**t)] == "PA_ERR_UNSUPPORTED"
    t = _prefill_tensors(hq=6, hkv=4)
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**t)] == "PA_ERR_UNSUPPORTED"
    t = _prefill_tensors(hq=130, hkv=1)
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**t)] == "PA_ERR_UNSUPPORTED"                 # ratio > 64
    t = _prefill_tensors()
    t["q"] = t["q"].transpose(1, 2).contiguous().transpose(1, 2)
    t["out"] = torch.empty_like(t["q"])
    assert B.STATUS_NAMES[B.paged_attn_check_prefill(**t)] == "PA_ERR_LAYOUT"


def test_prefill_ext_validation():
    """paged_attn_check_prefill_ext: the window is free (<= 0 is none);
    sinks are fp32 [Hq], 4-byte aligned."""
    def status(**over):
        t = _prefill_tensors()
        t.update(over)
        return B.STATUS_NAMES[B.paged_attn_check_prefill_ext(**t)]
    hq = _prefill_tensors()["q"].shape[1]
    assert status() == "PA_OK"
    assert status(sliding_window=128, sinks=torch.zeros(hq)) == "PA_OK"
    assert status(sliding_window=-1) == "PA_OK"
    assert status(sinks=torch.zeros(hq + 1)) == "PA_ERR_SHAPE"
    assert status(sinks=torch.zeros(hq, dtype=torch.bfloat16)) == "PA_ERR_DTYPE"
    assert status(sinks=torch.zeros(hq, 1)) == "PA_ERR_SHAPE"
    assert status(sinks=torch.zeros(2 * hq)[1::2]) == "PA_OK"                 # any stride


def test_prefill_flops_closed_form():
    from paged_attention_decode_attn_amd.workloads import prefill_flops
    # a whole prompt of n tokens: n (n + 1) / 2 (row, key) pairs
    assert prefill_flops([100], [100], 8, 64) == 4 * 64 * 8 * 5050
    # a chunk of 10 after 90 cached tokens: rows see 91 .. 100 keys
    assert prefill_flops([100], [10], 1, 1) == 4 * sum(range(91, 101))
    assert prefill_flops([5, 7], [0, 7], 2, 2) == 4 * 2 * 2 * 28


def test_prefill_flops_with_a_window_matches_counting():
    """With a sliding window w the row at position a sees min(a + 1, w) keys:
    the closed form against a plain count over the rows."""
    import random
    from paged_attention_decode_attn_amd.workloads import prefill_flops
    rng = random.Random(0)
    for _ in range(500):
        L = rng.randint(0, 300)
        n = rng.randint(0, L)
        w = rng.choice([0, -1, 1, 2, 3, 7, 50, 400])
        count = sum((a + 1) if w <= 0 else min(a + 1, w) for a in range(L - n, L))
        assert prefill_flops([L], [n], 1, 1, w) == 4 * count, (L, n, w)

"""GPU parity of the shape variants against the CPU oracle: cache blocks of
any multiple of 16 tokens, a sliding window, per-head attention sinks, and
their combinations with fp8 caches, speculative query rows and every split
of the work.  Same tolerance as the main parity suite: |gpu - ref| <= 1e-2 +
1e-2 |ref| on every produced element, relative L2 <= 1e-2, and rows past
query_len keep a canary."""
import numpy as np
import pytest
import torch

from _parity import check, compare, note, oracle_out, run_gpu
from paged_attention_decode_attn_amd import binding as B
from paged_attention_decode_attn_amd.workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _ragged(block_size=16, kv="bf16", qlen=2, qlen_lo=None, window=0, sinks=False, batch=6, ctx_hi=2000,
            hq=64, hkv=8, d=128, seed=5):
    blocks = batch * (-(-ctx_hi // block_size)) + 4
    return CONFIGS["mtp_verify"].replace(batch=batch, qlen=qlen, qlen_lo=qlen_lo, hq=hq, hkv=hkv, head_dim=d,
                                         kv_dtype=kv, ctx_lo=qlen, ctx_hi=ctx_hi, pool_blocks=blocks,
                                         block_size=block_size, sliding_window=window, sinks=sinks, seed=seed)


# --------------------------------------------------------------------------
# block sizes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [32, 48, 64, 256, 4096])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_block_sizes(bs, kv):
    w = generate(_ragged(bs, kv, d=128 if kv == "bf16" else 64))
    for groups in (0, 1, 7, 100000):
        check(w, groups, label=f"bs{bs}/{kv}/g{groups}")


@pytest.mark.parametrize("bs", [64, 256])
def test_block_size_edges_and_poison(bs):
    ctx = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1025]
    spec = CONFIGS["llama3_8b"].replace(batch=len(ctx), ctx_lo=1, ctx_hi=1025, block_size=bs,
                                        pool_blocks=len(ctx) * (-(-1025 // bs)) + 2)
    w = generate(spec, context_lens=ctx, poison=True)
    for groups in (0, 1, 5, 100000):
        check(w, groups, label=f"bs{bs}/edges/g{groups}")


# --------------------------------------------------------------------------
# sliding window and sinks
# --------------------------------------------------------------------------
SHAPES = {"q1": dict(qlen=1), "q2": dict(qlen=2), "q4_ragged": dict(qlen=4, qlen_lo=1)}


@pytest.mark.parametrize("window", [1, 5, 31, 32, 33, 128, 1000])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_sliding_window(window, shape):
    w = generate(_ragged(window=window, sinks=window % 2 == 1, seed=window, **SHAPES[shape]))
    for groups in (0, 7, 100000):
        check(w, groups, label=f"window{window}/{shape}/g{groups}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("bs", [16, 64])
def test_window_sinks_fp8_and_block_size(kv, bs):
    w = generate(_ragged(bs, kv, qlen=2, window=100, sinks=True, d=64, ctx_hi=1500, seed=20 + bs))
    for groups in (0, 1, 9, 100000):
        check(w, groups, label=f"window100+sinks/{kv}/bs{bs}/g{groups}")


@pytest.mark.parametrize("groups", [0, 1, 7, 100000])
def test_sinks_on_full_attention(groups):
    # direct rows (one share) add the sink in the partition kernel's
    # epilogue, split rows in the merge
    w = generate(_ragged(qlen=2, sinks=True, seed=31))
    check(w, groups, label=f"sinks/g{groups}")


def test_sink_extremes():
    w = generate(_ragged(qlen=1, sinks=True, batch=4, ctx_hi=800, seed=32))
    s = w.sinks.clone()
    s[0::4] = -float("inf")          # sink off
    s[1::4] = 60.0                   # dominates: output near zero
    s[2::4] = -60.0                  # negligible
    w.sinks = s
    for groups in (0, 1, 100000):
        check(w, groups, label=f"sink-extremes/g{groups}")


@pytest.mark.parametrize("bs", [16, 48])
@pytest.mark.parametrize("kv,d", [("bf16", 128), ("bf16", 64), ("fp8_e4m3fn", 64), ("fp8_e4m3fn", 128)])
def test_window_never_reads_what_lies_below_it(bs, kv, d):
    # Blocks wholly below the earliest row's window are freed in a windowed
    # cache: their table entries hold garbage ids and the blocks NaN.  The
    # token rows below the window in the block holding its first key hold
    # NaN as well (and, for fp8, NaN codes and scales).  The output must
    # equal the oracle's on the intact cache.
    window = 40
    spec = _ragged(bs, kv=kv, d=d, qlen=2, window=window, sinks=True, batch=5, ctx_hi=600, seed=33)
    lens = [2, 45, 100, 333, 600]
    w = generate(spec, context_lens=lens)
    ref = oracle_out(w)
    bad = generate(spec, context_lens=lens)
    t = bad.block_tables.clone()
    fp8 = kv != "bf16"

    def poison(blk, rows=slice(None)):
        for c in (bad.k_cache, bad.v_cache):
            if fp8:
                c[blk, rows].view(torch.uint8).fill_(0x7F)
            else:
                c[blk, rows].view(torch.int16).fill_(0x7FC0)
        if fp8:
            bad.k_scale[blk, rows] = float("nan")
            bad.v_scale[blk, rows] = float("nan")

    for b in range(spec.batch):
        L, n = int(bad.context_lens[b]), int(bad.query_lens[b])
        lo = max(0, L - n - window + 1)
        for i in range(lo // bs):
            poison(int(t[b, i]))
            t[b, i] = -7 if i % 2 else 1 << 30
        if lo % bs:
            poison(int(t[b, lo // bs]), slice(0, lo % bs))
    bad.block_tables = t
    for groups in (0, 1, 100000):
        note(f"[gpu] freed-below-window/{kv}/d{d}/bs{bs}/g{groups}")
        out = run_gpu(bad, groups)
        compare(out, ref, w.query_lens, label=f"freed-below-window/{kv}/d{d}/bs{bs}/g{groups}")


@pytest.mark.parametrize("hq,hkv,qlen", [(8, 8, 1), (32, 32, 2), (64, 1, 1), (16, 1, 4)])
def test_window_head_groupings(hq, hkv, qlen):
    w = generate(_ragged(qlen=qlen, hq=hq, hkv=hkv, window=70, sinks=True, batch=3, ctx_hi=700, seed=34))
    check(w, 0, label=f"window/heads{hq}/{hkv}/q{qlen}")
    check(w, 11, label=f"window/heads{hq}/{hkv}/q{qlen}/g11")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_whole_segments_with_window(kv, shape):
    # 64 sequences x 8 kv heads of short windowed ranges: one workgroup per
    # segment, no merge
    spec = _ragged(kv=kv, window=100, sinks=True, batch=64, ctx_hi=900, d=64 if kv != "bf16" else 128,
                   seed=40, **SHAPES[shape])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    max_ctx = 32 * (-(-(100 + spec.qlen - 1) // 32) + 1)
    plan = B.paged_attn_plan(spec.batch, spec.hq, spec.hkv, spec.head_dim, spec.qlen, max_ctx, kv, cus)
    assert plan["whole_segments"] == 1
    check(generate(spec), 0, label=f"whole/window/{kv}/{shape}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("bs", [16, 64])
def test_whole_segments_with_short_tables(kv, bs):
    # tables of at most 512 tokens and 64 sequences: whole segments without
    # a window (the general kernel variant with 16-token blocks)
    spec = _ragged(bs, kv, qlen=2, batch=64, ctx_hi=512, d=128, seed=41 + bs)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = B.paged_attn_plan(spec.batch, spec.hq, spec.hkv, spec.head_dim, spec.qlen,
                             bs * spec.table_width, kv, cus)
    assert plan["whole_segments"] == 1
    w = generate(spec)
    check(w, 0, label=f"whole/short/{kv}/bs{bs}")
    check(w, 5, label=f"whole/short/{kv}/bs{bs}/split")          # an override keeps the split


# --------------------------------------------------------------------------
# head_dim 256
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("hq,hkv,qlen,qlen_lo", [(16, 8, 1, None), (16, 2, 2, None), (8, 1, 2, 1), (4, 4, 4, None),
                                                 (16, 1, 1, None)])
def test_head_dim_256(kv, hq, hkv, qlen, qlen_lo):
    w = generate(_ragged(kv=kv, qlen=qlen, qlen_lo=qlen_lo, hq=hq, hkv=hkv, d=256, batch=4, ctx_hi=1200,
                         seed=50 + hq + qlen))
    for groups in (0, 1, 7, 100000):
        check(w, groups, label=f"d256/{hq}/{hkv}/q{qlen}/{kv}/g{groups}")


@pytest.mark.parametrize("bs", [16, 64])
def test_head_dim_256_window_sinks_and_whole_segments(bs):
    w = generate(_ragged(bs, qlen=2, hq=16, hkv=2, d=256, window=50, sinks=True, batch=4, ctx_hi=900, seed=60))
    for groups in (0, 3, 100000):
        check(w, groups, label=f"d256/window/bs{bs}/g{groups}")
    spec = _ragged(bs, qlen=1, hq=16, hkv=8, d=256, window=64, sinks=True, batch=64, ctx_hi=600, seed=61)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert B.paged_attn_plan(64, 16, 8, 256, 1, 128, "bf16", cus)["whole_segments"] == 1
    check(generate(spec), 0, label=f"d256/whole/bs{bs}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("hq,hkv,qlen,qlen_lo", [(32, 2, 2, None), (16, 2, 4, 1), (48, 8, 4, None), (64, 4, 4, None),
                                                 (32, 1, 2, None), (17 * 2, 2, 1, None)])
def test_head_dim_256_more_than_16_rows(kv, hq, hkv, qlen, qlen_lo):
    # ceil(rows / 16) waves per kv head, each one 16-row tile (24 rows: the
    # second tile half full; 17 rows: one row in the second tile)
    w = generate(_ragged(kv=kv, qlen=qlen, qlen_lo=qlen_lo, hq=hq, hkv=hkv, d=256, batch=4, ctx_hi=1200,
                         seed=70 + hq + qlen))
    for groups in (0, 1, 7, 100000):
        check(w, groups, label=f"d256/{hq}/{hkv}/q{qlen}/{kv}/g{groups}")


@pytest.mark.parametrize("hg", [1, 2])
def test_head_dim_256_32_rows_heads_per_group(hg):
    w = generate(_ragged(qlen=4, hq=32, hkv=4, d=256, batch=5, ctx_hi=900, seed=75))
    for groups in (0, 3, 100000):
        check(w, groups, label=f"d256/32rows/hg{hg}/g{groups}", heads_per_group=hg)


@pytest.mark.parametrize("bs", [16, 64])
def test_head_dim_256_32_rows_window_sinks_whole_segments_and_many_sequences(bs):
    w = generate(_ragged(bs, qlen=2, hq=32, hkv=2, d=256, window=50, sinks=True, batch=4, ctx_hi=900, seed=76))
    for groups in (0, 3, 100000):
        check(w, groups, label=f"d256/32rows/window/bs{bs}/g{groups}")
    spec = _ragged(bs, qlen=4, qlen_lo=1, hq=64, hkv=8, d=256, window=64, sinks=True, batch=64, ctx_hi=600, seed=77)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = B.paged_attn_plan(64, 64, 8, 256, 4, 128, "bf16", cus)
    assert plan["whole_segments"] == 1 and plan["row_waves"] == 2
    check(generate(spec), 0, label=f"d256/32rows/whole/bs{bs}")
    # more than 64 sequences: the chunk scan goes through LDS
    w = generate(_ragged(bs, qlen=2, hq=32, hkv=2, d=256, batch=70, ctx_hi=300, seed=78))
    for groups in (0, 5):
        check(w, groups, label=f"d256/32rows/b70/bs{bs}/g{groups}")


def test_ext_without_window_or_sinks_equals_decode_bitwise():
    w = generate(_ragged(qlen=2, seed=35)).to("cuda")
    a = torch.empty_like(w.q)
    b = torch.empty_like(w.q)
    note("[gpu] ext == decode")
    B.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.query_lens, w.scale,
                        None, None, a)
    B.paged_attn_decode_ext(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.query_lens, w.scale,
                            None, None, -1, None, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_window_graph_capture_replays_match_eager():
    w = generate(_ragged(qlen=2, window=64, sinks=True, seed=36))
    dev = w.to("cuda")
    s = torch.cuda.Stream()
    note("[gpu] window graph capture")
    eager = torch.empty_like(dev.q)
    with torch.cuda.stream(s):
        B.paged_attn_decode_ext(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                                dev.query_lens, dev.scale, None, None, 64, dev.sinks, eager)
    s.synchronize()
    compare(eager, oracle_out(w), w.query_lens, label="window-graph/eager")
    out = torch.empty_like(dev.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.paged_attn_decode_ext(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                                dev.query_lens, dev.scale, None, None, 64, dev.sinks, out)
    torch.cuda.synchronize()
    for r in range(3):
        out.view(torch.int16).fill_(0x7F7B)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"


def test_sinks_argument_errors_launch_nothing():
    w = generate(_ragged(qlen=1, sinks=True, batch=2, ctx_hi=100, seed=37)).to("cuda")
    out = torch.full_like(w.q, 3.0)
    note("[gpu] sinks argument errors")
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_decode_ext(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.query_lens,
                                w.scale, None, None, 0, w.sinks[:-1], out)
    assert e.value.name == "PA_ERR_SHAPE"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_decode_ext(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.query_lens,
                                w.scale, None, None, 0, w.sinks.to(torch.bfloat16), out)
    assert e.value.name == "PA_ERR_DTYPE"
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)

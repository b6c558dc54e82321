"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name, shapes and split overrides before it touches the
GPU.  The split overrides force the work division through its cases: one
workgroup (every segment whole, many per share, block-table windows
reloaded), a few workgroups (shares cut sequences at ragged points, so a
workgroup leaves partials in both its slots), and more workgroups than
chunks (one chunk per share, the most partials per row).  Tolerance: |gpu - ref| <= 1e-2 + 1e-2 |ref| on every produced element
(bf16 output vs the float64 oracle on the same stored bytes), plus a
relative-L2 bound of 1e-2; rows past query_len must keep a canary.
"""
import numpy as np
import pytest
import torch

from _parity import check, compare, note, oracle_out, run_gpu, small
from paged_attention_decode_attn_amd import binding as B
from paged_attention_decode_attn_amd.workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# the five workload shapes at oracle-friendly sizes (several tiles, ragged tails)
# --------------------------------------------------------------------------
SMALL = {
    "tiny": CONFIGS["tiny"],
    "llama3_8b": small("llama3_8b", ctx_lo=100, ctx_hi=1500, pool_blocks=400),
    "long_ctx": small("long_ctx", ctx_lo=20001, ctx_hi=20001, pool_blocks=1300),
    "fp8": small("fp8", batch=5, ctx_lo=100, ctx_hi=3000, pool_blocks=1000),
    "mtp_verify": small("mtp_verify", batch=6, ctx_lo=2, ctx_hi=2000, pool_blocks=800),
    # wider and ragged speculative verification (32 query rows per kv head)
    "mtp_verify_q4": small("mtp_verify_q4", batch=6, ctx_lo=4, ctx_hi=2000, pool_blocks=800),
    "mtp_verify_ragged": small("mtp_verify_ragged", batch=9, ctx_lo=4, ctx_hi=2000, pool_blocks=1200),
    # shape variants: 256-token blocks, multi-head, sliding window + sinks, sinks
    "long_ctx_bs256": small("long_ctx_bs256", ctx_lo=20001, ctx_hi=20001, pool_blocks=90),
    "mha": small("mha", batch=3, ctx_lo=100, ctx_hi=1500, pool_blocks=300),
    "swa_sinks": small("swa_sinks", batch=7, ctx_lo=1, ctx_hi=3000, pool_blocks=1400),
    "full_sinks": small("full_sinks", batch=5, ctx_lo=100, ctx_hi=3000, pool_blocks=1000),
    "d256": small("d256", batch=3, ctx_lo=100, ctx_hi=1500, pool_blocks=300),
    # head_dim 256 with 32 rows per kv head: two waves per kv head
    "d256_mtp": small("d256_mtp", batch=5, ctx_lo=4, ctx_hi=1500, pool_blocks=480),
}


# workgroup-count overrides: 0 = the planner's grid, 1 = one share for all,
# 7 / 100 = ragged cuts, 100000 = capped at one chunk per share
SPLITS = [0, 1, 7, 100, 100000]


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("groups", SPLITS)
def test_config_shapes(name, groups):
    w = generate(SMALL[name])
    check(w, groups, label=f"{name}/g{groups}")


@pytest.mark.parametrize("hg", [1, 2, 4, 8])
@pytest.mark.parametrize("groups", [13, 100000])
def test_heads_per_workgroup(hg, groups):
    # every kv-head grouping of the workgroups, ragged batches
    for name in ("mtp_verify", "fp8"):
        w = generate(SMALL[name])
        check(w, groups, label=f"hg{hg}/{name}/g{groups}", heads_per_group=hg)


def test_calls_of_different_shapes_alternate_on_one_stream():
    # one stream's workspace serves calls of every plan, whose layouts of
    # partials, log-sum-exps and chunk prefix differ
    names = ("long_ctx", "mtp_verify", "fp8", "llama3_8b", "mha", "d256", "d256_mtp", "long_ctx_bs256")
    ws = {n: generate(SMALL[n]) for n in names}
    refs = {n: oracle_out(w) for n, w in ws.items()}
    for rnd in range(3):
        for n in names if rnd % 2 == 0 else reversed(names):
            note(f"[gpu] alternating shapes: round {rnd} {n}")
            out = run_gpu(ws[n])
            compare(out, refs[n], ws[n].query_lens, label=f"alternate{rnd}/{n}")


@pytest.mark.parametrize("share", [2, 3, 40])
def test_min_share(share):
    for name in ("llama3_8b", "fp8", "long_ctx"):
        w = generate(SMALL[name])
        check(w, 0, label=f"share{share}/{name}", min_share=share)
        check(w, 100000, label=f"share{share}/{name}/g100000", min_share=share)


# --------------------------------------------------------------------------
# edge suite
# --------------------------------------------------------------------------
EDGE_CTX = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 1023, 1024, 1025]


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("groups", [0, 1, 5, 100000])
def test_context_length_edges(kv, groups):
    spec = CONFIGS["llama3_8b"].replace(batch=len(EDGE_CTX), ctx_lo=1, ctx_hi=1025,
                                        pool_blocks=300, kv_dtype=kv)
    w = generate(spec, context_lens=EDGE_CTX)
    check(w, groups, label=f"edges/{kv}/g{groups}")


@pytest.mark.parametrize("groups", [0, 1, 3, 100000])
def test_two_query_rows_short_and_ragged(groups):
    ctx = [2, 2, 3, 17, 33, 64, 100, 5]
    ql = [2, 1, 0, 2, 1, 2, 0, 2]
    spec = CONFIGS["mtp_verify"].replace(batch=8, ctx_lo=2, ctx_hi=100, pool_blocks=64)
    w = generate(spec, context_lens=ctx, query_lens=ql)
    check(w, groups, label=f"qlen2-ragged/g{groups}")


@pytest.mark.parametrize("batch", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("groups", [0, 7, 100000])
def test_batches_across_the_one_wave_scan(batch, groups):
    # up to 64 sequences every wave scans the chunk counts in its own lanes;
    # more go through the workgroup's LDS scan.  Ragged lengths with empty
    # sequences and query rows, contexts long enough for the split schedule.
    rng = np.random.default_rng(900 + batch)
    ctx = rng.integers(1, 1300, size=batch)
    ctx[rng.random(batch) < 0.1] = 0
    ql = np.minimum(rng.integers(0, 3, size=batch), ctx)
    spec = CONFIGS["mtp_verify"].replace(batch=batch, ctx_lo=1, ctx_hi=1300, hq=16, hkv=2, head_dim=64,
                                         pool_blocks=batch * 82 + 4)
    w = generate(spec, context_lens=ctx.tolist(), query_lens=ql.tolist())
    check(w, groups, label=f"batch{batch}/g{groups}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv,qlen", [(8, 8, 1), (8, 1, 1), (32, 8, 1), (64, 4, 1),
                                         (64, 8, 2), (16, 1, 2), (16, 1, 3), (32, 1, 2),
                                         (64, 1, 1), (12, 3, 3)])
def test_head_groupings(kv, d, hq, hkv, qlen):
    spec = CONFIGS["mtp_verify"].replace(batch=3, qlen=qlen, hq=hq, hkv=hkv, head_dim=d,
                                         kv_dtype=kv, ctx_lo=qlen, ctx_hi=300, pool_blocks=64)
    w = generate(spec)
    check(w, 0, label=f"heads{hq}/{hkv}/q{qlen}/d{d}/{kv}")
    check(w, 11, label=f"heads{hq}/{hkv}/q{qlen}/d{d}/{kv}/g11")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_nan_in_unread_memory_never_reaches_output(kv):
    spec = CONFIGS["mtp_verify"].replace(batch=5, ctx_lo=2, ctx_hi=500, pool_blocks=200, kv_dtype=kv)
    w = generate(spec, poison=True)
    for groups in (0, 1, 9, 100000):
        check(w, groups, label=f"poison/{kv}/g{groups}")


def test_shared_and_duplicated_blocks():
    spec = CONFIGS["mtp_verify"].replace(batch=3, ctx_lo=40, ctx_hi=200, pool_blocks=64)
    w = generate(spec, context_lens=[200, 180, 120])
    t = w.block_tables.clone()
    t[1, :5] = t[0, :5]           # shared prefix
    t[2, 3] = t[2, 1]             # duplicated entry within a row
    w.block_tables = t
    for groups in (0, 1, 100000):
        check(w, groups, label=f"shared/g{groups}")


@pytest.mark.parametrize("name", ["llama3_8b", "fp8", "mtp_verify", "swa_sinks", "d256"])
@pytest.mark.parametrize("scale", [-0.0883883, -0.5, 0.0])
def test_negative_and_zero_softmax_scale(name, scale):
    # a negative scale flips the sign of every logit (the kernels negate q);
    # zero makes every visible key weigh the same (the mean of V, or with
    # sinks the mean shrunk by e^s)
    w = generate(SMALL[name])
    w.scale = scale
    for groups in (0, 100000):
        check(w, groups, label=f"scale{scale}/{name}/g{groups}")


@pytest.mark.parametrize("factor", [4.0, 8.0])
def test_sharpened_queries(factor):
    for name in ("llama3_8b", "fp8", "mtp_verify"):
        w = generate(SMALL[name])
        w.q = (w.q.float() * factor).to(torch.bfloat16)     # power of two: exact
        check(w, 0, label=f"sharp{factor}/{name}")
        check(w, 100000, label=f"sharp{factor}/{name}/g100000")


def test_huge_logit_spread_between_heads():
    w = generate(SMALL["llama3_8b"].replace(batch=2))
    q = w.q.float()
    q[:, :, 0] *= 64.0
    w.q = q.to(torch.bfloat16)
    check(w, 0, label="logit-spread")
    check(w, 100000, label="logit-spread/g100000")


def test_rank3_query_and_strided_output():
    w = generate(SMALL["llama3_8b"])
    dev = w.to("cuda")
    big = torch.empty(w.q.shape[0], 3, w.q.shape[2], w.q.shape[3] + 64, dtype=torch.bfloat16,
                      device="cuda")
    big.fill_(7.0)
    out = big[:, 1, :, 32:32 + w.q.shape[3]]                 # rank 3, strided, 64 B aligned
    q3 = dev.q[:, 0]
    note("[gpu] rank3/strided")
    B.paged_attn_decode(q3, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                        None, w.scale, None, None, out)
    torch.cuda.synchronize()
    ref = oracle_out(w)
    compare(out[:, None], ref, torch.ones(w.q.shape[0], dtype=torch.int32), label="rank3")
    assert torch.all(big[:, 0] == 7.0) and torch.all(big[:, 2] == 7.0)
    assert torch.all(big[:, 1, :, :32] == 7.0) and torch.all(big[:, 1, :, 32 + w.q.shape[3]:] == 7.0)


def test_size_one_dims_may_carry_any_stride():
    # one sequence, one query row: the batch and query dims of q/out, the
    # table's row dim and the length vectors have size 1, so their strides
    # are never used, whatever they are (odd, huge); the output is bitwise
    # the contiguous call's
    w = generate(SMALL["tiny"])
    dev = w.to("cuda")
    assert dev.q.shape[:2] == (1, 1)
    ref = run_gpu(w)
    H, D = dev.q.shape[2], dev.q.shape[3]
    odd = 999999937
    q = torch.as_strided(dev.q, dev.q.shape, (odd, 12345, D, 1))
    out_buf = torch.empty(H * D, dtype=torch.bfloat16, device="cuda")
    out = torch.as_strided(out_buf, dev.q.shape, (odd, 777, D, 1))
    bt = torch.as_strided(dev.block_tables, dev.block_tables.shape, (odd, 1))
    ctx = torch.as_strided(dev.context_lens, (1,), (odd,))
    ql = torch.as_strided(dev.query_lens, (1,), (12345,))
    note("[gpu] size-1 dims with odd strides")
    B.paged_attn_decode(q, dev.k_cache, dev.v_cache, bt, ctx, ql, w.scale, None, None, out)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous().view(torch.int16).cpu(), ref.view(torch.int16).cpu())


def test_empty_batch_is_a_no_op():
    w = generate(SMALL["tiny"]).to("cuda")
    note("[gpu] empty batch")
    out = torch.empty_like(w.q[:0])
    B.paged_attn_decode(w.q[:0], w.k_cache, w.v_cache, w.block_tables[:0], w.context_lens[:0],
                        w.query_lens[:0], w.scale, None, None, out)
    torch.cuda.synchronize()


def test_fp8_every_code_decodes_exactly():
    # single-token context: the output row is the (scaled) value row itself
    spec = CONFIGS["fp8"].replace(batch=1, hq=4, hkv=4, head_dim=64, ctx_lo=1, ctx_hi=16,
                                  pool_blocks=4)
    w = generate(spec, context_lens=[1])
    blk = int(w.block_tables[0, 0])
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(4, 64)
    w.v_cache[blk, 0] = codes
    w.v_scale[blk, 0] = 1.0
    note("[gpu] fp8 codes")
    out = run_gpu(w).float().cpu()[0, 0]                       # [4 heads, 64]
    expect = codes.view(torch.float8_e4m3fn).float()
    nan = torch.isnan(expect)
    assert torch.equal(torch.isnan(out), nan)
    assert torch.equal(out[~nan], expect[~nan])
    # a power-of-two scale stays exact
    w.v_scale[blk, 0] = 0.25
    out = run_gpu(w).float().cpu()[0, 0]
    assert torch.equal(out[~nan], expect[~nan] * 0.25)


def test_bf16_single_token_returns_value_row_exactly():
    spec = CONFIGS["tiny"].replace(ctx_lo=1, ctx_hi=1, pool_blocks=4)
    w = generate(spec)
    note("[gpu] bf16 single token")
    out = run_gpu(w).cpu()[0, 0]                                # [32, 128]
    v = w.v_cache[int(w.block_tables[0, 0]), 0]                 # [8, 128]
    assert torch.equal(out.view(torch.int16), v.repeat_interleave(4, dim=0).view(torch.int16))


def test_repeat_calls_are_bitwise_identical_and_stream_ordered():
    w = generate(SMALL["mtp_verify"]).to("cuda")
    s = torch.cuda.Stream()
    outs = []
    note("[gpu] determinism / side stream")
    with torch.cuda.stream(s):
        for _ in range(3):
            o = torch.empty_like(w.q)
            B.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                w.query_lens, w.scale, None, None, o)
            outs.append(o)
    s.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_argument_errors_launch_nothing():
    w = generate(SMALL["tiny"]).to("cuda")
    out = torch.full_like(w.q, 3.0)
    note("[gpu] argument errors")
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                            w.query_lens, float("nan"), None, None, out)
    assert e.value.name == "PA_ERR_ARG"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_decode(w.q, w.k_cache, w.v_cache.float(), w.block_tables, w.context_lens,
                            w.query_lens, w.scale, None, None, out)
    assert e.value.name == "PA_ERR_DTYPE"
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_profile_events_measure_both_kernels():
    w = generate(SMALL["llama3_8b"]).to("cuda")
    note("[gpu] profile events")
    B.paged_attn_profile_begin(4)
    for _ in range(3):
        B.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                            w.query_lens, w.scale)
    r = B.paged_attn_profile_end()
    assert r["calls"] == 3 and r["partition_ms"] > 0 and r["reduce_ms"] > 0


# --------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark
# times, checked on sampled sequences
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,subset", [
    ("tiny", None), ("llama3_8b", None), ("long_ctx", None), ("fp8", [0, 7, 15]),
    ("mtp_verify", [0, 21, 63]), ("mtp_verify_q4", [0, 33, 63]), ("mtp_verify_ragged", [1, 30, 62]),
    ("long_ctx_bs256", None), ("mha", [0, 5]), ("swa_sinks", [0, 17, 40, 63]), ("full_sinks", [2, 9, 15]),
    ("d256", [0, 7]), ("d256_mtp", [0, 9, 15]),
])
def test_full_size_configs_sampled(name, subset):
    w = generate(CONFIGS[name])
    check(w, 0, batch_subset=subset, label=f"full/{name}")


# --------------------------------------------------------------------------
# graph capture: the call is graph-safe once its workspace exists
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["mtp_verify", "d256_mtp"])
def test_graph_capture_replays_match_eager(name):
    w = generate(SMALL[name])
    dev = w.to("cuda")
    ref = oracle_out(w)
    s = torch.cuda.Stream()
    note("[gpu] graph capture: eager warm-up on the capture stream")
    eager = torch.empty_like(dev.q)
    with torch.cuda.stream(s):
        B.paged_attn_decode(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                            dev.query_lens, dev.scale, None, None, eager)
    s.synchronize()
    compare(eager, ref, w.query_lens, label="graph/eager")
    out = torch.empty_like(dev.q)
    g = torch.cuda.CUDAGraph()
    note("[gpu] graph capture: capturing")
    with torch.cuda.graph(g, stream=s):
        B.paged_attn_decode(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                            dev.query_lens, dev.scale, None, None, out)
    torch.cuda.synchronize()
    for r in range(3):
        note(f"[gpu] graph capture: replay {r}")
        out.view(torch.int16).fill_(0x7F7B)                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"


def test_capture_without_workspace_is_refused():
    w = generate(SMALL["long_ctx"]).to("cuda")
    s = torch.cuda.Stream()                                  # no workspace on this stream yet
    out = torch.empty_like(w.q)
    g = torch.cuda.CUDAGraph()
    note("[gpu] capture without workspace")
    with pytest.raises(B.PagedAttnError) as e:
        with torch.cuda.graph(g, stream=s):
            B.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                w.query_lens, w.scale, None, None, out)
    assert e.value.name == "PA_ERR_CAPTURE"
    torch.cuda.synchronize()


def test_workspace_growth_keeps_captured_graphs_valid():
    # eager warm-up, capture at a small size, then an uncaptured call that
    # needs a larger workspace on the same stream: the graph keeps replaying
    # into the buffer it captured, which growth must not free
    small_w = generate(SMALL["mtp_verify"])
    big_w = generate(SMALL["long_ctx"].replace(ctx_lo=60001, ctx_hi=60001, pool_blocks=3800))
    ds, db = small_w.to("cuda"), big_w.to("cuda")
    s = torch.cuda.Stream()
    note("[gpu] workspace growth after capture: warm-up and capture at the small size")
    eager = torch.empty_like(ds.q)
    with torch.cuda.stream(s):
        B.paged_attn_decode(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.context_lens,
                            ds.query_lens, ds.scale, None, None, eager)
    s.synchronize()
    out = torch.empty_like(ds.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.paged_attn_decode(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.context_lens,
                            ds.query_lens, ds.scale, None, None, out)
    torch.cuda.synchronize()
    plan_s = B.paged_attn_plan(6, 64, 8, 128, 2, 16 * ds.block_tables.shape[1], "bf16",
                               torch.cuda.get_device_properties(0).multi_processor_count)
    plan_b = B.paged_attn_plan(1, 64, 8, 128, 1, 16 * db.block_tables.shape[1], "bf16",
                               torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan_b["workspace_bytes"] > 1.25 * plan_s["workspace_bytes"]
    note("[gpu] workspace growth after capture: the larger uncaptured call")
    big_out = torch.empty_like(db.q)
    with torch.cuda.stream(s):
        B.paged_attn_decode(db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                            db.query_lens, db.scale, None, None, big_out)
    s.synchronize()
    compare(big_out, oracle_out(big_w), big_w.query_lens, label="growth/big")
    # fresh device allocations that would land on freed memory
    filler = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(16)]
    for r in range(3):
        note(f"[gpu] workspace growth after capture: replay {r}")
        out.view(torch.int16).fill_(0x7F7B)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
    assert all(bool(torch.all(f == 7.0)) for f in filler)

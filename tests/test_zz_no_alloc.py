"""The no-allocation decode entry point (paged_attn_decode_noalloc) through
the C ABI: its output equals paged_attn_decode's bit for bit (the same
kernels and plan; only the workspace differs) and meets the oracle's
tolerance, on two calls in a row whose second input is smaller, under graph
capture without any reserve, and it refuses a plan larger than its static
scratch array before launching anything."""
import pytest
import torch

from _parity import CANARY, compare, note, oracle_out, small
from paged_attention_decode_attn_amd import binding as B
from paged_attention_decode_attn_amd.workloads import generate

pytestmark = pytest.mark.gpu


def _both(w):
    d = w.to("cuda")
    ref = torch.empty_like(d.q)
    got = torch.empty_like(d.q)
    ref.view(torch.int16).fill_(CANARY)
    got.view(torch.int16).fill_(CANARY)
    args = (d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, d.query_lens, d.scale,
            d.k_scale, d.v_scale)
    B.paged_attn_decode(*args, out=ref)
    B.paged_attn_decode_noalloc(*args, out=got)
    torch.cuda.synchronize()
    return d, ref, got, args


@pytest.mark.parametrize("first,second", [
    (("mtp_verify", dict(batch=24, ctx_lo=2, ctx_hi=6000, pool_blocks=9000)),
     ("mtp_verify", dict(batch=5, ctx_lo=2, ctx_hi=900, pool_blocks=300))),
    (("long_ctx", dict(ctx_lo=40000, ctx_hi=40000, pool_blocks=2600)),
     ("fp8", dict(batch=4, ctx_lo=100, ctx_hi=2000, pool_blocks=600))),
])
def test_two_calls_in_a_row_match_the_allocating_call(first, second):
    for name, kw in (first, second):
        w = generate(small(name, **kw))
        note(f"[gpu] noalloc {name} B={w.spec.batch} ctx={w.context_lens.tolist()[:6]}")
        _, ref, got, _ = _both(w)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name}: differs from paged_attn_decode"
        compare(got, oracle_out(w), w.query_lens, label=f"noalloc/{name}")


def test_graph_capture_without_reserve():
    w = generate(small("llama3_8b", ctx_lo=100, ctx_hi=3000, pool_blocks=900))
    note("[gpu] noalloc under graph capture")
    d, ref, _, args = _both(w)
    s = torch.cuda.Stream()
    out = torch.empty_like(d.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.paged_attn_decode_noalloc(*args, out=out, stream=s)
    for i in range(3):
        out.view(torch.int16).fill_(CANARY)
        # eager work between replays, the array shared with it
        other = generate(small("fp8", batch=3, ctx_lo=50, ctx_hi=1500, pool_blocks=400, seed=40 + i)).to("cuda")
        B.paged_attn_decode_noalloc(other.q, other.k_cache, other.v_cache, other.block_tables, other.context_lens,
                                    other.query_lens, other.scale, other.k_scale, other.v_scale,
                                    out=torch.empty_like(other.q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs"


def test_plan_larger_than_the_scratch_is_refused():
    # 64 rows per kv head over a full grid: the plan (from the table's
    # reach of 4000 tokens, not the short contexts) needs ~67 MB of partials
    w = generate(small("mtp_verify", batch=64, qlen=8, ctx_lo=9, ctx_hi=40, pool_blocks=200))
    d = w.to("cuda")
    wide = torch.zeros(64, 250, dtype=torch.int32, device="cuda")
    wide[:, :d.block_tables.shape[1]] = d.block_tables
    plan = B.paged_attn_plan(64, w.spec.hq, w.spec.hkv, w.spec.head_dim, 8, 16 * 250, w.spec.kv_dtype,
                             torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan["workspace_bytes"] > 48 << 20
    out = torch.empty_like(d.q)
    out.view(torch.int16).fill_(CANARY)
    note("[gpu] noalloc refusal")
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_decode_noalloc(d.q, d.k_cache, d.v_cache, wide, d.context_lens, d.query_lens,
                                    d.scale, d.k_scale, d.v_scale, out=out)
    assert e.value.name == "PA_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == CANARY)

"""GPU parity of paged prefill (paged_attn_prefill) against the CPU oracle:
packed variable-length chunks after cached prefixes, every q/kv head ratio,
head_dim 64 and 128, block sizes, chunk-length edges around the 32-key tile
and the 4-wave position block, NaN in unread memory.  Tolerance as for
decode: |gpu - ref| <= 1e-2 + 1e-2 |ref| on every produced element,
relative L2 <= 1e-2; rows outside every chunk keep a canary."""
import math

import numpy as np
import pytest
import torch

from _parity import ATOL, CANARY, REL_L2_MAX, RTOL, note
from oracle import paged_prefill_attention
from paged_attention_decode_attn_amd import binding as B
from paged_attention_decode_attn_amd.workloads import PREFILL_CONFIGS, generate_prefill

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _oracle(p, batch_subset=None, row_subset=None):
    c = p.cache
    fp8 = c.k_scale is not None
    return paged_prefill_attention(_bits(p.q), _bits(c.k_cache), _bits(c.v_cache), c.block_tables.numpy(),
                                   c.context_lens.numpy(), p.cu_seqlens.numpy(), p.scale,
                                   k_scale=c.k_scale.numpy() if fp8 else None,
                                   v_scale=c.v_scale.numpy() if fp8 else None,
                                   kv_dtype="fp8_e4m3fn" if fp8 else "bf16",
                                   batch_subset=batch_subset, row_subset=row_subset,
                                   sliding_window=p.sliding_window or None,
                                   sinks=None if c.sinks is None else c.sinks.numpy())


def _run(p, max_query_len=None, extra_rows=0, ext=None):
    """The plain call, or (ext: True, or None with a window or sinks in the
    workload) paged_attn_prefill_ext with the workload's window and sinks."""
    d = p.to("cuda")
    T, H, D = d.q.shape
    q = d.q
    if extra_rows:
        q = torch.cat([q, torch.zeros(extra_rows, H, D, dtype=q.dtype, device=q.device)])
    out = torch.empty_like(q)
    out.view(torch.int16).fill_(CANARY)
    mql = p.max_query_len if max_query_len is None else max_query_len
    c = d.cache
    if ext or (ext is None and (p.sliding_window or c.sinks is not None)):
        B.paged_attn_prefill_ext(q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, d.cu_seqlens, mql,
                                 p.scale, p.sliding_window, c.sinks, out, k_scale=c.k_scale, v_scale=c.v_scale)
    else:
        B.paged_attn_prefill(q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, d.cu_seqlens, mql, p.scale,
                             out, k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    return out.cpu()


def _compare(out, ref, label, rows=None):
    g = out.float().numpy().astype(np.float64)
    sel = np.arange(ref.shape[0]) if rows is None else np.asarray(rows)
    gb, rb = g[sel], ref[sel]
    assert np.all(np.isfinite(rb)), f"{label}: oracle rows not finite"
    err = np.abs(gb - rb)
    bad = ~(err <= ATOL + RTOL * np.abs(rb))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {bad.sum()} elements out of tolerance, first at row/head/d {tuple(i)}: "
                             f"gpu {gb[tuple(i)]!r} ref {rb[tuple(i)]!r}")
    rel = math.sqrt(float((err ** 2).sum()) / max(float((rb ** 2).sum()), 1e-300))
    assert rel <= REL_L2_MAX, f"{label}: relative L2 {rel:.3e}"


@pytest.mark.gpu
def test_size_one_dims_may_carry_any_stride():
    # one sequence: the table's row dim and the length vector have size 1,
    # so their strides are never used, whatever they are; the output is
    # bitwise the contiguous call's
    spec = PREFILL_CONFIGS["prefill_8k"].replace(ctx_lo=300, ctx_hi=300, pool_blocks=40)
    p = generate_prefill(spec)
    ref = _run(p)
    d = p.to("cuda")
    c = d.cache
    bt = torch.as_strided(c.block_tables, c.block_tables.shape, (999999937, 1))
    ctx = torch.as_strided(c.context_lens, (1,), (12345,))
    out = torch.empty_like(d.q)
    note("[gpu] prefill size-1 dims with odd strides")
    B.paged_attn_prefill(d.q, c.k_cache, c.v_cache, bt, ctx, d.cu_seqlens, p.max_query_len, p.scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16).cpu(), ref.view(torch.int16))



def _check(p, label, **kw):
    note(f"[gpu] prefill {label}: ctx={p.cache.context_lens.tolist()[:6]} chunks={p.chunk_lens.tolist()[:6]} "
         f"heads={p.spec.hq}/{p.spec.hkv} d={p.spec.head_dim} bs={p.spec.block_size} "
         f"window={p.sliding_window} sinks={p.sinks is not None} kv={p.spec.kv_dtype}")
    out = _run(p, **kw)
    _compare(out, _oracle(p), label)
    return out


SMALL = PREFILL_CONFIGS["chunked_prefill"].replace(batch=3, ctx_lo=1, ctx_hi=400, chunk_lo=1, chunk_hi=300,
                                                   pool_blocks=100)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (64, 8), (16, 1), (64, 1), (12, 4), (40, 8)])
def test_head_ratios(d, hq, hkv):
    p = generate_prefill(SMALL.replace(hq=hq, hkv=hkv, head_dim=d, seed=hq + hkv + d))
    _check(p, f"heads{hq}/{hkv}/d{d}")


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
def test_block_sizes(bs):
    p = generate_prefill(SMALL.replace(block_size=bs, pool_blocks=3 * (-(-400 // bs)) + 2, seed=30 + bs))
    _check(p, f"bs{bs}")


def test_whole_prompts():
    p = generate_prefill(SMALL.replace(chunk_lo=0, chunk_hi=0, seed=40))
    assert torch.equal(p.chunk_lens, p.cache.context_lens.to(torch.int32))
    _check(p, "whole prompts")


EDGE_CHUNKS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


@pytest.mark.parametrize("hq,hkv", [(8, 8), (64, 8)])
def test_chunk_length_edges(hq, hkv):
    ctx = [max(c, 1) + 37 * i for i, c in enumerate(EDGE_CHUNKS)]
    spec = SMALL.replace(batch=len(ctx), hq=hq, hkv=hkv, ctx_lo=1, ctx_hi=max(ctx), pool_blocks=400, seed=41)
    p = generate_prefill(spec, context_lens=ctx, chunk_lens=EDGE_CHUNKS)
    _check(p, f"edges/{hq}/{hkv}")


@pytest.mark.parametrize("batch", [2, 64, 70])
def test_launch_order_covers_every_row(batch):
    """Up to 64 sequences run in order of decreasing work (a per-workgroup
    search over the sequences), more in the plain order: mixed prefix and
    chunk lengths, empty chunks and whole prompts, every row produced once."""
    rng = np.random.default_rng(batch)
    ctx = rng.integers(1, 260, batch)
    chunks = [int(rng.integers(0, c + 1)) if i % 5 else (0 if i % 10 == 0 else int(c)) for i, c in enumerate(ctx)]
    spec = SMALL.replace(batch=batch, hq=16, hkv=4, head_dim=64, ctx_lo=1, ctx_hi=int(ctx.max()),
                         pool_blocks=int(sum(-(-int(c) // 16) for c in ctx)) + 8, seed=48 + batch)
    p = generate_prefill(spec, context_lens=[int(c) for c in ctx], chunk_lens=chunks)
    _check(p, f"order/B{batch}")


def test_larger_max_query_len_and_rows_outside_every_chunk():
    p = generate_prefill(SMALL.replace(seed=42))
    out = _run(p, max_query_len=p.max_query_len + 300, extra_rows=7)
    T = p.q.shape[0]
    _compare(out[:T], _oracle(p), "bigger max_query_len")
    assert torch.all(out[T:].view(torch.int16) == CANARY)


def test_nan_in_unread_memory_never_reaches_output():
    spec = SMALL.replace(seed=43)
    p = generate_prefill(spec)
    c = p.cache
    # poison every slot past each sequence's length in its last block, and
    # every unused block
    used = set()
    for b in range(spec.batch):
        L = int(c.context_lens[b])
        nb = -(-L // 16)
        used.update(int(x) for x in c.block_tables[b, :nb])
        last = int(c.block_tables[b, nb - 1])
        tail = L - (nb - 1) * 16
        c.k_cache[last, tail:].view(torch.int16).fill_(0x7FC0)
        c.v_cache[last, tail:].view(torch.int16).fill_(0x7FC0)
    for blk in range(spec.pool_blocks):
        if blk not in used:
            c.k_cache[blk].view(torch.int16).fill_(0x7FC0)
            c.v_cache[blk].view(torch.int16).fill_(0x7FC0)
    _check(p, "poison")


@pytest.mark.parametrize("factor", [4.0, 8.0])
def test_sharpened_queries(factor):
    p = generate_prefill(SMALL.replace(seed=44))
    p.q = (p.q.float() * factor).to(torch.bfloat16)
    _check(p, f"sharp{factor}")


@pytest.mark.parametrize("scale", [-0.3, 0.0])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_negative_and_zero_softmax_scale(scale, kv):
    p = generate_prefill(SMALL.replace(kv_dtype=kv, seed=51))
    p.scale = scale
    _check(p, f"scale{scale}/{kv}")
    p = generate_prefill(SWA.replace(kv_dtype=kv, sliding_window=60, sinks=True, seed=52))
    p.scale = scale
    _check(p, f"scale{scale}/{kv}/window-sinks")
    p = generate_prefill(SMALL.replace(hq=16, hkv=8, head_dim=256, kv_dtype=kv, seed=53))
    p.scale = scale
    _check(p, f"scale{scale}/{kv}/d256")


def test_repeat_calls_are_bitwise_identical():
    p = generate_prefill(SMALL.replace(seed=45))
    a = _run(p)
    b = _run(p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_graph_capture_replays_match_eager():
    p = generate_prefill(SMALL.replace(seed=46)).to("cuda")
    c = p.cache
    eager = torch.empty_like(p.q)
    note("[gpu] prefill graph capture")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        B.paged_attn_prefill(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                             p.max_query_len, p.scale, eager, stream=s)
    s.synchronize()
    out = torch.empty_like(p.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.paged_attn_prefill(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                             p.max_query_len, p.scale, out, stream=s)
    torch.cuda.synchronize()
    for r in range(3):
        out.view(torch.int16).fill_(CANARY)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"


def test_strided_tensors():
    """q and out as views into padded buffers, a block table that is a column
    slice of a wider one, and context lengths and row offsets with stride 2:
    the same bytes through every stride the kernel takes."""
    p = generate_prefill(SMALL.replace(kv_dtype="fp8_e4m3fn", sliding_window=90, sinks=True, seed=49))
    ref = _oracle(p)
    d = p.to("cuda")
    c = d.cache
    T, Hq, D = d.q.shape
    qbig = torch.zeros(T, Hq + 3, D + 64, dtype=torch.bfloat16, device="cuda")
    q = qbig[:, 1:1 + Hq, 32:32 + D]
    q.copy_(d.q)
    obig = torch.empty(T, Hq, 2 * D, dtype=torch.bfloat16, device="cuda")
    obig.view(torch.int16).fill_(CANARY)
    out = obig[:, :, D:]
    W = c.block_tables.shape[1]
    tbig = torch.zeros(c.block_tables.shape[0], W + 5, dtype=torch.int32, device="cuda")
    tbig[:, 2:2 + W] = c.block_tables
    ctx2 = torch.zeros(2 * len(c.context_lens), dtype=torch.int32, device="cuda")
    ctx2[::2] = c.context_lens
    cu2 = torch.zeros(2 * len(d.cu_seqlens), dtype=torch.int32, device="cuda")
    cu2[::2] = d.cu_seqlens
    note("[gpu] prefill strided tensors")
    B.paged_attn_prefill_ext(q, c.k_cache, c.v_cache, tbig[:, 2:2 + W], ctx2[::2], cu2[::2], p.max_query_len,
                             p.scale, p.sliding_window, c.sinks, out, k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    _compare(out.cpu(), ref, "strided")
    assert torch.all(obig[:, :, :D].view(torch.int16) == CANARY), "bytes outside the out view written"


def test_graph_capture_fp8_window_sinks():
    p = generate_prefill(SWA.replace(kv_dtype="fp8_e4m3fn", sliding_window=60, sinks=True, seed=50)).to("cuda")
    c = p.cache

    def call(out, s):
        B.paged_attn_prefill_ext(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                                 p.max_query_len, p.scale, p.sliding_window, c.sinks, out, stream=s,
                                 k_scale=c.k_scale, v_scale=c.v_scale)
    note("[gpu] prefill graph capture fp8/window/sinks")
    s = torch.cuda.Stream()
    eager = torch.empty_like(p.q)
    with torch.cuda.stream(s):
        call(eager, s)
    s.synchronize()
    out = torch.empty_like(p.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out, s)
    torch.cuda.synchronize()
    for r in range(3):
        out.view(torch.int16).fill_(CANARY)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"


def test_argument_errors_launch_nothing():
    p = generate_prefill(SMALL.replace(seed=47)).to("cuda")
    c = p.cache
    out = torch.full_like(p.q, 3.0)
    note("[gpu] prefill argument errors")
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_prefill(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens[:-1],
                             p.max_query_len, p.scale, out)
    assert e.value.name == "PA_ERR_SHAPE"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_prefill(p.q, c.k_cache.view(torch.uint8)[..., :p.spec.head_dim], c.v_cache, c.block_tables,
                             c.context_lens, p.cu_seqlens, p.max_query_len, p.scale, out)
    assert e.value.name in ("PA_ERR_UNSUPPORTED", "PA_ERR_DTYPE")
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# --------------------------------------------------------------------------
# sliding window and attention sinks (paged_attn_prefill_ext)
# --------------------------------------------------------------------------
SWA = SMALL.replace(hq=64, hkv=8, head_dim=64, ctx_hi=700, chunk_hi=300, pool_blocks=180)


@pytest.mark.parametrize("window", [1, 2, 31, 32, 33, 100, 128, 1000])
@pytest.mark.parametrize("with_sinks", [False, True])
def test_window_and_sinks(window, with_sinks):
    p = generate_prefill(SWA.replace(sliding_window=window, sinks=with_sinks, seed=60 + window + with_sinks))
    _check(p, f"window{window}/sinks{with_sinks}")


@pytest.mark.parametrize("hq,hkv,d", [(16, 8, 128), (64, 1, 64), (8, 8, 128)])
def test_window_and_sinks_head_ratios(hq, hkv, d):
    p = generate_prefill(SWA.replace(hq=hq, hkv=hkv, head_dim=d, sliding_window=77, sinks=True, seed=70 + hq))
    _check(p, f"window77/heads{hq}/{hkv}/d{d}")


def test_sinks_alone_and_chunk_edges_with_a_window():
    p = generate_prefill(SWA.replace(sinks=True, seed=74))
    _check(p, "sinks, no window")
    ctx = [max(c, 1) + 37 * i for i, c in enumerate(EDGE_CHUNKS)]
    spec = SWA.replace(batch=len(ctx), ctx_hi=max(ctx), pool_blocks=400, sliding_window=40, sinks=True, seed=75)
    p = generate_prefill(spec, context_lens=ctx, chunk_lens=EDGE_CHUNKS)
    _check(p, "window40 edges")


def test_blocks_freed_below_every_window_never_reach_output():
    """Blocks wholly below each sequence's first row's window hold NaN and
    their table entries point outside the pool; the output is that of the
    intact cache."""
    w = 48
    p = generate_prefill(SWA.replace(sliding_window=w, sinks=True, ctx_lo=200, seed=76))
    ref = _oracle(p)
    c = p.cache
    NB = c.k_cache.shape[0]
    freed = 0
    for b in range(p.spec.batch):
        L, n = int(c.context_lens[b]), int(p.chunk_lens[b])
        lo = max(0, L - n - w + 1)
        for i in range(lo // 16):
            blk = int(c.block_tables[b, i])
            c.k_cache[blk].view(torch.int16).fill_(0x7FC0)
            c.v_cache[blk].view(torch.int16).fill_(0x7FC0)
            c.block_tables[b, i] = NB + 5 if i % 2 else -7
            freed += 1
    assert freed > 0
    note(f"[gpu] prefill freed-below-window: {freed} blocks")
    _compare(_run(p), ref, "freed below window")


def test_ext_without_a_window_or_sinks_is_the_plain_call():
    p = generate_prefill(SMALL.replace(seed=77))
    plain = _run(p, ext=False)
    assert torch.equal(_run(p, ext=True).view(torch.int16), plain.view(torch.int16))
    # a window no row can exceed changes nothing either
    wide = generate_prefill(SMALL.replace(seed=77, sliding_window=1 << 20))
    assert torch.equal(_run(wide).view(torch.int16), plain.view(torch.int16))


def test_ext_argument_errors():
    p = generate_prefill(SWA.replace(sinks=True, seed=78)).to("cuda")
    c = p.cache
    out = torch.full_like(p.q, 3.0)
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_prefill_ext(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                                 p.max_query_len, p.scale, 32, c.sinks[:-1], out)
    assert e.value.name == "PA_ERR_SHAPE"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_prefill_ext(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                                 p.max_query_len, p.scale, 32, c.sinks.to(torch.bfloat16), out)
    assert e.value.name == "PA_ERR_DTYPE"
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# --------------------------------------------------------------------------
# head_dim 256 (one 16-row tile per wave: q_heads / kv_heads <= 16)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 8), (32, 2), (16, 1), (12, 4)])
def test_head_dim_256(hq, hkv):
    p = generate_prefill(SMALL.replace(hq=hq, hkv=hkv, head_dim=256, seed=100 + hq + hkv))
    _check(p, f"d256/heads{hq}/{hkv}")


def test_head_dim_256_fp8_window_sinks_and_edges():
    p = generate_prefill(SWA.replace(head_dim=256, hq=16, hkv=8, kv_dtype="fp8_e4m3fn", sliding_window=70,
                                     sinks=True, seed=106))
    _check(p, "d256/fp8/window70/sinks")
    ctx = [max(c, 1) + 37 * i for i, c in enumerate(EDGE_CHUNKS)]
    spec = SMALL.replace(head_dim=256, hq=16, hkv=8, batch=len(ctx), ctx_hi=max(ctx), pool_blocks=400, seed=107)
    _check(generate_prefill(spec, context_lens=ctx, chunk_lens=EDGE_CHUNKS), "d256 edges")


# --------------------------------------------------------------------------
# fp8 e4m3fn cache with per-token scales
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8), (64, 1)])
def test_fp8_cache(d, hq, hkv):
    p = generate_prefill(SMALL.replace(kv_dtype="fp8_e4m3fn", hq=hq, hkv=hkv, head_dim=d, seed=80 + hq + hkv + d))
    _check(p, f"fp8/heads{hq}/{hkv}/d{d}")


@pytest.mark.parametrize("bs", [16, 64])
def test_fp8_block_sizes_window_and_sinks(bs):
    p = generate_prefill(SWA.replace(kv_dtype="fp8_e4m3fn", block_size=bs, pool_blocks=3 * (-(-700 // bs)) + 2,
                                     sliding_window=50, sinks=True, seed=90 + bs))
    _check(p, f"fp8/bs{bs}/window50/sinks")


def test_fp8_sharpened_queries_and_chunk_edges():
    p = generate_prefill(SMALL.replace(kv_dtype="fp8_e4m3fn", seed=95))
    p.q = (p.q.float() * 8.0).to(torch.bfloat16)
    _check(p, "fp8 sharp8")
    ctx = [max(c, 1) + 37 * i for i, c in enumerate(EDGE_CHUNKS)]
    spec = SMALL.replace(kv_dtype="fp8_e4m3fn", batch=len(ctx), ctx_hi=max(ctx), pool_blocks=400, seed=96)
    _check(generate_prefill(spec, context_lens=ctx, chunk_lens=EDGE_CHUNKS), "fp8 edges")


def test_fp8_nan_scales_and_codes_in_unread_slots():
    """NaN codes (0x7F) and NaN scales past each sequence's length, and in
    unused blocks, never reach the output."""
    p = generate_prefill(SMALL.replace(kv_dtype="fp8_e4m3fn", seed=97))
    c = p.cache
    ref = _oracle(p)
    used = set()
    for b in range(p.spec.batch):
        L = int(c.context_lens[b])
        nb = -(-L // 16)
        used.update(int(x) for x in c.block_tables[b, :nb])
        last = int(c.block_tables[b, nb - 1])
        tail = L - (nb - 1) * 16
        c.k_cache[last, tail:] = 0x7F
        c.v_cache[last, tail:] = 0x7F
        c.k_scale[last, tail:] = float("nan")
        c.v_scale[last, tail:] = float("nan")
    for blk in range(p.spec.pool_blocks):
        if blk not in used:
            c.k_cache[blk] = 0x7F
            c.v_cache[blk] = 0x7F
            c.k_scale[blk] = float("nan")
            c.v_scale[blk] = float("nan")
    note("[gpu] prefill fp8 poison")
    _compare(_run(p), ref, "fp8 poison")


def test_fp8_argument_errors():
    p = generate_prefill(SMALL.replace(kv_dtype="fp8_e4m3fn", seed=98)).to("cuda")
    c = p.cache
    out = torch.full_like(p.q, 3.0)
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_prefill(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                             p.max_query_len, p.scale, out)                      # scales missing
    assert e.value.name == "PA_ERR_NULL"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_prefill(p.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, p.cu_seqlens,
                             p.max_query_len, p.scale, out, k_scale=c.k_scale[:, :8], v_scale=c.v_scale)
    assert e.value.name == "PA_ERR_SHAPE"
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# --------------------------------------------------------------------------
# the full-size workloads, in the benchmark's launch, checked on sampled rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,seq,rows", [
    ("prefill_8k", 0, [0, 1, 31, 32, 255, 256, 4095, 4096, 8190, 8191]),
    ("chunked_prefill", 1, [0, 1, 63, 64, 1000, 2047]),
    ("chunked_prefill", 3, [0, 511, 2047]),
    ("chunked_prefill_fp8", 0, [0, 1, 1000, 2047]),
    ("prefill_d256", 0, [0, 1, 63, 64, 4095, 8191]),
    ("prefill_swa_sinks", 0, [0, 1, 126, 127, 128, 129, 4095, 8191]),
    ("prefill_swa_sinks", 3, [0, 200, 8191]),
])
def test_full_size_sampled_rows(name, seq, rows):
    p = generate_prefill(PREFILL_CONFIGS[name])
    note(f"[gpu] prefill full {name}: seq {seq} rows {rows}")
    out = _run(p)
    ref = _oracle(p, batch_subset=[seq], row_subset=rows)
    base = int(p.cu_seqlens[seq])
    _compare(out, ref, f"full/{name}/{seq}", rows=[base + r for r in rows])

"""Pins of the oracle's shape variants (CPU only): block sizes other than 16,
a sliding window and per-head attention sinks.

The readings (the oracle's header states them): token j of a sequence is
slot ``j % BS`` of block ``bt[b, j // BS]``; a window ``w`` lets the row at
position ``p`` see keys ``p - w + 1 .. p``; a sink is one logit per query
head, in the units of the scaled scores, that joins the softmax normaliser
and carries no value.  Each pin below ties the oracle to something other than
itself: a relayout of the same tokens, a closed form, a pure-Python brute
force, or torch's float64 attention with an additive mask.
"""
import math

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, e4m3fn_bytes_to_f64, merge_states, paged_decode_attention, partial_state
from test_oracle import _bf16_bits


def _page_bs(seqs, hkv, d, bs, rng, dtype=np.uint16, scales=None, extra=2):
    """Scatter contiguous per-sequence rows [L_b, Hkv, D] into a permuted
    pool of blocks of `bs` tokens; with `scales` ([L_b, Hkv] per sequence)
    also the per-token scale pool.  Returns (pool, scale_pool, tables)."""
    nblk = [(len(x) + bs - 1) // bs for x in seqs]
    nb = sum(nblk) + extra
    W = max(max(nblk), 1)
    perm = rng.permutation(nb)
    pool = np.zeros((nb, bs, hkv, d), dtype=dtype)
    spool = np.ones((nb, bs, hkv), np.float32)
    tables = np.full((len(seqs), W), nb - 1, dtype=np.int32)
    off = 0
    for b, x in enumerate(seqs):
        for i in range(nblk[b]):
            blk = perm[off + i]
            tables[b, i] = blk
            r0, r1 = i * bs, min((i + 1) * bs, len(x))
            pool[blk, : r1 - r0] = x[r0:r1]
            if scales is not None:
                spool[blk, : r1 - r0] = scales[b][r0:r1]
        off += nblk[b]
    return pool, spool, tables


def _seqs(rng, lens, hkv, d):
    ks = [_bf16_bits(rng.standard_normal((L, hkv, d))) for L in lens]
    vs = [_bf16_bits(rng.standard_normal((L, hkv, d))) for L in lens]
    return ks, vs


def _paged(ks, vs, hkv, d, bs, seed):
    kp, _, t = _page_bs(ks, hkv, d, bs, np.random.default_rng(seed))
    vp, _, t2 = _page_bs(vs, hkv, d, bs, np.random.default_rng(seed))
    assert np.array_equal(t, t2)
    return kp, vp, t


def _brute(q, ks, vs, lens, qlens, scale, hq, hkv, window=None, sinks=None):
    """Pure-Python loops over contiguous sequences with math.exp: the
    window bounds the keys, the sink adds exp(sink) to the normaliser."""
    B, Qmax, _, D = q.shape
    G = hq // hkv
    out = np.full(q.shape, np.nan)
    qf = bf16_bits_to_f64(q)
    for b in range(B):
        L, n = int(lens[b]), int(qlens[b])
        kf, vf = bf16_bits_to_f64(ks[b]), bf16_bits_to_f64(vs[b])
        for t in range(n):
            p = L - n + t
            lo = 0 if not window or window <= 0 else max(0, p - window + 1)
            for h in range(hq):
                g = h // G
                xs = [scale * sum(qf[b, t, h, e] * kf[j, g, e] for e in range(D)) for j in range(lo, p + 1)]
                mx = max(xs)
                s = None if sinks is None else float(sinks[h])
                if s is not None:
                    mx = max(mx, s)
                ws = [math.exp(x - mx) for x in xs]
                den = sum(ws) + (0.0 if s is None else math.exp(s - mx))
                for e in range(D):
                    out[b, t, h, e] = sum(w * vf[lo + i, g, e] for i, w in enumerate(ws)) / den
    return out


def _sdpa_masked(q, ks, vs, lens, qlens, scale, hq, hkv, window=None, sinks=None):
    """torch float64 scaled_dot_product_attention with an additive mask: -inf
    outside the causal window, and one extra zero key/value column whose
    additive bias is the head's sink logit."""
    B, Qmax, _, D = q.shape
    G = hq // hkv
    out = np.full(q.shape, np.nan)
    qt = torch.from_numpy(bf16_bits_to_f64(q))
    for b in range(B):
        L, n = int(lens[b]), int(qlens[b])
        k = torch.from_numpy(bf16_bits_to_f64(ks[b])).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = torch.from_numpy(bf16_bits_to_f64(vs[b])).permute(1, 0, 2).repeat_interleave(G, dim=0)
        pos = torch.arange(n)[:, None] + (L - n)
        j = torch.arange(L)[None, :]
        ok = j <= pos
        if window and window > 0:
            ok &= j > pos - window
        bias = torch.where(ok, 0.0, -math.inf).to(torch.float64)[None].repeat(hq, 1, 1)   # [Hq, n, L]
        if sinks is not None:
            k = torch.cat([k, torch.zeros(hq, 1, D, dtype=torch.float64)], dim=1)
            v = torch.cat([v, torch.zeros(hq, 1, D, dtype=torch.float64)], dim=1)
            col = torch.from_numpy(np.asarray(sinks, np.float64))[:, None, None].expand(hq, n, 1)
            bias = torch.cat([bias, col], dim=2)
        qq = qt[b, :n].permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=bias, scale=float(scale))
        out[b, :n] = o.permute(1, 0, 2).numpy()
    return out


def _cmp(out, ref, atol=1e-12):
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(out[ok], ref[ok], rtol=0, atol=atol)


# ----------------------------------------------------------------------------
# block size
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [32, 48, 64, 256])
def test_block_size_relayout_is_bit_exact(bs):
    """The same tokens paged in blocks of `bs` and of 16 give the same output,
    bit for bit: the block size only changes where a token is stored."""
    rng = np.random.default_rng(bs)
    hq, hkv, d = 8, 2, 16
    lens, qlens = (1, 47, 64, 65, 300), (1, 2, 2, 1, 2)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((len(lens), 2, hq, d)))
    k16, v16, t16 = _paged(ks, vs, hkv, d, 16, 1)
    kb, vb, tb = _paged(ks, vs, hkv, d, bs, 2)
    ref = paged_decode_attention(q, k16, v16, t16, lens, qlens, 0.3)
    out = paged_decode_attention(q, kb, vb, tb, lens, qlens, 0.3)
    assert np.array_equal(out, ref, equal_nan=True)


def test_block_size_fp8_scales_follow_their_slots():
    rng = np.random.default_rng(5)
    hq, hkv, d, bs = 4, 2, 16, 64
    lens, qlens = (70, 129), (1, 2)
    k8 = [rng.integers(0, 0x7E, (L, hkv, d)).astype(np.uint8) for L in lens]
    v8 = [rng.integers(0x80, 0xFE, (L, hkv, d)).astype(np.uint8) for L in lens]
    ksc = [rng.uniform(0.01, 0.1, (L, hkv)).astype(np.float32) for L in lens]
    vsc = [rng.uniform(0.01, 0.1, (L, hkv)).astype(np.float32) for L in lens]
    q = _bf16_bits(rng.standard_normal((2, 2, hq, d)))
    outs = []
    for block in (16, bs):
        kp, kss, t = _page_bs(k8, hkv, d, block, np.random.default_rng(block), np.uint8, ksc)
        vp, vss, _ = _page_bs(v8, hkv, d, block, np.random.default_rng(block), np.uint8, vsc)
        outs.append(paged_decode_attention(q, kp, vp, t, lens, qlens, 0.25, kss, vss, "fp8_e4m3fn"))
    assert np.array_equal(outs[0], outs[1], equal_nan=True)
    # and both equal attention over the dequantised contiguous rows
    kf = [e4m3fn_bytes_to_f64(k) * s[..., None] for k, s in zip(k8, ksc)]
    vf = [e4m3fn_bytes_to_f64(v) * s[..., None] for v, s in zip(v8, vsc)]
    qf = bf16_bits_to_f64(q)
    for b, (L, n) in enumerate(zip(lens, qlens)):
        for t in range(n):
            p = L - n + t
            for h in range(hq):
                x = 0.25 * kf[b][: p + 1, h // 2] @ qf[b, t, h]
                w = np.exp(x - x.max())
                np.testing.assert_allclose(outs[1][b, t, h], w @ vf[b][: p + 1, h // 2] / w.sum(), rtol=0, atol=1e-12)


def test_block_size_one():
    rng = np.random.default_rng(8)
    hq, hkv, d = 4, 4, 8
    lens, qlens = (1, 9, 20), (1, 2, 1)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((3, 2, hq, d)))
    kp, vp, t = _paged(ks, vs, hkv, d, 1, 3)
    _cmp(paged_decode_attention(q, kp, vp, t, lens, qlens, 0.5), _brute(q, ks, vs, lens, qlens, 0.5, hq, hkv))



# ----------------------------------------------------------------------------
# sliding window and sinks: brute force and an independent library routine
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("window", [1, 2, 5, 16, 33])
@pytest.mark.parametrize("with_sinks", [False, True])
def test_window_and_sinks_match_brute_force(window, with_sinks):
    rng = np.random.default_rng(100 + window + 7 * with_sinks)
    hq, hkv, d, bs = 4, 2, 8, 32
    lens, qlens = (1, 6, 40, 70), (1, 2, 2, 1)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((4, 2, hq, d)))
    sinks = rng.uniform(-3, 3, hq).astype(np.float32) if with_sinks else None
    kp, vp, t = _paged(ks, vs, hkv, d, bs, 4)
    scale = np.float32(0.4)                     # the oracle takes the caller's float32 scale
    out = paged_decode_attention(q, kp, vp, t, lens, qlens, scale, sliding_window=window, sinks=sinks)
    _cmp(out, _brute(q, ks, vs, lens, qlens, float(scale), hq, hkv, window, sinks))


@pytest.mark.parametrize("window", [None, 3, 64, 200])
def test_window_and_sinks_match_torch_sdpa_with_additive_mask(window):
    rng = np.random.default_rng(7 + (window or 0))
    hq, hkv, d = 8, 2, 32
    lens, qlens = (1, 17, 129, 300), (1, 2, 2, 2)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((4, 2, hq, d)))
    sinks = rng.uniform(-4, 4, hq).astype(np.float32)
    sinks[3] = -np.inf                                          # this head has no sink
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 5)
    scale = np.float32(0.2)
    out = paged_decode_attention(q, kp, vp, t, lens, qlens, scale, sliding_window=window, sinks=sinks)
    _cmp(out, _sdpa_masked(q, ks, vs, lens, qlens, float(scale), hq, hkv, window, sinks))


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------
def test_window_one_returns_the_rows_own_value():
    rng = np.random.default_rng(11)
    hq, hkv, d = 4, 2, 16
    lens, qlens = (3, 50), (2, 2)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((2, 2, hq, d)) * 30)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 6)
    out = paged_decode_attention(q, kp, vp, t, lens, qlens, 1.0, sliding_window=1)
    for b, (L, n) in enumerate(zip(lens, qlens)):
        for r in range(n):
            for h in range(hq):
                assert np.array_equal(out[b, r, h], bf16_bits_to_f64(vs[b][L - n + r, h // 2]))


@pytest.mark.parametrize("window", [0, -1, 70, 10 ** 6])
def test_no_or_wide_window_equals_full_attention(window):
    rng = np.random.default_rng(12)
    hq, hkv, d = 4, 1, 16
    lens, qlens = (1, 64, 70), (1, 2, 2)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((3, 2, hq, d)))
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 7)
    ref = paged_decode_attention(q, kp, vp, t, lens, qlens, 0.3)
    out = paged_decode_attention(q, kp, vp, t, lens, qlens, 0.3, sliding_window=window)
    assert np.array_equal(out, ref, equal_nan=True)


@pytest.mark.parametrize("window", [2, 17, 40])
def test_window_equals_attention_over_the_truncated_sequence(window):
    """A windowed row equals unwindowed attention over a sequence that holds
    only the window's keys (query length 1, rebuilt block table)."""
    rng = np.random.default_rng(13 + window)
    hq, hkv, d = 4, 2, 16
    L, n = 90, 3
    ks, vs = _seqs(rng, (L,), hkv, d)
    q = _bf16_bits(rng.standard_normal((1, n, hq, d)))
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 8)
    out = paged_decode_attention(q, kp, vp, t, [L], [n], 0.3, sliding_window=window)
    for r in range(n):
        p = L - n + r
        lo = max(0, p - window + 1)
        kt, vt, tt = _paged([ks[0][lo: p + 1]], [vs[0][lo: p + 1]], hkv, d, 16, 9)
        ref = paged_decode_attention(q[:, r: r + 1], kt, vt, tt, [p + 1 - lo], [1], 0.3)
        np.testing.assert_allclose(out[0, r], ref[0, 0], rtol=0, atol=1e-12)


def test_sinks_with_zero_query_closed_form():
    """q = 0 makes every visible logit 0: out = sum of visible v / (count + e^sink)."""
    rng = np.random.default_rng(14)
    hq, hkv, d, window = 4, 2, 8, 5
    lens, qlens = (3, 40), (1, 2)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = np.zeros((2, 2, hq, d), np.uint16)
    sinks = np.array([0.0, 1.5, -2.0, math.log(3.0)], np.float32)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 10)
    for win in (None, window):
        out = paged_decode_attention(q, kp, vp, t, lens, qlens, 0.5, sliding_window=win, sinks=sinks)
        for b, (L, n) in enumerate(zip(lens, qlens)):
            for r in range(n):
                p = L - n + r
                lo = 0 if win is None else max(0, p - win + 1)
                for h in range(hq):
                    vsum = bf16_bits_to_f64(vs[b][lo: p + 1, h // 2]).sum(axis=0)
                    ref = vsum / ((p + 1 - lo) + math.exp(float(sinks[h])))
                    np.testing.assert_allclose(out[b, r, h], ref, rtol=1e-14, atol=1e-15)


def test_sink_of_minus_infinity_is_no_sink():
    rng = np.random.default_rng(15)
    hq, hkv, d = 4, 2, 16
    lens, qlens = (5, 33), (1, 2)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((2, 2, hq, d)))
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 11)
    ref = paged_decode_attention(q, kp, vp, t, lens, qlens, 0.3, sliding_window=7)
    out = paged_decode_attention(q, kp, vp, t, lens, qlens, 0.3, sliding_window=7,
                                 sinks=np.full(hq, -np.inf, np.float32))
    assert np.array_equal(out, ref, equal_nan=True)


def test_sinks_far_above_the_scores_stay_finite_and_shrink_the_output():
    rng = np.random.default_rng(16)
    hq, hkv, d = 2, 1, 16
    ks, vs = _seqs(rng, (20,), hkv, d)
    q = _bf16_bits(rng.standard_normal((1, 1, hq, d)))
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 12)
    base = paged_decode_attention(q, kp, vp, t, [20], [1], 0.3)
    out = paged_decode_attention(q, kp, vp, t, [20], [1], 0.3, sinks=np.array([1000.0, 5.0], np.float32))
    assert np.all(np.isfinite(out))
    assert np.all(np.abs(out[0, 0, 0]) < 1e-300)
    # a sink scales a head's output by sum e^x / (sum e^x + e^sink) < 1
    ratio = out[0, 0, 1] / base[0, 0, 1]
    assert np.allclose(ratio, ratio[0], rtol=1e-12, atol=0) and 0 < ratio[0] < 1


def test_sink_is_a_zero_valued_partial_in_the_merge():
    """The split-context merge of the key partials plus one partial (m=sink,
    l=1, o=0) equals attention with that sink."""
    rng = np.random.default_rng(17)
    x = rng.normal(0, 3, 50)
    v = rng.normal(0, 1, (50, 8))
    sink = 2.5
    parts = [partial_state(x[a:b], v[a:b]) for a, b in ((0, 13), (13, 14), (14, 50))]
    parts.append((sink, 1.0, np.zeros(8)))
    got = merge_states(parts)
    w = np.exp(x - x.max())
    ref = w @ v / (w.sum() + math.exp(sink - x.max()))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def variant_battery(orc) -> bool:
    """The pins above in brief, against a (possibly mutated) oracle copy;
    used by the planted-mistake check."""
    rng = np.random.default_rng(31)
    hq, hkv, d = 4, 2, 8
    lens, qlens = (6, 40, 70), (2, 2, 1)
    ks, vs = _seqs(rng, lens, hkv, d)
    q = _bf16_bits(rng.standard_normal((3, 2, hq, d)))
    sinks = np.array([0.5, -1.0, 2.0, -np.inf], np.float32)
    scale = np.float32(0.4)
    k64, v64, t64 = _paged(ks, vs, hkv, d, 64, 3)
    for window in (1, 5, None):
        out = orc.paged_decode_attention(q, k64, v64, t64, lens, qlens, scale, sliding_window=window, sinks=sinks)
        ref = _brute(q, ks, vs, lens, qlens, float(scale), hq, hkv, window, sinks)
        if not (np.array_equal(np.isnan(out), np.isnan(ref))
                and np.allclose(out[~np.isnan(ref)], ref[~np.isnan(ref)], rtol=0, atol=1e-12)):
            return False
    with np.errstate(all="ignore"):
        big = orc.paged_decode_attention(q, k64, v64, t64, lens, qlens, scale,
                                         sinks=np.full(hq, 1000.0, np.float32))
    return bool(np.all(np.isfinite(big[~np.isnan(big)])))

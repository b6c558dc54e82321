"""Pins of the prefill oracle (oracle/prefill.py), CPU only: packed
variable-length chunks over the paged cache against torch's float64
attention with a causal mask, a pure-Python brute force, the chunking
invariance of causal attention, and the agreement of its whole-sequence and
single-row evaluations."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, paged_prefill_attention
from test_oracle import _bf16_bits, _page, _sdpa_reference
from test_oracle_variants import _paged, _sdpa_masked, _seqs


def _pack(rng, lens, chunks, hq, d):
    """q rows of the last chunks[b] positions of each sequence, packed."""
    q = [_bf16_bits(rng.standard_normal((n, hq, d))) for n in chunks]
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return np.concatenate(q, axis=0) if sum(chunks) else np.zeros((0, hq, d), np.uint16), cu


def _sdpa_packed(qp, cu, ks, vs, lens, scale, hq, hkv):
    """torch float64 SDPA per sequence with an offset-causal boolean mask
    (is_causal for chunks that are the whole sequence)."""
    G = hq // hkv
    out = np.full(qp.shape, np.nan)
    for b in range(len(lens)):
        n, L = int(cu[b + 1] - cu[b]), int(lens[b])
        if n == 0:
            continue
        q = torch.from_numpy(bf16_bits_to_f64(qp[cu[b]:cu[b + 1]])).permute(1, 0, 2)     # [Hq, n, D]
        k = torch.from_numpy(bf16_bits_to_f64(ks[b])).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = torch.from_numpy(bf16_bits_to_f64(vs[b])).permute(1, 0, 2).repeat_interleave(G, dim=0)
        if n == L:
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
        else:
            mask = torch.arange(L)[None, :] <= (torch.arange(n)[:, None] + (L - n))
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        out[cu[b]:cu[b + 1]] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 1)])
def test_whole_and_chunked_prefill_match_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    d = 32
    lens = (1, 17, 64, 150, 300)
    chunks = (1, 17, 30, 150, 77)          # whole prompts and chunks after cached prefixes
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 3)
    scale = np.float32(0.2)
    out = paged_prefill_attention(qp, kp, vp, t, lens, cu, scale)
    ref = _sdpa_packed(qp, cu, ks, vs, lens, float(scale), hq, hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_prefill_matches_brute_force_tiny():
    rng = np.random.default_rng(5)
    hq, hkv, d = 4, 2, 8
    lens, chunks = (3, 20), (3, 6)
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 32, 4)
    out = paged_prefill_attention(qp, kp, vp, t, lens, cu, 0.5)
    qf = bf16_bits_to_f64(qp)
    for b, (L, n) in enumerate(zip(lens, chunks)):
        kf, vf = bf16_bits_to_f64(ks[b]), bf16_bits_to_f64(vs[b])
        for r in range(n):
            p = L - n + r
            for h in range(hq):
                xs = [0.5 * sum(qf[cu[b] + r, h, e] * kf[j, h // 2, e] for e in range(d)) for j in range(p + 1)]
                m = max(xs)
                w = [math.exp(x - m) for x in xs]
                ref = [sum(w[j] * vf[j, h // 2, e] for j in range(p + 1)) / sum(w) for e in range(d)]
                np.testing.assert_allclose(out[cu[b] + r, h], ref, rtol=0, atol=1e-12)


def test_chunking_a_prompt_does_not_change_its_rows():
    """Causal attention of a prompt done in one piece equals the same prompt
    done as two chunks, the second seeing the first through the cache."""
    rng = np.random.default_rng(6)
    hq, hkv, d, L = 8, 2, 32, 200
    ks, vs = _seqs(rng, (L,), hkv, d)
    q = _bf16_bits(rng.standard_normal((L, hq, d)))
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 5)
    whole = paged_prefill_attention(q, kp, vp, t, [L], [0, L], 0.3)
    first = paged_prefill_attention(q[:120], kp, vp, t, [120], [0, 120], 0.3)
    second = paged_prefill_attention(q[120:], kp, vp, t, [L], [0, L - 120], 0.3)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=0, atol=1e-12)


def test_single_row_evaluation_equals_whole_sequence_evaluation():
    rng = np.random.default_rng(7)
    hq, hkv, d = 4, 1, 16
    lens, chunks = (90, 40), (60, 40)
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 6)
    whole = paged_prefill_attention(qp, kp, vp, t, lens, cu, 0.25)
    rows = [0, 13, 59]
    part = paged_prefill_attention(qp, kp, vp, t, lens, cu, 0.25, batch_subset=[0], row_subset=rows)
    np.testing.assert_allclose(part[rows], whole[rows], rtol=0, atol=1e-12)
    assert np.isnan(part[60:]).all() and np.isnan(np.delete(part[:60], rows, axis=0)).all()


def test_empty_chunks_and_bad_offsets():
    rng = np.random.default_rng(8)
    hq, hkv, d = 4, 2, 8
    lens, chunks = (5, 30, 9), (0, 4, 0)
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 7)
    out = paged_prefill_attention(qp, kp, vp, t, lens, cu, 0.5)
    assert out.shape == (4, hq, d) and np.isfinite(out).all()
    with pytest.raises(ValueError):
        paged_prefill_attention(qp, kp, vp, t, lens, np.array([0, 4, 3, 4]), 0.5)
    with pytest.raises(ValueError):
        paged_prefill_attention(qp, kp, vp, t, lens, np.array([0, 1, 2, 3]), 0.5)


def _padded(qp, cu, chunks, hq, d):
    """Packed rows as a padded [B, max chunk, Hq, D] batch of query rows."""
    q = np.zeros((len(chunks), max(max(chunks), 1), hq, d), np.uint16)
    for b, n in enumerate(chunks):
        q[b, :n] = qp[cu[b]:cu[b + 1]]
    return q


@pytest.mark.parametrize("window", [1, 5, 16, 40, 1000])
def test_window_and_sinks_match_torch_sdpa(window):
    """A sliding window and sink logits on packed chunks: torch float64 SDPA
    with an additive mask (-inf outside each row's causal window) and one
    extra zero key/value column biased by the head's sink."""
    rng = np.random.default_rng(300 + window)
    hq, hkv, d = 8, 2, 16
    lens, chunks = (1, 37, 90, 150), (1, 37, 20, 64)
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 11)
    sinks = rng.uniform(-4, 4, hq).astype(np.float32)
    sinks[2] = -np.inf                                      # this head has no sink
    scale = np.float32(0.3)
    out = paged_prefill_attention(qp, kp, vp, t, lens, cu, scale, sliding_window=window, sinks=sinks)
    ref = _sdpa_masked(_padded(qp, cu, chunks, hq, d), ks, vs, lens, chunks, float(scale), hq, hkv, window, sinks)
    for b, n in enumerate(chunks):
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref[b, :n], rtol=0, atol=1e-12)
    # chosen rows alone agree with the whole-sequence evaluation
    part = paged_prefill_attention(qp, kp, vp, t, lens, cu, scale, sliding_window=window, sinks=sinks,
                                   batch_subset=[3], row_subset=[0, 31, 63])
    rows = [cu[3] + r for r in (0, 31, 63)]
    np.testing.assert_allclose(part[rows], out[rows], rtol=0, atol=1e-12)


def test_window_of_one_returns_the_rows_own_value():
    rng = np.random.default_rng(12)
    hq, hkv, d = 4, 1, 8
    lens, chunks = (20, 9), (7, 9)
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 12)
    out = paged_prefill_attention(qp, kp, vp, t, lens, cu, 0.7, sliding_window=1)
    for b, (L, n) in enumerate(zip(lens, chunks)):
        for r in range(n):
            np.testing.assert_array_equal(out[cu[b] + r], np.repeat(bf16_bits_to_f64(vs[b][L - n + r]), hq, axis=0))


def _fp8_case(rng, lens, chunks, hq, hkv, d):
    """Random e4m3fn codes (no NaN) and per-token scales for each sequence,
    paged into a pool with the scales following their slots."""
    ks8, vs8, kss, vss = [], [], [], []
    for L in lens:
        for store, sc in ((ks8, kss), (vs8, vss)):
            c = rng.integers(0, 256, (L, hkv, d)).astype(np.uint8)
            c[(c & 0x7F) == 0x7F] = 0x3A
            store.append(c)
            sc.append(rng.uniform(0.001, 0.02, (L, hkv)).astype(np.float32))
    kp, vp, t = _page(ks8, vs8, hkv, d, rng, dtype=np.uint8)
    ksc = np.ones((kp.shape[0], 16, hkv), np.float32)
    vsc = np.ones_like(ksc)
    for b, L in enumerate(lens):
        for j in range(L):
            ksc[t[b, j // 16], j % 16] = kss[b][j]
            vsc[t[b, j // 16], j % 16] = vss[b][j]
    return ks8, vs8, kss, vss, kp, vp, t, ksc, vsc


def test_fp8_cache_matches_torch_sdpa_on_dequantised_values():
    """An e4m3fn cache with per-token scales: torch float64 SDPA on the
    decoded codes times their scales (torch's own e4m3fn decoding)."""
    rng = np.random.default_rng(13)
    hq, hkv, d = 8, 2, 16
    lens, chunks = (3, 40, 90), (3, 15, 50)
    ks8, vs8, kss, vss, kp, vp, t, ksc, vsc = _fp8_case(rng, lens, chunks, hq, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    scale = np.float32(0.25)
    out = paged_prefill_attention(qp, kp, vp, t, lens, cu, scale, ksc, vsc, kv_dtype="fp8_e4m3fn")
    ref = _sdpa_reference(_padded(qp, cu, chunks, hq, d), ks8, vs8, lens, chunks, float(scale), hq, hkv, kss, vss,
                          fp8=True)
    for b, n in enumerate(chunks):
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref[b, :n], rtol=0, atol=1e-12)


def prefill_battery(orc) -> bool:
    """The pins above in brief, against a (possibly mutated) oracle copy."""
    rng = np.random.default_rng(9)
    hq, hkv, d = 4, 2, 16
    lens, chunks = (40, 70, 5), (40, 25, 5)
    ks, vs = _seqs(rng, lens, hkv, d)
    qp, cu = _pack(rng, lens, chunks, hq, d)
    kp, vp, t = _paged(ks, vs, hkv, d, 16, 8)
    scale = np.float32(0.3)
    out = orc.paged_prefill_attention(qp, kp, vp, t, lens, cu, scale)
    ref = _sdpa_packed(qp, cu, ks, vs, lens, float(scale), hq, hkv)
    if not np.allclose(out, ref, rtol=0, atol=1e-12):
        return False
    part = orc.paged_prefill_attention(qp, kp, vp, t, lens, cu, scale, batch_subset=[1], row_subset=[0, 24])
    if not np.allclose(part[[cu[1], cu[1] + 24]], ref[[cu[1], cu[1] + 24]], rtol=0, atol=1e-12):
        return False
    # a sliding window with sinks, whole sequences and a chosen row
    sinks = np.array([1.5, -1.0, 0.5, 3.0], np.float32)
    outw = orc.paged_prefill_attention(qp, kp, vp, t, lens, cu, scale, sliding_window=9, sinks=sinks)
    refw = _sdpa_masked(_padded(qp, cu, chunks, hq, d), ks, vs, lens, chunks, float(scale), hq, hkv, 9, sinks)
    for b, n in enumerate(chunks):
        if not np.allclose(outw[cu[b]:cu[b + 1]], refw[b, :n], rtol=0, atol=1e-12):
            return False
    partw = orc.paged_prefill_attention(qp, kp, vp, t, lens, cu, scale, batch_subset=[1], row_subset=[20],
                                        sliding_window=9, sinks=sinks)
    if not np.allclose(partw[cu[1] + 20], refw[1, 20], rtol=0, atol=1e-12):
        return False
    # an fp8 cache with per-token scales
    lens8, chunks8 = (20, 33), (20, 9)
    ks8, vs8, kss, vss, kp8, vp8, t8, ksc, vsc = _fp8_case(rng, lens8, chunks8, hq, hkv, d)
    qp8, cu8 = _pack(rng, lens8, chunks8, hq, d)
    out8 = orc.paged_prefill_attention(qp8, kp8, vp8, t8, lens8, cu8, scale, ksc, vsc, kv_dtype="fp8_e4m3fn")
    ref8 = _sdpa_reference(_padded(qp8, cu8, chunks8, hq, d), ks8, vs8, lens8, chunks8, float(scale), hq, hkv,
                           kss, vss, fp8=True)
    return all(np.allclose(out8[cu8[b]:cu8[b + 1]], ref8[b, :n], rtol=0, atol=1e-12) for b, n in enumerate(chunks8))

"""Pins of the CPU oracle against things other than itself.

Closed forms, invariants, brute force on tiny inputs and independent library
routines (PyTorch's dtype casts and its float64 scaled-dot-product
attention).  Each pin is chosen to catch a class of plausible oracle
mistakes: a wrong block/slot index, a wrong GQA head map, a missing softmax
scale, a wrong causal offset, a misapplied fp8 scale, a bad format decode.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f64, e4m3fn_bytes_to_f64, e4m3fn_table, merge_states,
                    paged_decode_attention, partial_state)

BS = 16


# ----------------------------------------------------------------------------
# format decoders
# ----------------------------------------------------------------------------
def test_bf16_decode_exhaustive_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros / infinities survive
    assert np.signbit(ours[0x8000]) and ours[0x8000] == 0
    assert ours[0x7F80] == np.inf and ours[0xFF80] == -np.inf
    assert ours[0x3F80] == 1.0 and ours[0xC000] == -2.0


def test_e4m3fn_table_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3fn_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0),
    (0x3C, 1.5), (0x06, 0.01171875),
])
def test_e4m3fn_format_definition_values(code, value):
    # OCP FP8 e4m3fn: bias 7, 3 mantissa bits, max normal 1.75 * 2^8 = 448,
    # smallest subnormal 2^-9, no infinities.
    assert e4m3fn_bytes_to_f64(np.array([code], np.uint8))[0] == value


def test_e4m3fn_negative_zero_and_monotone():
    t = e4m3fn_table()
    assert t[0x80] == 0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)          # codes 0x00..0x7E strictly increasing
    assert np.array_equal(t[0x80:0xFF], -pos)


# ----------------------------------------------------------------------------
# helpers: contiguous sequences -> random paged cache
# ----------------------------------------------------------------------------
def _bf16_bits(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _page(seqs_k, seqs_v, hkv, d, rng, extra_blocks=3, dtype=np.uint16):
    """Scatter per-sequence contiguous caches [L_b, Hkv, D] into a randomly
    permuted pool; returns (k_pool, v_pool, tables, perm_info)."""
    nblk = [(len(k) + BS - 1) // BS for k in seqs_k]
    nb = sum(nblk) + extra_blocks
    W = max(max(nblk), 1)
    perm = rng.permutation(nb)
    kp = np.zeros((nb, BS, hkv, d), dtype=dtype)
    vp = np.zeros((nb, BS, hkv, d), dtype=dtype)
    tables = np.zeros((len(seqs_k), W), dtype=np.int32)
    off = 0
    for b, (k, v) in enumerate(zip(seqs_k, seqs_v)):
        for i in range(nblk[b]):
            blk = perm[off + i]
            tables[b, i] = blk
            rows = slice(i * BS, min((i + 1) * BS, len(k)))
            nrow = rows.stop - rows.start
            kp[blk, :nrow] = k[rows]
            vp[blk, :nrow] = v[rows]
        off += nblk[b]
    return kp, vp, tables


def _case(rng, B=2, Qmax=2, hq=4, hkv=2, d=8, lens=(5, 37), qlens=(2, 1)):
    q = _bf16_bits(rng.standard_normal((B, Qmax, hq, d)))
    ks = [_bf16_bits(rng.standard_normal((L, hkv, d))) for L in lens]
    vs = [_bf16_bits(rng.standard_normal((L, hkv, d))) for L in lens]
    kp, vp, tables = _page(ks, vs, hkv, d, rng)
    return q, ks, vs, kp, vp, tables, np.array(lens, np.int32), np.array(qlens, np.int32)


def _brute_force(q, ks, vs, lens, qlens, scale, hq, hkv):
    """Pure-Python triple loop over contiguous sequences with math.exp."""
    B, Qmax, _, D = q.shape
    G = hq // hkv
    out = np.full(q.shape, np.nan)
    qf = bf16_bits_to_f64(q)
    for b in range(B):
        L, n = int(lens[b]), int(qlens[b])
        kf = bf16_bits_to_f64(ks[b])
        vf = bf16_bits_to_f64(vs[b])
        for t in range(n):
            last = L - n + t
            for h in range(hq):
                g = h // G
                xs = []
                for j in range(last + 1):
                    acc = 0.0
                    for dd in range(D):
                        acc += qf[b, t, h, dd] * kf[j, g, dd]
                    xs.append(scale * acc)
                mx = max(xs)
                ws = [math.exp(x - mx) for x in xs]
                den = sum(ws)
                for dd in range(D):
                    out[b, t, h, dd] = sum(w * vf[j, g, dd] for j, w in enumerate(ws)) / den
    return out


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_single_token_context_returns_v():
    rng = np.random.default_rng(0)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, B=1, Qmax=1, lens=(1,), qlens=(1,))
    out = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.37)
    v = bf16_bits_to_f64(vs[0])[0]                      # [Hkv, D]
    G = 2
    for h in range(4):
        assert np.array_equal(out[0, 0, h], v[h // G])


def test_identical_keys_give_mean_of_attended_values():
    rng = np.random.default_rng(1)
    L, hkv, d = 29, 2, 8
    key = _bf16_bits(rng.standard_normal((1, hkv, d)))
    ks = [np.repeat(key, L, axis=0)]
    vs = [_bf16_bits(rng.standard_normal((L, hkv, d)))]
    kp, vp, tables = _page(ks, vs, hkv, d, rng)
    q = _bf16_bits(rng.standard_normal((1, 2, 4, d)))
    out = paged_decode_attention(q, kp, vp, tables, [L], [2], 0.5)
    vf = bf16_bits_to_f64(vs[0])
    for t in range(2):
        last = L - 2 + t
        for h in range(4):
            np.testing.assert_allclose(out[0, t, h], vf[: last + 1, h // 2].mean(axis=0),
                                       rtol=0, atol=1e-12)


def test_two_keys_with_log2_gap_weight_one_third_two_thirds():
    # scores differ by exactly ln 2 -> softmax weights 1/3 and 2/3
    d = 2
    q = _bf16_bits(np.array([[[[1.0, 0.0]]]]))
    k = np.zeros((2, 1, d))
    k[1, 0, 0] = 1.0
    v = np.array([[[3.0, -6.0]], [[6.0, 9.0]]])
    kp, vp, tables = _page([_bf16_bits(k)], [_bf16_bits(v)], 1, d, np.random.default_rng(2))
    out = paged_decode_attention(q, kp, vp, tables, [2], [1], np.float32(math.log(2.0)))
    s = np.float64(np.float32(math.log(2.0)))           # the fp32 scale the call carries
    w1 = 1.0 / (1.0 + math.exp(s))
    expect = w1 * v[0, 0] + (1 - w1) * v[1, 0]
    np.testing.assert_allclose(out[0, 0, 0], expect, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, 0, 0], [5.0, 4.0], atol=1e-6)


def test_planted_key_dominates():
    rng = np.random.default_rng(3)
    L, hkv, d = 40, 1, 8
    qv = rng.standard_normal(d)
    k = rng.standard_normal((L, hkv, d)) * 0.1
    k[17, 0] = 64.0 * qv
    v = rng.standard_normal((L, hkv, d))
    kp, vp, tables = _page([_bf16_bits(k)], [_bf16_bits(v)], hkv, d, rng)
    q = _bf16_bits(qv[None, None, None, :])
    out = paged_decode_attention(q, kp, vp, tables, [L], [1], 1.0)
    np.testing.assert_allclose(out[0, 0, 0], bf16_bits_to_f64(_bf16_bits(v))[17, 0], atol=1e-9)


def test_linear_in_values():
    rng = np.random.default_rng(4)
    L, hkv, d = 23, 2, 8
    k = _bf16_bits(rng.standard_normal((L, hkv, d)))
    v1 = rng.integers(-8, 9, (L, hkv, d)).astype(np.float64)
    v2 = rng.integers(-8, 9, (L, hkv, d)).astype(np.float64)
    v3 = 2.0 * v1 - 3.0 * v2                            # small integers: exact in bf16
    q = _bf16_bits(rng.standard_normal((1, 2, 4, d)))
    outs = []
    for v in (v1, v2, v3):
        kp, vp, tables = _page([k], [_bf16_bits(v)], hkv, d, np.random.default_rng(9))
        outs.append(paged_decode_attention(q, kp, vp, tables, [L], [2], 0.3))
    np.testing.assert_allclose(outs[2], 2 * outs[0] - 3 * outs[1], rtol=0, atol=1e-12)


def test_large_logit_spread_between_rows_is_stable():
    # one query head with logits around 1e3, another around 1e-1: each row's
    # softmax must be shifted by its own maximum, or the small row underflows
    rng = np.random.default_rng(8)
    L, hkv, d = 37, 1, 8
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    kp, vp, tables = _page([_bf16_bits(k)], [_bf16_bits(v)], hkv, d, rng)
    qv = rng.standard_normal((1, 1, 2, d))
    qv[0, 0, 0] *= 400.0
    q = _bf16_bits(qv)
    out = paged_decode_attention(q, kp, vp, tables, [L], [1], 1.0)
    ref = _sdpa_reference(q, [_bf16_bits(k)], [_bf16_bits(v)], [L], [1], 1.0, 2, 1)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# paging invariants
# ----------------------------------------------------------------------------
def test_invariant_to_physical_block_placement_bit_exact():
    rng = np.random.default_rng(5)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, lens=(33, 48))
    ref = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.25)
    pi = rng.permutation(kp.shape[0])                    # relabel every physical block
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    out = paged_decode_attention(q, kp2, vp2, pi[tables], lens, qlens, 0.25)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    assert np.array_equal(out[~np.isnan(ref)], ref[~np.isnan(ref)])


def test_shared_and_duplicated_blocks_equal_private_copies():
    rng = np.random.default_rng(6)
    hkv, d = 2, 8
    prefix_k = _bf16_bits(rng.standard_normal((32, hkv, d)))
    prefix_v = _bf16_bits(rng.standard_normal((32, hkv, d)))
    sfx = [(_bf16_bits(rng.standard_normal((n, hkv, d))), _bf16_bits(rng.standard_normal((n, hkv, d))))
           for n in (5, 20)]
    # private copies
    ks = [np.concatenate([prefix_k, s[0]]) for s in sfx]
    vs = [np.concatenate([prefix_v, s[1]]) for s in sfx]
    lens = np.array([len(k) for k in ks], np.int32)
    kp, vp, tables = _page(ks, vs, hkv, d, rng)
    q = _bf16_bits(rng.standard_normal((2, 2, 4, d)))
    ref = paged_decode_attention(q, kp, vp, tables, lens, [2, 2], 0.4)
    # shared prefix blocks: sequence 1 points at sequence 0's first two blocks
    tables_sh = tables.copy()
    tables_sh[1, :2] = tables[0, :2]
    out = paged_decode_attention(q, kp, vp, tables_sh, lens, [2, 2], 0.4)
    assert np.array_equal(out, ref, equal_nan=True)
    # duplicated entries: a sequence whose content repeats one block twice
    rep_k = np.concatenate([prefix_k[:16], prefix_k[:16], prefix_k[:3]])
    rep_v = np.concatenate([prefix_v[:16], prefix_v[:16], prefix_v[:3]])
    kp1, vp1, t1 = _page([rep_k], [rep_v], hkv, d, rng)
    ref1 = paged_decode_attention(q[:1], kp1, vp1, t1, [35], [1], 0.4)
    t_dup = t1.copy()
    t_dup[0, 1] = t1[0, 0]
    out1 = paged_decode_attention(q[:1], kp1, vp1, t_dup, [35], [1], 0.4)
    assert np.array_equal(out1, ref1, equal_nan=True)


def test_unread_memory_does_not_matter():
    # NaN in unused blocks, tail slots and table padding never reaches the output
    rng = np.random.default_rng(7)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, lens=(5, 37))
    ref = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.3)
    kp2, vp2 = kp.copy(), vp.copy()
    used = set()
    for b, L in enumerate(lens):
        nb = (L + BS - 1) // BS
        used.update(tables[b, :nb].tolist())
        last, tail = tables[b, nb - 1], L - (nb - 1) * BS
        kp2[last, tail:] = 0x7FC0
        vp2[last, tail:] = 0x7FC0
    for blk in range(kp.shape[0]):
        if blk not in used:
            kp2[blk] = 0x7FC0
            vp2[blk] = 0x7FC0
    t2 = tables.copy()
    t2[0, 1:] = 10 ** 6                                  # padding past ceil(L/16) is never read
    out = paged_decode_attention(q, kp2, vp2, t2, lens, qlens, 0.3)
    assert np.array_equal(out, ref, equal_nan=True)


# ----------------------------------------------------------------------------
# brute force and an independent library routine
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (4, 1), (6, 3)])   # GQA, MHA, MQA
def test_matches_brute_force_tiny(hq, hkv):
    rng = np.random.default_rng(10 + hq * 7 + hkv)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, B=3, Qmax=2, hq=hq, hkv=hkv, d=8,
                                                   lens=(1, 17, 40), qlens=(1, 2, 2))
    scale = np.float32(0.35)
    out = paged_decode_attention(q, kp, vp, tables, lens, qlens, scale)
    ref = _brute_force(q, ks, vs, lens, qlens, float(scale), hq, hkv)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    np.testing.assert_allclose(out[~np.isnan(ref)], ref[~np.isnan(ref)], rtol=0, atol=1e-12)


def _sdpa_reference(q, seqs_k, seqs_v, lens, qlens, scale, hq, hkv, k_scales=None, v_scales=None,
                    fp8=False):
    """torch float64 SDPA on contiguous data, GQA by repeat_interleave,
    explicit offset-causal boolean mask."""
    B, Qmax, _, D = q.shape
    G = hq // hkv
    out = np.full(q.shape, np.nan)
    qt = torch.from_numpy(q.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    for b in range(B):
        L, n = int(lens[b]), int(qlens[b])
        if fp8:
            k = torch.from_numpy(seqs_k[b].copy()).view(torch.float8_e4m3fn).to(torch.float64)
            v = torch.from_numpy(seqs_v[b].copy()).view(torch.float8_e4m3fn).to(torch.float64)
            k = k * torch.from_numpy(k_scales[b]).to(torch.float64)[..., None]
            v = v * torch.from_numpy(v_scales[b]).to(torch.float64)[..., None]
        else:
            k = torch.from_numpy(seqs_k[b].view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
            v = torch.from_numpy(seqs_v[b].view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
        kk = k.permute(1, 0, 2).repeat_interleave(G, dim=0)          # [Hq, L, D]
        vv = v.permute(1, 0, 2).repeat_interleave(G, dim=0)
        qq = qt[b, :n].permute(1, 0, 2)                               # [Hq, n, D]
        rows = torch.arange(n)[:, None] + (L - n)
        mask = torch.arange(L)[None, :] <= rows                       # [n, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, scale=float(scale))
        out[b, :n] = o.permute(1, 0, 2).numpy()
    return out


def test_matches_torch_sdpa_float64_bf16():
    rng = np.random.default_rng(20)
    hq, hkv, d = 8, 2, 16
    lens, qlens = (1, 16, 17, 70, 129), (1, 2, 1, 2, 2)
    q, ks, vs, kp, vp, tables, L, n = _case(rng, B=5, Qmax=2, hq=hq, hkv=hkv, d=d, lens=lens, qlens=qlens)
    scale = np.float32(1 / math.sqrt(d))
    out = paged_decode_attention(q, kp, vp, tables, L, n, scale)
    ref = _sdpa_reference(q, ks, vs, L, n, float(scale), hq, hkv)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(out), ~ok)
    np.testing.assert_allclose(out[ok], ref[ok], rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64_fp8_with_per_token_scales():
    rng = np.random.default_rng(21)
    hq, hkv, d = 8, 4, 16
    lens, qlens = (3, 31, 64), (1, 2, 1)
    B, Qmax = 3, 2
    q = _bf16_bits(rng.standard_normal((B, Qmax, hq, d)))
    ks, vs, kss, vss = [], [], [], []
    for L in lens:
        for store, sc in ((ks, kss), (vs, vss)):
            codes = rng.integers(0, 256, (L, hkv, d)).astype(np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0x3A                      # no NaN codes in real rows
            store.append(codes)
            sc.append(rng.uniform(0.001, 0.02, (L, hkv)).astype(np.float32))
    kp, vp, tables = _page(ks, vs, hkv, d, rng, dtype=np.uint8)
    nb = kp.shape[0]
    ksc = np.ones((nb, BS, hkv), np.float32)
    vsc = np.ones((nb, BS, hkv), np.float32)
    for b, L in enumerate(lens):
        for j in range(L):
            ksc[tables[b, j // BS], j % BS] = kss[b][j]
            vsc[tables[b, j // BS], j % BS] = vss[b][j]
    scale = np.float32(0.25)
    out = paged_decode_attention(q, kp, vp, tables, lens, qlens, scale, ksc, vsc, kv_dtype="fp8_e4m3fn")
    ref = _sdpa_reference(q, ks, vs, lens, qlens, float(scale), hq, hkv, kss, vss, fp8=True)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(out), ~ok)
    np.testing.assert_allclose(out[ok], ref[ok], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# causality, row bookkeeping
# ----------------------------------------------------------------------------
def test_causal_rows_see_only_their_prefix():
    rng = np.random.default_rng(30)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, B=1, Qmax=2, lens=(21,), qlens=(2,))
    ref = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.3)
    kp2, vp2 = kp.copy(), vp.copy()
    last = tables[0, (21 - 1) // BS]
    slot = (21 - 1) % BS
    kp2[last, slot] = _bf16_bits(rng.standard_normal(kp.shape[2:]))
    vp2[last, slot] = _bf16_bits(rng.standard_normal(kp.shape[2:]))
    out = paged_decode_attention(q, kp2, vp2, tables, lens, qlens, 0.3)
    assert np.array_equal(out[0, 0], ref[0, 0])         # row 0 stops at position L-2
    assert not np.allclose(out[0, 1], ref[0, 1])         # row 1 sees position L-1


def test_rows_past_query_len_are_not_produced():
    rng = np.random.default_rng(31)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, lens=(9, 18), qlens=(1, 0))
    out = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.3)
    assert np.all(np.isnan(out[0, 1])) and np.all(np.isnan(out[1]))
    assert not np.any(np.isnan(out[0, 0]))


def test_batch_subset_matches_full():
    rng = np.random.default_rng(32)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, lens=(9, 40), qlens=(2, 2))
    full = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.3)
    part = paged_decode_attention(q, kp, vp, tables, lens, qlens, 0.3, batch_subset=[1])
    assert np.array_equal(part[1], full[1]) and np.all(np.isnan(part[0]))


def test_rejects_out_of_range_metadata():
    rng = np.random.default_rng(33)
    q, ks, vs, kp, vp, tables, lens, qlens = _case(rng, lens=(9, 40), qlens=(2, 2))
    with pytest.raises(ValueError):
        paged_decode_attention(q, kp, vp, tables, [1, 40], [2, 2], 0.3)     # n > L
    t2 = tables.copy()
    t2[0, 0] = kp.shape[0]
    with pytest.raises(ValueError):
        paged_decode_attention(q, kp, vp, t2, lens, qlens, 0.3)


# ----------------------------------------------------------------------------
# split-context merge algebra
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("cuts", [[0], [1], [7], [3, 3, 10], [0, 5, 5, 12, 19]])
def test_lse_merge_of_any_split_equals_whole(cuts):
    rng = np.random.default_rng(40 + len(cuts))
    J, D = 19, 6
    x = rng.standard_normal(J) * 3
    v = rng.standard_normal((J, D))
    whole = partial_state(x, v)[2]
    e = np.exp(x - x.max())
    np.testing.assert_allclose(whole, (e @ v) / e.sum(), rtol=0, atol=1e-13)
    bounds = [0] + sorted(cuts) + [J]
    parts = [partial_state(x[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    np.testing.assert_allclose(merge_states(parts), whole, rtol=0, atol=1e-12)


def test_empty_split_contributes_nothing():
    x = np.array([0.5, -1.0])
    v = np.array([[1.0, 2.0], [3.0, 4.0]])
    m, l, o = partial_state(x[:0], v[:0])
    assert m == -np.inf and l == 0
    np.testing.assert_allclose(merge_states([(m, l, o), partial_state(x, v)]),
                               partial_state(x, v)[2], atol=1e-15)

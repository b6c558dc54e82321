"""Planted-mistake check of the oracle's pins (CPU only).

Each case copies the oracle package into a temporary directory, plants one
plausible mistake in the copy (a wrong index, a dropped term, a swapped
operand, an off-by-one mask, a wrong format constant) and runs a battery of
the pins from ``test_oracle`` against the mutated copy.  Every mutant must
fail at least one pin; the unmutated copy must pass them all.
"""
import importlib.util
import os
import shutil
import sys

import numpy as np
import pytest
import torch

from test_oracle import _bf16_bits, _case, _page, _sdpa_reference
from test_oracle_prefill import prefill_battery
from test_oracle_variants import variant_battery

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = {
    "kv_head_of_keys": ("paged_attention.py", "K[:, g, :].T", "K[:, (g + 1) % Hkv, :].T"),
    "kv_head_of_values": ("paged_attention.py", "V[:, g, :])", "V[:, (g + 1) % Hkv, :])"),
    "gqa_group_slice": ("paged_attention.py", "Qg = Q[:, g * G:(g + 1) * G, :]",
                        "Qg = Q[:, g:g + G, :]"),
    "dropped_scale": ("paged_attention.py", "x = s * np.matmul", "x = np.matmul"),
    "causal_offset": ("paged_attention.py", "pos = L - n + np.arange(n)", "pos = np.arange(n) + L - 1"),
    "causal_off_by_one": ("paged_attention.py", "<= pos[:, None]", "< pos[:, None] + 0 * 1"),
    "block_index": ("paged_attention.py", "[j // bs]", "[(j // bs) % 2]"),
    "slot_index": ("paged_attention.py", "slot = j % bs", "slot = (j + 1) % bs"),
    "fp8_scale_head": ("paged_attention.py", "vals = vals * s[:, :, None]", "vals = vals * s[:, :1, None]"),
    "normaliser": ("paged_attention.py", "den = e.sum(axis=-1, keepdims=True)", "den = e.sum(axis=-1, keepdims=True).max()"),
    "values_are_keys": ("paged_attention.py", "np.matmul(e, V[:, g, :])", "np.matmul(e, K[:, g, :])"),
    "no_max_shift": ("paged_attention.py", "mx = x.max(axis=-1, keepdims=True)", "mx = x.max()"),
    "window_off_by_one": ("paged_attention.py", "> (pos - window)[:, None]", ">= (pos - window)[:, None]"),
    "sink_head_index": ("paged_attention.py", "sink[g * G:(g + 1) * G]", "sink[g:g + G]"),
    "sink_not_in_max": ("paged_attention.py", "mx = np.maximum(mx, sk)", "mx = mx + 0 * sk"),
    "sink_dropped": ("paged_attention.py", "+ np.exp(sk - mx)", "+ 0 * np.exp(sk - mx)"),
    "block_size_fixed": ("paged_attention.py", "bs = np.asarray(cache).shape[1]", "bs = 16"),
    "prefill_prefix_dropped": ("prefill.py", "[int(ctx[b])], [n], scale", "[n], [n], scale"),
    "prefill_row_position": ("prefill.py", "Lt = int(ctx[b]) - n + int(t) + 1", "Lt = int(ctx[b]) - n + int(t)"),
    "prefill_rows_reversed": ("prefill.py", "q_bits[cu[b]:cu[b + 1]][None]", "q_bits[cu[b]:cu[b + 1]][::-1][None]"),
    "prefill_window_dropped": ("prefill.py", "sliding_window=sliding_window, sinks=sinks)",
                               "sliding_window=None, sinks=sinks)"),
    "prefill_sinks_dropped": ("prefill.py", "sliding_window=sliding_window, sinks=sinks)",
                              "sliding_window=sliding_window, sinks=None)"),
    "prefill_fp8_scales_swapped": ("prefill.py", "scale, k_scale, v_scale, kv_dtype,",
                                   "scale, v_scale, k_scale, kv_dtype,"),
    "e4m3_subnormal": ("formats.py", "man_field * 2.0 ** -9", "man_field * 2.0 ** -10"),
    "e4m3_bias": ("formats.py", "2.0 ** (exp_field - 7)", "2.0 ** (exp_field - 8)"),
    "e4m3_mantissa": ("formats.py", "(1.0 + man_field / 8.0)", "(1.0 + man_field / 16.0)"),
    "bf16_shift": ("formats.py", "(u << np.uint32(16))", "(u << np.uint32(15))"),
}


def _load_copy(tmp_path, mutant):
    pkg = tmp_path / "oracle_copy"
    shutil.copytree(ORACLE_DIR, pkg, ignore=shutil.ignore_patterns("__pycache__"))
    if mutant is not None:
        fname, old, new = MUTANTS[mutant]
        path = pkg / fname
        src = path.read_text()
        assert src.count(old) >= 1, f"mutation site {old!r} not found"
        path.write_text(src.replace(old, new))
    name = f"oracle_copy_{mutant or 'clean'}"
    spec = importlib.util.spec_from_file_location(name, pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


def _battery(orc) -> bool:
    """True if the (possibly mutated) oracle passes every pin in the battery."""
    try:
        # decoders against torch, exhaustively
        codes16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        ref16 = torch.from_numpy(codes16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
        got16 = orc.bf16_bits_to_f64(codes16)
        ok = ~np.isnan(ref16)
        if not (np.array_equal(np.isnan(got16), ~ok) and np.array_equal(got16[ok], ref16[ok])):
            return False
        ref8 = torch.arange(256).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        got8 = orc.e4m3fn_table()
        ok = ~np.isnan(ref8)
        if not (np.array_equal(np.isnan(got8), ~ok) and np.array_equal(got8[ok], ref8[ok])):
            return False
        # bf16 attention vs float64 SDPA (GQA, ragged, causal qlen 2)
        rng = np.random.default_rng(123)
        hq, hkv, d = 8, 2, 16
        q, ks, vs, kp, vp, tables, L, n = _case(rng, B=4, Qmax=2, hq=hq, hkv=hkv, d=d,
                                                lens=(2, 17, 40, 70), qlens=(2, 1, 2, 2))
        scale = np.float32(0.3)
        out = orc.paged_decode_attention(q, kp, vp, tables, L, n, scale)
        ref = _sdpa_reference(q, ks, vs, L, n, float(scale), hq, hkv)
        ok = ~np.isnan(ref)
        if not (np.array_equal(np.isnan(out), ~ok) and np.allclose(out[ok], ref[ok], rtol=0, atol=1e-12)):
            return False
        # fp8 attention with per-token scales vs float64 SDPA
        lens, qlens = (5, 37), (2, 1)
        q8 = _bf16_bits(rng.standard_normal((2, 2, hq, d)))
        ks8, vs8, kss, vss = [], [], [], []
        for Lb in lens:
            for store, sc in ((ks8, kss), (vs8, vss)):
                c = rng.integers(0, 256, (Lb, hkv, d)).astype(np.uint8)
                c[(c & 0x7F) == 0x7F] = 0x3A
                store.append(c)
                sc.append(rng.uniform(0.001, 0.02, (Lb, hkv)).astype(np.float32))
        kp8, vp8, t8 = _page(ks8, vs8, hkv, d, rng, dtype=np.uint8)
        ksc = np.ones((kp8.shape[0], 16, hkv), np.float32)
        vsc = np.ones_like(ksc)
        for b, Lb in enumerate(lens):
            for j in range(Lb):
                ksc[t8[b, j // 16], j % 16] = kss[b][j]
                vsc[t8[b, j // 16], j % 16] = vss[b][j]
        out8 = orc.paged_decode_attention(q8, kp8, vp8, t8, lens, qlens, scale, ksc, vsc,
                                          kv_dtype="fp8_e4m3fn")
        ref8a = _sdpa_reference(q8, ks8, vs8, lens, qlens, float(scale), hq, hkv, kss, vss, fp8=True)
        ok = ~np.isnan(ref8a)
        if not (np.array_equal(np.isnan(out8), ~ok) and np.allclose(out8[ok], ref8a[ok], rtol=0, atol=1e-12)):
            return False
        # rows with very different logit magnitudes in one call
        k1 = rng.standard_normal((37, 1, 8))
        v1 = rng.standard_normal((37, 1, 8))
        kp1, vp1, t1 = _page([_bf16_bits(k1)], [_bf16_bits(v1)], 1, 8, rng)
        qv = rng.standard_normal((1, 1, 2, 8))
        qv[0, 0, 0] *= 400.0
        q1 = _bf16_bits(qv)
        with np.errstate(all="ignore"):
            o1 = orc.paged_decode_attention(q1, kp1, vp1, t1, [37], [1], 1.0)
        r1 = _sdpa_reference(q1, [_bf16_bits(k1)], [_bf16_bits(v1)], [37], [1], 1.0, 2, 1)
        if not (np.all(np.isfinite(o1)) and np.allclose(o1, r1, rtol=0, atol=1e-12)):
            return False
        # split/merge: a closed form with a large logit spread
        x = np.array([700.0, 0.0])
        m, l, o = orc.partial_state(x, np.eye(2))
        if not np.all(np.isfinite(o)):
            return False
        # block sizes, sliding window, sinks
        if not variant_battery(orc):
            return False
        # packed prefill chunks
        if not prefill_battery(orc):
            return False
    except Exception:
        return False
    return True


def test_clean_copy_passes_battery(tmp_path):
    assert _battery(_load_copy(tmp_path, None))


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_every_planted_mistake_is_caught(tmp_path, mutant):
    assert not _battery(_load_copy(tmp_path, mutant)), f"pins missed the planted mistake {mutant}"

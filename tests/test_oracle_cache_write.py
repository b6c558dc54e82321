"""Pins of the cache-write oracle (oracle/cache_write.py) against the format
definition, an independent library cast, closed forms and invariants."""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, e4m3fn_table, gather_sequence_kv
from oracle.cache_write import FP8_MAX, e4m3fn_encode, quantize_rows_e4m3fn, reshape_and_cache


def _torch_codes(y):
    """PyTorch's float32 -> float8_e4m3fn cast (round to nearest even)."""
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_finite_code_encodes_to_itself():
    table = e4m3fn_table()
    codes = np.array([c for c in range(256) if not np.isnan(table[c])], dtype=np.uint8)
    assert len(codes) == 254
    assert np.array_equal(e4m3fn_encode(table[codes]), codes)


def test_midpoints_round_to_the_even_code():
    table = e4m3fn_table()
    for c in range(0x7E):                        # neighbours c, c+1 among the positive codes
        mid = (table[c] + table[c + 1]) / 2.0
        even = c if c % 2 == 0 else c + 1
        assert int(e4m3fn_encode(np.float32(mid))) == even, hex(c)
        assert int(e4m3fn_encode(np.float32(-mid))) == even | 0x80, hex(c)
        # just off the midpoint: the nearer neighbour
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(np.inf))
        assert int(e4m3fn_encode(below)) == c and int(e4m3fn_encode(above)) == c + 1


def test_encoder_matches_the_library_cast():
    rng = np.random.default_rng(11)
    y = np.concatenate([
        rng.uniform(-FP8_MAX, FP8_MAX, 200000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 50000),          # subnormal range and its edge
        rng.normal(0, 4, 50000).clip(-FP8_MAX, FP8_MAX),
        [0.0, -0.0, FP8_MAX, -FP8_MAX, 2.0 ** -10, -2.0 ** -10, 2.0 ** -9 * 1.5],
    ]).astype(np.float32)
    assert np.array_equal(e4m3fn_encode(y), _torch_codes(y))


def test_row_quantisation_closed_forms():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (300, 8, 128)).astype(np.float32)
    codes, scale = quantize_rows_e4m3fn(x)
    amax = np.abs(x).max(-1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest magnitude of every row lands on +-448 (codes 0x7E / 0xFE)
    at = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes, at[..., None], -1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    # dequantisation error: half a step of 3 mantissa bits (relative 2^-4) in
    # the normal range, half the subnormal spacing (2^-10) times the scale below it
    dq = e4m3fn_table()[codes] * scale[..., None]
    err = np.abs(dq - x.astype(np.float64))
    assert np.all(err <= 2.0 ** -4 * np.abs(x) + scale[..., None] * 2.0 ** -10 + 1e-30)
    # an all-zero row: scale 1, codes +0
    c0, s0 = quantize_rows_e4m3fn(np.zeros((2, 64), np.float32))
    assert np.all(c0 == 0) and np.all(s0 == 1.0)


def _torch_row_quant(x):
    """The absmax/448 rule in PyTorch float32 on the CPU: scale = |x|max / 448
    (1 for an all-zero row), codes = float8_e4m3fn(clamp(x / scale, +-448)).
    PyTorch's division and its float8 cast, independent of the oracle."""
    x = torch.from_numpy(np.asarray(x, np.float32))
    a = x.abs().amax(dim=-1)
    s = torch.where(a > 0, a / 448.0, torch.ones_like(a))
    y = (x / s[..., None]).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s.numpy()


def _bf16_rows(rng, shape, spread=False):
    """N(0, 1) rows rounded to bf16 (the cache write's input), optionally
    with per-row magnitudes spread over 2^-40 .. 2^40."""
    x = rng.normal(0, 1, shape).astype(np.float32)
    if spread:
        x *= np.exp2(rng.integers(-40, 41, shape[:-1] + (1,))).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def test_row_quantisation_matches_torch_division_and_cast():
    rng = np.random.default_rng(31)
    x = np.concatenate([_bf16_rows(rng, (4000, 64)), _bf16_rows(rng, (2000, 128), spread=False)[:, :64],
                        _bf16_rows(rng, (2000, 64), spread=True)])
    codes, scale = quantize_rows_e4m3fn(x)
    tc, ts = _torch_row_quant(x)
    assert np.array_equal(scale, ts)
    assert np.array_equal(codes, tc)
    # the pin separates the division from the reciprocal product
    # x * (448 / absmax): on these rows the two round to different codes
    a = np.abs(x).max(-1, keepdims=True)
    y2 = np.clip(x * (np.float32(448) / a), -448, 448).astype(np.float32)
    assert np.count_nonzero(e4m3fn_encode(y2) != tc) > 100


def test_row_quantisation_of_extreme_rows_matches_torch():
    # rows mixing the largest and the smallest bf16 magnitudes (quotients in
    # float32's subnormal range), a single nonzero element, subnormal absmax
    tiny = np.float32(torch.tensor(2.0 ** -133, dtype=torch.bfloat16).float())
    rows = np.zeros((6, 64), np.float32)
    rows[0, 0], rows[0, 1:8] = 3.0e38, [tiny, -tiny, 1e-30, -1e-38, 2.0 ** -126, 1.0, -1.0]
    rows[1, 5] = -7.0
    rows[2, :] = tiny
    rows[2, 3] = -2 * tiny
    rows[3, 0], rows[3, 1] = 2.0 ** -120, 2.0 ** -130
    rows[4] = np.linspace(-1, 1, 64)
    rows[5, 0], rows[5, 1:] = 448.0, -2.0 ** -12
    rows = torch.from_numpy(rows).to(torch.bfloat16).float().numpy()
    codes, scale = quantize_rows_e4m3fn(rows)
    tc, ts = _torch_row_quant(rows)
    assert np.array_equal(scale, ts) and np.array_equal(codes, tc)
    assert np.all(scale > 0)


def test_quantisation_is_scale_invariant_by_powers_of_two():
    rng = np.random.default_rng(6)
    x = rng.normal(0, 1, (64, 64)).astype(np.float32)
    c1, s1 = quantize_rows_e4m3fn(x)
    c2, s2 = quantize_rows_e4m3fn(x * np.float32(8.0))     # exact in fp32
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * np.float32(8.0))


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("bs", [16, 64])
def test_write_touches_exactly_the_mapped_slots(kv, bs):
    rng = np.random.default_rng(9)
    NB, H, D, T = 6, 2, 64, 7
    kn = _bf16_bits(rng.normal(0, 1, (T, H, D)))
    vn = _bf16_bits(rng.normal(0, 1, (T, H, D)))
    # a negative slot and NB*bs (one past the pool) are skipped
    slots = np.array([5, -1, 17, NB * bs - 1, 40, NB * bs, 0])
    cdt = np.uint8 if kv == "fp8_e4m3fn" else np.uint16
    kc = np.full((NB, bs, H, D), 0x3C, cdt)
    vc = np.full((NB, bs, H, D), 0x3C, cdt)
    ks = np.full((NB, bs, H), 7.0, np.float32) if kv == "fp8_e4m3fn" else None
    vs = np.full((NB, bs, H), 7.0, np.float32) if kv == "fp8_e4m3fn" else None
    k2, v2, ks2, vs2 = reshape_and_cache(kn, vn, slots, kc, vc, ks, vs, kv)
    written = {5, 17, NB * bs - 1, 40, 0}
    for s in range(NB * bs):
        b, p = divmod(s, bs)
        if s in written:
            t = int(np.nonzero(slots == s)[0][0])
            for new, cache, sc in ((kn, k2, ks2), (vn, v2, vs2)):
                x = bf16_bits_to_f64(new[t])
                if kv == "bf16":
                    assert np.array_equal(cache[b, p], new[t])
                else:
                    dq = e4m3fn_table()[cache[b, p]] * sc[b, p][:, None]
                    assert np.all(np.abs(dq - x) <= 2.0 ** -4 * np.abs(x) + sc[b, p][:, None] * 2.0 ** -10)
        else:
            assert np.all(k2[b, p] == 0x3C) and np.all(v2[b, p] == 0x3C)
            if ks2 is not None:
                assert np.all(ks2[b, p] == 7.0) and np.all(vs2[b, p] == 7.0)
    assert np.all(kc == 0x3C)                                # inputs untouched


def test_written_tokens_read_back_through_the_attention_gather():
    rng = np.random.default_rng(12)
    NB, H, D = 10, 2, 64
    table = np.array([[7, 2, 9]], np.int32)
    L = 40
    kn = _bf16_bits(rng.normal(0, 1, (L, H, D)))
    vn = _bf16_bits(rng.normal(0, 1, (L, H, D)))
    pos = np.arange(L)
    slots = table[0, pos // 16].astype(np.int64) * 16 + pos % 16
    for kv, cdt in (("bf16", np.uint16), ("fp8_e4m3fn", np.uint8)):
        kc = np.zeros((NB, 16, H, D), cdt)
        vc = np.zeros((NB, 16, H, D), cdt)
        ks = np.ones((NB, 16, H), np.float32) if kv != "bf16" else None
        vs = np.ones((NB, 16, H), np.float32) if kv != "bf16" else None
        k2, v2, ks2, vs2 = reshape_and_cache(kn, vn, slots, kc, vc, ks, vs, kv)
        kr = gather_sequence_kv(k2, table[0], L, kv, ks2)               # [L, H, D]
        vr = gather_sequence_kv(v2, table[0], L, kv, vs2)
        if kv == "bf16":
            assert np.array_equal(kr, bf16_bits_to_f64(kn))
            assert np.array_equal(vr, bf16_bits_to_f64(vn))
        else:
            for got, new in ((kr, kn), (vr, vn)):
                codes, sc = quantize_rows_e4m3fn(bf16_bits_to_f64(new).astype(np.float32))
                assert np.array_equal(got, e4m3fn_table()[codes] * sc[..., None].astype(np.float64))


# --------------------------------------------------------------------------
# planted mistakes: every mutant of the cache-write oracle fails a pin
# --------------------------------------------------------------------------
import importlib.util  # noqa: E402
import os  # noqa: E402
import shutil  # noqa: E402
import sys  # noqa: E402

_ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
CW_MUTANTS = {
    "scale_max": ("np.where(nonzero, amax / np.float32(FP8_MAX)", "np.where(nonzero, amax / np.float32(224.0)"),
    "reciprocal_product": ("y = (x / scale[..., None])",
                           "y = (x * (np.float32(1.0) / scale[..., None]).astype(np.float32))"),
    "inverse_of_absmax": ("y = (x / scale[..., None])",
                          "y = (x * (np.float32(FP8_MAX) / np.where(nonzero, amax, np.float32(1))"
                          ".astype(np.float32))[..., None])"),
    "multiply_by_scale": ("y = (x / scale[..., None])", "y = (x * scale[..., None])"),
    "ties_away": ("(_POS_CODES[hi] % 2 == 0)", "(_POS_CODES[hi] >= 0)"),
    "truncate": ("take_hi = (d_hi < d_lo)", "take_hi = (d_hi < 0 * d_lo)"),
    "sign_lost": ("return (code | sign).astype(np.uint8)", "return code.astype(np.uint8)"),
    "slot_block_swap": ("blk, pos = int(s // bs), int(s % bs)",
                        "pos, blk = int(s // bs) % bs, int(s % bs) % nb"),
    "block_size_16": ("blk, pos = int(s // bs), int(s % bs)", "blk, pos = int(s // 16) % nb, int(s % 16)"),
    "v_from_k": ("((k_new_bits, kc, ks), (v_new_bits, vc, vs))", "((k_new_bits, kc, ks), (k_new_bits, vc, vs))"),
    "skip_slot_zero": ("if s < 0 or s >= nb * bs:", "if s <= 0 or s >= nb * bs:"),
    "zero_row_scale": ("amax / np.float32(FP8_MAX), np.float32(1.0))", "amax / np.float32(FP8_MAX), np.float32(0.0))"),
}


def _load_cw(tmp_path, mutant):
    pkg = tmp_path / f"oracle_cw_{mutant or 'clean'}"
    shutil.copytree(_ORACLE_DIR, pkg, ignore=shutil.ignore_patterns("__pycache__"))
    if mutant is not None:
        old, new = CW_MUTANTS[mutant]
        path = pkg / "cache_write.py"
        src = path.read_text()
        assert src.count(old) == 1, f"mutation site {old!r} not found once"
        path.write_text(src.replace(old, new))
    name = f"oracle_cw_copy_{mutant or 'clean'}"
    spec = importlib.util.spec_from_file_location(name, pkg / "__init__.py", submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return importlib.import_module(name + ".cache_write"), mod


def _cw_battery(cw, orc) -> bool:
    try:
        table = orc.e4m3fn_table()
        rng = np.random.default_rng(21)
        y = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000),
                            [(table[c] + table[c + 1]) / 2 for c in range(0x7E)]]).astype(np.float32)
        if not np.array_equal(cw.e4m3fn_encode(y), _torch_codes(y)):
            return False
        x = _bf16_rows(rng, (400, 4, 64))
        codes, scale = cw.quantize_rows_e4m3fn(x)
        tc, ts = _torch_row_quant(x)
        if not (np.array_equal(scale, ts) and np.array_equal(codes, tc)):
            return False
        c0, s0 = cw.quantize_rows_e4m3fn(np.zeros((1, 64), np.float32))
        if not (np.all(c0 == 0) and np.all(s0 == 1.0)):
            return False
        NB, H, D = 6, 2, 64
        kn = _bf16_bits(rng.normal(0, 1, (5, H, D)))
        vn = _bf16_bits(rng.normal(0, 1, (5, H, D)))
        slots = np.array([0, 17, 95, -1, 40])
        for kv, cdt in (("bf16", np.uint16), ("fp8_e4m3fn", np.uint8)):
            kc = np.zeros((NB, 16, H, D), cdt)
            vc = np.zeros((NB, 16, H, D), cdt)
            ks = np.ones((NB, 16, H), np.float32) if kv != "bf16" else None
            vs = np.ones((NB, 16, H), np.float32) if kv != "bf16" else None
            k2, v2, ks2, vs2 = cw.reshape_and_cache(kn, vn, slots, kc, vc, ks, vs, kv)
            for t, s in enumerate(slots):
                if s < 0:
                    continue
                b, p = divmod(int(s), 16)
                for new, cache, sc in ((kn, k2, ks2), (vn, v2, vs2)):
                    if kv == "bf16":
                        if not np.array_equal(cache[b, p], new[t]):
                            return False
                    else:
                        c, sref = _torch_row_quant(bf16_bits_to_f64(new[t]).astype(np.float32))
                        if not (np.array_equal(cache[b, p], c) and np.array_equal(sc[b, p], sref)):
                            return False
        # block size 64: slot s is position s % 64 of block s // 64
        kc = np.zeros((3, 64, H, D), np.uint16)
        slots64 = np.array([0, 63, 64, 130, 191])
        k2, _, _, _ = cw.reshape_and_cache(kn, vn, slots64, kc, kc.copy(), None, None, "bf16")
        for t, s in enumerate(slots64):
            b, p = divmod(int(s), 64)
            if not np.array_equal(k2[b, p], kn[t]):
                return False
        if np.count_nonzero(np.any(k2 != 0, axis=(2, 3))) != len(slots64):
            return False
        return True
    except Exception:
        return False


def test_clean_copy_passes_the_cache_write_battery(tmp_path):
    cw, orc = _load_cw(tmp_path, None)
    assert _cw_battery(cw, orc)


@pytest.mark.parametrize("mutant", sorted(CW_MUTANTS))
def test_every_planted_cache_write_mistake_is_caught(tmp_path, mutant):
    cw, orc = _load_cw(tmp_path, mutant)
    assert not _cw_battery(cw, orc), f"mutant {mutant} passed every pin"

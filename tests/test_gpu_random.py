"""Seeded random shapes through both attention calls, each against the CPU
oracle at the usual tolerance (|gpu - ref| <= 1e-2 + 1e-2 |ref| on every
produced element, relative L2 <= 1e-2): batch, q/kv heads, head_dim, KV
dtype, block size, query lengths (ragged), context and chunk lengths, a
sliding window and sinks are all drawn, so combinations no hand-written
case names still meet the oracle; a second decode set draws batches of
60-200 sequences and forced grids, a third head_dim 256 with 17-64 query
rows per kv head (several waves per kv head)."""
import numpy as np
import pytest

from _parity import check
from paged_attention_decode_attn_amd.workloads import CONFIGS, PREFILL_CONFIGS, generate, generate_prefill
from test_gpu_prefill import _check as check_prefill

pytestmark = pytest.mark.gpu

DECODE_CASES = 24
WIDE_DECODE_CASES = 24
D256_ROWS_CASES = 12
PREFILL_CASES = 24


def decode_spec(i):
    rng = np.random.default_rng(5000 + i)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    qlen = int(rng.integers(1, 5))
    max_rows = 16 if d == 256 else 64
    gs = [g for g in (1, 2, 4, 8, 16) if g * qlen <= max_rows]
    g = int(rng.choice(gs))
    bs = int(rng.choice([16, 16, 32, 64, 256]))
    batch = int(rng.integers(1, 7))
    ctx_hi = int(rng.integers(qlen, 1500))
    ctx_lo = int(rng.integers(qlen, ctx_hi + 1))
    window = int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    return CONFIGS["mtp_verify"].replace(
        name=f"random_decode_{i}", batch=batch, qlen=qlen, qlen_lo=int(rng.integers(1, qlen + 1)),
        hq=hkv * g, hkv=hkv, head_dim=d, kv_dtype=str(rng.choice(["bf16", "fp8_e4m3fn"])),
        ctx_lo=ctx_lo, ctx_hi=ctx_hi, block_size=bs, pool_blocks=batch * (-(-ctx_hi // bs)) + 4,
        seed=6000 + i, sliding_window=window, sinks=bool(rng.integers(0, 2)))


def wide_decode_spec(i):
    # batches on both sides of 64 sequences (the partition kernel scans the
    # chunk counts in the wave's lanes up to 64, in LDS beyond) and forced grids
    rng = np.random.default_rng(9000 + i)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    qlen = int(rng.integers(1, 5))
    max_rows = 16 if d == 256 else 64
    g = int(rng.choice([x for x in (1, 2, 4, 8, 16) if x * qlen <= max_rows]))
    bs = int(rng.choice([16, 16, 32, 64, 256]))
    batch = int(rng.choice([int(rng.integers(60, 70)), int(rng.integers(100, 200))]))
    ctx_hi = int(rng.integers(qlen, 400))
    ctx_lo = int(rng.integers(qlen, ctx_hi + 1))
    window = int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    spec = CONFIGS["mtp_verify"].replace(
        name=f"random_wide_decode_{i}", batch=batch, qlen=qlen, qlen_lo=int(rng.integers(1, qlen + 1)),
        hq=hkv * g, hkv=hkv, head_dim=d, kv_dtype=str(rng.choice(["bf16", "fp8_e4m3fn"])),
        ctx_lo=ctx_lo, ctx_hi=ctx_hi, block_size=bs, pool_blocks=batch * (-(-ctx_hi // bs)) + 4,
        seed=10000 + i, sliding_window=window, sinks=bool(rng.integers(0, 2)))
    grid = int(rng.choice([0, 0, int(rng.integers(1, 64)), int(rng.integers(64, 3000))]))
    return spec, grid


def d256_rows_spec(i):
    rng = np.random.default_rng(11000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    qlen = int(rng.integers(1, 5))
    g = int(rng.choice([x for x in range(1, 33) if 16 < x * qlen <= 64]))
    bs = int(rng.choice([16, 16, 32, 64, 256]))
    batch = int(rng.choice([int(rng.integers(1, 7)), int(rng.integers(60, 80))]))
    ctx_hi = int(rng.integers(qlen, 1500 if batch < 10 else 300))
    ctx_lo = int(rng.integers(qlen, ctx_hi + 1))
    window = int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    spec = CONFIGS["mtp_verify"].replace(
        name=f"random_d256_rows_{i}", batch=batch, qlen=qlen, qlen_lo=int(rng.integers(1, qlen + 1)),
        hq=hkv * g, hkv=hkv, head_dim=256, kv_dtype=str(rng.choice(["bf16", "fp8_e4m3fn"])),
        ctx_lo=ctx_lo, ctx_hi=ctx_hi, block_size=bs, pool_blocks=batch * (-(-ctx_hi // bs)) + 4,
        seed=12000 + i, sliding_window=window, sinks=bool(rng.integers(0, 2)))
    grid = int(rng.choice([0, 0, int(rng.integers(1, 64)), int(rng.integers(64, 3000))]))
    return spec, grid


def prefill_spec(i):
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16, 64]))
    if i % 6 == 5:                                  # head_dim 256 takes ratios up to 16
        d, g = 256, int(rng.choice([1, 2, 4, 16]))
    bs = int(rng.choice([16, 16, 32, 64, 256]))
    batch = int(rng.integers(1, 9))
    ctx_hi = int(rng.integers(1, 600))
    ctx_lo = int(rng.integers(1, ctx_hi + 1))
    whole = bool(rng.integers(0, 3) == 0)
    chunk_hi = 0 if whole else int(rng.integers(1, ctx_hi + 1))
    window = int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    return PREFILL_CONFIGS["chunked_prefill"].replace(
        name=f"random_prefill_{i}", batch=batch, hq=hkv * g, hkv=hkv, head_dim=d,
        kv_dtype=str(rng.choice(["bf16", "fp8_e4m3fn"])), ctx_lo=ctx_lo, ctx_hi=ctx_hi,
        chunk_lo=0 if whole else int(rng.integers(0, chunk_hi + 1)), chunk_hi=chunk_hi, block_size=bs,
        pool_blocks=batch * (-(-ctx_hi // bs)) + 4, seed=8000 + i, sliding_window=window,
        sinks=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("i", range(DECODE_CASES))
def test_random_decode(i):
    spec = decode_spec(i)
    check(generate(spec), label=f"{spec.name}: {spec.hq}/{spec.hkv} d{spec.head_dim} {spec.kv_dtype} "
                                f"qlen {spec.qlen_lo}..{spec.qlen}")


@pytest.mark.parametrize("i", range(WIDE_DECODE_CASES))
def test_random_wide_decode(i):
    spec, grid = wide_decode_spec(i)
    check(generate(spec), grid, label=f"{spec.name}: B{spec.batch} {spec.hq}/{spec.hkv} d{spec.head_dim} "
                                      f"{spec.kv_dtype} qlen {spec.qlen_lo}..{spec.qlen} grid {grid or 'auto'}")


@pytest.mark.parametrize("i", range(D256_ROWS_CASES))
def test_random_d256_many_rows(i):
    spec, grid = d256_rows_spec(i)
    check(generate(spec), grid, label=f"{spec.name}: B{spec.batch} {spec.hq}/{spec.hkv} {spec.kv_dtype} "
                                      f"qlen {spec.qlen_lo}..{spec.qlen} bs{spec.block_size} "
                                      f"window {spec.sliding_window} grid {grid or 'auto'}")


@pytest.mark.parametrize("i", range(PREFILL_CASES))
def test_random_prefill(i):
    spec = prefill_spec(i)
    check_prefill(generate_prefill(spec), f"{spec.name}: {spec.hq}/{spec.hkv} d{spec.head_dim} {spec.kv_dtype}")

"""GPU parity of the paged KV-cache write (paged_attn_reshape_and_cache)
against the CPU oracle: every byte of the caches and every scale of the
pool must be identical (bf16 copies and e4m3fn codes are exact decisions,
taken in float32 on both sides), and the write followed by the decode call
must match the oracle's attention over the oracle-written cache."""
import numpy as np
import pytest
import torch

from _parity import compare, note
from oracle import e4m3fn_table, paged_decode_attention
from oracle.cache_write import reshape_and_cache
from paged_attention_decode_attn_amd import binding as B
from paged_attention_decode_attn_amd.workloads import CONFIGS, generate_cache_write

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _oracle_write(cw):
    w = cw.base
    fp8 = w.spec.kv_dtype == "fp8_e4m3fn"
    return reshape_and_cache(_bits(cw.k_new), _bits(cw.v_new), cw.slot_mapping.numpy(),
                             _bits(w.k_cache), _bits(w.v_cache),
                             w.k_scale.numpy() if fp8 else None, w.v_scale.numpy() if fp8 else None,
                             w.spec.kv_dtype)


def _gpu_write(cw, k_new=None, v_new=None):
    d = cw.to("cuda")
    w = d.base
    B.paged_attn_reshape_and_cache(d.k_new if k_new is None else k_new, d.v_new if v_new is None else v_new,
                                   d.slot_mapping, w.k_cache, w.v_cache, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    return d


def _check_pool(cw, d, label):
    kc, vc, ks, vs = _oracle_write(cw)
    w = d.base
    assert np.array_equal(_bits(w.k_cache), kc), f"{label}: k_cache differs"
    assert np.array_equal(_bits(w.v_cache), vc), f"{label}: v_cache differs"
    if ks is not None:
        assert np.array_equal(w.k_scale.cpu().numpy(), ks), f"{label}: k_scale differs"
        assert np.array_equal(w.v_scale.cpu().numpy(), vs), f"{label}: v_scale differs"


SMALL = {
    "tiny": CONFIGS["tiny"],
    "llama3_8b": CONFIGS["llama3_8b"].replace(ctx_lo=100, ctx_hi=1500, pool_blocks=400),
    "fp8": CONFIGS["fp8"].replace(batch=5, ctx_lo=100, ctx_hi=3000, pool_blocks=1000),
    "mtp_verify": CONFIGS["mtp_verify"].replace(batch=6, ctx_lo=2, ctx_hi=2000, pool_blocks=800),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_decode_step_write_matches_oracle(name, kv):
    cw = generate_cache_write(SMALL[name].replace(kv_dtype=kv), pad=3)
    note(f"[gpu] cache write {name}/{kv}: T={cw.k_new.shape[0]}")
    d = _gpu_write(cw)
    _check_pool(cw, d, f"{name}/{kv}")


@pytest.mark.parametrize("pieces", [0, 2, 4])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("hkv,d", [(1, 64), (2, 128), (8, 64), (8, 128), (3, 128), (2, 256), (8, 256)])
def test_bulk_write_with_padding_and_out_of_pool_slots(kv, hkv, d, pieces):
    # pieces: 16-byte row pieces per thread (0: the library's choice, one
    # for writes this small); a ragged last round leaves threads idle
    spec = CONFIGS["llama3_8b"].replace(batch=2, hq=hkv, hkv=hkv, head_dim=d, kv_dtype=kv, ctx_lo=16,
                                        ctx_hi=64, pool_blocks=90)
    cw = generate_cache_write(spec, bulk_tokens=1000, pad=5)
    s = cw.slot_mapping.clone()
    s[3] = 90 * 16 + 7                                     # past the pool: skipped
    s[4] = -7                                              # any negative: skipped
    cw.slot_mapping = s
    note(f"[gpu] bulk cache write hkv={hkv} d={d} {kv} pieces={pieces}")
    B.paged_attn_set_write_pieces(pieces)
    try:
        d_ = _gpu_write(cw)
    finally:
        B.paged_attn_set_write_pieces(0)
    _check_pool(cw, d_, f"bulk/{hkv}/{d}/{kv}/{pieces}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("bs", [32, 48, 80, 256])
def test_bulk_write_block_sizes(kv, bs):
    # a slot's block and position come from a shift for power-of-two block
    # sizes and from a division otherwise
    nb = -(-1500 // bs) + 2
    spec = CONFIGS["llama3_8b"].replace(batch=2, hq=8, hkv=8, head_dim=64, kv_dtype=kv, block_size=bs, ctx_lo=16,
                                        ctx_hi=2 * bs, pool_blocks=nb)
    cw = generate_cache_write(spec, bulk_tokens=1000, pad=3)
    note(f"[gpu] bulk cache write block_size={bs} {kv}")
    d_ = _gpu_write(cw)
    _check_pool(cw, d_, f"bulk/bs{bs}/{kv}")


def test_fp8_quotients_for_every_pair_of_mantissas():
    # Every bf16 mantissa of the row's absolute maximum (the scale is
    # absmax / 448) against every bf16 mantissa of an element, at element
    # magnitudes that put the quotient anywhere from below the smallest
    # e4m3fn subnormal to 448, both signs: each code must be the rounding of
    # the correctly rounded float32 quotient, as the oracle's division gives
    D = 64
    man = 1.0 + np.arange(128) / 128.0                      # the 128 bf16 mantissas in [1, 2)
    xs = np.concatenate([man * 2.0 ** e for e in range(-20, 1)])
    xs = np.concatenate([xs, -xs])                          # 5376 elements of magnitude below 2
    per_row = D - 1
    rows = []
    for am in man:                                          # absmax in [1, 2): its scale am / 448
        for i in range(0, len(xs), per_row):
            r = np.zeros(D, np.float32)
            r[0] = am
            chunk = xs[i:i + per_row]
            r[1:1 + len(chunk)] = np.clip(chunk, -am, am)
            rows.append(r)
    x = np.stack(rows)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(xb.float(), torch.from_numpy(x))   # all exact bf16 values
    T = xb.shape[0]
    spec = CONFIGS["fp8"].replace(batch=1, hq=1, hkv=1, head_dim=D, ctx_lo=16, ctx_hi=16, pool_blocks=T // 16 + 4)
    cw = generate_cache_write(spec, bulk_tokens=T)
    cw.k_new = xb[:, None, :].contiguous()
    cw.v_new = (-xb * 2.0 ** -100)[:, None, :].contiguous()   # the same pairs at tiny magnitudes
    note(f"[gpu] fp8 mantissa-pair sweep: {T} rows")
    d = _gpu_write(cw)
    _check_pool(cw, d, "mantissa-pairs")


def test_strided_new_rows():
    cw = generate_cache_write(SMALL["mtp_verify"].replace(kv_dtype="fp8_e4m3fn"))
    T, H, D = cw.k_new.shape
    big = torch.zeros(T, 3, H, D, dtype=torch.bfloat16)
    big[:, 1] = cw.k_new
    bigv = torch.zeros(T, H, 2 * D, dtype=torch.bfloat16)
    bigv[:, :, D:] = cw.v_new
    note("[gpu] strided cache write")
    d = _gpu_write(cw, k_new=big.cuda()[:, 1], v_new=bigv.cuda()[:, :, D:])
    _check_pool(cw, d, "strided")


def test_fp8_rounding_of_every_code_midpoint_and_subnormal():
    # rows whose largest magnitude is 448 have scale exactly 1, so the codes
    # are the rounding of the bf16 values themselves
    tab = e4m3fn_table()
    vals = [tab[c] for c in range(0x7F)]
    vals += [(tab[c] + tab[c + 1]) / 2 for c in range(0x7E)]           # ties -> even code
    bf = lambda x: float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16))
    vals += [bf(np.nextafter(np.float32(v), np.float32(0))) for v in vals[:20]]
    vals = np.array([bf(v) for v in vals], dtype=np.float32)
    vals = np.concatenate([vals, -vals])
    D = 64
    rows = int(np.ceil(len(vals) / (D - 1)))
    x = np.zeros((rows, D), np.float32)
    x[:, 0] = 448.0
    x[:, 1:].flat[:len(vals)] = vals
    T = rows
    spec = CONFIGS["fp8"].replace(batch=1, hq=1, hkv=1, head_dim=D, ctx_lo=16, ctx_hi=16, pool_blocks=T + 2)
    cw = generate_cache_write(spec, bulk_tokens=T)
    cw.k_new = torch.from_numpy(x).to(torch.bfloat16)[:, None, :].contiguous()
    cw.v_new = torch.from_numpy(-x).to(torch.bfloat16)[:, None, :].contiguous()
    note(f"[gpu] fp8 rounding sweep: {len(vals)} values")
    d = _gpu_write(cw)
    _check_pool(cw, d, "rounding")
    ks = d.base.k_scale.cpu().numpy()
    written = cw.slot_mapping.numpy()
    assert np.all(ks[written // 16, written % 16, 0] == 1.0)


def test_fp8_quotients_round_as_correctly_rounded_divisions():
    # rows on which the quotient x / scale and the product x * (448 / absmax)
    # round to different codes, and rows mixing the largest and smallest bf16
    # magnitudes (quotients in float32's subnormal range, a subnormal absmax)
    rng = np.random.default_rng(77)
    D = 64
    x = rng.normal(0, 1, (600, D)).astype(np.float32)
    x[:200] *= np.exp2(rng.integers(-60, 61, (200, 1))).astype(np.float32)
    tiny = float(torch.tensor(2.0 ** -133, dtype=torch.bfloat16).float())
    x[590, :8] = [3.0e38, tiny, -tiny, 1e-30, -1e-38, 2.0 ** -126, 1.0, -1.0]
    x[591] = 0.0
    x[591, 5] = -7.0
    x[592] = tiny
    x[592, 3] = -2 * tiny
    x[593] = 0.0
    x[593, :2] = [2.0 ** -120, 2.0 ** -130]
    x[594, 0], x[594, 1:] = 448.0, -2.0 ** -12
    xb = torch.from_numpy(x).to(torch.bfloat16)
    T = xb.shape[0]
    spec = CONFIGS["fp8"].replace(batch=1, hq=1, hkv=1, head_dim=D, ctx_lo=16, ctx_hi=16, pool_blocks=T // 16 + 4)
    cw = generate_cache_write(spec, bulk_tokens=T)
    cw.k_new = xb[:, None, :].contiguous()
    cw.v_new = (-xb)[:, None, :].contiguous()
    note(f"[gpu] fp8 division sweep: {T} rows")
    d = _gpu_write(cw)
    _check_pool(cw, d, "division")


def test_all_zero_rows_get_unit_scale():
    spec = CONFIGS["fp8"].replace(batch=1, ctx_lo=32, ctx_hi=32, pool_blocks=40)
    cw = generate_cache_write(spec, bulk_tokens=17)
    cw.k_new = torch.zeros_like(cw.k_new)
    note("[gpu] zero rows")
    d = _gpu_write(cw)
    _check_pool(cw, d, "zero-rows")


@pytest.mark.parametrize("name", ["fp8", "mtp_verify", "llama3_8b"])
def test_write_then_decode_matches_oracle(name):
    cw = generate_cache_write(SMALL[name])
    d = _gpu_write(cw)
    w = d.base
    note(f"[gpu] write then decode {name}")
    out = B.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.query_lens,
                              w.scale, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    kc, vc, ks, vs = _oracle_write(cw)
    h = cw.base
    ref = paged_decode_attention(_bits(h.q), kc, vc, h.block_tables.numpy(), h.context_lens.numpy(),
                                 h.query_lens.numpy(), h.scale, ks, vs, h.spec.kv_dtype)
    compare(out, ref, h.query_lens, label=f"write+decode/{name}")


def test_write_argument_errors_launch_nothing():
    cw = generate_cache_write(SMALL["fp8"]).to("cuda")
    w = cw.base
    before = w.k_cache.clone()
    note("[gpu] cache write argument errors")
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_reshape_and_cache(cw.k_new, cw.v_new, cw.slot_mapping, w.k_cache, w.v_cache, None, None)
    assert e.value.name == "PA_ERR_NULL"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_reshape_and_cache(cw.k_new.float(), cw.v_new, cw.slot_mapping, w.k_cache, w.v_cache,
                                       w.k_scale, w.v_scale)
    assert e.value.name == "PA_ERR_DTYPE"
    with pytest.raises(B.PagedAttnError) as e:
        B.paged_attn_reshape_and_cache(cw.k_new, cw.v_new, cw.slot_mapping[:-1], w.k_cache, w.v_cache,
                                       w.k_scale, w.v_scale)
    assert e.value.name == "PA_ERR_SHAPE"
    torch.cuda.synchronize()
    assert torch.equal(w.k_cache, before)

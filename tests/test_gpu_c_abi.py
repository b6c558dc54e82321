"""The library called from plain C: pa_decode_cli (built beside the library
from c_example/pa_decode_cli.c; device memory from the HIP runtime API, the
call through include/paged_attn.h) runs paged_attn_decode on a seeded
workload written to raw files, and its output meets the oracle at the usual
tolerance.  The C program computes nothing itself."""
import os
import subprocess

import numpy as np
import pytest
import torch

from _parity import compare, note, oracle_out, small
from paged_attention_decode_attn_amd.build import CLI_PATH
from paged_attention_decode_attn_amd.workloads import generate

pytestmark = pytest.mark.gpu


def _write(w, d):
    s = w.spec
    B, Qmax, Hq, D = w.q.shape
    NB, BS, Hkv, _ = w.k_cache.shape
    fp8 = w.k_scale is not None
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"{B} {Qmax} {Hq} {Hkv} {D} {NB} {BS} {w.block_tables.shape[1]} {int(fp8)} {w.scale!r}\n")

    def raw(name, t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        t.numpy().tofile(os.path.join(d, name))
    raw("q.bin", w.q)
    raw("k_cache.bin", w.k_cache)
    raw("v_cache.bin", w.v_cache)
    raw("block_tables.bin", w.block_tables.to(torch.int32))
    raw("context_lens.bin", w.context_lens.to(torch.int32))
    raw("query_lens.bin", w.query_lens.to(torch.int32))
    if fp8:
        # physical [NB, Hkv, BS], the layout the program describes
        raw("k_scale.bin", w.k_scale.permute(0, 2, 1))
        raw("v_scale.bin", w.v_scale.permute(0, 2, 1))
    return (B, Qmax, Hq, D), s


@pytest.mark.parametrize("name", ["mtp_verify", "fp8"])
def test_decode_called_from_c(tmp_path, name):
    assert os.path.exists(CLI_PATH), f"{CLI_PATH} is missing: build the package first"
    w = generate(small(name, batch=3, ctx_lo=5, ctx_hi=300, pool_blocks=64))
    shape, _ = _write(w, str(tmp_path))
    note(f"[gpu] C caller: {name} {shape}")
    res = subprocess.run([CLI_PATH, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"pa_decode_cli exited {res.returncode}: {res.stderr}"
    bits = np.fromfile(os.path.join(tmp_path, "out.bin"), dtype=np.int16).reshape(shape)
    out = torch.from_numpy(bits).view(torch.bfloat16)
    compare(out, oracle_out(w), w.query_lens, label=f"C caller {name}")


def test_c_caller_reports_a_library_error(tmp_path):
    """A mismatched meta file (a head count the data does not have) comes
    back as the library's status, not a crash."""
    w = generate(small("mtp_verify", batch=2, ctx_lo=5, ctx_hi=100, pool_blocks=32))
    _write(w, str(tmp_path))
    meta = open(os.path.join(tmp_path, "meta.txt")).read().split()
    meta[2] = str(int(meta[3]) * 3 + 1)               # q heads not a multiple of kv heads
    # the q file must still be long enough for the (smaller or larger) shape
    need = int(meta[0]) * int(meta[1]) * int(meta[2]) * int(meta[4]) * 2
    np.zeros(need // 2, np.int16).tofile(os.path.join(tmp_path, "q.bin"))
    open(os.path.join(tmp_path, "meta.txt"), "w").write(" ".join(meta) + "\n")
    res = subprocess.run([CLI_PATH, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 50 + 4, (res.returncode, res.stderr)     # PA_ERR_UNSUPPORTED = -4
    assert "paged_attn_decode" in res.stderr

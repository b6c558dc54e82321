"""Seeded synthetic decode workloads (inputs only; no attention arithmetic).

This module is the one piece shared by the HIP path's callers (tests,
benchmark) and by the CPU oracle's callers: it draws every input from a
seeded ``torch.Generator`` on the host, so the GPU and the oracle read
identical bytes.  It holds none of the attention computation.

The shapes follow the decode regime the pages describe: one or a few new
query tokens per sequence, GQA head grouping, ragged context lengths, a
block-size-16 paged cache in bf16 or fp8 (ATOM configuration guide,
"Master configuration (Config)": ``kv_cache_block_size``,
``kv_cache_dtype``), and short causal query runs for MTP verification (ROCm
blog "Optimizing ATOM and vLLM-ATOM for High-Interactivity Inference",
"Multi-Token Prediction").  The pages measure on no public dataset for this
path; every value is N(0, 1) noise.

Generation order for a spec with seed ``s`` (``torch.Generator('cpu')``):

1. context lengths (constant, or uniform integers in ``[lo, hi]``), then,
   for specs with ``qlen_lo``, query lengths uniform in ``[qlen_lo, qlen]``;
2. one random permutation of the physical pool;
3. Q, float32 N(0, 1) rounded to bf16;
4. K for every used block, in table order (float32 N(0, 1)), then V the
   same way; bf16 caches round to bf16, fp8 caches quantise each
   (token, kv head) row of D values with scale ``absmax / 448`` (1 if the
   row is all zero) and ``torch``'s round-to-nearest-even cast to
   ``float8_e4m3fn``;
5. block tables: sequence ``b`` takes the next ``ceil(L_b / BS)`` entries of
   the permutation; unused table columns hold block 0 (or, with
   ``poison=True``, an unused block filled with NaN);
6. for specs with ``sinks``, one sink logit per query head, uniform in
   ``[-2, 8]`` (from about no effect to dominating a 128-token window's
   log-sum-exp).

Unused pool blocks hold zeros (NaN with ``poison=True``; the tail slots past
``L_b`` of each sequence's last block are NaN then as well).  Scales are
stored physically ``[NB, Hkv, BS]`` so that one (block, kv head) reads its
slots' scales contiguously, and handed out as the logical ``[NB, BS, Hkv]``
view.  ``BS`` is the spec's block size (16 unless stated).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import torch

BLOCK = 16
FP8_MAX = 448.0

__all__ = ["WorkloadSpec", "Workload", "CONFIGS", "CONFIG_ORDER", "NEXT_CONFIG_ORDER", "generate", "kv_bytes",
           "CacheWrite", "generate_cache_write", "write_bytes", "PrefillSpec", "Prefill", "PREFILL_CONFIGS",
           "generate_prefill", "prefill_flops"]


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    batch: int
    qlen: int
    hq: int
    hkv: int
    head_dim: int
    kv_dtype: str            # "bf16" or "fp8_e4m3fn"
    ctx_lo: int
    ctx_hi: int
    pool_blocks: int
    seed: int
    scale: Optional[float] = None   # None: 1 / sqrt(head_dim)
    qlen_lo: Optional[int] = None   # ragged query lengths, uniform in [qlen_lo, qlen]
    block_size: int = BLOCK         # tokens per cache block
    sliding_window: int = 0         # 0: none
    sinks: bool = False             # per-query-head sink logits

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    @property
    def table_width(self) -> int:
        return (self.ctx_hi + self.block_size - 1) // self.block_size

    def replace(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


# The five decode workloads (sizes and seeds fixed; seed k for the k-th).
CONFIGS = {
    "tiny": WorkloadSpec("tiny_b1_q32kv8_d128_ctx512_bf16", batch=1, qlen=1, hq=32, hkv=8,
                         head_dim=128, kv_dtype="bf16", ctx_lo=512, ctx_hi=512,
                         pool_blocks=64, seed=1, scale=1.0 / math.sqrt(128)),
    "llama3_8b": WorkloadSpec("llama3_8b_b4_q32kv8_d128_ctx1k-8k_bf16", batch=4, qlen=1,
                              hq=32, hkv=8, head_dim=128, kv_dtype="bf16", ctx_lo=1024,
                              ctx_hi=8192, pool_blocks=4096, seed=2),
    "long_ctx": WorkloadSpec("long_ctx_b1_q64kv8_d128_ctx131072_bf16", batch=1, qlen=1,
                             hq=64, hkv=8, head_dim=128, kv_dtype="bf16", ctx_lo=131072,
                             ctx_hi=131072, pool_blocks=16384, seed=3),
    "fp8": WorkloadSpec("fp8_b16_q64kv8_d64_ctx512-32k_e4m3fn", batch=16, qlen=1, hq=64,
                        hkv=8, head_dim=64, kv_dtype="fp8_e4m3fn", ctx_lo=512, ctx_hi=32768,
                        pool_blocks=32768, seed=4),
    "mtp_verify": WorkloadSpec("mtp_verify_b64_qlen2_q64kv8_d128_ctx256-16k_bf16", batch=64,
                               qlen=2, hq=64, hkv=8, head_dim=128, kv_dtype="bf16",
                               ctx_lo=256, ctx_hi=16384, pool_blocks=65536, seed=5),
}
CONFIG_ORDER = ["tiny", "llama3_8b", "long_ctx", "fp8", "mtp_verify"]

# Wider speculative verification (query length 4, and ragged query lengths
# 1..4 per sequence): the ROCm blog "Optimizing ATOM and vLLM-ATOM for
# High-Interactivity Inference" ("Multi-Token Prediction") verifies draft
# tokens in one decode step, and the model operations guide's paged-kernel
# envelope table bounds query length x q/kv head ratio; here 4 x 8 = 32 rows.
CONFIGS.update({
    "mtp_verify_q4": WorkloadSpec("mtp_verify_b64_qlen4_q64kv8_d128_ctx256-16k_bf16", batch=64, qlen=4,
                                  hq=64, hkv=8, head_dim=128, kv_dtype="bf16", ctx_lo=256, ctx_hi=16384,
                                  pool_blocks=65536, seed=6),
    "mtp_verify_ragged": WorkloadSpec("mtp_verify_b64_qlen1-4_q64kv8_d128_ctx256-16k_bf16", batch=64,
                                      qlen=4, hq=64, hkv=8, head_dim=128, kv_dtype="bf16", ctx_lo=256,
                                      ctx_hi=16384, pool_blocks=65536, seed=7, qlen_lo=1),
})
# Shape variants that the pages' decode dispatch and model table name: a
# larger cache block (the persistent decode kernel's block size 256), a
# multi-head (q_heads == kv_heads) model, and GPT-OSS-style sliding-window
# layers with attention sinks (the landing page's model table; 64 query /
# 8 kv heads of dimension 64 and a 128-token window are GPT-OSS's published
# attention shape) next to its full-attention layers with sinks.
CONFIGS.update({
    "long_ctx_bs256": WorkloadSpec("long_ctx_b1_q64kv8_d128_ctx131072_bf16_block256", batch=1, qlen=1,
                                   hq=64, hkv=8, head_dim=128, kv_dtype="bf16", ctx_lo=131072,
                                   ctx_hi=131072, pool_blocks=1024, seed=8, block_size=256),
    "mha": WorkloadSpec("mha_b8_q32kv32_d128_ctx1k-8k_bf16", batch=8, qlen=1, hq=32, hkv=32,
                        head_dim=128, kv_dtype="bf16", ctx_lo=1024, ctx_hi=8192, pool_blocks=4096,
                        seed=9),
    "swa_sinks": WorkloadSpec("swa128_sinks_b64_q64kv8_d64_ctx1k-16k_bf16", batch=64, qlen=1, hq=64,
                              hkv=8, head_dim=64, kv_dtype="bf16", ctx_lo=1024, ctx_hi=16384,
                              pool_blocks=70000, seed=10, sliding_window=128, sinks=True),
    "full_sinks": WorkloadSpec("sinks_b16_q64kv8_d64_ctx1k-32k_bf16", batch=16, qlen=1, hq=64, hkv=8,
                               head_dim=64, kv_dtype="bf16", ctx_lo=1024, ctx_hi=32768,
                               pool_blocks=34000, seed=11, sinks=True),
})
# head_dim 256 (the model operations guide routes head_dim != 128 to another
# decode kernel): a Gemma-2-9B-shaped layer, 16 query / 8 kv heads.
CONFIGS["d256"] = WorkloadSpec("d256_b8_q16kv8_ctx1k-8k_bf16", batch=8, qlen=1, hq=16, hkv=8, head_dim=256,
                               kv_dtype="bf16", ctx_lo=1024, ctx_hi=8192, pool_blocks=4096, seed=12)
# head_dim 256 with more than 16 query rows per kv head: a verify step of
# four tokens over a Qwen3-Next-shaped full-attention layer (the landing
# page's model table lists Qwen3-Next and its MTP module; 16 query / 2 kv
# heads of dimension 256 is its published attention shape), 8 x 4 = 32 rows.
CONFIGS["d256_mtp"] = WorkloadSpec("d256_mtp_b16_qlen4_q16kv2_ctx1k-16k_bf16", batch=16, qlen=4, hq=16, hkv=2,
                                   head_dim=256, kv_dtype="bf16", ctx_lo=1024, ctx_hi=16384,
                                   pool_blocks=16400, seed=13)
NEXT_CONFIG_ORDER = ["mtp_verify_q4", "mtp_verify_ragged", "long_ctx_bs256", "mha", "swa_sinks",
                     "full_sinks", "d256", "d256_mtp"]


@dataclass
class Workload:
    spec: WorkloadSpec
    q: torch.Tensor              # bf16 [B, Qmax, Hq, D]
    k_cache: torch.Tensor        # bf16 or uint8 (e4m3fn bytes) [NB, 16, Hkv, D]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]   # fp32 logical [NB, 16, Hkv] (physical [NB, Hkv, 16]) or None
    v_scale: Optional[torch.Tensor]
    block_tables: torch.Tensor   # int32 [B, W]
    context_lens: torch.Tensor   # int32 [B]
    query_lens: torch.Tensor     # int32 [B]
    scale: float
    sinks: Optional[torch.Tensor] = None   # fp32 [Hq] or None

    @property
    def sliding_window(self) -> int:
        return self.spec.sliding_window

    def to(self, device) -> "Workload":
        def mv(t):
            return None if t is None else _move(t, device)
        return Workload(self.spec, mv(self.q), mv(self.k_cache), mv(self.v_cache),
                        mv(self.k_scale), mv(self.v_scale), mv(self.block_tables),
                        mv(self.context_lens), mv(self.query_lens), self.scale, mv(self.sinks))

    def numpy_inputs(self) -> dict:
        """The same bytes as NumPy arrays (bf16 as uint16 bit patterns,
        e4m3fn as uint8), keyed like the attention call's arguments."""
        def bits(t):
            t = t.detach().cpu()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view("uint16")
            return t.numpy()
        d = dict(q_bits=bits(self.q), k_cache=bits(self.k_cache), v_cache=bits(self.v_cache),
                 block_tables=self.block_tables.cpu().numpy(),
                 context_lens=self.context_lens.cpu().numpy(),
                 query_lens=self.query_lens.cpu().numpy(), scale=self.scale,
                 kv_dtype=self.spec.kv_dtype, k_scale=None, v_scale=None,
                 sliding_window=self.spec.sliding_window or None,
                 sinks=None if self.sinks is None else self.sinks.cpu().numpy())
        if self.k_scale is not None:
            d["k_scale"] = self.k_scale.cpu().numpy()
            d["v_scale"] = self.v_scale.cpu().numpy()
        return d


def _move(t: torch.Tensor, device) -> torch.Tensor:
    """Copy to ``device`` keeping the storage layout (scale views stay views
    of a contiguous physical tensor)."""
    if t.is_contiguous():
        return t.to(device)
    # the scale tensors: logical [NB, BS, Hkv] view of physical [NB, Hkv, BS]
    phys = t.permute(0, 2, 1)
    assert phys.is_contiguous()
    return phys.to(device).permute(0, 2, 1)


def kv_bytes(context_lens, hkv: int, head_dim: int, kv_dtype: str, query_lens=None,
             sliding_window: int = 0) -> int:
    """Algorithmic KV bytes of one call: K and V rows of every attended
    token, plus the fp32 per-token scales of an fp8 cache.  With a sliding
    window a sequence's rows attend to at most window + query_len - 1
    tokens."""
    ctx = torch.as_tensor(context_lens).to(torch.int64)
    if sliding_window > 0:
        ql = torch.ones_like(ctx) if query_lens is None else torch.as_tensor(query_lens).to(torch.int64)
        ctx = torch.where(ql > 0, torch.minimum(ctx, sliding_window + ql - 1), torch.zeros_like(ctx))
    tokens = int(ctx.sum())
    elem = 1 if kv_dtype == "fp8_e4m3fn" else 2
    per_token = 2 * hkv * head_dim * elem
    if kv_dtype == "fp8_e4m3fn":
        per_token += 2 * hkv * 4
    return tokens * per_token


def _nan_pattern(kv_dtype: str):
    return (0x7F, torch.uint8) if kv_dtype == "fp8_e4m3fn" else (0x7FC0, torch.int16)


def _fill_cache(cache, scales, block_ids, gen, spec, chunk_blocks):
    """Draw N(0, 1) rows for ``block_ids`` (in order) and store them."""
    H, D, BS = spec.hkv, spec.head_dim, spec.block_size
    for start in range(0, block_ids.numel(), chunk_blocks):
        ids = block_ids[start:start + chunk_blocks]
        x = torch.randn(ids.numel(), BS, H, D, generator=gen, dtype=torch.float32)
        if spec.kv_dtype == "bf16":
            cache[ids] = x.to(torch.bfloat16)
        else:
            amax = x.abs().amax(dim=-1)                              # [n, BS, H]
            s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            y = (x / s[..., None]).clamp(-FP8_MAX, FP8_MAX)
            cache[ids] = y.to(torch.float8_e4m3fn).view(torch.uint8)
            scales[ids] = s.permute(0, 2, 1).contiguous()            # physical [n, H, BS]


def generate(spec: WorkloadSpec, *, seed: Optional[int] = None, poison: bool = False,
             context_lens=None, query_lens=None) -> Workload:
    """Draw one workload on the host.  ``context_lens`` overrides step 1 and
    ``query_lens`` the per-sequence query-row counts (edge-case tests; no
    random draw is spent on either); ``poison`` fills everything the call
    must not read with NaN."""
    gen = torch.Generator("cpu").manual_seed(spec.seed if seed is None else seed)
    B, Qn, Hq, H, D = spec.batch, spec.qlen, spec.hq, spec.hkv, spec.head_dim
    if Hq % H:
        raise ValueError("q heads must be a multiple of kv heads")
    NB, W, BS = spec.pool_blocks, spec.table_width, spec.block_size
    if BS < 1:
        raise ValueError("block size must be positive")

    # 1. context lengths
    if context_lens is not None:
        ctx = torch.as_tensor(context_lens, dtype=torch.int64).clone()
        if ctx.numel() != B:
            raise ValueError("context_lens must have one entry per sequence")
    elif spec.ctx_lo == spec.ctx_hi:
        ctx = torch.full((B,), spec.ctx_lo, dtype=torch.int64)
    else:
        ctx = torch.randint(spec.ctx_lo, spec.ctx_hi + 1, (B,), generator=gen, dtype=torch.int64)
    if ctx.numel() and int(ctx.max()) > BS * W:
        raise ValueError("a context is longer than the block table")
    if ctx.numel() and int(ctx.min()) < 0:
        raise ValueError("negative context length")
    if query_lens is None and spec.qlen_lo is not None:
        qls = torch.randint(spec.qlen_lo, Qn + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    elif query_lens is None:
        qls = torch.full((B,), Qn, dtype=torch.int32)
    else:
        qls = torch.as_tensor(query_lens, dtype=torch.int32).clone()
        if qls.numel() != B or (qls.numel() and (int(qls.min()) < 0 or int(qls.max()) > Qn)):
            raise ValueError("query_lens must be in [0, qlen], one per sequence")
    if bool((qls.to(torch.int64) > ctx).any()):
        raise ValueError("a sequence has more query rows than context tokens")
    nblk = (ctx + BS - 1) // BS
    used = int(nblk.sum())
    if used + (1 if poison else 0) > NB:
        raise ValueError(f"pool of {NB} blocks cannot hold {used} used blocks")

    # 2. pool placement
    perm = torch.randperm(NB, generator=gen)

    # 3. queries
    q = torch.randn(B, Qn, Hq, D, generator=gen, dtype=torch.float32).to(torch.bfloat16)

    # 4. caches
    fp8 = spec.kv_dtype == "fp8_e4m3fn"
    if spec.kv_dtype not in ("bf16", "fp8_e4m3fn"):
        raise ValueError(spec.kv_dtype)
    cdtype = torch.uint8 if fp8 else torch.bfloat16
    k_cache = torch.zeros(NB, BS, H, D, dtype=cdtype)
    v_cache = torch.zeros(NB, BS, H, D, dtype=cdtype)
    k_sc = torch.ones(NB, H, BS, dtype=torch.float32) if fp8 else None
    v_sc = torch.ones(NB, H, BS, dtype=torch.float32) if fp8 else None
    used_ids = perm[:used]
    if poison:
        pat, vdt = _nan_pattern(spec.kv_dtype)
        for c in (k_cache, v_cache):
            c.view(vdt).fill_(pat)
        for s in (k_sc, v_sc):
            if s is not None:
                s.fill_(float("nan"))
    chunk = max(1, (64 << 20) // (BS * H * D * 4))
    _fill_cache(k_cache, k_sc, used_ids, gen, spec, chunk)
    _fill_cache(v_cache, v_sc, used_ids, gen, spec, chunk)

    # 5. block tables
    pad_id = int(perm[used]) if poison else 0
    tables = torch.full((B, W), pad_id, dtype=torch.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        tables[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
        if poison and n:
            tail = int(ctx[b]) - (n - 1) * BS             # valid slots in the last block
            if tail < BS:
                last = int(tables[b, n - 1])
                pat, vdt = _nan_pattern(spec.kv_dtype)
                k_cache[last, tail:].view(vdt).fill_(pat)
                v_cache[last, tail:].view(vdt).fill_(pat)
                if fp8:
                    k_sc[last, :, tail:] = float("nan")
                    v_sc[last, :, tail:] = float("nan")

    # 6. sinks
    sinks = None
    if spec.sinks:
        sinks = torch.rand(Hq, generator=gen, dtype=torch.float32) * 10.0 - 2.0

    return Workload(
        spec=spec, q=q, k_cache=k_cache, v_cache=v_cache,
        k_scale=None if k_sc is None else k_sc.permute(0, 2, 1),
        v_scale=None if v_sc is None else v_sc.permute(0, 2, 1),
        block_tables=tables, context_lens=ctx.to(torch.int32),
        query_lens=qls, scale=spec.softmax_scale, sinks=sinks)


@dataclass
class CacheWrite:
    """Inputs of one paged KV-cache write: the new tokens' K/V rows and
    their slots, plus the workload whose pool (caches, scales) they go to."""
    base: Workload
    k_new: torch.Tensor          # bf16 [T, Hkv, D]
    v_new: torch.Tensor
    slot_mapping: torch.Tensor   # int32 [T]; -1 marks a padding token

    def to(self, device) -> "CacheWrite":
        return CacheWrite(self.base.to(device), self.k_new.to(device), self.v_new.to(device),
                          self.slot_mapping.to(device))


def generate_cache_write(spec: WorkloadSpec, *, bulk_tokens: Optional[int] = None, pad: int = 0,
                         seed: Optional[int] = None, **kw) -> CacheWrite:
    """A cache write shaped like the workload's decode step: the new tokens
    are the last ``query_lens[b]`` positions of every sequence (their slots
    through the block table), rows N(0, 1) rounded to bf16 from a generator
    seeded with ``seed`` (default: the workload's seed + 1000).  With
    ``bulk_tokens``, ``T`` tokens take distinct slots drawn from the whole
    pool instead (a prefill-sized write).  ``pad`` extra tokens carry slot
    -1 (padding, not written).  ``kw`` goes to ``generate``."""
    base = generate(spec, **kw)
    gen = torch.Generator("cpu").manual_seed((spec.seed + 1000) if seed is None else seed)
    if bulk_tokens is None:
        slots = []
        for b in range(spec.batch):
            L, n = int(base.context_lens[b]), int(base.query_lens[b])
            bs = spec.block_size
            for pos in range(L - n, L):
                slots.append(int(base.block_tables[b, pos // bs]) * bs + pos % bs)
        slots = torch.tensor(slots, dtype=torch.int64)
    else:
        total = spec.pool_blocks * spec.block_size
        if bulk_tokens > total:
            raise ValueError("more tokens than pool slots")
        slots = torch.randperm(total, generator=gen)[:bulk_tokens]
    if pad:
        at = torch.randint(0, slots.numel() + 1, (pad,), generator=gen)
        for p in sorted(at.tolist(), reverse=True):
            slots = torch.cat([slots[:p], torch.tensor([-1]), slots[p:]])
    T = slots.numel()
    k_new = torch.randn(T, spec.hkv, spec.head_dim, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    v_new = torch.randn(T, spec.hkv, spec.head_dim, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return CacheWrite(base, k_new, v_new, slots.to(torch.int32))


def write_bytes(slot_mapping, hkv: int, head_dim: int, kv_dtype: str, num_blocks: int,
                block_size: int = BLOCK) -> int:
    """Algorithmic bytes of one cache write: the bf16 K and V rows read, the
    cache rows written (and the fp32 scales for an fp8 cache), for the
    tokens whose slot lies in the pool."""
    s = torch.as_tensor(slot_mapping).to(torch.int64)
    n = int(((s >= 0) & (s < num_blocks * block_size)).sum())
    per_token = 2 * hkv * head_dim * 2
    if kv_dtype == "fp8_e4m3fn":
        per_token += 2 * hkv * head_dim + 2 * hkv * 4
    else:
        per_token += 2 * hkv * head_dim * 2
    return n * per_token


# ----------------------------------------------------------------------------
# prefill (chunked prefill) inputs
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillSpec:
    """Packed prefill chunks over a paged cache.  Sequence b's chunk holds
    the last n_b of its L_b tokens: L_b uniform in [ctx_lo, ctx_hi]; n_b =
    L_b for whole prompts (chunk_lo = chunk_hi = 0), else uniform in
    [chunk_lo, chunk_hi] clamped to L_b."""
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    ctx_lo: int
    ctx_hi: int
    chunk_lo: int
    chunk_hi: int
    pool_blocks: int
    seed: int
    block_size: int = BLOCK
    sliding_window: int = 0         # 0: none
    sinks: bool = False             # per-query-head sink logits (drawn as for decode)
    kv_dtype: str = "bf16"          # or "fp8_e4m3fn" (per-token scales, drawn as for decode)

    def cache_spec(self) -> WorkloadSpec:
        return WorkloadSpec(self.name, batch=self.batch, qlen=1, hq=self.hq, hkv=self.hkv,
                            head_dim=self.head_dim, kv_dtype=self.kv_dtype, ctx_lo=self.ctx_lo, ctx_hi=self.ctx_hi,
                            pool_blocks=self.pool_blocks, seed=self.seed, block_size=self.block_size,
                            sliding_window=self.sliding_window, sinks=self.sinks)

    def replace(self, **kw) -> "PrefillSpec":
        return dataclasses.replace(self, **kw)


@dataclass
class Prefill:
    spec: PrefillSpec
    cache: Workload              # its caches, tables and context lengths (its q is unused)
    q: torch.Tensor              # bf16 [T, Hq, D], packed
    cu_seqlens: torch.Tensor     # int32 [B + 1]
    max_query_len: int
    scale: float

    def to(self, device) -> "Prefill":
        return Prefill(self.spec, self.cache.to(device), self.q.to(device), self.cu_seqlens.to(device),
                       self.max_query_len, self.scale)

    @property
    def chunk_lens(self) -> torch.Tensor:
        return (self.cu_seqlens[1:] - self.cu_seqlens[:-1]).cpu()

    @property
    def sinks(self) -> Optional[torch.Tensor]:
        return self.cache.sinks

    @property
    def sliding_window(self) -> int:
        return self.spec.sliding_window


# A Llama-3-8B-shaped whole 8192-token prompt, and chunked prefill of four
# sequences (2048-token chunks after cached prefixes, up to 16k tokens),
# 64 query / 8 kv heads: the prefill shapes of the pages' engine (a
# variable-length prefill call over the paged cache).
PREFILL_CONFIGS = {
    "prefill_8k": PrefillSpec("prefill_b1_q32kv8_d128_prompt8192_bf16", batch=1, hq=32, hkv=8, head_dim=128,
                              ctx_lo=8192, ctx_hi=8192, chunk_lo=0, chunk_hi=0, pool_blocks=600, seed=21),
    "chunked_prefill": PrefillSpec("chunked_prefill_b4_q64kv8_d128_chunk2048_ctx2k-16k_bf16", batch=4, hq=64,
                                   hkv=8, head_dim=128, ctx_lo=2048, ctx_hi=16384, chunk_lo=2048,
                                   chunk_hi=2048, pool_blocks=4200, seed=22),
    # Gemma-2-9B-shaped head_dim 256 (16 query / 8 kv heads): one whole
    # 8192-token prompt
    "prefill_d256": PrefillSpec("prefill_b1_q16kv8_d256_prompt8192_bf16", batch=1, hq=16, hkv=8, head_dim=256,
                                ctx_lo=8192, ctx_hi=8192, chunk_lo=0, chunk_hi=0, pool_blocks=600, seed=24),
    # the chunked workload over an fp8 e4m3fn cache with per-token scales
    "chunked_prefill_fp8": PrefillSpec("chunked_prefill_b4_q64kv8_d128_chunk2048_ctx2k-16k_fp8", batch=4, hq=64,
                                       hkv=8, head_dim=128, ctx_lo=2048, ctx_hi=16384, chunk_lo=2048,
                                       chunk_hi=2048, pool_blocks=4200, seed=22, kv_dtype="fp8_e4m3fn"),
    # GPT-OSS-shaped sliding-window layers (64 query / 8 kv heads of 64, a
    # 128-token window and sink logits): four whole 8192-token prompts
    "prefill_swa_sinks": PrefillSpec("prefill_swa128_sinks_b4_q64kv8_d64_prompt8192_bf16", batch=4, hq=64, hkv=8,
                                     head_dim=64, ctx_lo=8192, ctx_hi=8192, chunk_lo=0, chunk_hi=0,
                                     pool_blocks=2100, seed=23, sliding_window=128, sinks=True),
}


def generate_prefill(spec: PrefillSpec, *, context_lens=None, chunk_lens=None) -> Prefill:
    """The cache as ``generate`` draws it for ``spec.cache_spec()`` (steps 1-5),
    then from a generator seeded with ``seed + 2000``: the chunk lengths
    (unless whole prompts or given) and the packed q rows (N(0, 1) -> bf16)."""
    cache = generate(spec.cache_spec(), context_lens=context_lens)
    gen = torch.Generator("cpu").manual_seed(spec.seed + 2000)
    L = cache.context_lens.to(torch.int64)
    if chunk_lens is not None:
        n = torch.as_tensor(chunk_lens, dtype=torch.int64).clone()
    elif spec.chunk_hi == 0:
        n = L.clone()
    else:
        n = torch.randint(spec.chunk_lo, spec.chunk_hi + 1, (spec.batch,), generator=gen, dtype=torch.int64)
    n = torch.minimum(n, L)
    if bool((n < 0).any()):
        raise ValueError("negative chunk length")
    cu = torch.zeros(spec.batch + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(n, 0)
    T = int(cu[-1])
    q = torch.randn(T, spec.hq, spec.head_dim, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return Prefill(spec, cache, q, cu.to(torch.int32), int(n.max()) if spec.batch else 0,
                   1.0 / math.sqrt(spec.head_dim))


def prefill_flops(context_lens, chunk_lens, hq: int, head_dim: int, sliding_window: int = 0) -> int:
    """Algorithmic flops of one prefill call: every (row, visible key, query
    head) pair costs 2 * D for the score and 2 * D for the value update; row
    t of a chunk of n rows in a sequence of L tokens sees a + 1 keys, a =
    L - n + t its position, or min(a + 1, w) with a sliding window w."""
    total = 0
    w = int(sliding_window)
    for L, n in zip(torch.as_tensor(context_lens).tolist(), torch.as_tensor(chunk_lens).tolist()):
        n = min(int(n), int(L))
        if n <= 0:
            continue
        a0, a1 = L - n, L - 1                    # first and last row position
        if w <= 0:
            total += n * (L - n) + n * (n + 1) // 2          # sum of a + 1 over the rows
            continue
        # rows below w - 1 see a + 1 keys, the rest w
        lo_end = min(a1, w - 2)
        if lo_end >= a0:
            total += (lo_end + 1) * (lo_end + 2) // 2 - a0 * (a0 + 1) // 2
        total += w * (a1 - max(a0, w - 1) + 1) if a1 >= max(a0, w - 1) else 0
    return 4 * head_dim * hq * total

"""Seeded synthetic decode batches for paged attention.

This module only *draws inputs*: context lengths, block tables over a shuffled
physical pool, and N(0,1) query / key / value data rounded to the 2-byte
storage type. It performs none of the attention arithmetic (no slot
computation, no gather, no softmax), so the CPU oracle and the HIP path can
both consume the very same arrays without sharing any of the method's code.

Shapes follow the cache layout of "01. PagedAttention 详解" (vLLM learning
book), §3: key_cache / value_cache are ``[num_blocks, block_size,
num_kv_heads, head_size]``; block tables are one int32 row per sequence,
packed into a single ``[num_seqs, max_blocks_per_seq]`` array (same page,
§10, questions on how the table reaches the GPU and on a 100k-token table).
A sequence of L tokens owns ceil(L / block_size) blocks ("PagedAttention 机制"
wiki, §5.3.2, the allocation rule of its BlockTable sketch).

Values are returned as numpy ``uint16`` bit patterns plus a dtype tag
("fp16" / "bf16"); both sides upcast them with their own code. A workload
with an FP8 cache ("fp8" cache dtype) keeps q and the new token's k/v in the
2-byte type and fills the pools with uint8 E4M3 codes of N(0,1) / scale,
produced by torch's float8_e4m3fn conversion (input preparation only; the
oracle has its own encoder).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

SEED_ROOT = 331
# Elements per independently seeded chunk of a bulk normal draw. Fixed, so the
# values do not depend on how many threads fill them.
_CHUNK = 1 << 22
# Seed-stream ids for the independent draws of one batch.
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_KNEW, _STREAM_VNEW = 1, 2, 3, 4, 5
_STREAM_PREFILL_POOL = 6

DTYPES = ("fp16", "bf16")


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and length distribution of one synthetic decode batch."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: str
    lengths: str                 # "uniform" | "lognormal"
    len_lo: int                  # inclusive bounds (uniform) or clip bounds (lognormal)
    len_hi: int
    len_median: float = 0.0      # lognormal only
    len_sigma: float = 1.0       # lognormal only
    num_blocks: Optional[int] = None   # fixed pool size; None -> ceil(1.1 * blocks used)
    shared_prefix_blocks: int = 0      # leading blocks common to every table
    partition_size: int = 0            # split-K partition the workload is quoted with (0: auto)
    cache_write: bool = True           # one new token per sequence written before attention
    seed_index: int = 0                # second word of the seed key
    cache_dtype: str = ""              # "" = dtype; "fp8" = E4M3 codes with kv_scale
    kv_scale: float = 2.0 ** -5        # fp32 scale of both FP8 cache tensors

    @property
    def cache_type(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_len(self) -> int:
        """Largest context length the distribution can produce."""
        if self.shared_prefix_blocks:
            return self.shared_prefix_blocks * self.block_size + self.len_hi
        return self.len_hi

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)


# The five decode workloads, in order. Lengths count the new token, which is
# written at position L-1 before the attention step reads positions [0, L)
# (decode flow of "01. PagedAttention 详解", §4).
CONFIGS = {
    "tiny_write": WorkloadSpec(
        name="tiny_write", num_seqs=4, num_q_heads=4, num_kv_heads=4, head_size=64,
        block_size=16, dtype="fp16", lengths="uniform", len_lo=1, len_hi=100,
        num_blocks=64, seed_index=1),
    "llama2_7b_mha": WorkloadSpec(
        name="llama2_7b_mha", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_size=128,
        block_size=16, dtype="fp16", lengths="uniform", len_lo=512, len_hi=2048,
        seed_index=2),
    "gqa_8b": WorkloadSpec(
        name="gqa_8b", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, dtype="bf16", lengths="lognormal", len_lo=16, len_hi=4096,
        len_median=1000.0, len_sigma=1.0, seed_index=3),
    "long_context_splitk": WorkloadSpec(
        name="long_context_splitk", num_seqs=4, num_q_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, dtype="fp16", lengths="uniform", len_lo=32768, len_hi=100000,
        partition_size=512, seed_index=4),
    "prefix_shared_write": WorkloadSpec(
        name="prefix_shared_write", num_seqs=128, num_q_heads=32, num_kv_heads=8, head_size=128,
        block_size=32, dtype="bf16", lengths="uniform", len_lo=16, len_hi=512,
        shared_prefix_blocks=32, seed_index=5),
    # FP8 (E4M3) caches of the MHA and GQA batches: same shapes and length
    # laws, q / out / new k, v in the 2-byte type.
    "llama2_7b_mha_fp8": WorkloadSpec(
        name="llama2_7b_mha_fp8", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_size=128,
        block_size=16, dtype="fp16", lengths="uniform", len_lo=512, len_hi=2048,
        seed_index=6, cache_dtype="fp8"),
    "gqa_8b_fp8": WorkloadSpec(
        name="gqa_8b_fp8", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, dtype="bf16", lengths="lognormal", len_lo=16, len_hi=4096,
        len_median=1000.0, len_sigma=1.0, seed_index=7, cache_dtype="fp8"),
}
CONFIG_ORDER = ("tiny_write", "llama2_7b_mha", "gqa_8b", "long_context_splitk",
                "prefix_shared_write")


@dataclass(frozen=True)
class PrefillSpec:
    """A prefill batch: each sequence holds ``ctx`` cached tokens and receives
    ``new`` prompt tokens (the book's §4 prefill phase; ctx = 0 is a whole
    prompt, ctx > 0 a later chunk of a chunked prompt)."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: str
    ctx_lo: int
    ctx_hi: int
    new_lo: int
    new_hi: int
    seed_index: int
    cache_dtype: str = ""              # "" = dtype; "fp8" = E4M3 codes with kv_scale
    kv_scale: float = 2.0 ** -5        # fp32 scale of both FP8 cache tensors

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads


PREFILL_CONFIGS = {
    # Llama-2-7B-shaped whole prompts of 512..2048 tokens.
    "llama2_7b_prefill": PrefillSpec(
        name="llama2_7b_prefill", num_seqs=4, num_q_heads=32, num_kv_heads=32, head_size=128,
        block_size=16, dtype="fp16", ctx_lo=0, ctx_hi=0, new_lo=512, new_hi=2048, seed_index=8),
    # GQA 8B-shaped chunked prefill: 0..2048 cached tokens plus a 64..512-token chunk.
    "gqa_8b_chunked_prefill": PrefillSpec(
        name="gqa_8b_chunked_prefill", num_seqs=16, num_q_heads=32, num_kv_heads=8,
        head_size=128, block_size=16, dtype="bf16", ctx_lo=0, ctx_hi=2048, new_lo=64, new_hi=512,
        seed_index=9),
}
# The same batches over FP8 (E4M3) caches: the same lengths (same seed),
# pools of E4M3 codes of N(0,1) / kv_scale as in the FP8 decode batches.
PREFILL_CONFIGS["llama2_7b_prefill_fp8"] = replace(PREFILL_CONFIGS["llama2_7b_prefill"],
                                                   name="llama2_7b_prefill_fp8", cache_dtype="fp8")
PREFILL_CONFIGS["gqa_8b_chunked_prefill_fp8"] = replace(
    PREFILL_CONFIGS["gqa_8b_chunked_prefill"], name="gqa_8b_chunked_prefill_fp8",
    cache_dtype="fp8")
PREFILL_ORDER = ("llama2_7b_prefill", "gqa_8b_chunked_prefill")
PREFILL_FP8_ORDER = ("llama2_7b_prefill_fp8", "gqa_8b_chunked_prefill_fp8")


@dataclass
class PrefillBatch:
    """Host arrays of one prefill batch. ``k_new`` / ``v_new`` are the new
    tokens' K/V, to be written before attention; the pool already holds the
    earlier context."""

    spec: PrefillSpec
    q: np.ndarray              # uint16 [T, Hq, D]
    key_cache: np.ndarray      # uint16 [NB, bs, Hkv, D]
    value_cache: np.ndarray
    block_tables: np.ndarray   # int32 [B, MB]
    context_lens: np.ndarray   # int32 [B], cached tokens after the new ones are written
    query_start: np.ndarray    # int32 [B + 1]
    k_new: np.ndarray          # uint16 [T, Hkv, D]
    v_new: np.ndarray
    scale: np.float32
    used_blocks: np.ndarray

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def cache_dtype(self) -> str:
        return self.spec.cache_dtype or self.spec.dtype

    @property
    def k_scale(self) -> np.float32:
        return np.float32(self.spec.kv_scale if self.cache_dtype == "fp8" else 1.0)

    @property
    def v_scale(self) -> np.float32:
        return self.k_scale

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def num_blocks(self) -> int:
        return int(self.key_cache.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def max_query_len(self) -> int:
        n = np.diff(self.query_start)
        return int(n.max()) if n.size else 0
FP8_ORDER = ("llama2_7b_mha_fp8", "gqa_8b_fp8")


@dataclass
class Batch:
    """One decode batch: every array is host memory (numpy)."""

    spec: WorkloadSpec
    q: np.ndarray              # uint16 [B, Hq, D]
    key_cache: np.ndarray      # uint16 [NB, bs, Hkv, D] (uint8 E4M3 codes for an FP8 cache)
    value_cache: np.ndarray    # same as key_cache
    block_tables: np.ndarray   # int32 [B, MB]
    context_lens: np.ndarray   # int32 [B]
    k_new: np.ndarray          # uint16 [B, Hkv, D]  (the new token's key)
    v_new: np.ndarray          # uint16 [B, Hkv, D]
    scale: np.float32
    used_blocks: np.ndarray    # int64 ids of physical blocks some table uses
    pad_block: int             # id stored in table entries past a sequence's blocks
    extra: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def cache_dtype(self) -> str:
        return self.spec.cache_type

    @property
    def k_scale(self) -> np.float32:
        return np.float32(self.spec.kv_scale if self.cache_dtype == "fp8" else 1.0)

    @property
    def v_scale(self) -> np.float32:
        return self.k_scale

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.extra.get("num_blocks", self.key_cache.shape[0]))

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 2-byte storage bits, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_bits(dtype: str) -> int:
    """A quiet-NaN bit pattern of the storage type (used to poison memory)."""
    return {"fp16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}[dtype]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_normal(shape: Sequence[int], dtype: str, key: Sequence[int]) -> np.ndarray:
    """N(0,1) float32 draws rounded to ``dtype``, as uint16 bits.

    The array is cut into fixed chunks of ``_CHUNK`` elements; chunk i draws
    from ``SeedSequence(key).spawn(...)[i]``, so the result depends only on
    ``key`` and ``shape``.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    nch = -(-n // _CHUNK)
    if nch == 0:
        return out.reshape(shape)
    kids = np.random.SeedSequence(list(key)).spawn(nch)

    def work(i: int) -> None:
        a = i * _CHUNK
        b = min(n, a + _CHUNK)
        x = np.random.default_rng(kids[i]).standard_normal(b - a, dtype=np.float32)
        out[a:b] = round_to_storage(x, dtype)

    if nch == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out.reshape(shape)


def fill_fp8(shape: Sequence[int], scale: float, key: Sequence[int]) -> np.ndarray:
    """E4M3 codes of N(0,1) / scale (torch's float8_e4m3fn conversion), uint8."""
    import torch
    bits16 = fill_normal(shape, "bf16", key)     # a seeded N(0,1) draw, as bf16 bits
    x = torch.from_numpy(bits16.view(np.int16)).view(torch.bfloat16).float() / float(scale)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(shape)


def draw_lengths(spec: WorkloadSpec, rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    """Context lengths (including the new token), int32 [num_seqs]."""
    if spec.lengths == "uniform":
        lens = rng.integers(spec.len_lo, spec.len_hi, size=num_seqs, endpoint=True)
    elif spec.lengths == "lognormal":
        z = rng.standard_normal(num_seqs)
        lens = np.rint(np.exp(math.log(spec.len_median) + spec.len_sigma * z))
        lens = np.clip(lens, spec.len_lo, spec.len_hi)
    else:
        raise ValueError(spec.lengths)
    lens = lens.astype(np.int64)
    if spec.shared_prefix_blocks:
        lens = lens + spec.shared_prefix_blocks * spec.block_size
    return lens.astype(np.int32)


def make_batch(spec: WorkloadSpec, *, lengths: Optional[Sequence[int]] = None,
               num_seqs: Optional[int] = None, seed: Optional[Sequence[int]] = None,
               max_blocks_per_seq: Optional[int] = None, values: bool = True) -> Batch:
    """Draw one batch for ``spec``.

    Draw order: lengths, then the pool permutation (both from
    ``default_rng([331, seed_index])``), then q, K pool, V pool, new k, new v
    (each from its own seed stream). ``lengths`` overrides the length draw
    (edge-case tests); ``num_seqs`` shrinks the batch. ``values=False`` draws
    only lengths and tables (the value arrays come back empty).
    """
    key = list(seed) if seed is not None else [SEED_ROOT, spec.seed_index]
    rng = np.random.default_rng(key)
    if lengths is not None:
        lens = np.asarray(lengths, dtype=np.int32)
    else:
        lens = draw_lengths(spec, rng, num_seqs if num_seqs is not None else spec.num_seqs)
    B = int(lens.shape[0])
    bs = spec.block_size
    if np.any(lens < 0):
        raise ValueError("negative context length")

    nblk = (lens.astype(np.int64) + bs - 1) // bs          # blocks each sequence owns
    shared = spec.shared_prefix_blocks
    if shared and B and np.any(nblk < shared):
        raise ValueError("a sequence is shorter than the shared prefix")
    private = nblk - shared if shared else nblk
    distinct = int(private.sum()) + (shared if B else 0)

    if spec.num_blocks is not None:
        NB = spec.num_blocks
        if NB < distinct + 1:
            raise ValueError("fixed pool too small")
    else:
        NB = max(distinct + 1, int(math.ceil(1.1 * distinct)))
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else max(
        spec.max_blocks_per_seq, int(nblk.max()) if B else 1)
    if B and int(nblk.max()) > MB:
        raise ValueError("max_blocks_per_seq too small")

    perm = rng.permutation(NB).astype(np.int64)
    pad_block = int(perm[distinct])            # never used by any sequence
    tables = np.full((B, MB), pad_block, dtype=np.int32)
    cursor = 0
    prefix = perm[:shared] if shared else perm[:0]
    cursor += shared if B else 0
    for s in range(B):
        row = []
        if shared:
            row.extend(prefix.tolist())
        n = int(private[s])
        row.extend(perm[cursor:cursor + n].tolist())
        cursor += n
        tables[s, :len(row)] = row
    used = perm[:distinct].copy()

    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_size
    dt = spec.dtype
    if values:
        q = fill_normal((B, Hq, D), dt, key + [_STREAM_Q])
        if spec.cache_type == "fp8":
            kc = fill_fp8((NB, bs, Hkv, D), spec.kv_scale, key + [_STREAM_K])
            vc = fill_fp8((NB, bs, Hkv, D), spec.kv_scale, key + [_STREAM_V])
        else:
            kc = fill_normal((NB, bs, Hkv, D), dt, key + [_STREAM_K])
            vc = fill_normal((NB, bs, Hkv, D), dt, key + [_STREAM_V])
        k_new = fill_normal((B, Hkv, D), dt, key + [_STREAM_KNEW])
        v_new = fill_normal((B, Hkv, D), dt, key + [_STREAM_VNEW])
    else:
        q = np.empty((0, Hq, D), np.uint16)
        kc = vc = np.empty((0, bs, Hkv, D), np.uint8 if spec.cache_type == "fp8" else np.uint16)
        k_new = v_new = np.empty((0, Hkv, D), np.uint16)
    scale = np.float32(1.0 / math.sqrt(D))
    return Batch(spec=spec, q=q, key_cache=kc, value_cache=vc, block_tables=tables,
                 context_lens=lens, k_new=k_new, v_new=v_new, scale=scale,
                 used_blocks=used, pad_block=pad_block, extra={"num_blocks": NB})


def small_variant(name: str, num_seqs: int) -> WorkloadSpec:
    """A config with fewer sequences (same shapes and length law)."""
    return replace(CONFIGS[name], num_seqs=num_seqs)


def relabel_contiguous(batch: Batch) -> Batch:
    """The same batch with its physical blocks renumbered so that every table
    row is a run of consecutive ids in sequence order: shared prefix blocks
    first, then each sequence's own blocks in table order (the contiguous
    layout a non-paged cache would have). Pool rows move with their ids, so
    every position keeps its K/V values and the attention result is the same;
    only the physical placement changes. Unused blocks keep the ids after the
    used ones; table entries past a sequence's blocks point at the pad block's
    new id."""
    bs = batch.spec.block_size
    NB = batch.key_cache.shape[0]
    order = []                       # old ids in their new order
    seen = np.zeros(NB, dtype=bool)
    for s in range(batch.num_seqs):
        n = -(-int(batch.context_lens[s]) // bs)
        for blk in batch.block_tables[s, :n].tolist():
            if not seen[blk]:
                seen[blk] = True
                order.append(blk)
    order.extend(np.flatnonzero(~seen).tolist())
    order = np.asarray(order, dtype=np.int64)
    new_id = np.empty(NB, dtype=np.int64)
    new_id[order] = np.arange(NB)
    return replace(batch, key_cache=batch.key_cache[order], value_cache=batch.value_cache[order],
                   block_tables=new_id[batch.block_tables].astype(np.int32),
                   used_blocks=new_id[batch.used_blocks], pad_block=int(new_id[batch.pad_block]))


def poison_unused_blocks(batch: Batch) -> None:
    """Fill every physical block no table uses (including the pad block) with NaN."""
    mask = np.ones(batch.num_blocks, dtype=bool)
    mask[batch.used_blocks] = False
    nb = nan_bits(batch.cache_dtype)
    batch.key_cache[mask] = nb
    batch.value_cache[mask] = nb


def make_prefill_batch(spec: PrefillSpec, *, ctx: Optional[Sequence[int]] = None,
                       new: Optional[Sequence[int]] = None,
                       num_seqs: Optional[int] = None) -> PrefillBatch:
    """Draw a prefill batch: ctx and new-token counts (uniform, inclusive) from
    ``default_rng([331, seed_index])``, tables over a shuffled pool of the
    blocks used plus 10%, then q / pool / new k, v from their own streams."""
    key = [SEED_ROOT, spec.seed_index]
    rng = np.random.default_rng(key)
    B = num_seqs if num_seqs is not None else spec.num_seqs
    c = np.asarray(ctx, np.int64) if ctx is not None else \
        rng.integers(spec.ctx_lo, spec.ctx_hi, size=B, endpoint=True)
    n = np.asarray(new, np.int64) if new is not None else \
        rng.integers(spec.new_lo, spec.new_hi, size=B, endpoint=True)
    lens = (c + n).astype(np.int32)
    dec = WorkloadSpec(name=spec.name, num_seqs=len(lens), num_q_heads=spec.num_q_heads,
                       num_kv_heads=spec.num_kv_heads, head_size=spec.head_size,
                       block_size=spec.block_size, dtype=spec.dtype, lengths="uniform",
                       len_lo=1, len_hi=max(1, int(lens.max()) if lens.size else 1),
                       seed_index=spec.seed_index, cache_dtype=spec.cache_dtype,
                       kv_scale=spec.kv_scale)
    b = make_batch(dec, lengths=lens, seed=key + [_STREAM_PREFILL_POOL])
    T = int(n.sum())
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_size
    q = fill_normal((T, Hq, D), spec.dtype, key + [_STREAM_Q])
    k_new = fill_normal((T, Hkv, D), spec.dtype, key + [_STREAM_KNEW])
    v_new = fill_normal((T, Hkv, D), spec.dtype, key + [_STREAM_VNEW])
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return PrefillBatch(spec=spec, q=q, key_cache=b.key_cache, value_cache=b.value_cache,
                        block_tables=b.block_tables, context_lens=lens, query_start=qs,
                        k_new=k_new, v_new=v_new, scale=np.float32(1.0 / math.sqrt(D)),
                        used_blocks=b.used_blocks)

"""Plain fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The HIP library never calls it and
shares no code with it; the two meet only in the seeded input arrays.

What it computes, with the passage each step follows:

* Cache layout ``key_cache / value_cache [num_blocks, block_size,
  num_kv_heads, head_size]`` -- "01. PagedAttention 详解" (vLLM learning
  book), §3 (storage layout).
* Logical position t of a sequence lives in physical block
  ``block_table[t // block_size]`` at offset ``t % block_size`` --
  "PagedAttention 机制" wiki, §5.3.4 (its conceptual paged_attention loop),
  and the book's §3 figure (request A's tokens 0..47 over blocks 42, 17, 99).
* Decode order: the new token's k/v are appended to the next free slot of the
  last block, then q attends over all cached positions -- book §4, decode
  phase. So with context length L the newest token sits at position L-1.
* Attention for one query head: logits ``scale * (q . k_t)`` for t < L,
  softmax over t, weighted sum of v_t. The wiki's §5.3.4 sketch scales by
  1/sqrt(head_dim) but omits the exponentiation and normalisation, and the
  book's §4 formula did not survive extraction; the standard softmax
  attention is the reading taken here.
* Query head h reads kv head ``h // (num_q_heads // num_kv_heads)``
  (grouped-query attention; the book's self-check Q2 only uses GQA as a size
  effect, so consecutive query heads sharing one kv head is a reading).
* L = 0 leaves the output at zero (the wiki sketch starts from
  ``zeros_like(query)`` and its loop body never runs).
* Split-K recombination (the book's §4 and §9 say v2 splits long sequences
  across partitions): each partition keeps (max, exp-sum, normalised output)
  and the combine rescales by exp(m_p - M). This is an exact identity and is
  provided so its algebra can be checked against the unsplit definition.

Storage values arrive as uint16 bit patterns with a dtype tag; they are
upcast exactly to float64. ``scale`` is the float32 value handed to the
library, upcast. Results are float64 and unrounded.

An FP8 cache (the article's §4.3 FP8 K/V; encoding in :mod:`oracle.fp8`)
holds uint8 E4M3 codes and one fp32 scale per tensor: a cached row stands for
``decode(code) * scale``, computed exactly in float64. The query and the
output keep their 2-byte type.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "to_float64", "physical_slot", "slot_mapping", "cache_write",
    "gather_positions", "decode", "decode_one", "attention_weights",
    "decode_partitioned", "decode_two_level", "prefill", "prefill_slot_mapping",
    "blocks_needed",
]


def to_float64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of fp16 / bf16 bit patterns (or E4M3 codes) to float64."""
    if dtype == "fp8":
        from .fp8 import e4m3_decode
        return e4m3_decode(bits)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bf16 is the top half of an IEEE binary32.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies (wiki §5.3.2 allocate rule)."""
    return (int(num_tokens) + block_size - 1) // block_size


def physical_slot(table_row: np.ndarray, position: int, block_size: int) -> int:
    """Flat slot index of logical ``position``: block id times block size plus offset."""
    position = int(position)
    return int(table_row[position // block_size]) * block_size + position % block_size


def slot_mapping(block_tables: np.ndarray, context_lens: np.ndarray,
                 block_size: int) -> np.ndarray:
    """Slot of each sequence's newest token (position L-1); -1 when L == 0."""
    out = np.empty(len(context_lens), dtype=np.int32)
    for s, L in enumerate(np.asarray(context_lens).tolist()):
        out[s] = physical_slot(block_tables[s], L - 1, block_size) if L > 0 else -1
    return out


def cache_write(key_cache: np.ndarray, value_cache: np.ndarray,
                k: np.ndarray, v: np.ndarray,
                slots: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the caches with token i's k/v stored at ``slots[i]``.

    ``k, v`` are ``[num_tokens, num_kv_heads, head_size]`` bit patterns; a
    negative slot means "no write" for that token. Slots must be distinct.
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    bs = kc.shape[1]
    live = [int(x) for x in np.asarray(slots).tolist() if x >= 0]
    assert len(live) == len(set(live)), "cache_write: duplicate slots"
    for i, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        kc[slot // bs, slot % bs] = k[i]
        vc[slot // bs, slot % bs] = v[i]
    return kc, vc


def gather_positions(cache: np.ndarray, table_row: np.ndarray, length: int,
                     kv_head: int, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Rows ``cache[table[t // bs], t % bs, kv_head, :]`` for t < length, as float64.

    For an FP8 cache each row is multiplied by the tensor's scale.
    """
    bs = cache.shape[1]
    t = np.arange(int(length), dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[t // bs]
    rows = to_float64(cache[blocks, t % bs, kv_head, :], dtype)
    return rows * float(np.float32(scale)) if dtype == "fp8" else rows


def _softmax_attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray,
                    scale: float) -> Tuple[np.ndarray, np.ndarray]:
    logits = scale * (K @ qv)
    m = logits.max()
    w = np.exp(logits - m)
    p = w / w.sum()
    return p @ V, p


def _row_operands(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                  block_tables: np.ndarray, context_lens: np.ndarray, dtype: str,
                  seq: int, head: int, cache_dtype: Optional[str], k_scale: float,
                  v_scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """q row, and the K / V rows of positions < L of its kv head, as float64."""
    cdt = cache_dtype or dtype
    Hq = q.shape[1]
    Hkv = key_cache.shape[2]
    g = head // (Hq // Hkv)
    L = int(context_lens[seq])
    K = gather_positions(key_cache, block_tables[seq], L, g, cdt, k_scale)
    V = gather_positions(value_cache, block_tables[seq], L, g, cdt, v_scale)
    return to_float64(q[seq, head], dtype), K, V


def decode_one(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
               block_tables: np.ndarray, context_lens: np.ndarray, scale,
               dtype: str, seq: int, head: int, cache_dtype: Optional[str] = None,
               k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Output row ``out[seq, head, :]`` in float64."""
    if int(context_lens[seq]) == 0:
        return np.zeros(q.shape[2], dtype=np.float64)
    qv, K, V = _row_operands(q, key_cache, value_cache, block_tables, context_lens, dtype,
                             seq, head, cache_dtype, k_scale, v_scale)
    out, _ = _softmax_attend(qv, K, V, float(np.float32(scale)))
    return out


def decode(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale,
           dtype: str, seqs: Optional[Iterable[int]] = None,
           cache_dtype: Optional[str] = None, k_scale: float = 1.0,
           v_scale: float = 1.0) -> np.ndarray:
    """``out[s, h, :] = softmax(scale * q[s,h] . K_g^T) V_g`` over positions < L_s.

    Returns float64 ``[len(seqs), Hq, D]`` (all sequences by default). Each kv
    head's rows are gathered once and reused by its query-head group.
    ``dtype`` is the query's storage type; ``cache_dtype`` (default: the
    same) is the caches', and an FP8 cache's rows are scaled by
    ``k_scale`` / ``v_scale``.
    """
    cdt = cache_dtype or dtype
    B, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    seqs = list(range(B)) if seqs is None else list(seqs)
    sc = float(np.float32(scale))
    out = np.zeros((len(seqs), Hq, D), dtype=np.float64)
    for i, s in enumerate(seqs):
        L = int(context_lens[s])
        if L == 0:
            continue
        for g in range(Hkv):
            K = gather_positions(key_cache, block_tables[s], L, g, cdt, k_scale)
            V = gather_positions(value_cache, block_tables[s], L, g, cdt, v_scale)
            for h in range(g * G, (g + 1) * G):
                out[i, h], _ = _softmax_attend(to_float64(q[s, h], dtype), K, V, sc)
    return out


def attention_weights(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                      block_tables: np.ndarray, context_lens: np.ndarray, scale, dtype: str,
                      seq: int, head: int, cache_dtype: Optional[str] = None,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """The softmax weights over positions < L that :func:`decode_one` applies
    to the V rows of one (sequence, query head): the same gathered operands
    and the same ``_softmax_attend`` call, so ``weights @ V`` is that output
    row. Empty for L == 0."""
    if int(context_lens[seq]) == 0:
        return np.zeros(0, dtype=np.float64)
    qv, K, V = _row_operands(q, key_cache, value_cache, block_tables, context_lens, dtype,
                             seq, head, cache_dtype, k_scale, v_scale)
    _, p = _softmax_attend(qv, K, V, float(np.float32(scale)))
    return p


def decode_partitioned(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                       block_tables: np.ndarray, context_lens: np.ndarray, scale,
                       dtype: str, partition_size: int,
                       seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Same result as :func:`decode`, computed partition by partition.

    Partition p covers positions [p*P, min((p+1)*P, L)). It keeps its own max
    m_p, exp-sum Z_p and normalised output o_p; the combine takes
    M = max m_p, c_p = Z_p * exp(m_p - M) and returns sum c_p o_p / sum c_p.
    """
    B, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    P = int(partition_size)
    seqs = list(range(B)) if seqs is None else list(seqs)
    sc = float(np.float32(scale))
    out = np.zeros((len(seqs), Hq, D), dtype=np.float64)
    for i, s in enumerate(seqs):
        L = int(context_lens[s])
        if L == 0:
            continue
        for g in range(Hkv):
            K = gather_positions(key_cache, block_tables[s], L, g, dtype)
            V = gather_positions(value_cache, block_tables[s], L, g, dtype)
            for h in range(g * G, (g + 1) * G):
                qv = to_float64(q[s, h], dtype)
                parts: List[Tuple[float, float, np.ndarray]] = []
                for a in range(0, L, P):
                    logits = sc * (K[a:a + P] @ qv)
                    m_p = logits.max()
                    w = np.exp(logits - m_p)
                    Z_p = w.sum()
                    parts.append((m_p, Z_p, (w @ V[a:a + P]) / Z_p))
                M = max(m for m, _, _ in parts)
                c = np.array([Z * np.exp(m - M) for m, Z, _ in parts])
                o = np.stack([o for _, _, o in parts])
                out[i, h] = (c @ o) / c.sum()
    return out


def decode_two_level(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                     block_tables: np.ndarray, context_lens: np.ndarray, scale, dtype: str,
                     prefix_len: int, seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Same result as :func:`decode`, with the shared prefix taken separately.

    When every table starts with the same blocks (the book's §6: one copy of
    a shared prompt referenced by many requests), positions [0, prefix_len)
    can be attended through one table for all sequences and the rest through
    each sequence's own. Each part keeps (max, exp-sum, normalised output) over
    its positions below the sequence's length, and the two are merged with the
    exp(m - M) rescale of :func:`decode_partitioned`.
    """
    B, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    seqs = list(range(B)) if seqs is None else list(seqs)
    sc = float(np.float32(scale))
    shared_row = block_tables[0]
    out = np.zeros((len(seqs), Hq, D), dtype=np.float64)
    for i, s in enumerate(seqs):
        L = int(context_lens[s])
        if L == 0:
            continue
        lp = min(L, int(prefix_len))
        for g in range(Hkv):
            Kp = gather_positions(key_cache, shared_row, lp, g, dtype)
            Vp = gather_positions(value_cache, shared_row, lp, g, dtype)
            K = gather_positions(key_cache, block_tables[s], L, g, dtype)[lp:]
            V = gather_positions(value_cache, block_tables[s], L, g, dtype)[lp:]
            for h in range(g * G, (g + 1) * G):
                qv = to_float64(q[s, h], dtype)
                parts = []
                for Kx, Vx in ((Kp, Vp), (K, V)):
                    if len(Kx) == 0:
                        continue
                    logits = sc * (Kx @ qv)
                    m_p = logits.max()
                    w = np.exp(logits - m_p)
                    parts.append((m_p, w.sum(), (w @ Vx) / w.sum()))
                M = max(m for m, _, _ in parts)
                c = np.array([Z * np.exp(m - M) for m, Z, _ in parts])
                o = np.stack([o for _, _, o in parts])
                out[i, h] = (c @ o) / c.sum()
    return out


def prefill(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
            block_tables: np.ndarray, context_lens: np.ndarray, query_start: np.ndarray,
            scale, dtype: str, cache_dtype: Optional[str] = None, k_scale: float = 1.0,
            v_scale: float = 1.0) -> np.ndarray:
    """Causal attention of each sequence's new tokens over its paged cache.

    The book's §4 prefill phase: the N new tokens' K and V are first written
    into the blocks the table points to, then attention runs over them. With
    chunked prompts a sequence may already hold earlier tokens, so sequence s
    has ``n = query_start[s+1] - query_start[s]`` new tokens (rows
    ``query_start[s] .. query_start[s+1]-1`` of ``q``) at positions
    ``L - n .. L - 1`` of its ``L = context_lens[s]`` cached positions. The
    new token at position ``p`` attends to positions ``0 .. p``.
    ``cache_dtype`` (default: ``dtype``) is the caches' type, as in
    :func:`decode`: an FP8 cache's rows are its codes' values times
    ``k_scale`` / ``v_scale``.
    Returns float64 ``[num_tokens, Hq, D]``.
    """
    T, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qs = np.asarray(query_start, dtype=np.int64)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        a, b = int(qs[s]), int(qs[s + 1])
        n = b - a
        if n == 0:
            continue
        assert n <= L, "more new tokens than cached positions"
        for g in range(Hkv):
            K = gather_positions(key_cache, block_tables[s], L, g, cache_dtype or dtype, k_scale)
            V = gather_positions(value_cache, block_tables[s], L, g, cache_dtype or dtype, v_scale)
            for i in range(n):
                pos = L - n + i
                for h in range(g * G, (g + 1) * G):
                    out[a + i, h], _ = _softmax_attend(to_float64(q[a + i, h], dtype),
                                                       K[:pos + 1], V[:pos + 1], sc)
    return out


def prefill_slot_mapping(block_tables: np.ndarray, context_lens: np.ndarray,
                         query_start: np.ndarray, block_size: int) -> np.ndarray:
    """Slot of every new token: row ``query_start[s] + i`` holds position
    ``L - n + i`` of sequence s (the book's §4 prefill writes the new tokens'
    K/V in order into the blocks the table points to)."""
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.empty(int(qs[-1]), dtype=np.int32)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        n = int(qs[s + 1] - qs[s])
        for i in range(n):
            out[qs[s] + i] = physical_slot(block_tables[s], L - n + i, block_size)
    return out

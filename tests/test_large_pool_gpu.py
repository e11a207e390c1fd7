"""GPU parity with every block a batch uses placed above 2**31 elements of the
pool (above 2**31 bytes for FP8 caches), so that the cache addressing of
every kernel must run in 64 bits. A 288 GB device holds pools that size; the
slots themselves stay int32 (num_blocks * block_size <= INT32_MAX).

The batches are the small seeded ones of the other tests. Their compact
pools are copied into a device pool of T + n blocks, block c at T + perm[c]
with T = ceil(2**31 / elements per block), the rest zero, and the tables are
renumbered the same way; the oracle runs on the compact arrays. Written rows
are compared bit-exactly at their renumbered slots.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.block_pool import copy_blocks as oracle_copy_blocks
from paged_kv_cache_331_amd import pa, workloads as wl

from _paged import (TOL, down16, down8, max_err, oracle_caches, oracle_decode, say, tdtype, up16,
                    up32, up8)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pa.load()
    assert torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class BigPool:
    """A compact pool [n, bs, Hkv, D] moved to block ids T .. T + n - 1 of a
    device pool of T + n blocks."""

    def __init__(self, kc: np.ndarray, vc: np.ndarray, bt: np.ndarray, dtype: str, fp8: bool,
                 seed: int):
        n, bs, Hkv, D = kc.shape
        self.first = -(-(2 ** 31) // (bs * Hkv * D))      # T: offsets of block T are >= 2**31
        self.perm = self.first + np.random.default_rng([331, 900, seed]).permutation(n)
        nb = self.first + n
        assert nb * bs <= 2 ** 31 - 1
        shape = (nb, bs, Hkv, D)
        tdt = torch.uint8 if fp8 else tdtype(dtype)
        self.kc = torch.zeros(shape, dtype=tdt, device="cuda")
        self.vc = torch.zeros(shape, dtype=tdt, device="cuda")
        ids = torch.from_numpy(self.perm.astype(np.int64)).cuda()
        up = up8 if fp8 else (lambda a: up16(a, dtype))
        self.kc[ids] = up(kc)
        self.vc[ids] = up(vc)
        self.fp8 = fp8
        self.bt = up32(self.table(bt))
        self.bs = bs

    def table(self, bt: np.ndarray) -> np.ndarray:
        out = bt.astype(np.int64).copy()
        used = (out >= 0) & (out < len(self.perm))
        out[used] = self.perm[out[used]]
        return out.astype(np.int32)

    def slot(self, compact_slot: int) -> int:
        c = int(compact_slot)
        return int(self.perm[c // self.bs]) * self.bs + c % self.bs

    def rows(self, cache: torch.Tensor, compact_slots) -> np.ndarray:
        """The rows at the renumbered slots, as host arrays of the storage type."""
        sl = [self.slot(c) for c in compact_slots]
        idx_b = torch.tensor([s // self.bs for s in sl], device="cuda")
        idx_o = torch.tensor([s % self.bs for s in sl], device="cuda")
        r = cache[idx_b, idx_o]
        return down8(r) if self.fp8 else down16(r)


def _decode_batch(name, nseq):
    b = wl.make_batch(wl.small_variant(name, nseq))
    assert int(b.key_cache.shape[0]) < 4096
    return b


@pytest.mark.parametrize("name,nseq,P,one_call", [
    ("llama2_7b_mha", 6, 0, False),        # VALU item, three calls
    ("llama2_7b_mha", 6, 512, True),       # VALU item, split, one call
    ("gqa_8b", 10, 0, True),               # matrix-core item
    ("gqa_8b", 10, 256, False),            # matrix-core item, split
    ("gqa_8b_fp8", 10, 0, True),           # FP8 matrix-core item
    ("llama2_7b_mha_fp8", 6, 512, False),  # FP8 VALU item, split
])
def test_decode_above_2g_elements(name, nseq, P, one_call):
    b = _decode_batch(name, nseq)
    fp8 = b.cache_dtype == "fp8"
    pool = BigPool(b.key_cache, b.value_cache, b.block_tables, b.dtype, fp8, seed=nseq + P)
    say(f"large pool {name} B={b.num_seqs} P={P} one_call={one_call} first block {pool.first}")
    dt = b.dtype
    q, kn, vn = up16(b.q, dt), up16(b.k_new, dt), up16(b.v_new, dt)
    lens = up32(b.context_lens)
    if one_call:
        if fp8:
            out = pa.decode_append_fp8(q, kn, vn, pool.kc, pool.vc, pool.bt, lens, float(b.scale),
                                       float(b.k_scale), float(b.v_scale), b.max_context_len,
                                       partition_size=P)
        else:
            out = pa.decode_append(q, kn, vn, pool.kc, pool.vc, pool.bt, lens, float(b.scale),
                                   b.max_context_len, partition_size=P)
    else:
        slots = pa.decode_slot_mapping(pool.bt, lens, b.spec.block_size)
        if fp8:
            pa.cache_write_fp8(kn, vn, pool.kc, pool.vc, slots, float(b.k_scale),
                               float(b.v_scale))
            out = pa.decode_fp8(q, pool.kc, pool.vc, pool.bt, lens, float(b.scale),
                                float(b.k_scale), float(b.v_scale), b.max_context_len,
                                partition_size=P)
        else:
            pa.cache_write(kn, vn, pool.kc, pool.vc, slots)
            out = pa.decode(q, pool.kc, pool.vc, pool.bt, lens, float(b.scale),
                            b.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    kc, vc, ref_slots = oracle_caches(b, True)
    ref = oracle_decode(b, kc, vc)
    err = max_err(out, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[dt]
    live = [int(x) for x in ref_slots if x >= 0]
    bs = b.spec.block_size
    kref = np.stack([kc[s // bs, s % bs] for s in live])
    vref = np.stack([vc[s // bs, s % bs] for s in live])
    assert np.array_equal(pool.rows(pool.kc, live), kref)
    assert np.array_equal(pool.rows(pool.vc, live), vref)


@pytest.mark.parametrize("P", [0, 256])
def test_cascade_above_2g_elements(P):
    spec = wl.small_variant("prefix_shared_write", 6)
    b = wl.make_batch(spec)
    pool = BigPool(b.key_cache, b.value_cache, b.block_tables, b.dtype, False, seed=50 + P)
    say(f"large pool cascade B={b.num_seqs} P={P} first block {pool.first}")
    dt = b.dtype
    q, kn, vn = up16(b.q, dt), up16(b.k_new, dt), up16(b.v_new, dt)
    lens = up32(b.context_lens)
    slots = pa.decode_slot_mapping(pool.bt, lens, spec.block_size)
    pa.cache_write(kn, vn, pool.kc, pool.vc, slots)
    out = pa.decode_cascade(q, pool.kc, pool.vc, pool.bt, lens, float(b.scale), b.max_context_len,
                            spec.shared_prefix_blocks, partition_size=P)
    torch.cuda.synchronize()
    kc, vc, _ = oracle_caches(b, True)
    ref = oracle.decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, b.dtype)
    err = max_err(out, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("name,ctx,new", [
    ("llama2_7b_prefill", [0, 300], [200, 90]),
    ("gqa_8b_chunked_prefill", [900, 0, 129], [80, 300, 1]),
])
def test_prefill_above_2g_elements(name, ctx, new):
    b = wl.make_prefill_batch(wl.PREFILL_CONFIGS[name], ctx=ctx, new=new)
    pool = BigPool(b.key_cache, b.value_cache, b.block_tables, b.dtype, False, seed=len(ctx))
    say(f"large pool prefill {name} T={b.num_tokens} first block {pool.first}")
    dt = b.dtype
    q, kn, vn = up16(b.q, dt), up16(b.k_new, dt), up16(b.v_new, dt)
    lens, qs = up32(b.context_lens), up32(b.query_start)
    bs = b.spec.block_size
    slots = pa.prefill_slot_mapping(pool.bt, lens, qs, b.num_tokens, b.max_query_len, bs,
                                    b.max_context_len)
    pa.cache_write(kn, vn, pool.kc, pool.vc, slots)
    out = pa.prefill(q, pool.kc, pool.vc, pool.bt, lens, qs, float(b.scale), b.max_query_len,
                     b.max_context_len)
    torch.cuda.synchronize()
    ref_slots = oracle.prefill_slot_mapping(b.block_tables, b.context_lens, b.query_start, bs)
    kc, vc = oracle.cache_write(b.key_cache, b.value_cache, b.k_new, b.v_new, ref_slots)
    assert np.array_equal(slots.cpu().numpy(), [pool.slot(x) for x in ref_slots])
    ref = oracle.prefill(b.q, kc, vc, b.block_tables, b.context_lens, b.query_start, b.scale,
                         b.dtype)
    err = max_err(out, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[dt]


def test_copy_blocks_above_2g_elements():
    b = _decode_batch("gqa_8b", 4)
    pool = BigPool(b.key_cache, b.value_cache, b.block_tables, b.dtype, False, seed=77)
    n = b.key_cache.shape[0]
    pairs_c = np.array([[0, n - 1], [n - 2, 1]], dtype=np.int32)   # compact (src, dst)
    pairs = torch.from_numpy(pool.perm[pairs_c].astype(np.int32)).cuda()
    say(f"large pool copy_blocks pairs {pool.perm[pairs_c].tolist()}")
    pa.copy_blocks(pool.kc, pool.vc, pairs)
    torch.cuda.synchronize()
    kc, vc = oracle_copy_blocks(b.key_cache, b.value_cache, pairs_c.tolist())
    for c in range(n):
        blk = int(pool.perm[c])
        assert np.array_equal(down16(pool.kc[blk]), kc[c])
        assert np.array_equal(down16(pool.vc[blk]), vc[c])


def test_prefill_fp8_above_2g_bytes():
    b = wl.make_prefill_batch(wl.PREFILL_CONFIGS["gqa_8b_chunked_prefill_fp8"], ctx=[900, 0, 129],
                              new=[80, 300, 1])
    pool = BigPool(b.key_cache, b.value_cache, b.block_tables, b.dtype, True, seed=88)
    say(f"large pool prefill fp8 T={b.num_tokens} first block {pool.first}")
    dt, ks, vs = b.dtype, float(b.k_scale), float(b.v_scale)
    q, kn, vn = up16(b.q, dt), up16(b.k_new, dt), up16(b.v_new, dt)
    lens, qs = up32(b.context_lens), up32(b.query_start)
    bs = b.spec.block_size
    slots = pa.prefill_slot_mapping(pool.bt, lens, qs, b.num_tokens, b.max_query_len, bs,
                                    b.max_context_len)
    pa.cache_write_fp8(kn, vn, pool.kc, pool.vc, slots, ks, vs)
    out = pa.prefill_fp8(q, pool.kc, pool.vc, pool.bt, lens, qs, float(b.scale), ks, vs,
                         b.max_query_len, b.max_context_len)
    torch.cuda.synchronize()
    ref_slots = oracle.prefill_slot_mapping(b.block_tables, b.context_lens, b.query_start, bs)
    kc, vc = oracle.cache_write_fp8(b.key_cache, b.value_cache, b.k_new, b.v_new, ref_slots, dt,
                                    ks, vs)
    assert np.array_equal(pool.rows(pool.kc, ref_slots), kc[ref_slots // bs, ref_slots % bs])
    ref = oracle.prefill(b.q, kc, vc, b.block_tables, b.context_lens, b.query_start, b.scale, dt,
                         cache_dtype="fp8", k_scale=ks, v_scale=vs)
    err = max_err(out, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[dt]

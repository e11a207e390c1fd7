"""Shared helpers for the GPU parity tests: upload a seeded batch, run the HIP
path through the C-ABI binding, run the oracle on the same host arrays, and
compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from paged_kv_cache_331_amd import pa, workloads as wl

TOL = {"fp16": 2e-3, "bf16": 1e-2}   # max abs error vs the fp64 oracle


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(dtype: str) -> torch.dtype:
    return torch.float16 if dtype == "fp16" else torch.bfloat16


def up16(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdtype(dtype)).cuda()


def up32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def down16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def up8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def down8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


class Device:
    """The batch's arrays on the GPU."""

    def __init__(self, b: wl.Batch):
        dt = b.dtype
        self.q = up16(b.q, dt)
        if b.cache_dtype == "fp8":
            self.kc = up8(b.key_cache)
            self.vc = up8(b.value_cache)
        else:
            self.kc = up16(b.key_cache, dt)
            self.vc = up16(b.value_cache, dt)
        self.bt = up32(b.block_tables)
        self.lens = up32(b.context_lens)
        self.k_new = up16(b.k_new, dt)
        self.v_new = up16(b.v_new, dt)


def gpu_step(b: wl.Batch, d: Device, *, write: bool, partition_size: int = 0):
    """Slot mapping + cache write (optional) + decode; returns (slots, out)."""
    slots = pa.decode_slot_mapping(d.bt, d.lens, b.spec.block_size)
    if b.cache_dtype == "fp8":
        if write:
            pa.cache_write_fp8(d.k_new, d.v_new, d.kc, d.vc, slots, float(b.k_scale),
                               float(b.v_scale))
        out = pa.decode_fp8(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), float(b.k_scale),
                            float(b.v_scale), b.max_context_len, partition_size=partition_size)
    else:
        if write:
            pa.cache_write(d.k_new, d.v_new, d.kc, d.vc, slots)
        out = pa.decode(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), b.max_context_len,
                        partition_size=partition_size)
    torch.cuda.synchronize()
    return slots, out


def oracle_caches(b: wl.Batch, write: bool):
    if not write:
        return b.key_cache, b.value_cache, None
    slots = oracle.slot_mapping(b.block_tables, b.context_lens, b.spec.block_size)
    if b.cache_dtype == "fp8":
        kc, vc = oracle.cache_write_fp8(b.key_cache, b.value_cache, b.k_new, b.v_new, slots,
                                        b.dtype, b.k_scale, b.v_scale)
    else:
        kc, vc = oracle.cache_write(b.key_cache, b.value_cache, b.k_new, b.v_new, slots)
    return kc, vc, slots


def oracle_decode(b: wl.Batch, kc, vc, seqs=None):
    """The oracle's output for the batch with the given caches (any cache type)."""
    return oracle.decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, b.dtype, seqs=seqs,
                         cache_dtype=b.cache_dtype, k_scale=b.k_scale, v_scale=b.v_scale)


def oracle_decode_one(b: wl.Batch, kc, vc, s, h):
    return oracle.decode_one(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, b.dtype, s, h,
                             cache_dtype=b.cache_dtype, k_scale=b.k_scale, v_scale=b.v_scale)


# Half an ulp of the 2-byte output type, relative: a result of magnitude x is
# stored with an error up to HALF_ULP_REL * x on top of the path's own error.
HALF_ULP_REL = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def excess_err(gpu_out: torch.Tensor, ref: np.ndarray, dtype: str) -> float:
    """Largest error beyond TOL + the output's own rounding at |ref|, or <= 0."""
    out = to_f64(gpu_out)
    return float(np.max(np.abs(out - ref) - TOL[dtype] - HALF_ULP_REL[dtype] * np.abs(ref)))


def max_err(gpu_out: torch.Tensor, ref: np.ndarray) -> float:
    return float(np.max(np.abs(to_f64(gpu_out) - ref))) if ref.size else 0.0


def poison_tails(b: wl.Batch, write: bool) -> None:
    """NaN into every slot at a position >= L inside each sequence's last block
    (after the newest token, which the write fills)."""
    nb = wl.nan_bits(b.cache_dtype)
    bs = b.spec.block_size
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        if L == 0:
            continue
        last_end = oracle.blocks_needed(L, bs) * bs
        for t in range(L, last_end):
            slot = oracle.physical_slot(b.block_tables[s], t, bs)
            b.key_cache[slot // bs, slot % bs] = nb
            b.value_cache[slot // bs, slot % bs] = nb

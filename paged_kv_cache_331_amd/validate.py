"""Host-side checks of the preconditions the decode calls leave unchecked.

The kernels validate shapes on the host, but they do not read the tables or
the lengths there (those live on the device, and a step must not
synchronise). include/pa.h lists what a call assumes about them; breaking an
assumption gives undefined output rather than a fault. This module checks
host copies of those arrays, for debugging a caller. It is not used by any
call of the library.

What is checked (the layout of "01. PagedAttention 详解" §3: position t of a
sequence lives in block table[t // bs] at offset t % bs; §6: a block shared
by several tables is copied before it is written):
  * every length lies in [0, max_context_len] and fits the table row;
  * every table entry a sequence uses (its first ceil(L / bs)) is in
    [0, num_blocks);
  * for a write of each sequence's newest token (pa_cache_write after
    pa_decode_slot_mapping, or pa_decode_append): the slots are distinct, and
    the block receiving a new token is used by no other table;
  * for a cascade: the first shared_prefix_blocks entries of every table
    are equal, and a new token lies past the shared prefix.
"""
from __future__ import annotations

from typing import List

import numpy as np


def _host(a) -> np.ndarray:
    if hasattr(a, "detach"):                     # a torch tensor, possibly on the GPU
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def decode_input_problems(block_tables, context_lens, *, max_context_len: int, num_blocks: int,
                          block_size: int, writes_new_token: bool = False,
                          shared_prefix_blocks: int = 0, limit: int = 20) -> List[str]:
    """Every broken precondition found (at most ``limit`` messages), or []."""
    bt = _host(block_tables).astype(np.int64)
    lens = _host(context_lens).astype(np.int64)
    if bt.ndim != 2 or lens.ndim != 1 or bt.shape[0] != lens.shape[0]:
        return [f"block_tables {bt.shape} and context_lens {lens.shape} do not match"]
    B, MB = bt.shape
    bs = int(block_size)
    out: List[str] = []

    def add(msg: str) -> bool:
        out.append(msg)
        return len(out) >= limit

    cap = min(int(max_context_len), MB * bs)
    for s in np.flatnonzero((lens < 0) | (lens > cap)):
        if add(f"sequence {s}: length {lens[s]} outside [0, {cap}]"):
            return out
    L = np.clip(lens, 0, cap)
    used = (L + bs - 1) // bs                      # entries each sequence reads
    cols = np.arange(MB)[None, :]
    mask = cols < used[:, None]
    bad = mask & ((bt < 0) | (bt >= num_blocks))
    for s, j in zip(*np.nonzero(bad)):
        if add(f"sequence {s}: table entry {j} = {bt[s, j]} outside [0, {num_blocks})"):
            return out

    pre = int(shared_prefix_blocks)
    if pre > 0 and B > 0:
        if pre > MB:
            return out + [f"shared_prefix_blocks {pre} exceeds the table width {MB}"]
        diff = np.flatnonzero(np.any(bt[:, :pre] != bt[0:1, :pre], axis=1))
        for s in diff:
            if add(f"sequence {s}: its first {pre} entries differ from sequence 0's"):
                return out

    if writes_new_token:
        live = np.flatnonzero(L > 0)
        pos = L[live] - 1
        blk = bt[live, pos // bs]
        slots = blk * bs + pos % bs
        uniq, counts = np.unique(slots, return_counts=True)
        for v in uniq[counts > 1]:
            who = live[slots == v].tolist()
            if add(f"sequences {who} write the same slot {v}"):
                return out
        # How many tables use each block among their read entries.
        refs = np.bincount(bt[mask].clip(0, max(num_blocks - 1, 0)),
                           minlength=max(num_blocks, 1)) if mask.any() else np.zeros(1, int)
        for i, s in enumerate(live):
            b = int(blk[i])
            if 0 <= b < num_blocks and refs[b] > 1:
                if add(f"sequence {s}: its new token goes into block {b}, which "
                       f"{refs[b] - 1} other table entr{'y' if refs[b] == 2 else 'ies'} "
                       f"also read (copy it first)"):
                    return out
            if pre > 0 and pos[i] < pre * bs:
                if add(f"sequence {s}: its new token (position {pos[i]}) lies inside the "
                       f"shared prefix of {pre * bs} positions"):
                    return out
    return out


def check_decode_inputs(block_tables, context_lens, **kw) -> None:
    """Raise ValueError listing the broken preconditions, if any."""
    problems = decode_input_problems(block_tables, context_lens, **kw)
    if problems:
        raise ValueError("decode inputs break the call's preconditions:\n  " +
                         "\n  ".join(problems))

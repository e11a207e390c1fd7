"""GPU: the persistent schedule of split decode calls.

A split call's work items (kv head, sequence, partition) are taken by a
fixed grid of work-groups. On a workspace whose scheduler word (its first 8
bytes) holds the state a finished call left there, later items come from a
counter; on a fresh workspace (random bytes here) the first call walks them
with a fixed stride. Each item is computed the same way whichever
work-group takes it, so both schedules must give bitwise-equal outputs,
within the oracle bar, and every call must leave the counter at zero.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_331_amd import pa, workloads as wl

from _paged import TOL, Device, max_err, oracle_caches, oracle_decode_one, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pa.load()
    assert torch.cuda.is_available()


SCHED_HEAD_BYTES = 256   # the workspace's leading scheduler words (include/pa.h)


def _random_workspace(nbytes: int, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)


def _counter(ws: torch.Tensor) -> int:
    """The work counter: high half of the little-endian 64-bit scheduler word."""
    return int(ws[4:8].view(torch.int32).item())


def _persistent_expected(b, P: int) -> bool:
    """The library's choice: persistent when the call splits into partitions
    of at least 1024 tokens, at most 8192 (kv head, sequence, partition)
    items, the (sequence, kv head) pairs fill the chip, and the cache is
    2-byte, or FP8 with one query head per kv head."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    spec = b.spec
    if P == 0:
        P = pa.decode_partition_size(b.num_seqs, spec.num_kv_heads, b.max_context_len,
                                     1 if b.cache_dtype == "fp8" else 2)
    if P < 0:
        return False
    parts = -(-b.max_context_len // P)
    group = spec.num_q_heads // spec.num_kv_heads
    return (parts > 1 and P >= 1024 and b.num_seqs * spec.num_kv_heads * parts <= 8192
            and b.num_seqs * spec.num_kv_heads >= cus
            and (b.cache_dtype != "fp8" or group == 1))


def _head_rewritten(ws: torch.Tensor, before: torch.Tensor) -> bool:
    """Only the persistent path's combine writes the tag over the random head."""
    return not torch.equal(ws[:4], before)


def _decode(b, d, ws, P):
    if b.cache_dtype == "fp8":
        out = pa.decode_fp8(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), float(b.k_scale),
                            float(b.v_scale), b.max_context_len, partition_size=P, workspace=ws)
    else:
        out = pa.decode(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), b.max_context_len,
                        partition_size=P, workspace=ws)
    torch.cuda.synchronize()
    return out


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# Batches of at least 256 (sequence, kv head) pairs with 1024-token partitions
# take the persistent schedule (except FP8 GQA); the others check that the
# one-per-item path leaves the workspace head alone.
@pytest.mark.parametrize("name,seqs,P", [
    ("llama2_7b_mha", 8, 1024), ("gqa_8b", 32, 1024), ("llama2_7b_mha_fp8", 8, 1024),
    ("gqa_8b_fp8", 32, 1024), ("llama2_7b_mha", 8, 256), ("long_context_splitk", 1, 512),
    ("tiny_write", 4, 32), ("llama2_7b_mha", 4, 128),
])
def test_workspace_reuse_small_all_outputs(name, seqs, P):
    spec = wl.small_variant(name, seqs)
    b = wl.make_batch(spec)
    kc, vc, _ = oracle_caches(b, False)
    ref = oracle.decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, b.dtype,
                        cache_dtype=b.cache_dtype, k_scale=b.k_scale, v_scale=b.v_scale)
    d = Device(b)
    ws = _random_workspace(pa.decode_workspace_size(b.num_seqs, spec.num_q_heads, spec.head_size,
                                                    b.max_context_len, P), 5)
    head = ws[:8].clone()
    persistent = _persistent_expected(b, P)
    say(f"schedule reuse {name} B={b.num_seqs} P={P} persistent={persistent}")
    outs = [_decode(b, d, ws, P) for _ in range(3)]
    assert _head_rewritten(ws, head[:4]) == persistent
    if persistent:
        assert _counter(ws) == 0
    else:
        assert torch.equal(ws[:8], head)
    assert _same(outs[0], outs[1]) and _same(outs[1], outs[2])
    err = max_err(outs[1], ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[b.dtype]


def test_workspace_shared_by_calls_of_different_shapes():
    """One workspace, sized for the larger call, alternates between two batches
    of different sizes and partition counts; every output matches its first
    (fixed-stride) run and the oracle."""
    b1 = wl.make_batch(wl.small_variant("gqa_8b", 40))
    b2 = wl.make_batch(wl.small_variant("llama2_7b_mha", 9))
    P1, P2 = 1024, 1024
    assert _persistent_expected(b1, P1) and _persistent_expected(b2, P2)
    n = max(pa.decode_workspace_size(b.num_seqs, b.spec.num_q_heads, b.spec.head_size,
                                     b.max_context_len, P)
            for b, P in ((b1, P1), (b2, P2)))
    ws = _random_workspace(n, 9)
    d1, d2 = Device(b1), Device(b2)
    first = {}
    for rnd in range(3):
        for key, b, d, P in (("a", b1, d1, P1), ("b", b2, d2, P2)):
            out = _decode(b, d, ws, P)
            assert _counter(ws) == 0
            if key in first:
                assert _same(out, first[key]), (rnd, key)
            else:
                first[key] = out
    for key, b in (("a", b1), ("b", b2)):
        ref = oracle.decode(b.q, b.key_cache, b.value_cache, b.block_tables, b.context_lens,
                            b.scale, b.dtype)
        assert max_err(first[key], ref) <= TOL[b.dtype]


def test_cascade_workspace_reuse():
    """Suffixes of up to 2500 tokens in 1024-token partitions, one workspace of
    random bytes reused: the one-launch cascade runs its suffix items one
    work-group per item beside the prefix work-groups, so it leaves the
    scheduler words as it found them, and every call gives the same output."""
    spec = dataclasses.replace(wl.CONFIGS["prefix_shared_write"], num_seqs=32, len_hi=2500)
    b = wl.make_batch(spec)
    d = Device(b)
    pfx = spec.shared_prefix_blocks
    P = 1024
    n = pa.decode_cascade_workspace_size(b.num_seqs, spec.num_q_heads, spec.head_size,
                                         spec.block_size, b.max_context_len, pfx, P)
    ws = _random_workspace(n, 11)
    words = ws[:SCHED_HEAD_BYTES].clone()
    say(f"schedule reuse cascade B={b.num_seqs} prefix_blocks={pfx}")
    outs = []
    for _ in range(3):
        outs.append(pa.decode_cascade(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale),
                                      b.max_context_len, pfx, partition_size=P, workspace=ws))
        torch.cuda.synchronize()
    assert torch.equal(ws[:SCHED_HEAD_BYTES], words)
    assert _same(outs[0], outs[1]) and _same(outs[1], outs[2])
    ref = oracle.decode(b.q, b.key_cache, b.value_cache, b.block_tables, b.context_lens, b.scale,
                        b.dtype)
    assert max_err(outs[2], ref) <= TOL[b.dtype]


def test_concurrent_calls_on_two_streams():
    """Two persistent-grid calls in flight at once on two streams, each with
    its own workspace (the rule for concurrent calls): both match their
    results from one stream, several times over."""
    b1 = wl.make_batch(wl.small_variant("gqa_8b", 40))
    b2 = wl.make_batch(wl.small_variant("llama2_7b_mha", 9))
    P = 1024
    assert _persistent_expected(b1, P) and _persistent_expected(b2, P)
    d1, d2 = Device(b1), Device(b2)
    ws = [_random_workspace(pa.decode_workspace_size(b.num_seqs, b.spec.num_q_heads,
                                                     b.spec.head_size, b.max_context_len, P), 21 + i)
          for i, b in enumerate((b1, b2))]
    ref1, ref2 = _decode(b1, d1, ws[0], P), _decode(b2, d2, ws[1], P)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            o1 = pa.decode(d1.q, d1.kc, d1.vc, d1.bt, d1.lens, float(b1.scale), b1.max_context_len,
                           partition_size=P, workspace=ws[0])
        with torch.cuda.stream(s2):
            o2 = pa.decode(d2.q, d2.kc, d2.vc, d2.bt, d2.lens, float(b2.scale), b2.max_context_len,
                           partition_size=P, workspace=ws[1])
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert _same(o1, ref1) and _same(o2, ref2)
    assert _counter(ws[0]) == 0 and _counter(ws[1]) == 0


def _done_count(ws: torch.Tensor) -> int:
    """The finish count of a counted walk, 32 bits at byte offset 128."""
    return int(ws[128:132].view(torch.int32).item())


@pytest.mark.parametrize("name", ["llama2_7b_mha", "llama2_7b_mha_fp8"])
def test_append_new_token_only_partitions_both_schedules(name):
    """Fused append on the persistent grid with lengths L = 1 (mod 1024), so
    that some items' partitions hold only the new token and skip the table
    loop (and its barriers). The first call on a random workspace walks the
    items with the fixed stride, the next ones draw tickets: every call must
    equal the oracle (whole pools bitwise, every output within the bar) and
    the calls must be bitwise equal to each other."""
    lens = [1025, 2049, 1, 1024, 1026, 2048, 1537, 1025]
    spec = wl.small_variant(name, len(lens))
    b = wl.make_batch(spec, lengths=lens)
    P = 1024
    assert _persistent_expected(b, P)
    kc_ref, vc_ref, slots_ref = oracle_caches(b, True)
    ref = oracle.decode(b.q, kc_ref, vc_ref, b.block_tables, b.context_lens, b.scale, b.dtype,
                        cache_dtype=b.cache_dtype, k_scale=b.k_scale, v_scale=b.v_scale)
    d = Device(b)
    n = pa.decode_workspace_size(b.num_seqs, spec.num_q_heads, spec.head_size,
                                 b.max_context_len, P)
    ws = _random_workspace(n, 31)
    fp8 = b.cache_dtype == "fp8"
    say(f"append schedules {name} lens={lens} P={P}")
    outs = []
    for _ in range(3):
        slots = torch.full((b.num_seqs,), 12345, dtype=torch.int32, device="cuda")
        if fp8:
            out = pa.decode_append_fp8(d.q, d.k_new, d.v_new, d.kc, d.vc, d.bt, d.lens,
                                       float(b.scale), float(b.k_scale), float(b.v_scale),
                                       b.max_context_len, slot_mapping=slots, partition_size=P,
                                       workspace=ws)
        else:
            out = pa.decode_append(d.q, d.k_new, d.v_new, d.kc, d.vc, d.bt, d.lens,
                                   float(b.scale), b.max_context_len, 0, slot_mapping=slots,
                                   partition_size=P, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(slots.cpu().numpy(), slots_ref)
        assert _counter(ws) == 0 and _done_count(ws) == 0
        outs.append(out)
    down = (lambda t: t.cpu().numpy()) if fp8 else (
        lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(down(d.kc), kc_ref) and np.array_equal(down(d.vc), vc_ref)
    assert _same(outs[0], outs[1]) and _same(outs[1], outs[2])
    err = max_err(outs[0], ref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[b.dtype]

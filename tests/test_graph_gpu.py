"""GPU: the hot path captured in a HIP graph and replayed.

A decode step (slot of the new token, cache write, attention; as three calls
and as one pa_decode_append call) and a prefill step are captured once
through torch.cuda.graph and replayed several times,
with unrelated eager work and synchronisations between the replays. Every
replay must give the eager result bitwise. The library enqueues kernels only
(no memset, no allocation, no host synchronisation), and the persistent
decode grid's scheduler word is carried from call to call by kernel writes,
so replays see the same state as eager calls.
"""
import dataclasses

import pytest
import torch

from paged_kv_cache_331_amd import pa, workloads as wl

from _paged import Device, say
from test_prefill_gpu import Dev as PrefillDev

pytestmark = pytest.mark.gpu

REPLAYS = 5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pa.load()
    assert torch.cuda.is_available()


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _eager_noise():
    x = torch.randn(1 << 20, device="cuda")
    return float((x * 2).sum().item())


def _decode_step(b, d, out, slots, ws, P, cascade, append=False):
    bs = b.spec.block_size
    if append:
        if b.cache_dtype == "fp8":
            pa.decode_append_fp8(d.q, d.k_new, d.v_new, d.kc, d.vc, d.bt, d.lens, float(b.scale),
                                 float(b.k_scale), float(b.v_scale), b.max_context_len, out=out,
                                 slot_mapping=slots, partition_size=P, workspace=ws)
        else:
            pa.decode_append(d.q, d.k_new, d.v_new, d.kc, d.vc, d.bt, d.lens, float(b.scale),
                             b.max_context_len, b.spec.shared_prefix_blocks if cascade else 0,
                             out=out, slot_mapping=slots, partition_size=P, workspace=ws)
        return
    pa.decode_slot_mapping(d.bt, d.lens, bs, out=slots)
    if b.cache_dtype == "fp8":
        pa.cache_write_fp8(d.k_new, d.v_new, d.kc, d.vc, slots, float(b.k_scale),
                           float(b.v_scale))
        pa.decode_fp8(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), float(b.k_scale),
                      float(b.v_scale), b.max_context_len, out=out, partition_size=P,
                      workspace=ws)
    elif cascade:
        pa.cache_write(d.k_new, d.v_new, d.kc, d.vc, slots)
        pa.decode_cascade(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), b.max_context_len,
                          b.spec.shared_prefix_blocks, out=out, partition_size=P, workspace=ws)
    else:
        pa.cache_write(d.k_new, d.v_new, d.kc, d.vc, slots)
        pa.decode(d.q, d.kc, d.vc, d.bt, d.lens, float(b.scale), b.max_context_len, out=out,
                  partition_size=P, workspace=ws)


CASES = [
    ("mha_persistent", dataclasses.replace(wl.CONFIGS["llama2_7b_mha"], num_seqs=8), 1024, False,
     False),
    ("gqa", wl.small_variant("gqa_8b", 32), 0, False, False),
    ("fp8_mha", dataclasses.replace(wl.CONFIGS["llama2_7b_mha_fp8"], num_seqs=8), 1024, False,
     False),
    ("cascade", dataclasses.replace(wl.CONFIGS["prefix_shared_write"], num_seqs=32, len_hi=2500),
     1024, True, False),
    ("append_mha_persistent", dataclasses.replace(wl.CONFIGS["llama2_7b_mha"], num_seqs=8), 1024,
     False, True),
    ("append_gqa", wl.small_variant("gqa_8b", 32), 0, False, True),
    ("append_fp8_gqa", wl.small_variant("gqa_8b_fp8", 32), 0, False, True),
    ("append_cascade", dataclasses.replace(wl.CONFIGS["prefix_shared_write"], num_seqs=32,
                                           len_hi=2500), 1024, True, True),
]


@pytest.mark.parametrize("name,spec,P,cascade,append", CASES, ids=[c[0] for c in CASES])
def test_decode_step_graph_replays(name, spec, P, cascade, append):
    b = wl.make_batch(spec)
    d = Device(b)
    Hq, D = spec.num_q_heads, spec.head_size
    if cascade:
        n = pa.decode_cascade_workspace_size(b.num_seqs, Hq, D, spec.block_size,
                                             b.max_context_len, spec.shared_prefix_blocks, P)
    else:
        n = pa.decode_workspace_size(b.num_seqs, Hq, D, b.max_context_len, P)
    ws = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d.q)
    slots = torch.empty(b.num_seqs, dtype=torch.int32, device="cuda")
    say(f"graph decode step {name} B={b.num_seqs} P={P}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            _decode_step(b, d, out, slots, ws, P, cascade, append)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    ref_k = d.kc.clone()
    ref_v = d.vc.clone()
    ref_slots = slots.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode_step(b, d, out, slots, ws, P, cascade, append)
    for r in range(REPLAYS):
        out.fill_(0)
        slots.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref), f"replay {r}"
        assert _same(d.kc, ref_k) and _same(d.vc, ref_v)
        assert torch.equal(slots, ref_slots)
        _eager_noise()
        torch.cuda.synchronize()


def test_prefill_step_graph_replays():
    b = wl.make_prefill_batch(wl.PREFILL_CONFIGS["gqa_8b_chunked_prefill"], ctx=[100, 0, 700, 33],
                              new=[40, 130, 65, 1])
    d = PrefillDev(b)
    out = torch.empty_like(d.q)
    slots = torch.empty(b.num_tokens, dtype=torch.int32, device="cuda")
    bs = b.spec.block_size

    def step():
        pa.prefill_slot_mapping(d.bt, d.lens, d.qs, b.num_tokens, b.max_query_len, bs,
                                b.max_context_len, out=slots)
        pa.cache_write(d.k_new, d.v_new, d.kc, d.vc, slots)
        pa.prefill(d.q, d.kc, d.vc, d.bt, d.lens, d.qs, float(b.scale), b.max_query_len,
                   b.max_context_len, out=out)

    say(f"graph prefill step T={b.num_tokens}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref), f"replay {r}"
        _eager_noise()
        torch.cuda.synchronize()

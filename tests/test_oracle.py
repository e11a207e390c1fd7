"""Pins of the fp64 oracle against facts outside itself (CPU only).

Each pin is a function of the decode callable, so the same pin can also be
run against deliberately broken variants ("planted mistakes" at the bottom)
to show it would catch that mistake.

Independent references used here: explicit Python loops plus
``scipy.special.softmax`` (brute force), ``torch``'s float64 CPU
``scaled_dot_product_attention`` on contiguous K/V, closed forms, and the
worked examples printed in "01. PagedAttention 详解" (vLLM learning book).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from oracle import paged_attention as opa
from paged_kv_cache_331_amd import workloads as wl

from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers

def _torch_upcast(bits, dtype):
    """Upcast with torch's own dtype views (independent of the oracle's)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.to(torch.float64).numpy()


def _random_case(rng, B, Hkv, G, D, bs, lens, dtype="fp16", spare=3):
    """Tiny batch with a shuffled pool; returns the pieces as a dict."""
    nblk = [(L + bs - 1) // bs for L in lens]
    NB = sum(nblk) + spare
    MB = max(max(nblk), 1)
    perm = rng.permutation(NB)
    tables = np.full((B, MB), perm[-1], dtype=np.int32)
    c = 0
    for s in range(B):
        tables[s, :nblk[s]] = perm[c:c + nblk[s]]
        c += nblk[s]
    Hq = Hkv * G
    f = lambda *shape: wl.round_to_storage(rng.standard_normal(shape).astype(np.float32), dtype)
    return dict(q=f(B, Hq, D), key_cache=f(NB, bs, Hkv, D), value_cache=f(NB, bs, Hkv, D),
                block_tables=tables, context_lens=np.asarray(lens, np.int32),
                scale=np.float32(1.0 / math.sqrt(D)), dtype=dtype)


def _call(decode_fn, c, **over):
    a = dict(c)
    a.update(over)
    return decode_fn(a["q"], a["key_cache"], a["value_cache"], a["block_tables"],
                     a["context_lens"], a["scale"], a["dtype"])


def _bruteforce(c):
    """Explicit loops over tokens, flat-slot addressing, scipy softmax."""
    q = _torch_upcast(c["q"], c["dtype"])
    kc = _torch_upcast(c["key_cache"], c["dtype"])
    vc = _torch_upcast(c["value_cache"], c["dtype"])
    NB, bs, Hkv, D = kc.shape
    kflat = kc.reshape(NB * bs, Hkv, D)
    vflat = vc.reshape(NB * bs, Hkv, D)
    B, Hq, _ = q.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for s in range(B):
        L = int(c["context_lens"][s])
        for h in range(Hq):
            g = h // G
            Ks, Vs = [], []
            for t in range(L):
                slot = int(c["block_tables"][s][t // bs]) * bs + (t % bs)
                Ks.append(kflat[slot, g])
                Vs.append(vflat[slot, g])
            if L == 0:
                continue
            K = np.array(Ks)
            V = np.array(Vs)
            p = scipy.special.softmax(float(c["scale"]) * (K @ q[s, h]))
            out[s, h] = p @ V
    return out


# ------------------------------------------------------------------- pins

def pin_bruteforce(decode_fn, seed=0):
    """P1: equals brute-force attention on several tiny random cases."""
    rng = np.random.default_rng(seed)
    ok = True
    for (B, Hkv, G, D, bs, dtype) in [(3, 2, 2, 8, 4, "fp16"), (2, 1, 4, 4, 2, "bf16"),
                                      (2, 2, 1, 8, 16, "fp16"), (1, 2, 2, 4, 4, "bf16")]:
        lens = rng.integers(1, 40, size=B).tolist()
        c = _random_case(rng, B, Hkv, G, D, bs, lens, dtype)
        ok &= np.allclose(_call(decode_fn, c), _bruteforce(c), rtol=0, atol=1e-13)
    return ok


def pin_single_token(decode_fn):
    """P2: with L = 1 the output is the single cached value row, exactly."""
    rng = np.random.default_rng(1)
    c = _random_case(rng, 3, 2, 2, 8, 4, [1, 1, 1])
    out = _call(decode_fn, c)
    ok = True
    for s in range(3):
        for h in range(4):
            v = _torch_upcast(c["value_cache"][c["block_tables"][s, 0], 0, h // 2], "fp16")
            ok &= np.array_equal(out[s, h], v)
    return ok


def pin_uniform(decode_fn):
    """P3: q = 0 gives equal weights, so the output is the mean value row."""
    rng = np.random.default_rng(2)
    c = _random_case(rng, 2, 2, 2, 8, 4, [7, 13])
    c["q"] = np.zeros_like(c["q"])
    out = _call(decode_fn, c)
    ok = True
    kvf = _torch_upcast(c["value_cache"], "fp16")
    for s in range(2):
        L = int(c["context_lens"][s])
        for h in range(4):
            rows = [kvf[c["block_tables"][s][t // 4], t % 4, h // 2] for t in range(L)]
            ok &= np.allclose(out[s, h], np.mean(rows, axis=0), rtol=0, atol=1e-14)
    return ok


def pin_hardmax(decode_fn):
    """P4: a huge scale turns softmax into argmax."""
    rng = np.random.default_rng(3)
    c = _random_case(rng, 2, 1, 2, 8, 4, [11, 9])
    c["scale"] = np.float32(1e4)
    out = _call(decode_fn, c)
    q = _torch_upcast(c["q"], "fp16")
    kf = _torch_upcast(c["key_cache"], "fp16")
    vf = _torch_upcast(c["value_cache"], "fp16")
    ok = True
    for s in range(2):
        L = int(c["context_lens"][s])
        for h in range(2):
            rows = [(c["block_tables"][s][t // 4], t % 4) for t in range(L)]
            dots = np.array([kf[b, o, 0] @ q[s, h] for b, o in rows])
            order = np.sort(dots)
            assert order[-1] - order[-2] > 1e-3  # the seed gives a clear winner
            b, o = rows[int(np.argmax(dots))]
            ok &= np.allclose(out[s, h], vf[b, o, 0], rtol=0, atol=1e-12)
    return ok


def pin_permutation(decode_fn):
    """P6: relabelling physical blocks (moving the pool rows and rewriting the tables)
    leaves the output bitwise unchanged."""
    rng = np.random.default_rng(4)
    c = _random_case(rng, 3, 2, 2, 8, 4, [5, 16, 23], spare=5)
    NB = c["key_cache"].shape[0]
    pi = rng.permutation(NB)                     # old id b moves to new id pi[b]
    kc = np.empty_like(c["key_cache"])
    vc = np.empty_like(c["value_cache"])
    kc[pi] = c["key_cache"]
    vc[pi] = c["value_cache"]
    bt = pi[c["block_tables"]].astype(np.int32)
    a = _call(decode_fn, c)
    b = _call(decode_fn, c, key_cache=kc, value_cache=vc, block_tables=bt)
    return np.array_equal(a, b)


def pin_contiguous(decode_fn):
    """P7: an identity table over a contiguous region equals ordinary attention
    (torch float64 scaled_dot_product_attention) on that region."""
    rng = np.random.default_rng(5)
    B, Hkv, G, D, bs = 2, 2, 2, 8, 4
    lens = [10, 16]
    nblk = [3, 4]
    c = _random_case(rng, B, Hkv, G, D, bs, lens)
    NB = c["key_cache"].shape[0]
    bt = np.zeros((B, 4), np.int32)
    bt[0, :3] = [0, 1, 2]
    bt[1, :4] = [3, 4, 5, 6]
    c["block_tables"] = bt
    out = _call(decode_fn, c)
    q = torch.from_numpy(_torch_upcast(c["q"], "fp16"))
    kf = torch.from_numpy(_torch_upcast(c["key_cache"], "fp16")).reshape(NB * bs, Hkv, D)
    vf = torch.from_numpy(_torch_upcast(c["value_cache"], "fp16")).reshape(NB * bs, Hkv, D)
    ok = True
    starts = [0, 3 * bs]
    for s in range(B):
        L = lens[s]
        K = kf[starts[s]:starts[s] + L].permute(1, 0, 2)          # [Hkv, L, D]
        V = vf[starts[s]:starts[s] + L].permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[s][:, None, :], K, V, scale=float(c["scale"]))[:, 0, :]
        ok &= np.allclose(out[s], ref.numpy(), rtol=0, atol=1e-13)
    return ok


def pin_sharing(decode_fn):
    """P8: the book's §6 sharing figure. B = [42, 17, 88] shares blocks 42 and
    17 with A = [42, 17, 99]; copying the shared blocks into private blocks
    (03 and 55, the spare blocks of the §3 figure) changes nothing."""
    fig = _golden("book_sharing_figure.json")
    bs = fig["block_size"]
    rng = np.random.default_rng(6)
    NB, Hkv, D = 100, 2, 8
    f = lambda *shape: wl.round_to_storage(rng.standard_normal(shape).astype(np.float32), "fp16")
    kc, vc, q = f(NB, bs, Hkv, D), f(NB, bs, Hkv, D), f(2, 4, D)
    bt = np.array([fig["tables"]["A"], fig["tables"]["B"]], np.int32)
    lens = np.array([48, 40], np.int32)
    sc = np.float32(1 / math.sqrt(D))
    shared = decode_fn(q, kc, vc, bt, lens, sc, "fp16")
    kc2, vc2 = kc.copy(), vc.copy()
    for src, dst in [(42, 3), (17, 55)]:
        kc2[dst] = kc[src]
        vc2[dst] = vc[src]
    bt2 = bt.copy()
    bt2[1, :2] = [3, 55]
    private = decode_fn(q, kc2, vc2, bt2, lens, sc, "fp16")
    return np.array_equal(shared, private)


def pin_gqa(decode_fn):
    """P9: GQA equals MHA after repeating each kv head for its query group."""
    rng = np.random.default_rng(7)
    c = _random_case(rng, 2, 2, 4, 8, 4, [9, 14], dtype="bf16")
    out = _call(decode_fn, c)
    kc = np.repeat(c["key_cache"], 4, axis=2)
    vc = np.repeat(c["value_cache"], 4, axis=2)
    mha = _call(decode_fn, c, key_cache=kc, value_cache=vc)
    return np.allclose(out, mha, rtol=0, atol=1e-15)


ALL_DECODE_PINS = [pin_bruteforce, pin_single_token, pin_uniform, pin_hardmax,
                   pin_permutation, pin_contiguous, pin_sharing, pin_gqa]


@pytest.mark.parametrize("pin", ALL_DECODE_PINS, ids=lambda p: p.__name__)
def test_oracle_decode_pins(pin):
    assert pin(oracle.decode)


# ------------------------------------------------------ hypothesis sweep

@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.data())
def test_oracle_matches_bruteforce_hypothesis(data):
    B = data.draw(st.integers(1, 4))
    bs = data.draw(st.sampled_from([2, 4, 16]))
    D = data.draw(st.sampled_from([4, 8, 64]))
    G = data.draw(st.sampled_from([1, 2, 4]))
    Hkv = data.draw(st.integers(1, 2))
    dtype = data.draw(st.sampled_from(["fp16", "bf16"]))
    lens = data.draw(st.lists(st.integers(0, 70), min_size=B, max_size=B))
    seed = data.draw(st.integers(0, 2**31))
    c = _random_case(np.random.default_rng(seed), B, Hkv, G, D, bs, lens, dtype)
    assert np.allclose(_call(oracle.decode, c), _bruteforce(c), rtol=0, atol=1e-13)


# --------------------------------------------------------- other pins

def test_zero_length_gives_zero():
    """L = 0: the wiki's §5.3.4 sketch returns its zeros_like(query) start."""
    rng = np.random.default_rng(8)
    c = _random_case(rng, 2, 1, 2, 8, 4, [0, 5])
    out = _call(oracle.decode, c)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_weights_sum_to_one(name):
    """P5: softmax weights sum to 1 for every (sequence, head) -- small draws of each workload."""
    spec = wl.small_variant(name, 2)
    b = wl.make_batch(spec)
    for s in range(b.num_seqs):
        for h in range(spec.num_q_heads):
            p = oracle.attention_weights(b.q, b.key_cache, b.value_cache, b.block_tables,
                                         b.context_lens, b.scale, b.dtype, s, h)
            assert p.shape == (int(b.context_lens[s]),)
            assert abs(p.sum() - 1.0) <= 1e-14 and np.all(p >= 0)


def _bruteforce_weights(c, s, h):
    """Weights of one (sequence, head) by explicit loops over tokens, flat-slot
    addressing and scipy's softmax (independent of the oracle's gather)."""
    q = _torch_upcast(c["q"], c["dtype"])
    kc = _torch_upcast(c["key_cache"], c["dtype"])
    NB, bs, Hkv, D = kc.shape
    kflat = kc.reshape(NB * bs, Hkv, D)
    g = h // (q.shape[1] // Hkv)
    L = int(c["context_lens"][s])
    logits = []
    for t in range(L):
        slot = int(c["block_tables"][s][t // bs]) * bs + (t % bs)
        logits.append(float(c["scale"]) * float(kflat[slot, g] @ q[s, h]))
    return scipy.special.softmax(np.array(logits))


def pin_weights_bruteforce(weights_fn, seed=5):
    """P5b: the weights equal brute-force softmax weights, position by position,
    and weights @ (brute-force gathered V) is the brute-force output row."""
    rng = np.random.default_rng(seed)
    ok = True
    for (B, Hkv, G, D, bs, dtype) in [(3, 2, 2, 8, 4, "fp16"), (2, 1, 4, 4, 2, "bf16"),
                                      (2, 2, 1, 8, 16, "fp16"), (2, 2, 4, 8, 4, "bf16")]:
        lens = rng.integers(1, 40, size=B).tolist()
        c = _random_case(rng, B, Hkv, G, D, bs, lens, dtype)
        bf_out = _bruteforce(c)
        vc = _torch_upcast(c["value_cache"], c["dtype"])
        vflat = vc.reshape(-1, Hkv, D)
        for s in range(B):
            for h in range(Hkv * G):
                p = weights_fn(c["q"], c["key_cache"], c["value_cache"], c["block_tables"],
                               c["context_lens"], c["scale"], c["dtype"], s, h)
                ref = _bruteforce_weights(c, s, h)
                if p.shape != ref.shape or not np.allclose(p, ref, rtol=0, atol=1e-15):
                    return False
                L = int(c["context_lens"][s])
                V = np.array([vflat[int(c["block_tables"][s][t // bs]) * bs + t % bs, h // G]
                              for t in range(L)])
                ok &= np.allclose(p @ V, bf_out[s, h], rtol=0, atol=1e-13)
    return ok


def test_weights_match_bruteforce():
    assert pin_weights_bruteforce(oracle.attention_weights)


def test_weights_are_decodes_weights():
    """weights @ V of the oracle's own gather is the oracle's decode row (both
    come from one computation), on a small draw of every workload shape."""
    for name in wl.CONFIG_ORDER:
        b = wl.make_batch(wl.small_variant(name, 2))
        ref = oracle.decode(b.q, b.key_cache, b.value_cache, b.block_tables, b.context_lens,
                            b.scale, b.dtype)
        G = b.spec.num_q_heads // b.spec.num_kv_heads
        for s in range(b.num_seqs):
            for h in (0, b.spec.num_q_heads - 1):
                p = oracle.attention_weights(b.q, b.key_cache, b.value_cache, b.block_tables,
                                             b.context_lens, b.scale, b.dtype, s, h)
                V = opa.gather_positions(b.value_cache, b.block_tables[s],
                                         int(b.context_lens[s]), h // G, b.dtype)
                assert np.array_equal(p @ V, ref[s, h])


def _weights_mutant_head_map(q, kc, vc, bt, lens, scale, dtype, s, h):
    Hkv = kc.shape[2]
    G = q.shape[1] // Hkv
    # query head h read kv head h % Hkv instead of h // G: swap to the head of that map
    h2 = (h % Hkv) * G + (h // Hkv) % G
    p = oracle.attention_weights(q[:, [h] * q.shape[1]], kc, vc, bt, lens, scale, dtype, s, h2)
    return p


@pytest.mark.parametrize("name", ["no_scale", "swapped_block_offset", "off_by_one_length",
                                  "no_normalisation", "logit_sign", "wrong_gqa_head_map"])
def test_weights_pin_catches_planted_mistake(name, monkeypatch):
    """Each planted mistake, placed where the weights are computed, fails P5b."""
    if name == "wrong_gqa_head_map":
        fn = _weights_mutant_head_map
    else:
        MUTANTS[name](monkeypatch)
        fn = opa.attention_weights
    assert not pin_weights_bruteforce(fn)


def test_book_figure_slots():
    """P10: the book's §3 figure -- tokens 0..15 in block 42, 16..31 in 17, 32..47 in 99."""
    fig = _golden("book_block_table_figure.json")
    bs = fig["block_size"]
    row = np.array(fig["table"], np.int32)
    for lo, hi, phys in fig["token_ranges"]:
        for t in range(lo, hi + 1):
            slot = oracle.physical_slot(row, t, bs)
            assert slot // bs == phys and slot % bs == t - lo
    # the newest token of a 48-token request sits in the last slot of block 99
    sm = oracle.slot_mapping(row[None, :], np.array([48], np.int32), bs)
    assert sm[0] == 99 * bs + 15
    # and a 33-token request writes its newest token at the first slot of block 99
    sm = oracle.slot_mapping(row[None, :], np.array([33], np.int32), bs)
    assert sm[0] == 99 * bs + 0
    assert oracle.slot_mapping(row[None, :], np.array([0], np.int32), bs)[0] == -1


def test_book_table_size_arithmetic():
    """P11: the book's self-check Q2 -- a 100k-token request at block size 16 needs
    6250 int32 entries, 25000 bytes; 100001 tokens need one more."""
    g = _golden("book_size_arithmetic.json")
    n = oracle.blocks_needed(g["tokens"], g["block_size"])
    assert n == g["table_entries"]
    assert n * g["table_entry_bytes"] == g["table_bytes"]
    assert oracle.blocks_needed(g["tokens"] + 1, g["block_size"]) == n + 1
    # a table of exactly 6250 entries serves the newest token of a 100k request
    row = np.arange(n, dtype=np.int32)
    assert oracle.slot_mapping(row[None], np.array([g["tokens"]], np.int32), 16)[0] == g["tokens"] - 1


def test_write_round_trip_and_nothing_else_changes():
    """P13: writing at the newest slot then gathering position L-1 returns k, v
    bitwise, and no other element of either pool changes."""
    rng = np.random.default_rng(9)
    c = _random_case(rng, 4, 2, 1, 8, 4, [1, 4, 5, 17])
    kn = wl.round_to_storage(rng.standard_normal((4, 2, 8)).astype(np.float32), "fp16")
    vn = wl.round_to_storage(rng.standard_normal((4, 2, 8)).astype(np.float32), "fp16")
    slots = oracle.slot_mapping(c["block_tables"], c["context_lens"], 4)
    kc, vc = oracle.cache_write(c["key_cache"], c["value_cache"], kn, vn, slots)
    for s in range(4):
        L = int(c["context_lens"][s])
        for g in range(2):
            got_k = oracle.gather_positions(kc, c["block_tables"][s], L, g, "fp16")[L - 1]
            got_v = oracle.gather_positions(vc, c["block_tables"][s], L, g, "fp16")[L - 1]
            assert np.array_equal(got_k, _torch_upcast(kn[s, g], "fp16"))
            assert np.array_equal(got_v, _torch_upcast(vn[s, g], "fp16"))
    changed = np.argwhere(np.any(kc != c["key_cache"], axis=(2, 3)))
    flat = sorted(int(b) * 4 + int(o) for b, o in changed)
    assert flat == sorted(int(x) for x in slots)
    # a negative slot writes nothing
    kc2, _ = oracle.cache_write(c["key_cache"], c["value_cache"], kn, vn,
                                np.array([-1, -1, -1, -1], np.int32))
    assert np.array_equal(kc2, c["key_cache"])


@pytest.mark.parametrize("P", [1, 3, 4, 16, 512])
def test_split_partition_identity(P):
    """P14: the partition-and-combine algebra reproduces the unsplit result."""
    rng = np.random.default_rng(10)
    c = _random_case(rng, 3, 2, 2, 8, 4, [1, 37, 70])
    a = _call(oracle.decode, c)
    b = oracle.decode_partitioned(c["q"], c["key_cache"], c["value_cache"], c["block_tables"],
                                  c["context_lens"], c["scale"], "fp16", P)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_decode_one_matches_decode():
    b = wl.make_batch(wl.small_variant("gqa_8b", 3))
    full = oracle.decode(b.q, b.key_cache, b.value_cache, b.block_tables, b.context_lens,
                         b.scale, b.dtype)
    for s, h in [(0, 0), (1, 7), (2, 31)]:
        one = oracle.decode_one(b.q, b.key_cache, b.value_cache, b.block_tables,
                                b.context_lens, b.scale, b.dtype, s, h)
        assert np.array_equal(one, full[s, h])


def test_upcast_exact():
    """Storage upcast: a few bit patterns with known values."""
    assert oracle.to_float64(np.array([0x3C00, 0xC000, 0x0001], np.uint16), "fp16").tolist() == \
        [1.0, -2.0, 2.0 ** -24]
    assert oracle.to_float64(np.array([0x3F80, 0xC040, 0x0001], np.uint16), "bf16").tolist() == \
        [1.0, -3.0, 2.0 ** -133]


# ----------------------------------------------------- planted mistakes

def _mutant_no_scale(monkeypatch):
    orig = opa._softmax_attend
    monkeypatch.setattr(opa, "_softmax_attend", lambda q, K, V, scale: orig(q, K, V, 1.0))


def _mutant_swapped_index(monkeypatch):
    def gather(cache, row, length, kv_head, dtype, scale=1.0):
        bs = cache.shape[1]
        t = np.arange(int(length))
        # block and offset roles exchanged (a transposed operand of the indirection)
        blk = np.asarray(row, np.int64)[np.minimum(t % bs, len(row) - 1)]
        return opa.to_float64(cache[blk, np.minimum(t // bs, bs - 1), kv_head, :], dtype)
    monkeypatch.setattr(opa, "gather_positions", gather)


def _mutant_off_by_one(monkeypatch):
    orig = opa.gather_positions
    monkeypatch.setattr(opa, "gather_positions",
                        lambda cache, row, length, g, dt, sc=1.0: orig(cache, row, max(length - 1, 1),
                                                                       g, dt, sc))


def _mutant_no_normalise(monkeypatch):
    def attend(q, K, V, scale):
        logits = scale * (K @ q)
        w = np.exp(logits - logits.max())
        return w @ V, w
    monkeypatch.setattr(opa, "_softmax_attend", attend)


def _mutant_no_max_shift_sign(monkeypatch):
    def attend(q, K, V, scale):
        logits = -scale * (K @ q)       # sign error on the logit
        w = np.exp(logits - logits.max())
        p = w / w.sum()
        return p @ V, p
    monkeypatch.setattr(opa, "_softmax_attend", attend)


def _mutant_wrong_head_map(monkeypatch):
    orig = opa.decode

    def decode(q, kc, vc, bt, lens, scale, dtype, seqs=None):
        Hq, Hkv = q.shape[1], kc.shape[2]
        G = Hq // Hkv
        # query head h read kv head h % Hkv instead of h // G
        order = [(h % Hkv) * G + (h // Hkv) for h in range(Hq)]
        out = orig(q[:, order], kc, vc, bt, lens, scale, dtype, seqs)
        inv = np.argsort(order)
        return out[:, inv]
    return decode


MUTANTS = {
    "no_scale": _mutant_no_scale,
    "swapped_block_offset": _mutant_swapped_index,
    "off_by_one_length": _mutant_off_by_one,
    "no_normalisation": _mutant_no_normalise,
    "logit_sign": _mutant_no_max_shift_sign,
    "wrong_gqa_head_map": _mutant_wrong_head_map,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    fn = MUTANTS[name](monkeypatch)
    decode_fn = fn if fn is not None else opa.decode
    failed = [p.__name__ for p in ALL_DECODE_PINS if not p(decode_fn)]
    assert failed, f"no pin caught the planted mistake {name}"



@pytest.mark.parametrize("prefix_blocks", [1, 2, 3])
def test_two_level_prefix_identity(prefix_blocks):
    """The shared-prefix reformulation equals the plain definition, including
    sequences shorter than the prefix and an empty one."""
    spec = wl.WorkloadSpec(name="pfx", num_seqs=5, num_q_heads=4, num_kv_heads=2, head_size=16,
                           block_size=16, dtype="fp16", lengths="uniform", len_lo=1, len_hi=40,
                           shared_prefix_blocks=prefix_blocks, seed_index=77)
    b = wl.make_batch(spec)
    pfx = prefix_blocks * 16
    lens = b.context_lens.copy()
    lens[0], lens[1], lens[2] = 0, max(1, pfx // 2), pfx
    assert np.all(b.block_tables[:, :prefix_blocks] == b.block_tables[0, :prefix_blocks])
    ref = oracle.decode(b.q, b.key_cache, b.value_cache, b.block_tables, lens, b.scale, b.dtype)
    got = oracle.decode_two_level(b.q, b.key_cache, b.value_cache, b.block_tables, lens, b.scale,
                                  b.dtype, pfx)
    assert np.max(np.abs(got - ref)) <= 1e-12
    assert np.all(got[0] == 0)

"""Host-side logic of bench.py (CPU): the algorithmic byte count and the
one-GPU guard."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from paged_kv_cache_331_amd import workloads as wl

from conftest import GOLDEN, ROOT


def test_bytes_per_token_match_book_arithmetic():
    """The book's self-check Q2: hidden size 4096 in fp16 holds 16384 bytes of
    K+V per token per layer, 524288 over 32 layers. The Llama-2-7B-shaped
    workload has 32 kv heads x head size 128 = 4096."""
    g = json.load(open(os.path.join(GOLDEN, "book_size_arithmetic.json")))
    spec = wl.CONFIGS["llama2_7b_mha"]
    assert spec.num_kv_heads * spec.head_size == g["hidden_size"]
    nb = bench.algorithmic_bytes(spec, np.array([1], np.int32))
    assert nb["per_token_head"] * spec.num_kv_heads == g["kv_bytes_per_token_per_layer"]
    assert nb["kv"] * g["num_layers"] == g["kv_bytes_per_token_all_layers"]
    # 100k tokens over 32 layers: 48.8 GiB; a quarter of that with 8 of 32 kv heads
    gib = 100000 * g["kv_bytes_per_token_all_layers"] / 2**30
    assert round(gib, 1) == g["kv_gib_100k_tokens"]
    assert round(gib * g["gqa_kv_heads_of_32"] / 32, 1) == g["gqa_kv_gib_100k_tokens"]


def test_algorithmic_bytes_components():
    spec = wl.CONFIGS["prefix_shared_write"]
    L = np.array([1024 + 16, 1024 + 33], np.int32)
    nb = bench.algorithmic_bytes(spec, L)
    per = 2 * 128 * 2
    assert nb["kv"] == int(L.sum()) * 8 * per
    assert nb["kv_unique"] == (16 + 33 + 1024) * 8 * per
    assert nb["tables"] == (33 + 34) * 4
    assert nb["q_out"] == 2 * 2 * 32 * 128 * 2
    assert nb["total"] == nb["kv"] + nb["q_out"] + nb["tables"] + nb["lens"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_oracle_timing_forks_workers_and_counts_items():
    """The CPU baseline's process pool: every worker takes its own items and
    the reported rate is items over the slowest worker's time."""
    seen = []
    rate, done, dt = bench.run_oracle_timed(lambda i: seen.append(i), 5, 0.05, 2)
    assert done > 0 and dt >= 0.05 and abs(rate - done / dt) < 1e-9
    assert seen == []          # the items ran in the forked workers, not here
    rate1, done1, dt1 = bench.run_oracle_timed(lambda i: seen.append(i), 5, 0.02, 1)
    assert done1 == len(seen) and seen[:5] == [0, 1, 2, 3, 4]
    assert 1 <= bench.cpu_workers() <= 16

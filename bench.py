#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step is one pass of the whole decode hot path over a synthetic batch
already resident in HBM: the newest token's slot, the cache write of its k/v,
then paged attention over every cached position (automatic single-pass /
split-K choice). By default the step is one pa_decode_append call (the cascade
form for a batch whose tables share a prefix, the FP8 form for an FP8 cache);
--separate times it as pa_decode_slot_mapping + pa_cache_write + pa_decode.

Default workload: the Llama-2-7B-shaped single-layer decode batch (64
sequences, 32 query = 32 kv heads, head size 128, block size 16, fp16,
context lengths uniform in [512, 2048], shuffled block tables over a pool of
the blocks used plus 10%).

Prints ONE JSON line: tokens/s for the whole job (one new token per sequence
per step), the decode call's achieved HBM bandwidth against MI355X's 8 TB/s
peak (from HIP events recorded on the launch stream inside the timed
region), the counter-measured HBM traffic per call when profiles/ holds it
for these kernel sources, the same call timed HBM-cold (after a cache flush,
outside the timed region), and the fp64 CPU oracle timed on a bounded sample
of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD's published figure
METRIC = "decode attn tokens/s + effective KV HBM GB/s (% of MI355X peak), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCES = ("paged_kv_cache_331_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_331_amd/csrc/pa_device.h",
                  "paged_kv_cache_331_amd/csrc/pa_launch.h",
                  "paged_kv_cache_331_amd/csrc/pa_mq.h",
                  "paged_kv_cache_331_amd/csrc/pa_prefix.h",
                  "paged_kv_cache_331_amd/csrc/pa_api.hip")


def algorithmic_bytes(spec, context_lens: np.ndarray) -> dict:
    """Bytes the decode step must move at least once.

    Per (token, kv head): K and V rows, 2 * head_size * 2 bytes. Plus q and
    out (num_seqs * num_q_heads * head_size * 2 bytes each), the table entries
    actually used (4 bytes per block) and the lengths (4 bytes per sequence).
    Positions >= L and split-K scratch are overhead, not counted.
    """
    L = context_lens.astype(np.int64)
    esz = 2                                             # q / out element bytes
    kv_esz = 1 if spec.cache_type == "fp8" else 2       # cache element bytes
    per_token_head = 2 * spec.head_size * kv_esz
    kv = int(L.sum()) * spec.num_kv_heads * per_token_head
    if spec.shared_prefix_blocks:
        pre = spec.shared_prefix_blocks * spec.block_size
        kv_unique = (int((L - pre).sum()) + pre) * spec.num_kv_heads * per_token_head
    else:
        kv_unique = kv
    qo = 2 * len(L) * spec.num_q_heads * spec.head_size * esz
    tables = int(((L + spec.block_size - 1) // spec.block_size).sum()) * 4
    lens = 4 * len(L)
    return {"kv": kv, "kv_unique": kv_unique, "q_out": qo, "tables": tables, "lens": lens,
            "total": kv + qo + tables + lens,
            "total_unique": kv_unique + qo + tables + lens,
            "per_token_head": per_token_head}


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_key(workload: str, separate: bool) -> str:
    """Key of a traffic record: the workload, and which form of the step ran."""
    return workload + (":separate" if separate else "")


def load_traffic(workload: str):
    """Counter-measured HBM traffic per decode call, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha") != kernel_source_sha():
        return None
    return entry.get("bytes_per_launch")


def _pmc_rows(path: str):
    import csv
    with open(path) as f:
        for r in csv.DictReader(f):
            yield r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])


def ingest_pmc(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
               copy_write_csv: str, copy_bytes: int = 1 << 30) -> dict:
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE dispatch records into bytes per decode call.

    Each counter is scaled by what it reads for a device copy of
    ``copy_bytes`` (the calibration run, ``--copy-probe``): the copy fetches
    and writes exactly ``copy_bytes``. A decode call is the partition kernel
    (one work-group per item, or the persistent grid) plus, when split, the
    reduce kernel; a cascade is its one launch of suffix items and prefix
    work-groups plus the reduce kernel. The median over dispatches of each is
    summed. The record is keyed to the kernel sources' hash so that it
    stops being reported once the kernels change.
    """
    def median_kib(path, counter, match):
        vals = [v for k, c, v in _pmc_rows(path) if c == counter and match(k)]
        if not vals:
            raise ValueError(f"no {counter} rows for the kernel in {path}")
        return float(np.median(vals)), len(vals)

    copy_kib = copy_bytes / 1024.0
    is_copy = lambda k: "copyBuffer" in k
    cf, _ = median_kib(copy_fetch_csv, "FETCH_SIZE", is_copy)
    cw, _ = median_kib(copy_write_csv, "WRITE_SIZE", is_copy)
    f_fetch, f_write = copy_kib / cf, copy_kib / cw
    rec = {"kernel_source_sha": kernel_source_sha(), "fetch_scale": f_fetch,
           "write_scale": f_write, "kernels": {}}
    total = 0.0
    for tag in ("cascade_fused_kernel", "decode_partition_kernel", "decode_mma_kernel",
                "decode_persistent_kernel",
                "decode_reduce_kernel", "decode_reduce_few_kernel"):
        m = lambda k, tag=tag: tag in k
        try:
            fk, n = median_kib(fetch_csv, "FETCH_SIZE", m)
        except ValueError:
            continue
        wk, _ = median_kib(write_csv, "WRITE_SIZE", m)
        fb, wb = fk * f_fetch * 1024, wk * f_write * 1024
        rec["kernels"][tag] = {"dispatches": n, "fetch_kib_raw": fk, "write_kib_raw": wk,
                               "fetch_bytes": fb, "write_bytes": wb}
        total += fb + wb
    rec["bytes_per_launch"] = total
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec[workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


# The oracle's work item and item count, set before the worker processes are
# forked (they inherit it; nothing is pickled).
_CPU_JOB = None


def host_cpus() -> int:
    """CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_workers() -> int:
    """Worker processes for the oracle: every CPU this process may run on,
    at most 16 (the host cores that go with one GPU on an 8-GPU node)."""
    return max(1, min(host_cpus(), 16))


def _oracle_worker(w: int, n: int, budget_s: float):
    """Items w, w + n, w + 2n, ... (wrapping round) until ``budget_s`` seconds
    have passed; one BLAS thread. Returns (items done, seconds)."""
    fn, count = _CPU_JOB
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        ctx = None
    done = 0
    t0 = time.perf_counter()
    try:
        i = w
        while True:
            fn(i % count)
            done += 1
            i += n
            if time.perf_counter() - t0 >= budget_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return done, time.perf_counter() - t0


def run_oracle_timed(fn, count: int, budget_s: float, workers: int):
    """Time ``fn(i)`` over items 0..count-1 in ``workers`` processes forked
    from this one (which must not have touched the GPU yet). Returns
    (items per second, items done, seconds)."""
    global _CPU_JOB
    _CPU_JOB = (fn, count)
    if workers <= 1:
        res = [_oracle_worker(0, 1, budget_s)]
    else:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(workers) as pool:
            res = pool.starmap(_oracle_worker, [(w, workers, budget_s) for w in range(workers)])
    done = sum(r[0] for r in res)
    dt = max(r[1] for r in res)
    return done / dt, done, dt


def cpu_baseline(batch, budget_s: float) -> dict:
    """Time the fp64 oracle (as it stands) on a bounded sample of the batch.

    One item is one sequence's decode: the slot of its newest token and
    attention over every cached position. Items are taken in order, wrapping
    round, for ``budget_s`` seconds in one process per host CPU (at most 16),
    each with one BLAS thread, and then for ``budget_s / 2`` seconds in one
    process with one thread. The rate is decoded tokens (one per sequence
    visited) per second.
    """
    import oracle
    b = batch

    def one(s):
        oracle.slot_mapping(b.block_tables[s:s + 1], b.context_lens[s:s + 1], b.spec.block_size)
        oracle.decode(b.q, b.key_cache, b.value_cache, b.block_tables, b.context_lens, b.scale,
                      b.dtype, seqs=[s], cache_dtype=b.cache_dtype, k_scale=b.k_scale,
                      v_scale=b.v_scale)

    n = cpu_workers()
    rate, done, dt = run_oracle_timed(one, b.num_seqs, budget_s, n)
    rate1, done1, dt1 = run_oracle_timed(one, b.num_seqs, budget_s / 2, 1)
    return {"value": rate, "unit": "tokens/s", "cores": n, "host_cpus": host_cpus(),
            "blas_threads_per_worker": 1, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle (slot of the newest token + attention over every "
                       f"cached position) in {n} forked processes, one BLAS thread each: "
                       f"{done} sequence decodes = {done / b.num_seqs:.2f} passes over the "
                       f"{b.num_seqs}-sequence batch in {dt:.1f} s; one decoded token per "
                       f"sequence"),
            "single_thread": {"value": rate1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{done1} sequence decodes in {dt1:.1f} s, one thread"}}


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 20) -> dict:
    """Device-to-device copy of ``nbytes`` (torch ``copy_``), timed with events.

    Reported as (read + write bytes) / time: the practical HBM ceiling the
    decode kernel is compared with, and the known-size copy that calibrates
    the FETCH_SIZE / WRITE_SIZE counters.
    """
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        ms.append((e0, e1))
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ms])) * 1e-3
    del src, dst
    return {"bytes": nbytes, "GBs": 2 * nbytes / t / 1e9, "ms": t * 1e3}


def cold_calls(step, reps: int = 20, flush_bytes: int = 1 << 30) -> list:
    """Event-timed calls, each after a read of a ``flush_bytes`` buffer.

    The read (outside the event pair) replaces the L2 and last-level cache
    contents with clean lines of another buffer, so the timed call finds none
    of its own bytes there and writes nothing back: HBM-cold numbers, beside
    the back-to-back steps of the main loop. Returns milliseconds per call.
    """
    import torch
    buf = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")   # summed as is: a pure read
    evs = []
    for _ in range(reps):
        buf.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        step(e0, e1)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del buf
    return [a.elapsed_time(b) for a, b in evs]


PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 matrix peak, AMD's published figure
PREFILL_METRIC = "prefill tokens/s + TFLOP/s (% of MI355X dense fp16/bf16 MFMA peak), 1 GPU"


def prefill_flops(spec, context_lens: np.ndarray, query_start: np.ndarray) -> int:
    """Causal attention FLOPs: 4 * head_size per (new token, query head, visible position)."""
    total = 0
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        n = int(query_start[s + 1] - query_start[s])
        # positions L-n .. L-1 see L-n+1 .. L keys
        total += n * (L - n) + n * (n + 1) // 2
    return 4 * spec.head_size * spec.num_q_heads * total


def prefill_cpu_baseline(batch, budget_s: float) -> dict:
    """The fp64 oracle's prefill arithmetic row by row (one new token, all its
    heads, at its own length), rows in a fixed random order, timed like
    :func:`cpu_baseline`."""
    import oracle
    b = batch
    qs = b.query_start
    rows = [(s, i) for s in range(b.num_seqs) for i in range(int(qs[s + 1] - qs[s]))]
    order = np.random.default_rng(0).permutation(len(rows))

    def one(j):
        s, i = rows[order[j]]
        n = int(qs[s + 1] - qs[s])
        L1 = np.array([int(b.context_lens[s]) - n + i + 1], np.int32)
        oracle.decode(b.q[qs[s] + i][None], b.key_cache, b.value_cache,
                      b.block_tables[s:s + 1], L1, b.scale, b.dtype,
                      cache_dtype=b.cache_dtype, k_scale=b.k_scale, v_scale=b.v_scale)

    n = cpu_workers()
    rate, done, dt = run_oracle_timed(one, len(rows), budget_s, n)
    rate1, done1, dt1 = run_oracle_timed(one, len(rows), budget_s / 2, 1)
    return {"value": rate, "unit": "tokens/s", "cores": n, "host_cpus": host_cpus(),
            "blas_threads_per_worker": 1, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle in {n} forked processes, one BLAS thread each: "
                       f"{done} new-token rows (all query heads of a token at its own causal "
                       f"length), drawn at random from the {len(rows)}-token batch, in "
                       f"{dt:.1f} s"),
            "single_thread": {"value": rate1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{done1} rows in {dt1:.1f} s, one thread"}}


def run_prefill(args) -> int:
    """One step = slots of the new tokens + their cache write + causal prefill."""
    import torch
    from paged_kv_cache_331_amd import pa, workloads as wl
    spec = wl.PREFILL_CONFIGS[args.workload]
    print(f"# generating {spec.name}", file=sys.stderr, flush=True)
    b = wl.make_prefill_batch(spec)
    # The oracle's worker processes are forked before this process touches the GPU.
    base = None
    if args.cpu_budget > 0:
        print("# cpu baseline", file=sys.stderr, flush=True)
        base = prefill_cpu_baseline(b, args.cpu_budget)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    pa.load()          # the HIP library must be built; there is no fallback
    tdt = torch.float16 if spec.dtype == "fp16" else torch.bfloat16
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(tdt).cuda()
    fp8 = b.cache_dtype == "fp8"
    q, k_new, v_new = up(b.q), up(b.k_new), up(b.v_new)
    if fp8:
        kc, vc = torch.from_numpy(b.key_cache).cuda(), torch.from_numpy(b.value_cache).cuda()
    else:
        kc, vc = up(b.key_cache), up(b.value_cache)
    ks, vs = float(b.k_scale), float(b.v_scale)
    bt = torch.from_numpy(b.block_tables).cuda()
    lens = torch.from_numpy(b.context_lens).cuda()
    qs = torch.from_numpy(b.query_start).cuda()
    out = torch.empty_like(q)
    slots = torch.empty(b.num_tokens, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    T, mq, ml = b.num_tokens, b.max_query_len, b.max_context_len

    def step(ev0=None, ev1=None):
        pa.prefill_slot_mapping(bt, lens, qs, T, mq, spec.block_size, ml, out=slots, stream=stream)
        if fp8:
            pa.cache_write_fp8(k_new, v_new, kc, vc, slots, ks, vs, stream=stream)
        else:
            pa.cache_write(k_new, v_new, kc, vc, slots, stream=stream)
        if ev0 is not None:
            ev0.record(stream)
        if fp8:
            pa.prefill_fp8(q, kc, vc, bt, lens, qs, float(b.scale), ks, vs, mq, ml, out=out,
                           stream=stream)
        else:
            pa.prefill(q, kc, vc, bt, lens, qs, float(b.scale), mq, ml, out=out, stream=stream)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        step(e0, e1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    pf_ms = float(np.mean(ms))
    ms_per_step = wall * 1e3 / args.steps
    flops = prefill_flops(spec, b.context_lens, b.query_start)
    achieved = flops / (pf_ms * 1e-3) / 1e12
    line = {
        "metric": PREFILL_METRIC, "value": T / (ms_per_step * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block tables)",
        "config": {"workload": spec.name, "num_seqs": b.num_seqs, "new_tokens": T,
                   "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_size": spec.head_size, "block_size": spec.block_size,
                   "cached_before": f"uniform [{spec.ctx_lo}, {spec.ctx_hi}]",
                   "new_per_seq": f"uniform [{spec.new_lo}, {spec.new_hi}]",
                   "cache": (f"fp8 (E4M3), scale {spec.kv_scale}" if fp8 else spec.dtype),
                   "step": "prefill slot mapping + cache write + causal prefill",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma",
                     "kernel": ("pa_prefill_fp8" if fp8 else "pa_prefill")
                               + " (events around the call on its stream)",
                     "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_TFLOPS, "traffic": None,
                     "algorithmic_flops_per_launch": flops,
                     "prefill_ms_mean": pf_ms, "prefill_ms_min": float(np.min(ms))},
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2_7b_mha")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="0 automatic, <0 single pass, >0 split-K partition tokens")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work on all host CPUs for the CPU baseline, then "
                         "half that on one thread (0 to skip)")
    ap.add_argument("--separate", action="store_true",
                    help="time the step as three calls (slot mapping, cache write, decode) "
                         "instead of one pa_decode_append call")
    ap.add_argument("--no-cascade", action="store_true",
                    help="decode a shared-prefix batch with pa_decode instead of pa_decode_cascade")
    ap.add_argument("--no-contiguous", action="store_true",
                    help="skip the same step over the contiguously renumbered pool")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the streaming-read and gather-read ceilings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only time a 1 GiB device copy (the counter calibration run)")
    ap.add_argument("--ingest-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="record the traffic of --workload from rocprofv3 counter_collection "
                         "CSVs (no GPU needed)")
    args = ap.parse_args(argv)
    if args.ingest_pmc:
        print(json.dumps(ingest_pmc(traffic_key(args.workload, args.separate), *args.ingest_pmc),
                         indent=1))
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("steps must be >= 1 and warmup >= 0", file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_331_amd import workloads as wl

    if args.copy_probe:
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            return 1
        print(json.dumps({"copy_probe": copy_bandwidth()}), flush=True)
        return 0
    if args.workload in wl.PREFILL_CONFIGS:
        return run_prefill(args)
    spec = wl.CONFIGS[args.workload]
    print(f"# generating {spec.name}", file=sys.stderr, flush=True)
    batch = wl.make_batch(spec)

    # The oracle runs first, in processes forked before anything here has
    # touched the GPU (or loaded the HIP library).
    base = None
    if args.cpu_budget > 0:
        print("# cpu baseline", file=sys.stderr, flush=True)
        base = cpu_baseline(batch, args.cpu_budget)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    from paged_kv_cache_331_amd import pa
    pa.load()          # the HIP library must be built; there is no fallback
    fp8 = spec.cache_type == "fp8"
    maxlen = batch.max_context_len
    # A batch whose tables share a prefix (the scheduler knows it: one physical
    # copy referenced by every sequence) is decoded with the cascade.
    cascade = spec.shared_prefix_blocks > 0 and not args.no_cascade and not fp8
    fused = not args.separate
    run = StepRunner(batch, args, cascade, fused)
    dec_ms, ms_per_step = run.time(args.warmup, args.steps)
    decode_ms = float(np.mean(dec_ms))
    print(f"# timed {args.steps} steps: {ms_per_step:.4f} ms/step, decode mean {decode_ms:.4f} ms"
          f" (median {np.median(dec_ms):.4f}, min {np.min(dec_ms):.4f}, max {np.max(dec_ms):.4f})",
          file=sys.stderr, flush=True)

    cold_ms = cold_calls(run.step)
    part_used = (args.partition_size if args.partition_size != 0 else
                 pa.decode_partition_size(batch.num_seqs, spec.num_kv_heads, maxlen,
                                          1 if fp8 else 2))
    probes = read_ceilings(run, part_used) if not args.no_probes else None
    run.release()
    copy = copy_bandwidth()

    # The same step over the same values with the pool renumbered so that
    # every table is a run of consecutive blocks (the layout of an unpaged
    # cache): what the scattered placement of the blocks costs.
    contig = None
    if not args.no_contiguous:
        print("# contiguous layout", file=sys.stderr, flush=True)
        crun = StepRunner(wl.relabel_contiguous(batch), args, cascade, fused)
        c_ms, _ = crun.time(args.warmup, args.steps)
        crun.release()
        c_mean = float(np.mean(c_ms))
        contig = {"layout": "same values, blocks renumbered so every table row is consecutive",
                  "decode_ms_mean": c_mean, "decode_ms_median": float(np.median(c_ms)),
                  "paged_over_contiguous": decode_ms / c_mean}

    nbytes = algorithmic_bytes(spec, batch.context_lens)
    # A block shared by many tables must come from HBM at least once, so the
    # roofline counts the shared prefix once; the per-sequence (logical)
    # rate is reported beside it.
    # The one-call step also reads the new k/v rows, stores them and writes
    # the slots: those bytes join the timed call's numerator.
    app = 0
    if fused:
        kv_esz = 1 if fp8 else 2
        app = batch.num_seqs * (2 * spec.num_kv_heads * spec.head_size * (2 + kv_esz) + 4)
    achieved = (nbytes["total_unique"] + app) / (decode_ms * 1e-3) / 1e9
    logical = (nbytes["total"] + app) / (decode_ms * 1e-3) / 1e9
    traffic = load_traffic(traffic_key(spec.name, args.separate))
    tokens_per_s = batch.num_seqs / (ms_per_step * 1e-3)
    roof = {
        "bound": "hbm",
        "kernel": ("decode with append" if fused else "pa_decode") +
                  " (events around the call on its stream)",
        "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": achieved / PEAK_HBM_GBS,
        "traffic": traffic,
        "algorithmic_bytes_per_launch": nbytes["total_unique"] + app,
        "append_bytes_per_launch": app,
        "logical_bytes_per_launch": nbytes["total"] + app, "logical_GBs": logical,
        "bytes_per_token_per_kv_head": nbytes["per_token_head"],
        "decode_ms_mean": decode_ms, "decode_ms_median": float(np.median(dec_ms)),
        "decode_ms_min": float(np.min(dec_ms)),
        "measured_copy_GBs": copy["GBs"], "frac_of_copy": achieved / copy["GBs"],
        "cold": {"flush": "1 GiB read before each call, outside the events",
                 "calls": len(cold_ms), "ms_mean": float(np.mean(cold_ms)),
                 "ms_median": float(np.median(cold_ms)),
                 "GBs": (nbytes["total_unique"] + app) / (float(np.mean(cold_ms)) * 1e-3) / 1e9,
                 "frac": (nbytes["total_unique"] + app) / (float(np.mean(cold_ms)) * 1e-3)
                         / 1e9 / PEAK_HBM_GBS}}
    if probes is not None:
        roof["read_ceilings"] = probes
        roof["frac_of_stream_read"] = achieved / probes["stream_read_GBs"]
        if probes.get("gather_read_GBs"):
            roof["frac_of_gather_read"] = achieved / probes["gather_read_GBs"]
    if contig is not None:
        roof["contiguous"] = contig

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype if not fp8 else f"fp8_e4m3 K/V, {spec.dtype} q/out",
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block tables)",
        "config": {
            "workload": spec.name, "num_seqs": batch.num_seqs, "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads, "head_size": spec.head_size,
            "block_size": spec.block_size, "context_lens": f"uniform [{spec.len_lo}, {spec.len_hi}]"
            if spec.lengths == "uniform" else "lognormal", "num_blocks": batch.num_blocks,
            "max_context_len": maxlen, "partition_size": args.partition_size,
            "partition_tokens_used": part_used,
            "step": ("one call (pa_decode_append" + ("_fp8" if fp8 else "") + "): slot mapping + "
                     "cache write + " if fused else "slot mapping + cache write + ") +
                    ("cascade decode (shared prefix)" if cascade else "decode"),
            "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)
    return 0


class StepRunner:
    """One decode batch on the GPU and the step the benchmark times."""

    def __init__(self, batch, args, cascade: bool, fused: bool):
        import torch
        from paged_kv_cache_331_amd import pa
        self.torch, self.pa = torch, pa
        self.batch, self.args, self.cascade, self.fused = batch, args, cascade, fused
        spec = batch.spec
        self.spec = spec
        tdt = torch.float16 if spec.dtype == "fp16" else torch.bfloat16
        up16 = lambda a: torch.from_numpy(a.view(np.int16)).view(tdt).cuda()
        self.fp8 = spec.cache_type == "fp8"
        self.q = up16(batch.q)
        if self.fp8:
            self.kc = torch.from_numpy(batch.key_cache).cuda()
            self.vc = torch.from_numpy(batch.value_cache).cuda()
        else:
            self.kc, self.vc = up16(batch.key_cache), up16(batch.value_cache)
        self.ks, self.vs = float(batch.k_scale), float(batch.v_scale)
        self.k_new, self.v_new = up16(batch.k_new), up16(batch.v_new)
        self.bt = torch.from_numpy(batch.block_tables).cuda()
        self.lens = torch.from_numpy(batch.context_lens).cuda()
        self.out = torch.empty_like(self.q)
        self.slots = torch.empty(batch.num_seqs, dtype=torch.int32, device="cuda")
        self.maxlen = batch.max_context_len
        P = args.partition_size
        if cascade:
            ws_bytes = pa.decode_cascade_workspace_size(batch.num_seqs, spec.num_q_heads,
                                                        spec.head_size, spec.block_size,
                                                        self.maxlen, spec.shared_prefix_blocks, P)
        else:
            ws_bytes = pa.decode_workspace_size(batch.num_seqs, spec.num_q_heads, spec.head_size,
                                                self.maxlen, P)
        self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        self.scale = float(batch.scale)
        self.stream = torch.cuda.current_stream()

    def step(self, ev0=None, ev1=None):
        pa, a, st = self.pa, self.args, self.stream
        P = a.partition_size
        pfx = self.spec.shared_prefix_blocks if self.cascade else 0
        if self.fused:
            # The whole step in one call: slots, the new rows stored, attention.
            if ev0 is not None:
                ev0.record(st)
            if self.fp8:
                pa.decode_append_fp8(self.q, self.k_new, self.v_new, self.kc, self.vc, self.bt,
                                     self.lens, self.scale, self.ks, self.vs, self.maxlen,
                                     out=self.out, slot_mapping=self.slots, partition_size=P,
                                     workspace=self.ws, stream=st)
            else:
                pa.decode_append(self.q, self.k_new, self.v_new, self.kc, self.vc, self.bt,
                                 self.lens, self.scale, self.maxlen, pfx, out=self.out,
                                 slot_mapping=self.slots, partition_size=P, workspace=self.ws,
                                 stream=st)
            if ev1 is not None:
                ev1.record(st)
            return
        pa.decode_slot_mapping(self.bt, self.lens, self.spec.block_size, out=self.slots, stream=st)
        if self.fp8:
            pa.cache_write_fp8(self.k_new, self.v_new, self.kc, self.vc, self.slots, self.ks,
                               self.vs, stream=st)
        else:
            pa.cache_write(self.k_new, self.v_new, self.kc, self.vc, self.slots, stream=st)
        if ev0 is not None:
            ev0.record(st)
        if self.fp8:
            pa.decode_fp8(self.q, self.kc, self.vc, self.bt, self.lens, self.scale, self.ks,
                          self.vs, self.maxlen, out=self.out, partition_size=P,
                          workspace=self.ws, stream=st)
        elif self.cascade:
            pa.decode_cascade(self.q, self.kc, self.vc, self.bt, self.lens, self.scale,
                              self.maxlen, self.spec.shared_prefix_blocks, out=self.out,
                              partition_size=P, workspace=self.ws, stream=st)
        else:
            pa.decode(self.q, self.kc, self.vc, self.bt, self.lens, self.scale, self.maxlen,
                      out=self.out, partition_size=P, workspace=self.ws, stream=st)
        if ev1 is not None:
            ev1.record(st)

    def time(self, warmup: int, steps: int):
        """Warm-up steps, then ``steps`` steps bracketed by device syncs.
        Returns (event-timed decode-call ms per step, wall ms per step)."""
        torch = self.torch
        print(f"# warmup {warmup}", file=sys.stderr, flush=True)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            self.step(e0, e1)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return [e0.elapsed_time(e1) for e0, e1 in evs], wall * 1e3 / steps

    def release(self):
        for k in ("q", "kc", "vc", "k_new", "v_new", "bt", "lens", "out", "slots", "ws"):
            setattr(self, k, None)
        self.torch.cuda.empty_cache()


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_331_amd", "libpa_probe_gfx950.so")


def read_ceilings(run: "StepRunner", part_tokens: int, reps: int = 30) -> dict:
    """Practical read ceilings from the probe kernels (libpa_probe_gfx950.so):
    a 4 GiB buffer streamed once, and this batch's K/V rows gathered through
    its tables with the decode kernel's load shape (partitions of
    ``part_tokens``; one work-group per item, and fixed-stride grids of 2 and
    4 work-groups per CU; the best is the gather ceiling). Median of ``reps``
    event-timed launches each; bytes = the buffer, or the K/V bytes of
    positions < L."""
    import ctypes
    torch = run.torch
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_probe_stream_read.restype = ctypes.c_int
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p]
    lib.pa_probe_gather_read.restype = ctypes.c_int
    lib.pa_probe_gather_read.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 4 + [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p]
    st = run.stream

    def timed(launch):
        for _ in range(3):
            launch()
        evs = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            launch()
            e1.record(st)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3

    nbytes = 4 << 30
    grid = 32768               # the best of 1024 .. 32768 work-groups in a sweep
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(grid * 4, dtype=torch.int32, device="cuda")

    def stream_launch():
        if lib.pa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid,
                                    st.cuda_stream) != 0:
            raise RuntimeError("pa_probe_stream_read failed")

    t_stream = timed(stream_launch)
    del buf, sink
    out = {"stream_read_GBs": nbytes / t_stream / 1e9, "stream_read_bytes": nbytes,
           "stream_grid": grid}
    b, spec = run.batch, run.spec
    row_bytes = spec.head_size * (1 if run.fp8 else 2)
    if not run.cascade and spec.block_size % 16 == 0 and row_bytes in (128, 256):
        P = part_tokens if part_tokens > 0 else -(-run.maxlen // spec.block_size) * spec.block_size
        P = -(-P // 16) * 16
        items = spec.num_kv_heads * b.num_seqs * -(-run.maxlen // P)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        kv = int(b.context_lens.astype(np.int64).sum()) * spec.num_kv_heads * 2 * row_bytes
        rates = {}
        for label, g in (("one_per_item", 0), ("persistent_2_per_cu", 2 * cus),
                         ("persistent_4_per_cu", 4 * cus)):
            gsink = torch.empty(4 * (items if g == 0 else min(g, items)), dtype=torch.int32,
                                device="cuda")

            def gather_launch(g=g, gsink=gsink):
                if lib.pa_probe_gather_read(run.kc.data_ptr(), run.vc.data_ptr(),
                                            run.bt.data_ptr(), run.lens.data_ptr(), b.num_seqs,
                                            spec.num_kv_heads, row_bytes, spec.block_size,
                                            b.num_blocks, b.max_blocks_per_seq, run.maxlen, P,
                                            g, gsink.data_ptr(), st.cuda_stream) != 0:
                    raise RuntimeError("pa_probe_gather_read failed")

            rates[label] = kv / timed(gather_launch) / 1e9
        out.update({"gather_read_GBs": max(rates.values()), "gather_read_by_grid_GBs": rates,
                    "gather_read_bytes": kv, "gather_partition_tokens": P})
    return out


if __name__ == "__main__":
    sys.exit(main())

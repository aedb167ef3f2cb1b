"""Benchmark of one paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is the whole hot path for one layer of a decode batch: the write of
each sequence's new K/V row at its slot, then paged decode attention with
split-KV.  By default the step is pa_append_decode's two launches called one
by one: pa_append_decode_partials (the decode workers also store the step's
rows; timed with HIP events as the dominant kernel), then pa_decode_merge.
With --separate-write the rows go through pa_write_kv first and the decode
is pa_decode_partials + pa_decode_merge.  The partition size defaults to one at least as long as the
workload's longest context (so records only arise where a worker's slice
cuts a pair); the long-context workload keeps its 512-token partitions.
The shared-prefix workloads decode with pa_decode_shared_prefix (rows
appended), told which sequences share their prefix blocks, so each shared
block is streamed once per KV head; ``--no-groups`` decodes them as any other
batch instead, with PA_DECODE_SHARED_BLOCKS so that the shared blocks stay
cacheable.  Otherwise K/V tiles are streamed (``--shared-blocks`` overrides
the choice).  Bytes: a slot read by several sequences counts once
(``value``, roofline); ``logical_*`` fields count every sequence's reads.

The default workload is the Llama-3-8B-shaped decode layer: 64 sequences,
32 query / 8 KV heads, head_dim 128, bf16, B=16, context lengths uniform on
[512, 4096], pool 1.25x the blocks needed, shuffled.

Inputs are synthetic (seeded) and resident in HBM before timing starts.  To
keep the 256 MB last-level cache from serving K/V across steps, the step
rotates over ``--layers`` independent copies of the cache (a model's layers;
at most one per warmup step, so that each is read before the timed steps),
so every step reads its K/V from HBM.

Output: one JSON line (metric, value = GB/s of algorithmic bytes per step
time, roofline of the dominant kernel from HIP events, CPU-oracle baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "paged decode attention achieved HBM GB/s (% of peak) + tokens/s"
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE) over this script's run of each workload, each
# scaled by what the same counter reads for pa_copy_blocks on a known byte
# count (run with --copy-calibration): FETCH_SIZE x 1.99183, WRITE_SIZE x 1.0.
# Summaries and commands: profiles/copy_blocks_calibration_hbm_bytes.md and
# the profiles/*_hbm_bytes.md file of each workload.  Keyed by (workload,
# partition, appending step, shared-block loads, prefix groups); the figures
# hold only for the kernel sources they were measured with (their hash).
KERNEL_SOURCES = ["paged_kv_cache_307_amd/csrc/decode_mfma.hip", "paged_kv_cache_307_amd/csrc/schedule.h",
                  "paged_kv_cache_307_amd/csrc/device_common.h", "paged_kv_cache_307_amd/csrc/internal.h",
                  "paged_kv_cache_307_amd/csrc/api.hip", "paged_kv_cache_307_amd/build.py"]
MEASURED_TRAFFIC_SHA256 = "ed5dc107157bb0ec170e860cad13cd3f9d2ea2076cf9b5054b91598699d0b7d0"
MEASURED_TRAFFIC = {
    ("llama3_8b_decode", 4096, True, False, False): {
        "bytes": 553875718, "fetch_bytes": 549047654, "write_bytes": 4828064},
    ("long_context", 512, True, False, False): {
        "bytes": 2719792933, "fetch_bytes": 2696453283, "write_bytes": 23339650},
    ("shared_prefix_steady", 4096, True, False, True): {
        "bytes": 480424679, "fetch_bytes": 453690791, "write_bytes": 26733888},
    ("shared_prefix_fork", 4096, True, False, True): {
        "bytes": 210521474, "fetch_bytes": 177291217, "write_bytes": 33230257},
    ("mixed_lengths_B8", 8192, True, False, False): {
        "bytes": 1659140015, "fetch_bytes": 1645690641, "write_bytes": 13449374},
    ("mixed_lengths_B16", 8192, True, False, False): {
        "bytes": 1660488179, "fetch_bytes": 1642844503, "write_bytes": 17643676},
    ("mixed_lengths_B32", 8192, True, False, False): {
        "bytes": 1675116276, "fetch_bytes": 1653133340, "write_bytes": 21982936},
}
# The same two passes over `bench.py --workload llama3_8b_prefill` for
# pa_prefill (summary: profiles/prefill_llama3_8b_prefill_hbm_bytes.md).
PREFILL_SOURCES = ["paged_kv_cache_307_amd/csrc/prefill.hip", "paged_kv_cache_307_amd/csrc/device_common.h",
                   "paged_kv_cache_307_amd/csrc/internal.h", "paged_kv_cache_307_amd/csrc/api.hip",
                   "paged_kv_cache_307_amd/build.py"]
PREFILL_TRAFFIC_SHA256 = "9987b1b7b3fefdf83f6fac768495e20876b555a3c553e3f242a456fa801a3396"
PREFILL_TRAFFIC = {
    "llama3_8b_prefill": {"bytes": 297510225, "fetch_bytes": 230376054, "write_bytes": 67134171},
}


def make_workload(name):
    """(workload, default partition size)."""
    import workloads as W
    table = {
        "llama3_8b_decode": (W.llama3_8b_decode, 4096),
        "long_context": (W.long_context, 512),
        "shared_prefix_steady": (lambda: W.shared_prefix("steady"), 4096),
        "shared_prefix_fork": (lambda: W.shared_prefix("fork"), 4096),
        "mixed_lengths_B8": (lambda: W.mixed_lengths(8), 8192),
        "mixed_lengths_B16": (lambda: W.mixed_lengths(16), 8192),
        "mixed_lengths_B32": (lambda: W.mixed_lengths(32), 8192),
    }
    make, partition = table[name]
    return make(), partition


def unique_kv_tokens(w):
    """Distinct cache slots the step reads: over every physical block in use,
    the most tokens any sequence reads from it (a sequence reads a block's
    slots 0 .. n-1).  Equal to the sum of context lengths when no block is
    shared; a block shared by a group of sequences (the pages' reference-
    counted prefix) counts once."""
    B = w.block_size
    ids, n = [], []
    for s, L in enumerate(w.context_lens):
        L = int(L)
        nb = -(-L // B)
        if nb == 0:
            continue
        ids.append(w.block_tables[s, :nb].astype(np.int64))
        fill = np.full(nb, B, np.int64)
        fill[-1] = L - (nb - 1) * B
        n.append(fill)
    if not ids:
        return 0
    ids, n = np.concatenate(ids), np.concatenate(n)
    most = np.zeros(int(ids.max()) + 1, np.int64)
    np.maximum.at(most, ids, n)
    return int(most.sum())


def algorithmic_bytes(w, unique=True):
    """Bytes one step must move at minimum: K and V of the live tokens read
    once (the step's own row included), q, out, the table entries in use, the
    context lengths, and the step's K/V rows stored to the cache.  With
    ``unique`` a slot read by several sequences (a shared prefix block) counts
    once: that is what HBM must deliver, and what a roofline fraction is taken
    on.  Without it every sequence's reads count (logical bytes)."""
    e = w.elem_bytes
    L = w.context_lens.astype(np.int64)
    tokens = unique_kv_tokens(w) if unique else int(L.sum())
    kv = tokens * w.num_kv_heads * w.head_dim * 2 * e
    q = w.num_seqs * w.num_heads * w.head_dim * e
    table = int(sum(-(-int(x) // w.block_size) for x in L)) * 4
    # copy-on-write before the step (the shared-prefix fork step): each pair
    # reads and writes one whole block of K and of V
    copy = len(w.copy_pairs) * 2 * 2 * w.num_kv_heads * w.block_size * w.head_dim * e
    return {"kv": kv, "q": q, "out": q, "table": table, "context_lens": 4 * w.num_seqs,
            "write": int((L > 0).sum()) * w.num_kv_heads * w.head_dim * e * 2, "copy": copy}


def capacity_figures(w):
    """What paging costs and saves on this batch (the pages' capacity
    arithmetic): unused tail slots of the last blocks, the fragmentation
    proxy 1 - used / allocated slots, and the slots a max-length contiguous
    reservation (the table's capacity) would leave unused."""
    B = w.block_size
    L = w.context_lens.astype(np.int64)
    alloc = int(sum(-(-int(x) // B) * B for x in L))
    used = int(L.sum())
    max_len = w.max_blocks_per_seq * B
    return {"tail_waste_slots": alloc - used,
            "fragmentation_proxy": round(1.0 - used / alloc, 6) if alloc else 0.0,
            "max_len": max_len, "prealloc_waste_slots": int(w.num_seqs * max_len - used)}


def kernel_sources_sha256(sources=None):
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def shares_blocks(w):
    """Whether some physical block is read by more than one sequence."""
    ids = [w.block_tables[s, :-(-int(L) // w.block_size)] for s, L in enumerate(w.context_lens)]
    ids = np.concatenate(ids) if ids else np.zeros(0, np.int32)
    return len(np.unique(ids)) < len(ids)


def measured_traffic(workload, partition, append, shared, groups=False):
    """Counter-derived HBM bytes per launch, or None when there is no
    measurement for this workload and step or the kernel changed since."""
    rec = MEASURED_TRAFFIC.get((workload, partition, append, shared, groups))
    if rec is None or MEASURED_TRAFFIC_SHA256 != kernel_sources_sha256():
        return None
    return rec["bytes"]


# The CPU baseline's state, set before its worker processes fork so that
# they share it (pools in shared memory: the parent's per-step writes and
# copies are what the workers read).
_CPU = {}


def _shared_like(a):
    """A copy of array ``a`` in anonymous shared memory (inherited by forked
    workers, writes visible both ways)."""
    import mmap
    buf = mmap.mmap(-1, max(a.nbytes, 1))
    out = np.frombuffer(buf, dtype=a.dtype, count=a.size).reshape(a.shape)
    out[...] = a
    return out


def _cpu_decode_units(units):
    """Worker: the oracle's decode of (sequence, [KV heads]) units; returns
    the rows it computed."""
    import oracle
    st = _CPU
    w = st["w"]
    G = w.num_heads // w.num_kv_heads
    got = []
    for s, heads in units:
        out = oracle.decode(st["q"], st["k"], st["v"], w.block_tables, w.context_lens, w.scale,
                            w.num_kv_heads, w.block_size, w.dtype, seqs=[s], kv_heads=heads)
        got.append((s, heads, np.stack([out[s, g * G:(g + 1) * G] for g in heads])))
    return got


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    # one BLAS thread per worker process, kept for the worker's life
    _CPU["limits"] = threadpool_limits(limits=1)


def _split_units(w, n):
    """(sequence, KV head) units cut into n contiguous ranges of about equal
    tokens, each as a list of (sequence, [KV heads]) runs."""
    units = [(s, g) for s in range(w.num_seqs) for g in range(w.num_kv_heads)]
    cost = np.array([max(int(w.context_lens[s]), 1) for s, _ in units], np.float64)
    cum = np.cumsum(cost)
    cuts = np.searchsorted(cum, cum[-1] * np.arange(1, n) / n)
    chunks = []
    for part in np.split(np.arange(len(units)), cuts):
        runs = []
        for i in part:
            s, g = units[i]
            if runs and runs[-1][0] == s:
                runs[-1][1].append(g)
            else:
                runs.append((s, [g]))
        if runs:
            chunks.append(runs)
    return chunks


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers():
    """Worker processes for the CPU baseline: the host cores this process may
    run on, at most 16 (one GPU's share of a shared host)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def cpu_baseline(w, cpu_seconds=24.0):
    """The oracle (fp64 NumPy, as it is) on this host's cores: full steps of
    the same workload (copies if any, write, decode), the decode's (sequence,
    KV head) units spread over a pool of worker processes with one BLAS
    thread each, repeated for about ``cpu_seconds`` of CPU time in all."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import oracle
    B = w.block_size
    n = cpu_workers()
    with threadpool_limits(limits=1):
        k_pool, v_pool = oracle.new_pools(w.num_blocks, w.num_kv_heads, B, w.head_dim, w.dtype)
        hs = oracle.slot_mapping(w.hist_block_tables, w.hist_seq, w.hist_pos, B)
        oracle.write_kv(k_pool, v_pool, oracle.to_bits(w.hist_key, w.dtype),
                        oracle.to_bits(w.hist_value, w.dtype), hs, B)
    _CPU.clear()
    _CPU.update(w=w, q=oracle.to_bits(w.q, w.dtype), k=_shared_like(k_pool), v=_shared_like(v_pool))
    del k_pool, v_pool
    chunks = _split_units(w, n)
    new_k, new_v = oracle.to_bits(w.new_key, w.dtype), oracle.to_bits(w.new_value, w.dtype)
    budget = max(cpu_seconds / n, 1.0)
    ctx = mp.get_context("fork")
    with ctx.Pool(n, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_worker_init_probe, range(n))  # every worker started before timing
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.copy_blocks(_CPU["k"], _CPU["v"], w.copy_pairs)  # the fork step's copies
            ns = oracle.slot_mapping(w.block_tables, w.new_seq, w.new_pos, B)
            oracle.write_kv(_CPU["k"], _CPU["v"], new_k, new_v, ns, B)
            parts = pool.map(_cpu_decode_units, chunks)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 50:
                break
    assert sum(len(p) for p in parts) == sum(len(c) for c in chunks)
    _CPU.clear()
    step_s = el / reps
    ab = algorithmic_bytes(w)
    step_bytes = sum(ab.values())
    return {"value": round(step_bytes / step_s / 1e9, 4), "unit": "GB/s", "cores": n,
            "cpu_model": cpu_model(), "kind": "oracle",
            "tokens_per_s": round(w.num_seqs / step_s, 2),
            "sample": f"{reps} full steps (copies if any, write + decode of all {w.num_seqs} "
                      f"sequences) of the same workload, {el:.1f} s wall; the decode's "
                      f"(sequence, KV head) units over {n} worker processes, one BLAS thread "
                      f"each; copies and writes in the parent, pools in shared memory",
            "block_manager_us_per_step": model_block_manager_timing(w)}


def _cpu_worker_init_probe(_):
    return os.getpid()


def model_block_manager_timing(w, steps=50):
    """The CPU model of the block manager on the same pattern as
    host_block_manager_timing: us per 64-sequence append plus table export."""
    from oracle import block_manager as bm

    B, S = w.block_size, w.num_seqs
    grow = -(-steps // B) + 1
    mb = w.max_blocks_per_seq + grow
    nb = int(sum(-(-max(int(L) - 1, 0) // B) for L in w.context_lens)) + S * grow
    mgr = bm.BlockManager(nb, B, S, mb, np.random.default_rng(0).permutation(nb))
    for s_ in range(S):
        assert mgr.allocate(s_, int(w.context_lens[s_]) - 1)[0] == 0
    seqs = list(range(S))
    t0 = time.perf_counter()
    for _ in range(steps):
        assert mgr.append(seqs)[0] == 0
        mgr.block_tables(seqs)
    return round((time.perf_counter() - t0) * 1e6 / steps, 2)


def copy_calibration(pairs=2048, reps=5):
    """Run pa_copy_blocks on a known number of bytes (for scaling the HBM
    byte counters of a profiler: each launch reads and writes
    pairs * 2 pools * 32 KiB)."""
    import torch

    import paged_kv_cache_307_amd as pa
    dev = torch.device("cuda", 0)
    k, v = pa.empty_kv_cache(2 * pairs, 8, 16, 128, torch.bfloat16, dev, fill=1.0)
    m = torch.stack([torch.arange(pairs), torch.arange(pairs) + pairs], 1).to(dev)
    for _ in range(reps):
        pa.copy_blocks(k, v, m)
    torch.cuda.synchronize()
    block = 8 * 16 * 128 * 2
    print(json.dumps({"copy_calibration": {"launches": reps, "read_bytes_per_launch": pairs * 2 * block,
                                           "write_bytes_per_launch": pairs * 2 * block}}), flush=True)


def host_block_manager_timing(w, steps=200):
    """Host cost of producing one decode step's metadata with the native block
    manager for this batch: pa_bm_append (slots and copy pairs) plus
    pa_bm_block_tables (the rows the decode reads), through the Python binding."""
    import paged_kv_cache_307_amd as pa

    B, S = w.block_size, w.num_seqs
    grow = -(-steps // B) + 1
    mb = w.max_blocks_per_seq + grow
    # every sequence gets private blocks here (no sharing), plus room to grow
    nb = int(sum(-(-max(int(L) - 1, 0) // B) for L in w.context_lens)) + S * grow
    mgr = pa.BlockManager(nb, B, S, mb, np.random.default_rng(0).permutation(nb))
    for s in range(S):
        st, _ = mgr.allocate(s, int(w.context_lens[s]) - 1)
        assert st == 0
    seqs = np.arange(S, dtype=np.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        st, _, _ = mgr.append(seqs)
        assert st == 0
        mgr.block_tables(seqs)
    us = (time.perf_counter() - t0) * 1e6 / steps
    return {"us_per_step": round(us, 2), "steps": steps, "batch": S,
            "calls": "pa_bm_append + pa_bm_block_tables via the Python binding, host only"}


MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_WORKLOADS = {"llama3_8b_prefill"}


def prefill_traffic(workload):
    """Counter-derived HBM bytes per pa_prefill launch, or None when there is
    no measurement or the kernel changed since."""
    rec = PREFILL_TRAFFIC.get(workload)
    if rec is None or PREFILL_TRAFFIC_SHA256 != kernel_sources_sha256(PREFILL_SOURCES):
        return None
    return rec["bytes"]


def prefill_flops(w):
    """Algorithmic flops of a prefill: for every (query row, query head) and
    every token the row sees, 2 D for q.k and 2 D for p.v."""
    f = 0
    for s in range(w.num_seqs):
        L, n = int(w.context_lens[s]), int(w.query_lens[s])
        f += sum(max(L - n + i + 1, 0) for i in range(n))
    return f * w.num_heads * 4 * w.head_dim


def _cpu_prefill_units(units):
    """Worker: the oracle's prefill of (sequence, KV head) units; returns the
    flops they hold."""
    import oracle
    st = _CPU
    w = st["w"]
    G = w.num_heads // w.num_kv_heads
    flops = 0
    for s, g in units:
        oracle.prefill(st["q"], st["k"], st["v"], w.block_tables, w.context_lens,
                       w.query_start, w.scale, w.num_kv_heads, w.block_size, w.dtype,
                       seqs=[s], kv_heads=[g])
        L, n = int(w.context_lens[s]), int(w.query_lens[s])
        flops += sum(max(L - n + i + 1, 0) for i in range(n)) * G * 4 * w.head_dim
    return flops


def prefill_cpu_baseline(w, cpu_seconds=48.0):
    """The oracle's prefill (fp64 NumPy, as it is) on this host's cores: the
    workload's (sequence, KV head) units dealt to a pool of worker processes
    with one BLAS thread each, one unit per worker per round, for about
    ``cpu_seconds`` of CPU time in all; scaled to TFLOP/s."""
    import multiprocessing as mp

    import oracle
    n = cpu_workers()
    r = oracle.run_prefill(w, seqs=[], kv_heads=[])
    _CPU.clear()
    _CPU.update(w=w, q=oracle.to_bits(w.q, w.dtype), k=r["k_pool"], v=r["v_pool"])
    del r
    units = [(s, g) for s in range(w.num_seqs) for g in range(w.num_kv_heads)]
    budget = max(cpu_seconds / n, 1.0)
    ctx = mp.get_context("fork")
    done, flops = 0, 0
    with ctx.Pool(n, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_worker_init_probe, range(n))  # every worker started before timing
        t0 = time.perf_counter()
        while True:
            batch = [[units[(done + i) % len(units)]] for i in range(n)]
            flops += sum(pool.map(_cpu_prefill_units, batch))
            done += n
            dt = time.perf_counter() - t0
            if dt >= budget:
                break
    _CPU.clear()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} (sequence, KV head) units of the same workload over {n} worker "
                      f"processes (one BLAS thread each), {dt:.1f} s"}


def run_prefill_bench(args):
    """One chunked-prefill step of a layer: the chunk's K/V rows stored with
    pa_write_kv, then pa_prefill.  Prints one JSON line (TFLOP/s)."""
    import workloads as W

    w = {"llama3_8b_prefill": W.llama3_8b_prefill}[args.workload]()
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(w)

    import torch

    import paged_kv_cache_307_amd as pa
    pa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def t(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    B = w.block_size
    bt, cl, qs = t(w.block_tables), t(w.context_lens), t(w.query_start)
    k0, v0 = pa.empty_kv_cache(w.num_blocks, w.num_kv_heads, B, w.head_dim, torch.bfloat16, dev,
                               fill=float("nan"))
    slots = pa.slot_mapping(bt, t(w.kv_seq), t(w.kv_pos), B)
    pa.write_kv(k0, v0, t(w.key), t(w.value), slots)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.layers - 1)]
    # the chunk's rows: positions L - n .. L - 1 of each sequence
    chunk = np.concatenate([np.nonzero((w.kv_seq == s) & (w.kv_pos >= int(w.context_lens[s]) -
                                                          int(w.query_lens[s])))[0]
                            for s in range(w.num_seqs)])
    c_slots = pa.slot_mapping(bt, t(w.kv_seq[chunk]), t(w.kv_pos[chunk]), B)
    c_key, c_value = t(w.key[chunk]), t(w.value[chunk])
    q = t(w.q)
    out = torch.empty_like(q)
    mcl, mql = w.max_context_len, w.max_query_len

    def attend(i):
        k, v = layers[i % len(layers)]
        pa.prefill(q, k, v, bt, cl, qs, mcl, mql, w.scale, out=out)

    def step(i):
        k, v = layers[i % len(layers)]
        pa.write_kv(k, v, c_key, c_value, c_slots)
        attend(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        attend(i)
    ev1.record()
    torch.cuda.synchronize()
    attend_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = elapsed * 1e3 / args.steps
    F = prefill_flops(w)
    tflops = F / (ms_per_step * 1e-3) / 1e12
    k_tflops = F / (attend_ms * 1e-3) / 1e12
    L = w.context_lens
    rec = {
        "metric": "paged prefill attention TFLOP/s + query tokens/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.num_seqs, "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": B,
            "context_len_min": int(L.min()), "context_len_max": int(L.max()),
            "query_rows": w.num_query_tokens, "chunk": int(w.query_lens.max()),
            "num_blocks": w.num_blocks, "layers_rotated": args.layers,
            "step": "pa_write_kv (chunk rows) + pa_prefill",
        },
        "query_tokens_per_s": round(w.num_query_tokens / (ms_per_step * 1e-3), 1),
        "flops_per_step": F,
        "roofline": {
            "kernel": "prefill_bf16_mfma_kernel<128,16,4,2>, 1 wave per workgroup, Q in LDS, S on 16x16x32, P.V on 32x32x16 (pa_prefill)", "bound": "mfma",
            "achieved": round(k_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(k_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "avg_us": round(attend_ms * 1e3, 3),
            "flops_per_launch": F, "traffic": prefill_traffic(w.name),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def run_cp_bench(args):
    """Context-parallel decode of the 64-sequence layer over W ranks emulated
    on one GPU (one pool per rank): each rank's pa_decode_lse over the tokens
    it owns, then pa_merge_states.  Prints one JSON line; value = one rank's
    decode GB/s (a rank runs on its own GPU in a real deployment)."""
    import workloads as W_

    import torch

    import paged_kv_cache_307_amd as pa
    pa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    world, inter = args.cp_world, 1
    w = W_.llama3_8b_decode()
    B = w.block_size
    # --partition 0: single pass (one launch, no merge).  By default a rank
    # whose sequences hold 512 tokens or fewer on average runs single pass:
    # on the 64-sequence layer split-KV won at W = 2 (52.0 against 62.8 us),
    # tied at W = 4 (33.0 / 32.4) and lost at W = 8 (24.6 against 18.4), where
    # its fixed cost (the record merge launch) outweighs the balance it buys.
    P = args.partition
    if P is None:
        share = [-(-int(L) // (B * world)) * B for L in w.context_lens]  # tokens per rank, rounded up
        P = 0 if float(np.mean(share)) <= 512 else 4096
    # the oracle computes the same result unsplit; its rate per KV byte does
    # not depend on which tokens a rank holds
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)

    def t(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    # one table for every rank: virtual blocks of B * world tokens, shuffled ids
    nvb = [-(-int(L) // (B * world)) for L in w.context_lens]
    ids = np.random.default_rng(307_390).permutation(sum(nvb))
    table = np.full((w.num_seqs, max(nvb)), -1, dtype=np.int32)
    k = 0
    for s_, n in enumerate(nvb):
        table[s_, :n] = ids[k:k + n]
        k += n
    seq = np.concatenate([w.hist_seq, w.new_seq])
    pos = np.concatenate([w.hist_pos, w.new_pos])
    key = t(np.concatenate([w.hist_key, w.new_key]))
    val = t(np.concatenate([w.hist_value, w.new_value]))
    bt, cl, q = t(table), t(w.context_lens), t(w.q)
    ranks = []
    for r in range(world):
        kc, vc = pa.empty_kv_cache(len(ids), w.num_kv_heads, B, w.head_dim, torch.bfloat16, dev,
                                   fill=float("nan"))
        pa.write_kv(kc, vc, key, val, pa.cp_slot_mapping(bt, t(seq), t(pos), B, world, r, inter))
        local = pa.cp_context_lens(cl, B, world, r, inter)
        mcl = int(local.max().item())
        ws = pa.alloc_workspace(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, mcl,
                                P, dev) if P > 0 else None
        # the rank's pool in args.layers copies, rotated per step like the
        # decode bench, so K/V come from HBM rather than the last-level cache
        pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(args.layers - 1)]
        ranks.append((pools, local, mcl, ws))
    outs = torch.empty((world,) + tuple(q.shape), dtype=q.dtype, device=dev)
    lses = torch.empty((world, w.num_seqs, w.num_heads), dtype=torch.float32, device=dev)
    merged = torch.empty_like(q)

    def rank_decode(r, i):
        pools, local, mcl, ws = ranks[r]
        kc, vc = pools[i % len(pools)]
        pa.decode(q, kc, vc, bt, local, mcl, w.scale, partition_size=P, workspace=ws,
                  out=outs[r], lse=lses[r])

    def step(i):
        for r in range(world):
            rank_decode(r, i)
        pa.merge_states(outs, lses, out=merged)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for i in range(args.steps):
        rank_decode(0, i)
    ev[1].record()
    for _ in range(args.steps):
        pa.merge_states(outs, lses, out=merged)
    ev[2].record()
    torch.cuda.synchronize()
    rank_ms = ev[0].elapsed_time(ev[1]) / args.steps
    merge_ms = ev[1].elapsed_time(ev[2]) / args.steps
    local0 = ranks[0][1].cpu().numpy().astype(np.int64)
    e = 2
    rank_bytes = int(local0.sum()) * w.num_kv_heads * w.head_dim * 2 * e + 2 * q.numel() * e
    gbs = rank_bytes / (rank_ms * 1e-3) / 1e9
    rec = {
        "metric": "context-parallel paged decode: one rank's HBM GB/s", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(rank_ms + merge_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3_8b_decode over {world} context-parallel ranks",
                   "batch": w.num_seqs, "cp_world": world, "interleave": inter,
                   "layers_rotated": args.layers,
                   "rank0_tokens": int(local0.sum()), "partition_size": P,
                   "step": "per rank pa_decode_lse (" + ("partials + merge" if P else "single pass")
                           + "); pa_merge_states"},
        "rank_decode_us": round(rank_ms * 1e3, 3), "merge_states_us": round(merge_ms * 1e3, 3),
        "roofline": {"kernel": "pa_decode_lse of rank 0 (" + ("decode + merge launches" if P else "one launch")
                     + ")", "bound": "hbm",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "avg_us": round(rank_ms * 1e3, 3),
                     "bytes_per_launch": rank_bytes, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_decode")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-KV partition size (default: per workload)")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-write", action="store_true",
                    help="write the step's rows with pa_write_kv, then pa_decode_partials")
    ap.add_argument("--shared-blocks", choices=["auto", "on", "off"], default="auto",
                    help="PA_DECODE_SHARED_BLOCKS: auto = when the tables share blocks and "
                         "the decode is not told the groups")
    ap.add_argument("--no-groups", action="store_true",
                    help="shared-prefix workloads: decode with pa_append_decode_partials "
                         "(every sequence reads its shared blocks) instead of "
                         "pa_decode_shared_prefix")
    ap.add_argument("--cp-world", type=int, default=0,
                    help="context-parallel ranks to emulate on the decode layer (0 = off)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run pa_copy_blocks on a known byte count (profiler calibration)")
    args = ap.parse_args()
    # Every rotated copy of the cache is read in the warmup steps, so that no
    # first touch of a copy (its page-table walks) falls in the timed steps.
    # Two or more copies, each far larger than the 256 MB last-level cache,
    # already keep every step's K/V reads on HBM.
    args.layers = max(1, min(args.layers, max(args.warmup, 2)))
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the path is single-GPU); --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload in PREFILL_WORKLOADS:
        run_prefill_bench(args)
        return
    if args.cp_world > 0:
        run_cp_bench(args)
        return

    w, default_partition = make_workload(args.workload)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)

    import torch

    import paged_kv_cache_307_amd as pa
    pa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def t(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B = w.block_size
    P = default_partition if args.partition is None else args.partition
    # shared-prefix workloads: the decode is told which sequences share their
    # prefix blocks (each such block is then streamed once per KV head)
    groups = "prefix_len" in w.extra and not args.no_groups and not args.separate_write
    shared = (shares_blocks(w) and not groups) if args.shared_blocks == "auto" \
        else args.shared_blocks == "on"
    # some pair spans more than one partition (selects the kernel variant)
    multi_part = -(-min(w.max_context_len, w.max_blocks_per_seq * B) // P) > 1
    hist_bt, bt, cl = t(w.hist_block_tables), t(w.block_tables), t(w.context_lens)
    k0, v0 = pa.empty_kv_cache(w.num_blocks, w.num_kv_heads, B, w.head_dim, dt, dev,
                               fill=float("nan"))
    hist_slots = pa.slot_mapping(hist_bt, t(w.hist_seq), t(w.hist_pos), B)
    pa.write_kv(k0, v0, t(w.hist_key), t(w.hist_value), hist_slots)
    if len(w.copy_pairs):
        pa.copy_blocks(k0, v0, t(w.copy_pairs))
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.layers - 1)]
    new_slots = pa.slot_mapping(bt, t(w.new_seq), t(w.new_pos), B)
    new_k, new_v, q = t(w.new_key), t(w.new_value), t(w.q)
    out = torch.empty_like(q)
    mcl = w.max_context_len
    # the fork step copies each shared partial block into its branch's
    # private block first; repeating the copy every step restores the same
    # state (the sources never change, and each branch then rewrites its slot)
    copies = t(w.copy_pairs) if len(w.copy_pairs) else None
    if groups:
        ng, br = w.extra["num_groups"], w.extra["branches"]
        gs = torch.arange(0, ng * br + 1, br, dtype=torch.int32, device=dev)
        pl = torch.full((ng,), w.extra["prefix_len"], dtype=torch.int32, device=dev)
        ws = pa.alloc_shared_prefix_workspace(w.num_seqs, w.num_heads, w.num_kv_heads,
                                              w.head_dim, mcl, P, ng, dev)
    else:
        ws = pa.alloc_workspace(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, mcl, P, dev)
    torch.cuda.synchronize()

    def partials(i):
        k, v = layers[i % len(layers)]
        if groups:
            pa.decode_shared_prefix(q, k, v, bt, cl, gs, pl, mcl, w.scale, P, ws, out, key=new_k,
                                    value=new_v, shared_blocks=shared, partials_only=True)
        elif args.separate_write:
            pa.decode_partials(q, k, v, bt, cl, mcl, w.scale, P, ws, out, shared_blocks=shared)
        else:
            pa.append_decode_partials(q, new_k, new_v, k, v, bt, cl, mcl, w.scale, P, ws, out,
                                      shared_blocks=shared)

    def step(i):
        k, v = layers[i % len(layers)]
        if copies is not None:
            pa.copy_blocks(k, v, copies)
        if args.separate_write:
            pa.write_kv(k, v, new_k, new_v, new_slots)
        partials(i)
        if groups:
            pa.decode_shared_prefix_merge(out, cl, gs, pl, w.num_kv_heads, B,
                                          w.max_blocks_per_seq, mcl, P, ws)
        else:
            pa.decode_merge(out, cl, w.num_kv_heads, B, w.max_blocks_per_seq, mcl, P, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps back to back, nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # The dominant kernel alone: K of its launches back to back on the
    # launch stream, between two HIP events (an event record between
    # launches would add a gap of its own to each).  Successive launches
    # are independent: each reads its layer's cache and rewrites the
    # workspace records.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        partials(i)
    ev1.record()
    torch.cuda.synchronize()
    part_avg_ms = ev0.elapsed_time(ev1) / args.steps
    # Per-launch distribution of the same kernel: an event pair around each
    # launch (each pair adds its own small gap, so these read a few percent
    # above the back-to-back average).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        partials(i)
        e1.record()
    torch.cuda.synchronize()
    per_launch_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    launch_pct = {f"p{q}": round(float(np.percentile(per_launch_us, q)), 3) for q in (10, 50, 90)}
    copy_us = None
    if copies is not None:  # the copy launch alone, the same way
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            k, v = layers[i % len(layers)]
            pa.copy_blocks(k, v, copies)
        ev1.record()
        torch.cuda.synchronize()
        copy_us = round(ev0.elapsed_time(ev1) / args.steps * 1e3, 3)

    ms_per_step = elapsed * 1e3 / args.steps
    # unique bytes (a shared block counts once) set `value` and the roofline
    # fraction; logical bytes (every sequence's reads) are reported beside
    ab = algorithmic_bytes(w)
    ab_logical = algorithmic_bytes(w, unique=False)
    step_bytes = sum(ab.values())
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    def kernel_bytes(b):
        # the timed kernel: reads K/V, q, table entries and lengths; in the
        # appending step it also stores the rows (the merge writes most of out)
        return b["kv"] + b["q"] + b["table"] + b["context_lens"] + \
            (0 if args.separate_write else b["write"])

    part_bytes = kernel_bytes(ab)
    part_gbs = part_bytes / (part_avg_ms * 1e-3) / 1e9
    L = w.context_lens
    rec = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.num_seqs, "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": B,
            "context_len_min": int(L.min()), "context_len_max": int(L.max()),
            "context_len_mean": round(float(L.mean()), 1), "num_blocks": w.num_blocks,
            "partition_size": P, "layers_rotated": args.layers,
            "kv_loads": "cached (PA_DECODE_SHARED_BLOCKS)" if shared else "streamed (nontemporal)",
            "step": (("pa_copy_blocks + " if copies is not None else "") +
                     ("pa_decode_shared_prefix_partials (rows appended) + "
                      "pa_decode_shared_prefix_merge" if groups else
                      "pa_write_kv + pa_decode_partials + pa_decode_merge" if args.separate_write
                      else "pa_append_decode_partials + pa_decode_merge")),
            "prefix_groups": ({"groups": w.extra["num_groups"], "members": w.extra["branches"],
                               "shared_tokens": w.extra["prefix_len"]} if groups else None),
            "copy_pairs": len(w.copy_pairs),
        },
        "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": step_bytes,
        "logical_bytes_per_step": sum(ab_logical.values()),
        "logical_gbs": round(sum(ab_logical.values()) / (ms_per_step * 1e-3) / 1e9, 2),
        "copy_blocks_us": copy_us,
        "capacity": capacity_figures(w),
        "roofline": {
            "kernel": f"decode_bf16_mfma_kernel<{w.head_dim},{B},true,{str(not shared).lower()},"
                      f"{str(multi_part or groups).lower()},{str(groups).lower()}> (" +
                      ("pa_decode_shared_prefix_partials" if groups else
                       "pa_decode_partials" if args.separate_write else
                       "pa_append_decode_partials") + ")",
            "bound": "hbm", "achieved": round(part_gbs, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(part_gbs / HBM_PEAK_GBS, 4),
            "avg_us": round(part_avg_ms * 1e3, 3), "per_launch_us": launch_pct,
            "bytes_per_launch": part_bytes,
            "logical_bytes_per_launch": kernel_bytes(ab_logical),
            "traffic": measured_traffic(w.name, P, not args.separate_write, shared, groups),
            "traffic_source": "rocprofv3 FETCH_SIZE and WRITE_SIZE passes of this workload's "
                              "step, recorded for the current kernel sources (null once they "
                              "change)",
        },
        "cpu_baseline": cpu,
        "host_block_manager": host_block_manager_timing(w),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

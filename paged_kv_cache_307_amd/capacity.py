"""Capacity and fragmentation of a paged KV pool versus max-length
preallocation, on a synthetic serving trace.  Host-side simulation.

What is compared (the pages' experiment section, "PagedAttention学习笔记",
实验部分 / 内存利用率评估, and "KV cache 显存管理", sections 最直观的做法 and
为什么固定大小 block 可以减少浪费):

* max-length preallocation: each admitted request reserves ``max_len``
  contiguous token slots for its whole life, so a request that ends at 512
  of 4096 tokens leaves 3584 slots unused;
* paged allocation: the native block manager (``pa_bm_*``) gives a request
  ceil(L / B) blocks and one more block only when its tail block is full, so
  at most B - 1 slots of a request are unused.

Both run the same trace of requests (arrival step, prompt tokens, output
tokens) on the same number of token slots.  Each step: finished requests
release their memory; waiting requests are admitted first come first served
while memory allows (paged: the prompt's blocks, the pages' admission test;
preallocation: ``max_len`` free slots); every running request generates one
token.  When a paged decode step does not fit, the most recently admitted
request is preempted (its blocks freed, the request requeued at the head of
the waiting queue to restart), which is the recompute form of preemption the
pages name.

Metrics per policy: requests running per step (mean over the steady window,
peak), the fragmentation proxy 1 - used slots / held slots (the pages'
proxy: held = allocated blocks x B for paged, reserved slots for
preallocation), KV bytes per request at the mean and P95 final length, the
largest tail waste of any request, preemptions and finished requests.  A
per-block fill histogram (how many written tokens each allocated block holds)
summarises the pages' suggested fill heat map at the end of the window.
"""

from __future__ import annotations

import dataclasses
import json
import math
import sys
from collections import deque

import numpy as np

from .block_manager import PA_ERR_NO_BLOCKS, BlockManager


@dataclasses.dataclass
class Request:
    arrival: int
    prompt: int
    output: int


def synthetic_trace(seed: int = 307_700, num_requests: int = 2000, rate: float = 2.0,
                    prompt_median: int = 512, prompt_sigma: float = 1.0,
                    output_range=(16, 1024), max_len: int = 4096):
    """Seeded requests: Poisson arrivals (``rate`` per step), lognormal prompt
    lengths (median ``prompt_median``), uniform output lengths; prompt +
    output clipped to ``max_len``."""
    rng = np.random.default_rng(seed)
    per_step = rng.poisson(rate, size=int(2 * num_requests / rate) + 16)
    arrivals = np.repeat(np.arange(per_step.size), per_step)[:num_requests]
    prompts = np.clip(np.rint(np.exp(np.log(prompt_median) +
                                     prompt_sigma * rng.standard_normal(num_requests))),
                      1, max_len - 1).astype(int)
    outputs = rng.integers(output_range[0], output_range[1], size=num_requests, endpoint=True)
    outputs = np.minimum(outputs, max_len - prompts)
    return [Request(int(a), int(p), int(o)) for a, p, o in zip(arrivals, prompts, outputs)]


def _summary(running, used, held, final_lens, bytes_per_token, held_per_req, extra):
    running = np.asarray(running, dtype=np.float64)
    used = np.asarray(used, dtype=np.float64)
    held = np.asarray(held, dtype=np.float64)
    win = slice(len(running) // 4, 3 * len(running) // 4)  # steady window
    frag = 1.0 - used[win] / np.maximum(held[win], 1)
    lens = np.asarray(final_lens, dtype=np.float64)
    mean_len, p95_len = float(lens.mean()), float(np.percentile(lens, 95))
    out = {
        "mean_running": round(float(running[win].mean()), 2),
        "peak_running": int(running.max()),
        "fragmentation_proxy_mean": round(float(frag.mean()), 5),
        "fragmentation_proxy_max": round(float(frag.max()), 5),
        "kv_bytes_per_request_at_mean_len": int(held_per_req(mean_len) * bytes_per_token),
        "kv_bytes_per_request_at_p95_len": int(held_per_req(p95_len) * bytes_per_token),
        "mean_final_len": round(mean_len, 1),
        "p95_final_len": round(p95_len, 1),
    }
    out.update(extra)
    return out


def simulate_paged(trace, total_slots: int, block_size: int, max_len: int,
                   bytes_per_token: int, max_running: int = 4096, make_manager=None,
                   fill_snapshot_step=None):
    """Paged allocation through a block manager (native by default)."""
    B = block_size
    nb = total_slots // B
    mb = -(-max_len // B)
    make = make_manager or (lambda: BlockManager(nb, B, max_running, mb))
    mgr = make()
    order = sorted(range(len(trace)), key=lambda i: trace[i].arrival)
    pending = deque(order)
    waiting = deque()
    running = {}                   # request -> (row, generated)
    free_rows = list(range(max_running - 1, -1, -1))
    admitted_at = {}
    done = 0
    preemptions = 0
    max_tail_waste = 0
    hist_running, hist_used, hist_held, final_lens = [], [], [], []
    fill_hist = None
    step = 0
    while (pending or waiting or running) and step < 100_000:
        while pending and trace[pending[0]].arrival <= step:
            waiting.append(pending.popleft())
        # finished requests release their blocks
        for r in [r for r, (_, g) in running.items() if g >= trace[r].output]:
            row, _ = running.pop(r)
            final_lens.append(mgr.context_len(row))
            assert mgr.free_seq(row) == 0
            free_rows.append(row)
            done += 1
        # admissions, first come first served, while the prompt's blocks fit
        while waiting and free_rows and mgr.can_allocate(trace[waiting[0]].prompt):
            r = waiting.popleft()
            row = free_rows.pop()
            st, _ = mgr.allocate(row, trace[r].prompt)
            assert st == 0
            running[r] = (row, 0)
            admitted_at[r] = step
        # one token for every running request; preempt the newest on shortage
        while running:
            rows = [running[r][0] for r in running]
            st, _, _ = mgr.append(rows)
            if st == 0:
                break
            assert st == PA_ERR_NO_BLOCKS
            victim = max(running, key=lambda r: (admitted_at[r], r))
            row, _ = running.pop(victim)
            assert mgr.free_seq(row) == 0
            free_rows.append(row)
            waiting.appendleft(victim)
            preemptions += 1
        for r in running:
            row, g = running[r]
            running[r] = (row, g + 1)
        lens = [mgr.context_len(running[r][0]) for r in running]
        held = (nb - mgr.num_free()) * B
        hist_running.append(len(running))
        hist_used.append(sum(lens))
        hist_held.append(held)
        for L in lens:
            max_tail_waste = max(max_tail_waste, -(-L // B) * B - L)
        if fill_snapshot_step is not None and step == fill_snapshot_step:
            fill_hist = np.zeros(B + 1, dtype=np.int64)
            for L in lens:
                full, part = divmod(L, B)
                fill_hist[B] += full
                if part:
                    fill_hist[part] += 1
        step += 1
    return _summary(hist_running, hist_used, hist_held, final_lens, bytes_per_token,
                    lambda L: math.ceil(L / B) * B,
                    {"policy": f"paged B={B}", "steps": step, "finished": done,
                     "preemptions": preemptions, "max_tail_waste_slots": int(max_tail_waste),
                     "block_fill_histogram": None if fill_hist is None else fill_hist.tolist()})


def simulate_prealloc(trace, total_slots: int, max_len: int, bytes_per_token: int):
    """Each admitted request reserves max_len contiguous slots."""
    capacity = total_slots // max_len
    order = sorted(range(len(trace)), key=lambda i: trace[i].arrival)
    pending = deque(order)
    waiting = deque()
    running = {}                   # request -> tokens held
    done = 0
    hist_running, hist_used, hist_held, final_lens = [], [], [], []
    step = 0
    while (pending or waiting or running) and step < 100_000:
        while pending and trace[pending[0]].arrival <= step:
            waiting.append(pending.popleft())
        for r in [r for r, L in running.items() if L - trace[r].prompt >= trace[r].output]:
            final_lens.append(running.pop(r))
            done += 1
        while waiting and len(running) < capacity:
            r = waiting.popleft()
            running[r] = trace[r].prompt
        for r in running:
            running[r] += 1
        hist_running.append(len(running))
        hist_used.append(sum(running.values()))
        hist_held.append(len(running) * max_len)
        step += 1
    return _summary(hist_running, hist_used, hist_held, final_lens, bytes_per_token,
                    lambda L: max_len,
                    {"policy": f"max-length preallocation ({max_len})", "steps": step,
                     "finished": done, "preemptions": 0,
                     "max_tail_waste_slots": int(max_len - min(final_lens)) if final_lens else 0,
                     "block_fill_histogram": None})


def compare(seed=307_700, num_requests=2000, rate=2.0, max_len=4096, slots_per_max_len=64,
            block_sizes=(8, 16, 32), num_kv_heads=8, head_dim=128, elem_bytes=2, layers=32):
    """The same trace under preallocation and paged allocation at each block
    size, on ``slots_per_max_len`` x ``max_len`` token slots."""
    trace = synthetic_trace(seed, num_requests, rate, max_len=max_len)
    total = slots_per_max_len * max_len
    bpt = layers * num_kv_heads * head_dim * 2 * elem_bytes  # bytes per token, all layers
    res = {"trace": {"seed": seed, "requests": num_requests, "rate_per_step": rate,
                     "max_len": max_len, "token_slots": total, "bytes_per_token": bpt},
           "prealloc": simulate_prealloc(trace, total, max_len, bpt)}
    for B in block_sizes:
        res[f"paged_B{B}"] = simulate_paged(trace, total, B, max_len, bpt,
                                            fill_snapshot_step=trace[-1].arrival // 2)
    return res


if __name__ == "__main__":
    print(json.dumps(compare(**({"num_requests": int(sys.argv[1])} if len(sys.argv) > 1 else {}))))

"""The split-KV work schedule, modelled on the host (no GPU).

The decode workers cut one line of 16-token tiles -- all (sequence, KV head)
pairs in (sequence, head, tile) order -- into equal slices, one per worker,
and cut each slice further at pair and partition boundaries.  A piece that
is not a whole pair leaves a record at index (global partition index +
worker); the merge scans, for each pair, the index range
[first partition + worker of the pair's first tile,
 last partition + worker of the pair's last tile].

This module restates that arithmetic in Python and checks the properties the
kernels rely on, over random length mixes and worker counts:

* the pieces of all workers cover every tile of every pair exactly once;
* record indices are distinct and below (partitions + workers), the
  workspace's record capacity;
* every record of a pair lies in the range the merge scans for it, and no
  record of another pair does (indices grow along the line);
* a pair is "whole" (one piece, output written directly) exactly when the
  merge range has a single index and the pair has one partition;
* with the first PAIR_SLOTS records of each pair (numbered k from the start
  of its merge range) moved to slots indexed by the pair, slots stay
  distinct and within the workspace, and the merge's slots for k < count
  hold exactly the pair's records (or nothing of this launch).
"""

import numpy as np
import pytest

TILE = 16
PAIR_SLOTS = 4


def slice_start(n, workers, b):
    return n * b // workers


def owner_of(n, workers, x):
    return ((x + 1) * workers - 1) // n


def pieces(lengths, hkv, partition, workers):
    """All pieces, as (worker, s, g, first tile, tiles, whole, record)."""
    tiles = [-(-int(L) // TILE) for L in lengths]
    parts = [-(-int(L) // partition) for L in lengths]
    pref_t = np.concatenate([[0], np.cumsum(tiles)])
    pref_p = np.concatenate([[0], np.cumsum(parts)])
    n = int(pref_t[-1]) * hkv
    tpp = partition // TILE
    out = []
    if n == 0:
        return out, n
    for b in range(workers):
        x0, x1 = slice_start(n, workers, b), slice_start(n, workers, b + 1)
        cur = x0
        while cur < x1:
            s = int(np.searchsorted(pref_t * hkv, cur, side="right") - 1)
            while tiles[s] == 0:  # sequences with no tiles own no line positions
                s += 1
            sbase = int(pref_t[s]) * hkv
            off = cur - sbase
            g, tin = divmod(off, tiles[s])
            part = tin // tpp
            end = min(sbase + (g + 1) * tiles[s], sbase + g * tiles[s] + (part + 1) * tpp, x1)
            ntile = end - cur
            whole = tin == 0 and ntile == tiles[s]
            rec = int(pref_p[s]) * hkv + g * parts[s] + part + b
            out.append((b, s, g, tin, ntile, whole, rec))
            cur = end
    return out, n


def merge_range(lengths, hkv, partition, workers, n, s, g):
    tiles = [-(-int(L) // TILE) for L in lengths]
    parts = [-(-int(L) // partition) for L in lengths]
    pref_t = int(sum(tiles[:s]))
    pref_p = int(sum(parts[:s]))
    base = pref_t * hkv + g * tiles[s]
    gp0 = pref_p * hkv + g * parts[s]
    b_first = owner_of(n, workers, base)
    b_last = owner_of(n, workers, base + tiles[s] - 1)
    return gp0 + b_first, gp0 + parts[s] - 1 + b_last, b_first == b_last and parts[s] == 1


CASES = [
    # (lengths, Hkv, partition, workers)
    ([1, 17, 40, 100], 2, 16, 768),
    ([1, 17, 40, 100], 2, 64, 3),
    (list(range(1, 41)) + [63, 64, 65, 127, 128, 129, 255, 257, 511, 512, 513, 700], 8, 32, 768),
    ([0, 33, 0, 129, 16], 2, 16, 5),
    ([0, 0, 0], 4, 512, 768),
]


def random_cases():
    rng = np.random.default_rng(307_300)
    out = []
    for _ in range(25):
        S = int(rng.integers(1, 40))
        lengths = [int(x) for x in rng.integers(0, 3000, size=S)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, S))] = int(rng.integers(20000, 40000))
        hkv = int(rng.choice([1, 2, 4, 8]))
        partition = int(rng.choice([16, 32, 64, 512, 4096]))
        workers = int(rng.choice([1, 2, 7, 64, 768, 3000]))
        out.append((lengths, hkv, partition, workers))
    return out


@pytest.mark.parametrize("case", CASES + random_cases())
def test_schedule_invariants(case):
    lengths, hkv, partition, workers = case
    ps, n = pieces(lengths, hkv, partition, workers)
    tiles = [-(-int(L) // TILE) for L in lengths]
    parts = [-(-int(L) // partition) for L in lengths]

    # every tile of every pair exactly once
    seen = {}
    for b, s, g, tin, ntile, whole, rec in ps:
        assert ntile >= 1
        for t in range(tin, tin + ntile):
            key = (s, g, t)
            assert key not in seen
            seen[key] = b
    assert len(seen) == sum(tiles) * hkv

    # a piece never crosses a partition boundary of its pair
    tpp = partition // TILE
    for b, s, g, tin, ntile, whole, rec in ps:
        assert tin // tpp == (tin + ntile - 1) // tpp

    # record indices: distinct, within capacity, inside their pair's merge range
    recs = [(rec, s, g) for b, s, g, tin, ntile, whole, rec in ps if not whole]
    idx = [r for r, _, _ in recs]
    assert len(idx) == len(set(idx))
    capacity = sum(parts) * hkv + workers
    assert all(0 <= r < capacity for r in idx)
    owner = {r: (s, g) for r, s, g in recs}
    for s in range(len(lengths)):
        if tiles[s] == 0:
            continue
        for g in range(hkv):
            first, last, whole = merge_range(lengths, hkv, partition, workers, n, s, g)
            mine = [r for r, ss, gg in recs if (ss, gg) == (s, g)]
            n_pieces = sum(1 for p in ps if (p[1], p[2]) == (s, g))
            assert whole == (n_pieces == 1)
            if whole:
                assert not mine
                continue
            assert mine and min(mine) == first and max(mine) == last
            for r in range(first, last + 1):  # indices in range: this pair's, or unused
                assert owner.get(r, (s, g)) == (s, g)

    # pair slots: record k of a pair (k = line index - first index of its
    # merge range) goes to pair * PAIR_SLOTS + k when k < PAIR_SLOTS, else to
    # the overflow region at S * Hkv * PAIR_SLOTS + its line index
    S = len(lengths)
    slot_of = {}
    for r, s_, g_ in recs:
        first, last, _ = merge_range(lengths, hkv, partition, workers, n, s_, g_)
        k = r - first
        assert 0 <= k <= last - first
        slot_of[r] = (s_ * hkv + g_) * PAIR_SLOTS + k if k < PAIR_SLOTS else S * hkv * PAIR_SLOTS + r
    slots = list(slot_of.values())
    assert len(slots) == len(set(slots))
    assert all(0 <= x < S * hkv * (PAIR_SLOTS + max(parts + [1])) + workers for x in slots)
    by_slot = {x: r for r, x in slot_of.items()}
    for s in range(len(lengths)):
        if tiles[s] == 0:
            continue
        for g in range(hkv):
            first, last, whole = merge_range(lengths, hkv, partition, workers, n, s, g)
            if whole:
                continue
            seen_recs = set()
            for k in range(last - first + 1):
                x = (s * hkv + g) * PAIR_SLOTS + k if k < PAIR_SLOTS else S * hkv * PAIR_SLOTS + first + k
                r = by_slot.get(x)
                if r is not None:
                    assert owner[r] == (s, g)
                    seen_recs.add(r)
            assert seen_recs == {r for r, ss, gg in recs if (ss, gg) == (s, g)}


def test_workspace_record_bound_is_tight_enough():
    """The host sizes the records as S * Hkv * ceil(L_max / P) + 4096; with
    every sequence at L_max and 4096 workers the largest index fits."""
    lengths = [4096] * 8
    ps, n = pieces(lengths, 8, 512, 4096)
    cap = 8 * 8 * (4096 // 512) + 4096
    assert max(p[6] for p in ps if not p[5]) < cap


def test_double_floor_division_is_exact_below_2_53():
    """The schedule divides line positions with one IEEE double division and
    a floor (p < 2^53, q < 2^53); Python floats are IEEE doubles, so this
    checks the claim that the result equals integer floor division."""
    import math
    rng = np.random.default_rng(307_301)
    cases = []
    for _ in range(20000):
        q = int(rng.integers(1, 1 << int(rng.integers(1, 53))))
        p = int(rng.integers(0, 1 << 53))
        cases.append((p, q))
        k = p // q
        for d in (-1, 0, 1):       # next to multiples of q
            if 0 <= k * q + d < (1 << 53):
                cases.append((k * q + d, q))
    # the largest operands the decode forms: N < 2^40 tiles, W <= 4096
    for n in ((1 << 40) - 1, (1 << 40) - 3, 3 * (1 << 38) + 7):
        for w in (4096, 4095, 768, 1):
            cases += [(n * w, w), (n * w - 1, n), ((n - 1 + 1) * w - 1, n)]
    for p, q in cases:
        assert math.floor(float(p) / float(q)) == p // q, (p, q)

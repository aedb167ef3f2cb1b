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


def pieces(lengths, hkv, partition, workers, lead=0, wt=1):
    """All pieces, as (worker, s, g, first tile, tiles, whole, record).  A
    pair takes span = lead + tiles * wt line positions (0 without tiles);
    its tile t sits at lead + t * wt from the pair's start, owned by the
    worker whose slice holds that position."""
    tiles = [-(-int(L) // TILE) for L in lengths]
    parts = [-(-int(L) // partition) for L in lengths]
    spans = [lead + t * wt if t else 0 for t in tiles]
    pref_t = np.concatenate([[0], np.cumsum(spans)]).astype(np.int64)
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
            while spans[s] == 0:  # sequences with no tiles own no line positions
                s += 1
            sbase = int(pref_t[s]) * hkv
            g = (cur - sbase) // spans[s]
            pair_base = sbase + g * spans[s]
            end = min(pair_base + spans[s], x1)
            first_pos = pair_base + lead
            tin = 0 if cur <= first_pos else -(-(cur - first_pos) // wt)
            tend = 0 if end <= first_pos else min(tiles[s], -(-(end - first_pos) // wt))
            t = tin
            while t < tend:
                part = t // tpp
                e = min(tend, (part + 1) * tpp)
                whole = tin == 0 and tend == tiles[s] and parts[s] == 1
                rec = int(pref_p[s]) * hkv + g * parts[s] + part + b
                out.append((b, s, g, t, e - t, whole, rec))
                t = e
            cur = end
    return out, n


def merge_range(lengths, hkv, partition, workers, n, s, g, lead=0, wt=1):
    tiles = [-(-int(L) // TILE) for L in lengths]
    parts = [-(-int(L) // partition) for L in lengths]
    spans = [lead + t * wt if t else 0 for t in tiles]
    pref_t = int(sum(spans[:s]))
    pref_p = int(sum(parts[:s]))
    base = pref_t * hkv + g * spans[s] + lead
    gp0 = pref_p * hkv + g * parts[s]
    b_first = owner_of(n, workers, base)
    b_last = owner_of(n, workers, base + (tiles[s] - 1) * wt)
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


@pytest.mark.parametrize("weights", [(0, 1), (12, 4), (20, 4), (3, 2)])
@pytest.mark.parametrize("case", CASES + random_cases())
def test_schedule_invariants(case, weights):
    lengths, hkv, partition, workers = case
    lead, wt = weights
    ps, n = pieces(lengths, hkv, partition, workers, lead, wt)
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
            first, last, whole = merge_range(lengths, hkv, partition, workers, n, s, g, lead, wt)
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
        first, last, _ = merge_range(lengths, hkv, partition, workers, n, s_, g_, lead, wt)
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
            first, last, whole = merge_range(lengths, hkv, partition, workers, n, s, g, lead, wt)
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


# ---------------------------------------------------------------- grouped lines

def _group_info(group_start, prefix_lens, lengths, members_cap, i):
    S = len(lengths)
    s0 = min(max(int(group_start[i]), 0), S)
    s1 = min(max(int(group_start[i + 1]), 0), S)
    members = max(0, min(s1 - s0, members_cap))
    plen = 0
    if members > 0:
        plen = min(max(int(prefix_lens[i]), 0), int(lengths[s0])) // 16 * 16
    return s0, members, plen


def _seq_prefix(group_start, prefix_lens, lengths, members_cap, s):
    n = len(prefix_lens)
    if n == 0 or group_start[0] > s:
        return 0, -1, -1
    lo, hi = 0, n - 1
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if group_start[mid] <= s:
            lo = mid
        else:
            hi = mid - 1
    first, members, plen = _group_info(group_start, prefix_lens, lengths, members_cap, lo)
    m = s - first
    if m < 0 or m >= members:
        return 0, -1, -1
    return min(plen, int(lengths[s])), lo, m


def _unit_shapes(group_start, prefix_lens, lengths, members_cap, partition, tail_lead=0,
                 prefix_lead=0, prefix_wt=1, tail_wt=1):
    """(tiles, parts, tok0, lead, wt, span) of every unit: prefix units, then
    tails.  A pair takes span = lead + tiles * wt line positions (0 without
    tiles); tile t sits at lead + t * wt from the pair's start."""
    units = []
    for i in range(len(prefix_lens)):
        _, _, plen = _group_info(group_start, prefix_lens, lengths, members_cap, i)
        t = plen // TILE
        units.append((t, 0, 0, prefix_lead, prefix_wt, prefix_lead + t * prefix_wt if t else 0))
    for s, L in enumerate(lengths):
        t0, _, _ = _seq_prefix(group_start, prefix_lens, lengths, members_cap, s)
        n = int(L) - t0
        t = -(-n // TILE)
        units.append((t, -(-n // partition), t0, tail_lead, tail_wt,
                      tail_lead + t * tail_wt if t else 0))
    return units


def grouped_pieces(group_start, prefix_lens, lengths, hkv, partition, workers, members_cap,
                   tail_lead=0, prefix_lead=0, prefix_wt=1, tail_wt=1):
    units = _unit_shapes(group_start, prefix_lens, lengths, members_cap, partition, tail_lead,
                         prefix_lead, prefix_wt, tail_wt)
    ng = len(prefix_lens)
    spans = [u[5] for u in units]
    parts = [u[1] for u in units]
    pref_t = np.concatenate([[0], np.cumsum(spans)]).astype(np.int64)
    pref_p = np.concatenate([[0], np.cumsum(parts)]).astype(np.int64)
    n = int(pref_t[-1]) * hkv
    tpp = partition // TILE
    out = []
    for b in range(workers if n else 0):
        x0, x1 = slice_start(n, workers, b), slice_start(n, workers, b + 1)
        cur = x0
        while cur < x1:
            u = int(np.searchsorted(pref_t * hkv, cur, side="right") - 1)
            while spans[u] == 0:
                u += 1
            tiles, _, tok0, lead, wt, span = units[u]
            ubase = int(pref_t[u]) * hkv
            g = (cur - ubase) // span
            pair_base = ubase + g * span
            end = min(pair_base + span, x1)
            first_pos = pair_base + lead
            tin = 0 if cur <= first_pos else -(-(cur - first_pos) // wt)
            tend = 0 if end <= first_pos else min(tiles, -(-(end - first_pos) // wt))
            b_first = owner_of(n, workers, first_pos)
            t = tin
            while t < tend:  # tail runs are cut further at partition ends
                if u < ng:
                    out.append(("prefix", b, u, g, t, tend - t, u * hkv + g + b))
                    break
                part = t // tpp
                e = min(tend, (part + 1) * tpp)
                k = part + b - b_first
                slot = ((u - ng) * hkv + g) * PAIR_SLOTS + k if k < PAIR_SLOTS else \
                    len(lengths) * hkv * PAIR_SLOTS + int(pref_p[u]) * hkv + g * parts[u] + \
                    b_first + k
                whole = tin == 0 and tend == tiles and parts[u] == 1 and tok0 == 0
                out.append(("tail", b, u, g, t, e - t, None if whole else slot))
                t = e
            cur = end
    return out, n, units, pref_t, pref_p


@pytest.mark.parametrize("weights", [(0, 0, 1, 1), (4, 0, 1, 1), (3, 2, 2, 1), (1, 0, 3, 1),
                                     (14, 14, 5, 4), (14, 0, 5, 4), (23, 52, 6, 4)])
@pytest.mark.parametrize("seed", range(12))
def test_grouped_line_covers_and_indexes(seed, weights):
    tail_lead, prefix_lead, prefix_wt, tail_wt = weights
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8, 16]))
    members_cap = 64 // G
    partition = int(rng.choice([16, 32, 512]))
    workers = int(rng.choice([1, 3, 64, 768, 1024]))
    sizes = rng.integers(0, 20, size=int(rng.integers(0, 6)))
    group_start = np.concatenate([[int(rng.integers(0, 3))], np.cumsum(sizes) +
                                  int(rng.integers(0, 3))]).astype(np.int64)
    S = int(group_start[-1] + rng.integers(0, 4))
    lengths = rng.integers(0, 700, size=S)
    prefix_lens = rng.integers(-5, 600, size=len(sizes))
    ps, n, units, pref_t, pref_p = grouped_pieces(group_start, prefix_lens, lengths, hkv,
                                                  partition, workers, members_cap, tail_lead,
                                                  prefix_lead, prefix_wt, tail_wt)
    ng = len(prefix_lens)
    # every tile of every unit and KV head exactly once
    seen = {}
    for kind, b, u, g, tin, nt, slot in ps:
        for t in range(tin, tin + nt):
            assert (u, g, t) not in seen
            seen[(u, g, t)] = b
    assert len(seen) == sum(u[0] for u in units) * hkv
    for (u, g, t), b in seen.items():  # a tile belongs to the owner of its position
        tiles, _, _, lead, wt, span = units[u]
        assert b == owner_of(n, workers, int(pref_t[u]) * hkv + g * span + lead + t * wt)
    # each member's tokens: the prefix unit's plus its tail's
    for s, L in enumerate(lengths):
        t0, grp, m = _seq_prefix(group_start, prefix_lens, lengths, members_cap, s)
        tail = units[ng + s]
        assert tail[2] == t0 and t0 + tail[0] * TILE >= L > t0 + (tail[0] - 1) * TILE - 1 \
            if tail[0] else L == t0
        if grp >= 0:
            assert t0 == min(units[grp][0] * TILE, int(L))
    # wide slots distinct, within the wide region, and in the merge's range
    wide = [p for p in ps if p[0] == "prefix"]
    slots = [p[6] for p in wide]
    assert len(set(slots)) == len(slots)
    assert all(0 <= x < ng * hkv + workers for x in slots)
    for kind, b, u, g, tin, nt, slot in wide:
        tiles, _, _, lead, wt, span = units[u]
        base = int(pref_t[u]) * hkv + g * span + lead
        bf, bl = owner_of(n, workers, base), owner_of(n, workers, base + (tiles - 1) * wt)
        assert u * hkv + g + bf <= slot <= u * hkv + g + bl
    # tail records distinct, within the record region, and each in the
    # merge's range for its pair (k < parts + b_last - b_first)
    recs = [p for p in ps if p[0] == "tail" and p[6] is not None]
    assert len(set(p[6] for p in recs)) == len(recs)
    max_parts = max(1, -(-int(lengths.max(initial=0)) // partition))
    assert all(0 <= p[6] < S * hkv * (PAIR_SLOTS + max_parts) + workers for p in recs)
    for kind, b, u, g, tin, nt, slot in recs:
        tiles, parts, _, lead, wt, span = units[u]
        base = int(pref_t[u]) * hkv + g * span + lead
        bf, bl = owner_of(n, workers, base), owner_of(n, workers, base + (tiles - 1) * wt)
        k = tin // (partition // TILE) + b - bf
        assert 0 <= k < parts + bl - bf
    # whole pairs: one worker owns every tile, and the merge agrees
    for kind, b, u, g, tin, nt, slot in ps:
        if kind == "tail" and slot is None:
            tiles, parts, tok0, lead, wt, span = units[u]
            base = int(pref_t[u]) * hkv + g * span + lead
            assert owner_of(n, workers, base) == owner_of(n, workers, base + (tiles - 1) * wt)
            assert parts == 1 and tok0 == 0

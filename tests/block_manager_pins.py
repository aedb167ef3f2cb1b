"""Checks that pin a block manager to what the pages fix.

Each ``check_*`` takes a factory ``make(num_blocks, block_size, max_seqs,
max_blocks_per_seq, free_order=None)`` that returns a manager with the
interface of ``oracle.block_manager.BlockManager``.  The same checks run
against the CPU model, against copies of it with a planted mistake (each must
fail at least one check), and against the native manager of ``libpa.so``.

None of them restates the manager's rules.  They compare it with the pages'
printed examples, and with a content model: a map from slot to the token that
slot holds, moved only by what the manager hands out (slots to write, block
pairs to copy).  After every operation each live sequence must read back,
through its own table, exactly the tokens it was given, in order; that is what
"sharing without corrupting state" ([P1] section 共享但不污染状态) means for
the caller.  Structural invariants (reference counts equal table membership,
free blocks are exactly those nobody references, ceil(L/B) blocks per
sequence, at most B-1 unused tail slots, writes only into private blocks)
are checked alongside.
"""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
OK, ERR_INVALID_ARG, ERR_NO_BLOCKS, ERR_STATE = 0, -1, -5, -6


def _golden():
    with open(os.path.join(GOLDEN, "block_manager_examples.json")) as f:
        return json.load(f)


class World:
    """A manager under test plus the content model and the expected tokens."""

    def __init__(self, mgr, num_blocks, B, max_seqs, max_blocks):
        self.m, self.NB, self.B, self.S, self.MB = mgr, num_blocks, B, max_seqs, max_blocks
        self.cells = {}        # slot -> token identity
        self.expect = {}       # live sequence -> token identities, position order
        self.next_token = 0

    def _token(self):
        self.next_token += 1
        return self.next_token

    # ---- operations, mirrored into the content model
    def allocate(self, seq, n):
        st, slots = self.m.allocate(seq, n)
        if st == OK:
            assert len(slots) == n
            toks = [self._token() for _ in range(n)]
            for s, t in zip(slots, toks):
                self.cells[int(s)] = t
            self.expect[seq] = toks
        return st, slots

    def fork(self, parent, child):
        st = self.m.fork(parent, child)
        if st == OK:
            self.expect[child] = list(self.expect[parent])
        return st

    def append(self, seqs):
        before_ref = [self.m.ref_count(b) for b in range(self.NB)]
        st, slots, pairs = self.m.append(seqs)
        if st != OK:
            return st, slots, pairs
        assert len(slots) == len(seqs)
        assert len(set(int(s) for s in slots)) == len(slots), "two rows write one slot"
        dsts = [int(d) for _, d in pairs]
        assert len(set(dsts)) == len(dsts), "copy destinations repeat"
        for src, dst in pairs:
            assert before_ref[int(dst)] == 0, "copy into a block that was in use"
            assert before_ref[int(src)] > 1, "copy of a block nobody else referenced"
        # a step copies first, then writes (copy-on-write)
        for src, dst in pairs:
            for o in range(self.B):
                v = self.cells.get(int(src) * self.B + o)
                if v is None:
                    self.cells.pop(int(dst) * self.B + o, None)
                else:
                    self.cells[int(dst) * self.B + o] = v
        for s, slot in zip(seqs, slots):
            t = self._token()
            self.cells[int(slot)] = t
            self.expect[s].append(t)
        for slot in slots:
            assert self.m.ref_count(int(slot) // self.B) == 1, "write into a shared block"
        return st, slots, pairs

    def free(self, seq):
        st = self.m.free_seq(seq)
        if st == OK:
            del self.expect[seq]
        return st

    # ---- what must hold after every operation
    def snapshot(self):
        rows, lens = self.m.block_tables(list(range(self.S)))
        return ([list(map(int, r)) for r in rows], list(map(int, lens)),
                [self.m.ref_count(b) for b in range(self.NB)], self.m.num_free())

    def verify(self):
        rows, lens, refs, nfree = self.snapshot()
        members = [0] * self.NB
        for seq in range(self.S):
            live = seq in self.expect
            assert (self.m.context_len(seq) >= 0) == live
            if not live:
                assert all(b == -1 for b in rows[seq]) and lens[seq] == 0
                continue
            L = len(self.expect[seq])
            assert lens[seq] == L == self.m.context_len(seq)
            used = [b for b in rows[seq] if b != -1]
            nblk = -(-L // self.B)
            assert rows[seq][:nblk] == used and len(used) == nblk, "table is not ceil(L/B) blocks"
            assert len(set(used)) == len(used), "a block twice in one table"
            assert 0 <= nblk * self.B - L <= self.B - 1, "more than B-1 unused tail slots"
            for b in used:
                assert 0 <= b < self.NB
                members[b] += 1
            for pos, tok in enumerate(self.expect[seq]):
                slot = rows[seq][pos // self.B] * self.B + pos % self.B
                assert self.cells.get(slot) == tok, f"sequence {seq} lost token {pos}"
        assert refs == members, "reference counts differ from table membership"
        assert nfree == sum(1 for r in refs if r == 0), "free count differs from unreferenced blocks"


def _rows(m, seqs):
    rows, lens = m.block_tables(seqs)
    return [list(map(int, r)) for r in rows], list(map(int, lens))


def _world(make, NB, B, S, MB, free_order=None):
    return World(make(NB, B, S, MB, free_order), NB, B, S, MB)


# ------------------------------------------------------------ printed examples

def check_forty_token_table(make):
    """P3: 40 tokens at B=16 -> 3 blocks; with the free blocks 7, 2, 15 first in
    line, the table is 7 -> 2 -> 15 and token 39 lands in block 15, offset 7."""
    g = _golden()
    B = g["printed"]["block_size"]
    order = g["printed"]["forty_tokens"]["block_table"]
    order = order + [b for b in range(32) if b not in order]
    w = _world(make, 32, B, 4, 8, order)
    st, slots = w.allocate(0, 40)
    assert st == OK
    rows, lens = _rows(w.m, [0])
    assert list(rows[0][:3]) == g["printed"]["forty_tokens"]["block_table"]
    assert lens[0] == 40 and list(rows[0][3:]) == [-1] * 5
    for pos, slot in g["derived"]["forty_token_slots"].items():
        assert int(slots[int(pos)]) == slot
    w.verify()


def check_seventeen_tokens_tail_first(make):
    """P3: 17 tokens at B=16 take 2 blocks, the second holding 1 token; P1:
    decode fills that tail block before asking for a new one."""
    g = _golden()
    B = g["printed"]["block_size"]
    w = _world(make, 8, B, 2, 8)
    assert w.allocate(0, 17)[0] == OK
    rows, _ = _rows(w.m, [0])
    nblk = sum(1 for b in rows[0] if b != -1)
    assert nblk == g["printed"]["seventeen_tokens"]["num_blocks"]
    assert 17 - (nblk - 1) * B == g["printed"]["seventeen_tokens"]["tokens_in_last_block"]
    assert nblk * B - 17 == g["printed"]["max_wasted_slots_per_request"]
    free0 = w.m.num_free()
    for _ in range(g["derived"]["appends_without_new_block_from_17"]):
        assert w.m.blocks_needed_to_append([0]) == 0
        assert w.append([0])[0] == OK
        assert w.m.num_free() == free0
    assert w.m.blocks_needed_to_append([0]) == 1
    st, slots, pairs = w.append([0])
    assert st == OK and pairs == [] and w.m.num_free() == free0 - 1
    w.verify()


# ------------------------------------------------------------ sharing

def check_fork_then_copy_on_write(make):
    """P1: a sequence about to write into a shared partial block gets a private
    copy; only its table changes and the other sequence still reads its own
    tokens."""
    w = _world(make, 16, 16, 4, 4)
    assert w.allocate(0, 20)[0] == OK
    assert w.fork(0, 1) == OK
    rows, _ = _rows(w.m, [0, 1])
    assert list(rows[0]) == list(rows[1])
    assert all(w.m.ref_count(b) == 2 for b in rows[0] if b != -1)
    w.verify()
    assert w.m.blocks_needed_to_append([1]) == 1
    st, slots, pairs = w.append([1])
    assert st == OK and len(pairs) == 1 and int(pairs[0][0]) == rows[0][1]
    after, _ = _rows(w.m, [0, 1])
    assert list(after[0]) == list(rows[0]), "the other sequence's table changed"
    assert after[1][0] == rows[0][0] and after[1][1] != rows[0][1]
    assert w.m.ref_count(rows[0][0]) == 2 and w.m.ref_count(rows[0][1]) == 1
    w.verify()
    st, slots, pairs = w.append([0])          # now the only referrer: in place
    assert st == OK and pairs == [] and int(slots[0]) == rows[0][1] * 16 + 4
    w.verify()


def check_fork_at_block_boundary_copies_nothing(make):
    """Full shared blocks are never written again: a branch forked at a block
    boundary opens a fresh block and copies nothing."""
    w = _world(make, 16, 16, 4, 4)
    assert w.allocate(0, 32)[0] == OK and w.fork(0, 1) == OK
    st, _, pairs = w.append([1, 0])
    assert st == OK and pairs == []
    rows, _ = _rows(w.m, [0, 1])
    assert rows[0][:2] == rows[1][:2] and rows[0][2] != rows[1][2]
    w.verify()


def check_group_of_branches_in_one_batch(make):
    """k branches sharing a partial tail, appending together, need k-1 private
    blocks; the last referrer writes in place."""
    k = 16
    w = _world(make, 64, 16, k, 8)
    assert w.allocate(0, 16 * 3 + 5)[0] == OK
    for c in range(1, k):
        assert w.fork(0, c) == OK
    seqs = list(range(k))
    assert w.m.blocks_needed_to_append(seqs) == k - 1
    free0 = w.m.num_free()
    st, slots, pairs = w.append(seqs)
    assert st == OK and len(pairs) == k - 1 and w.m.num_free() == free0 - (k - 1)
    w.verify()


def check_free_returns_blocks_only_when_unreferenced(make):
    """P2 state diagram: free drops a reference; a block rejoins the free pool
    when its count reaches zero."""
    w = _world(make, 16, 16, 4, 4)
    assert w.allocate(0, 40)[0] == OK and w.fork(0, 1) == OK
    assert w.append([1])[0] == OK             # CoW: one private block
    n = w.m.num_free()
    assert w.free(0) == OK
    assert w.m.num_free() == n + 1            # only 0's own tail was unshared
    w.verify()
    assert w.free(1) == OK
    assert w.m.num_free() == 16
    w.verify()
    assert w.free(1) == ERR_STATE


# ------------------------------------------------------------ failure

def check_shortage_is_reported_and_changes_nothing(make):
    """P1: a failed allocation is reported and never overwrites another
    sequence's state; P3: a decode batch whose new blocks exceed the free ones
    cannot be scheduled as a whole."""
    w = _world(make, 4, 16, 4, 8)
    assert w.allocate(0, 40)[0] == OK          # 3 of 4 blocks
    snap = w.snapshot()
    assert not w.m.can_allocate(17) and w.m.can_allocate(16)
    assert w.allocate(1, 17)[0] == ERR_NO_BLOCKS
    assert w.snapshot() == snap
    assert w.allocate(1, 16)[0] == OK          # last block
    for _ in range(8):
        assert w.append([0])[0] == OK         # fills 40..47 in place
    snap = w.snapshot()
    assert w.m.blocks_needed_to_append([0, 1]) == 2
    assert w.append([0, 1])[0] == ERR_NO_BLOCKS
    assert w.snapshot() == snap
    w.verify()
    assert w.free(1) == OK                     # preempt one: the other proceeds
    assert w.append([0])[0] == OK
    w.verify()


def check_bad_arguments(make):
    w = _world(make, 8, 16, 4, 2)
    assert w.allocate(4, 1)[0] == ERR_INVALID_ARG
    assert w.allocate(0, -1)[0] == ERR_INVALID_ARG
    assert w.allocate(0, 33)[0] == ERR_INVALID_ARG     # more blocks than a table row holds
    assert w.allocate(0, 32)[0] == OK
    assert w.allocate(0, 1)[0] == ERR_STATE
    assert w.append([0])[0] == ERR_INVALID_ARG           # row is full
    assert w.append([1])[0] == ERR_STATE
    assert w.allocate(1, 0)[0] == OK                     # live, empty table
    assert w.append([1, 1])[0] == ERR_INVALID_ARG
    assert w.fork(2, 3) == ERR_STATE and w.fork(0, 1) == ERR_STATE
    assert w.fork(0, 9) == ERR_INVALID_ARG
    w.verify()


# ------------------------------------------------------------ random traces

def run_trace(make, seed, steps=150, NB=48, B=4, S=24, MB=24, log=None):
    """A seeded serving-like trace: admissions, parallel-sampling forks,
    decode batches, preemption on shortage, finishes.  Verifies after every
    operation; appends every result to ``log`` when given."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(NB)
    w = _world(make, NB, B, S, MB, order)

    def rec(*x):
        if log is not None:
            log.append(x)

    for _ in range(steps):
        live = sorted(w.expect)
        idle = [s for s in range(S) if s not in w.expect]
        r = rng.random()
        if r < 0.25 and idle:
            seq, n = int(rng.choice(idle)), int(rng.integers(0, 3 * B * 2))
            rec("can_allocate", n, bool(w.m.can_allocate(n)))
            st, slots = w.allocate(seq, n)
            rec("allocate", seq, n, st, [int(x) for x in slots])
        elif r < 0.4 and live and idle:
            parent = int(rng.choice(live))
            kids = [int(c) for c in rng.permutation(idle)[: int(rng.integers(1, 5))]]
            for c in kids:
                rec("fork", parent, c, w.fork(parent, c))
        elif r < 0.85 and live:
            batch = [int(s) for s in rng.permutation(live)[: int(rng.integers(1, len(live) + 1))]]
            batch = [s for s in batch if len(w.expect[s]) < MB * B]
            if not batch:
                continue
            rec("needed", batch, w.m.blocks_needed_to_append(batch))
            st, slots, pairs = w.append(batch)
            rec("append", batch, st, [int(x) for x in slots], [tuple(map(int, p)) for p in pairs])
            if st == ERR_NO_BLOCKS:
                victim = int(rng.choice(batch))
                rec("preempt", victim, w.free(victim))
        elif live:
            seq = int(rng.choice(live))
            rec("free", seq, w.free(seq))
        w.verify()
        rec("state", w.snapshot())
    return w


def check_random_traces(make):
    for seed in range(6):
        run_trace(make, 307_400 + seed)
    run_trace(make, 307_410, B=16, NB=40, MB=8)


ALL_CHECKS = [
    check_forty_token_table,
    check_seventeen_tokens_tail_first,
    check_fork_then_copy_on_write,
    check_fork_at_block_boundary_copies_nothing,
    check_group_of_branches_in_one_batch,
    check_free_returns_blocks_only_when_unreferenced,
    check_shortage_is_reported_and_changes_nothing,
    check_bad_arguments,
    check_random_traces,
]

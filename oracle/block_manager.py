"""Plain CPU model of the KV block manager.  TEST INFRASTRUCTURE ONLY.

This module is a checker, not the product: only ``tests/`` may import it.  It
shares no code with the native block manager in ``libpa.so``; the tests drive
both with the same seeded operation traces and compare every result.

What the pages ask of a block manager:

* [P3] "KV cache 显存管理：为什么 PagedAttention 是 vLLM 的核心", section
  "Block manager 是 PagedAttention 的前置条件" (the block manager is the
  precondition of PagedAttention): it keeps the free physical blocks, gives
  blocks to new requests, adds a block to a request during decode, keeps each
  sequence's block table, frees the blocks when the request ends, and decides
  whether memory can take a new request.  Section "对 Scheduler 的影响" (effect
  on the scheduler): a prefill needs blocks for all prompt tokens; a decode
  needs a new block only when the current one is full; if many running
  requests need new blocks at once and the free blocks do not cover them, the
  batch cannot be scheduled as a whole.
* [P1] "什么是 PagedAttention？", section 映射逻辑块与物理块 (logical to
  physical blocks): prefill asks for blocks by input length; decode appends to
  the partly filled tail block first and asks for a new block only once it is
  full; a failed allocation must be reported (admission control, preemption,
  swap or refusal), never served by overwriting another sequence's state.
  Section 共享但不污染状态 (sharing without corrupting state): sequences may
  reference the same immutable blocks (a common prefix, parallel-sampling
  branches), with a reference count deciding when a block is reclaimed; a
  sequence about to write into a shared partial block gets a private block,
  the valid entries are copied into it, and only that sequence's table changes.
* [P2] "PagedAttention学习笔记", section 2.1 (ceil(L/B) logical blocks; logical
  block i holds tokens [iB, min((i+1)B, L)); new blocks only when a sequence
  crosses a block boundary; parallel samples or beams share the prefix blocks
  before they fork; ref_cnt per block, and a block whose count drops to zero
  returns to the free queue), and its state diagram (free pool -> allocated on
  allocate, back to the free pool on free once the count is zero).

Readings where the pages leave a choice open:

* The free queue is first-in first-out: allocation takes from its head, a
  block whose count reaches zero joins its tail, so the block freed longest
  ago is reused first.  The initial order is given by the caller (ascending
  ids by default).  Blocks of a freed sequence are released in logical order.
* A sequence is a row index in [0, max_seqs) of the block table.
* Appending to a batch is all or nothing: if the free blocks do not cover the
  whole batch, nothing changes and the call reports the shortage.  Within a
  batch, sequences are served in list order; the copy-on-write test reads the
  reference count as earlier members of the batch left it, so of k sequences
  sharing one partial tail block and all appending in one batch, the first k-1
  get private copies and the last writes in place.
* A copy-on-write copies the whole block (entries past the valid ones are
  unused slots and never read).
* Allocation of zero tokens makes a live sequence with an empty table.
* Prefix hashing, swapping and eviction of cached blocks are not modelled:
  every block whose count is zero is free.
"""

from __future__ import annotations

from collections import deque

OK = 0
ERR_INVALID_ARG = -1
ERR_NO_BLOCKS = -5
ERR_STATE = -6


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class BlockManager:
    """Free queue, reference counts and per-sequence block tables."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int,
                 free_order=None):
        self.B = int(block_size)
        self.num_blocks = int(num_blocks)
        self.max_seqs = int(max_seqs)
        self.max_blocks = int(max_blocks_per_seq)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "free order must be a permutation"
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables = {}      # sequence -> list of physical block ids, logical order
        self.lens = {}        # sequence -> number of tokens held

    # ------------------------------------------------------------ queries
    def num_free(self) -> int:
        return len(self.free)

    def ref_count(self, block: int) -> int:
        return self.ref[block]

    def context_len(self, seq: int) -> int:
        """Tokens held by ``seq``; -1 if it is not live."""
        return self.lens.get(seq, -1)

    def slot(self, seq: int, pos: int) -> int:
        """[P2] BlockTable walkthrough: slot = table[pos // B] * B + pos % B."""
        return self.tables[seq][pos // self.B] * self.B + pos % self.B

    def can_allocate(self, num_tokens: int) -> bool:
        need = _ceil_div(num_tokens, self.B)
        return need <= self.max_blocks and need <= len(self.free)

    def _valid_seq(self, seq: int) -> bool:
        return 0 <= seq < self.max_seqs

    # ---------------------------------------------------------- prefill
    def allocate(self, seq: int, num_tokens: int):
        """A new sequence of ``num_tokens`` tokens: ceil(L/B) fresh blocks.
        Returns (status, slots of positions 0..L-1)."""
        if not self._valid_seq(seq) or num_tokens < 0:
            return ERR_INVALID_ARG, []
        if seq in self.tables:
            return ERR_STATE, []
        need = _ceil_div(num_tokens, self.B)
        if need > self.max_blocks:
            return ERR_INVALID_ARG, []
        if need > len(self.free):
            return ERR_NO_BLOCKS, []
        table = []
        for _ in range(need):
            b = self.free.popleft()
            self.ref[b] = 1
            table.append(b)
        self.tables[seq] = table
        self.lens[seq] = num_tokens
        return OK, [self.slot(seq, t) for t in range(num_tokens)]

    # ------------------------------------------------------------ fork
    def fork(self, parent: int, child: int) -> int:
        """``child`` references every block of ``parent``; counts go up by one."""
        if not (self._valid_seq(parent) and self._valid_seq(child)):
            return ERR_INVALID_ARG
        if parent not in self.tables or child in self.tables:
            return ERR_STATE
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return OK

    # ----------------------------------------------------------- decode
    def _plan(self, seqs):
        """Walk the batch in order and say, per sequence, whether its next token
        needs a fresh block and whether that block replaces a shared tail."""
        pending = {}          # block -> count as earlier batch members left it
        plan = []
        for s in seqs:
            pos = self.lens[s]
            if pos % self.B == 0:
                plan.append(("new", None))
                continue
            tail = self.tables[s][pos // self.B]
            count = pending.get(tail, self.ref[tail])
            if count > 1:
                pending[tail] = count - 1
                plan.append(("cow", tail))
            else:
                plan.append(("in_place", tail))
        return plan

    def blocks_needed_to_append(self, seqs) -> int:
        return sum(1 for kind, _ in self._plan(seqs) if kind != "in_place")

    def append(self, seqs):
        """One more token for each sequence in ``seqs`` (decode).  Returns
        (status, slots, copy pairs (src, dst)); on failure nothing changes."""
        seqs = [int(s) for s in seqs]
        if any(not self._valid_seq(s) for s in seqs) or len(set(seqs)) != len(seqs):
            return ERR_INVALID_ARG, [], []
        if any(s not in self.tables for s in seqs):
            return ERR_STATE, [], []
        if any(self.lens[s] >= self.max_blocks * self.B for s in seqs):
            return ERR_INVALID_ARG, [], []
        plan = self._plan(seqs)
        if sum(1 for kind, _ in plan if kind != "in_place") > len(self.free):
            return ERR_NO_BLOCKS, [], []
        slots, pairs = [], []
        for s, (kind, tail) in zip(seqs, plan):
            pos = self.lens[s]
            if kind == "new":
                b = self.free.popleft()
                self.ref[b] = 1
                self.tables[s].append(b)
            elif kind == "cow":
                b = self.free.popleft()
                self.ref[b] = 1
                self.ref[tail] -= 1
                self.tables[s][pos // self.B] = b
                pairs.append((tail, b))
            slots.append(self.slot(s, pos))
            self.lens[s] = pos + 1
        return OK, slots, pairs

    # ------------------------------------------------------------- free
    def free_seq(self, seq: int) -> int:
        """Drop the sequence; blocks whose count reaches zero return to the
        tail of the free queue, in logical order."""
        if not self._valid_seq(seq):
            return ERR_INVALID_ARG
        if seq not in self.tables:
            return ERR_STATE
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]
        return OK

    # ----------------------------------------------------------- export
    def block_tables(self, seqs):
        """Rows of the int32 [rows, max_blocks_per_seq] table, padded with -1,
        and the context lengths (0 for a sequence that is not live)."""
        rows, lens = [], []
        for s in seqs:
            t = self.tables.get(int(s), [])
            rows.append(list(t) + [-1] * (self.max_blocks - len(t)))
            lens.append(self.lens.get(int(s), 0))
        return rows, lens

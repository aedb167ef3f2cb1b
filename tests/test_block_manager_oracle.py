"""The CPU model of the block manager against the pages' examples and the
content model (no GPU), and planted mistakes that those checks must catch."""

import os
import types

import pytest

import block_manager_pins as pins
from oracle import block_manager as bm

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "block_manager.py")


def _make(module):
    def make(num_blocks, block_size, max_seqs, max_blocks, free_order=None):
        return module.BlockManager(num_blocks, block_size, max_seqs, max_blocks, free_order)
    return make


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_block_manager_oracle_pin(check):
    check(_make(bm))


MUTANTS = {
    "copy_on_write_skipped": ("            if count > 1:\n", "            if count > 999:\n"),
    "copy_pair_reversed": ("pairs.append((tail, b))", "pairs.append((b, tail))"),
    "batch_order_ignored": ("count = pending.get(tail, self.ref[tail])", "count = self.ref[tail]"),
    "fork_takes_no_reference": ("            self.ref[b] += 1\n", "            pass\n"),
    "free_ignores_references": ("            if self.ref[b] == 0:\n", "            if True:\n"),
    "new_block_every_decode": ("            if pos % self.B == 0:\n", "            if True:\n"),
    "ceil_becomes_floor": ("need = _ceil_div(num_tokens, self.B)\n        if need > self.max_blocks",
                           "need = num_tokens // self.B\n        if need > self.max_blocks"),
    "slot_offset_from_block": ("* self.B + pos % self.B", "* self.B + pos // self.B"),
    "shortage_not_checked": ("        if need > len(self.free):\n            return ERR_NO_BLOCKS, []\n",
                             ""),
    "shared_tail_counted_once": ("                pending[tail] = count - 1\n", ""),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("block_manager_mutant")
    exec(compile(src.replace(old, new, 1), "block_manager_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_manager_mutant_is_caught(name):
    make = _make(_mutant(*MUTANTS[name]))
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(make)
        except Exception as e:  # AssertionError or a crash both count as caught
            failures.append((check.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every check"

"""The oracle's prefill against its pins (no GPU), and planted mistakes that
the pins must catch."""

import os
import types

import pytest

import oracle
import prefill_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "paged_attention.py")


@pytest.mark.parametrize("check", prefill_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_prefill_oracle_pin(check):
    check(oracle)


MUTANTS = {
    "visible_off_by_one": ("visible = max(L - n + i + 1, 0)", "visible = max(L - n + i, 0)"),
    "position_from_chunk_start": ("visible = max(L - n + i + 1, 0)", "visible = max(i + 1, 0)"),
    "no_causal_mask": ("visible = max(L - n + i + 1, 0)", "visible = max(L, 0)"),
    "query_row_shifted": ("attend(q[q0 + i, g * G:(g + 1) * G]", "attend(q[q0 + n - 1 - i, g * G:(g + 1) * G]"),
    "gqa_modulo": ("out[q0 + i, g * G:(g + 1) * G] = attend(q[q0 + i, g * G:(g + 1) * G]",
                   "out[q0 + i, g::num_kv_heads] = attend(q[q0 + i, g::num_kv_heads]"),
    "rows_of_next_sequence": ("q0, q1 = int(query_start[s]), int(query_start[s + 1])",
                              "q0, q1 = int(query_start[s]), int(query_start[min(s + 2, S)])"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("oracle_prefill_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_prefill_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prefill_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failures = []
    for check in prefill_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            failures.append((check.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every check"

"""The oracle's context-parallel pieces against their pins (no GPU), and
planted mistakes that the pins must catch."""

import os
import types

import pytest

import cp_pins
import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "paged_attention.py")


@pytest.mark.parametrize("check", cp_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_cp_oracle_pin(check):
    check(oracle)


MUTANTS = {
    "owner_without_wrap": ("return (p % (B * W)) // I % W", "return (p % (B * W)) // I % (W + 1)"),
    "local_offset_ignores_interleave": ("return vo // (I * W) * I + vo % I", "return vo // W"),
    "virtual_block_is_one_block": ("out[i] = int(block_tables[s][p // (B * W)]) * B",
                                   "out[i] = int(block_tables[s][p // B]) * B"),
    "lse_without_denominator": ("return (w @ Vs) / den, (m + np.log(den))[:, 0]",
                                "return (w @ Vs) / den, m[:, 0]"),
    "merge_without_weights": ("num = (w[..., None] * outs).sum(axis=0)", "num = outs.sum(axis=0) * den[..., None] / len(outs)"),
    "kernel_block_not_scaled": ("kt[r, i * k + j] = mt[r, i] * k + j", "kt[r, i * k + j] = mt[r, i] + j"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("oracle_cp_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_cp_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_cp_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failures = []
    for check in cp_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            failures.append((check.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every check"

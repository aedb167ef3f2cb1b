"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and require that at least one pin check fails: the pins must be able to see
a dropped term, a wrong index, a wrong sign or a transposed operand."""

import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "paged_attention.py")

MUTANTS = {
    "offset_off_by_one": ("off = t % B\n", "off = (t + 1) % B\n"),
    "block_and_offset_swapped": ("lb = t // B\n    off = t % B\n", "lb = t % B\n    off = t // B\n"),
    "slot_uses_logical_block": ("return pb * B + off", "return _lb * B + off"),
    "ceil_becomes_floor": ("return (L + B - 1) // B", "return L // B"),
    "range_end_not_clipped": ("return i * B, min((i + 1) * B, L)", "return i * B, (i + 1) * B"),
    "scale_dropped": ("logits = (q_rows @ Ks.T) * scale", "logits = (q_rows @ Ks.T)"),
    "logit_sign_flipped": ("logits = (q_rows @ Ks.T) * scale", "logits = -(q_rows @ Ks.T) * scale"),
    "no_normalisation": ("return (w @ Vs) / w.sum(axis=1, keepdims=True)", "return (w @ Vs)"),
    "gqa_modulo": ("out[s, g * G:(g + 1) * G] = attend(q[s, g * G:(g + 1) * G], Ks, Vs, scale)",
                   "out[s, g::num_kv_heads] = attend(q[s, g::num_kv_heads], Ks, Vs, scale)"),
    "v_not_transposed": ("Vs[lo:hi] = widen(v_pool[pb, kv_head, :, :n], dtype).T",
                         "Vs[lo:hi] = widen(v_pool[pb, kv_head, :n, :], dtype)"),
    "write_ignores_skip": ("        if slot < 0:\n            continue\n        b, o", "        b, o"),
    "copy_reversed": ("k_pool[int(dst)] = k_pool[int(src)]", "k_pool[int(src)] = k_pool[int(dst)]"),
    "v_write_wrong_axis": ("v_pool[b, :, :, o] = value_bits[i]", "v_pool[b, :, o % v_pool.shape[2], :] = value_bits[i][..., :v_pool.shape[3]]"),
    "empty_not_zero": ("        return np.zeros((q_rows.shape[0], Vs.shape[1]), dtype=np.float64)\n",
                       "        return np.full((q_rows.shape[0], Vs.shape[1]), np.nan)\n"),
    "gather_misses_last_block": ("for i in range(blocks_needed(L, B)):\n        lo, hi",
                                 "for i in range(max(blocks_needed(L, B) - 1, 1)):\n        lo, hi"),
    "bf16_widen_wrong_shift": ("(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)"),
    "kv_bytes_counts_k_only": ("return layers * tokens * kv_heads * head_dim * 2 * dtype_size",
                               "return layers * tokens * kv_heads * head_dim * dtype_size"),
    "kv_bytes_ignores_layers": ("return layers * tokens * kv_heads * head_dim * 2 * dtype_size",
                                "return tokens * kv_heads * head_dim * 2 * dtype_size"),
    "kv_bytes_ignores_dtype": ("return layers * tokens * kv_heads * head_dim * 2 * dtype_size",
                               "return layers * tokens * kv_heads * head_dim * 2 * 2"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            failures.append((check.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every pin"

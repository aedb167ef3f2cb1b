"""Structure and determinism of the seeded workloads (no GPU)."""

import math

import numpy as np
import pytest

import oracle
import workloads as W


def _rows(w, tables=None):
    t = w.block_tables if tables is None else tables
    return [[int(b) for b in t[s] if b >= 0] for s in range(w.num_seqs)]


def _check_tables(w, tables=None, private=True):
    t = w.block_tables if tables is None else tables
    for s in range(w.num_seqs):
        n = oracle.blocks_needed(int(w.context_lens[s]), w.block_size)
        row = t[s]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < w.num_blocks)
        assert np.all(row[n:] == -1)
    if private:
        ids = [b for r in _rows(w, t) for b in r]
        assert len(ids) == len(set(ids))


def _check_history(w):
    """Every slot written by the history and the step is distinct, and every
    position a sequence attends to is written exactly once (shared positions
    once per sharing group)."""
    B = w.block_size
    hs = oracle.slot_mapping(w.hist_block_tables, w.hist_seq, w.hist_pos, B)
    ns = oracle.slot_mapping(w.block_tables, w.new_seq, w.new_pos, B)
    assert np.all(hs >= 0) and np.all(ns >= 0)
    assert len(set(hs.tolist())) == len(hs)
    assert len(set(ns.tolist())) == len(ns)
    assert np.array_equal(w.new_pos, w.context_lens - 1)
    assert w.hist_key.shape == (len(w.hist_seq), w.num_kv_heads, w.head_dim)
    assert w.new_key.shape == (w.num_seqs, w.num_kv_heads, w.head_dim)
    assert w.q.shape == (w.num_seqs, w.num_heads, w.head_dim)


def test_tiny_config():
    w = W.tiny_f32()
    assert w.context_lens.tolist() == [1, 17, 40, 100]
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size) == (4, 2, 64, 16)
    assert w.num_blocks == 32 and w.max_blocks_per_seq == 7 and w.dtype == "f32"
    assert abs(w.scale - 1 / 8) < 1e-15
    _check_tables(w)
    _check_history(w)
    assert len(w.hist_seq) == sum(w.context_lens) - 4


def test_deterministic():
    a, b = W.tiny_f32(), W.tiny_f32()
    for f in ("block_tables", "q", "hist_key", "hist_value", "new_key", "new_value"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = W.tiny_f32(seed=1)
    assert not np.array_equal(a.q, c.q)


def test_llama_config_full_size():
    w = W.llama3_8b_decode()
    assert w.num_seqs == 64 and w.context_lens.min() >= 512 and w.context_lens.max() <= 4096
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.dtype) == (32, 8, 128, 16, "bf16")
    need = sum(oracle.blocks_needed(int(L), 16) for L in w.context_lens)
    assert w.num_blocks == math.ceil(1.25 * need)
    assert w.max_blocks_per_seq == 256
    _check_tables(w)
    for r in _rows(w):
        assert not all(b - a == 1 for a, b in zip(r, r[1:]))
    hs = oracle.slot_mapping(w.block_tables, w.new_seq, w.new_pos, 16)
    assert len(set(hs.tolist())) == 64


def test_bf16_values_look_normal():
    w = W.llama3_8b_decode(num_seqs=4, min_len=600, max_len=700)
    x = oracle.widen(w.hist_key, "bf16")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert np.abs(x).max() < 4.4 and not np.isnan(x).any()


def test_long_context_structure():
    w = W.long_context(num_seqs=2, min_len=3000, max_len=5000)
    _check_tables(w)
    _check_history(w)
    assert w.partition_size == 512 and w.max_blocks_per_seq == 5000 // 16 + 1


@pytest.mark.parametrize("phase", ["fork", "steady", "aligned"])
def test_shared_prefix_structure(phase):
    w = W.shared_prefix(phase, num_groups=3, branches=4, prefix_len=64, max_tail=40)
    G, Br = 3, 4
    _check_tables(w, private=False)
    _check_tables(w, w.hist_block_tables, private=False)
    _check_history(w)
    n_pre = 64 // 16
    for g in range(G):
        rows = [w.block_tables[g * Br + b] for b in range(Br)]
        for r in rows:
            assert np.array_equal(r[:n_pre], rows[0][:n_pre])
    prefixes = [tuple(w.block_tables[g * Br, :n_pre]) for g in range(G)]
    assert len(set(b for p in prefixes for b in p)) == G * n_pre
    if phase == "fork":
        assert len(w.copy_pairs) == G * (Br - 1)
        assert len(set(w.copy_pairs[:, 1].tolist())) == len(w.copy_pairs)
        hist_ids = set(int(b) for b in w.hist_block_tables.ravel() if b >= 0)
        assert not (set(w.copy_pairs[:, 1].tolist()) & hist_ids)
        for s in range(w.num_seqs):
            diff = np.nonzero(w.block_tables[s] != w.hist_block_tables[s])[0]
            assert len(diff) == (0 if s % Br == 0 else 1)
            assert 1 <= w.context_lens[s] - 64 - 1 <= 15
    else:
        assert len(w.copy_pairs) == 0
        assert np.array_equal(w.block_tables, w.hist_block_tables)
    if phase == "aligned":
        assert np.all(w.context_lens == 65)


def test_shared_prefix_full_counts():
    w = W.shared_prefix("fork")
    assert w.num_seqs == 256 and len(w.copy_pairs) == 240
    assert w.num_blocks == math.ceil(1.25 * 16 * (128 + 1 + 15))


def test_mixed_lengths_across_block_sizes():
    ws = {B: W.mixed_lengths(B, num_seqs=32) for B in (8, 16, 32)}
    for B, w in ws.items():
        assert w.block_size == B
        assert w.context_lens.min() >= 16 and w.context_lens.max() <= 8192
        _check_tables(w)
        _check_history(w)
    for f in ("context_lens", "q", "hist_key", "hist_value", "new_key", "new_value"):
        assert np.array_equal(getattr(ws[8], f), getattr(ws[32], f))
    full = W.mixed_lengths(16)
    # sample median of 256 lognormal(sigma=1) draws: standard error ~ 8% of 1024
    assert 780 < np.median(full.context_lens) < 1300


def test_pool_exhaustion_raises():
    with pytest.raises(RuntimeError):
        W.custom([40, 40], 2, 1, 8, 16, pool_factor=0.5)

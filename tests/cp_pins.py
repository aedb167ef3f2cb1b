"""Checks that pin the oracle's context-parallel pieces: rank ownership and
local slots, per-rank partial attention with its log-sum-exp, the merge of
the ranks' partials, and allocator-to-kernel block tables.

The central pin is the log-sum-exp identity: W ranks that each attend over
the tokens they own and are merged must give the unsplit decode of the same
sequence, which the decode's own pins fix."""

import math

import numpy as np

import workloads as W_


def _unsplit_and_ranks(o, w, world, interleave, kv_heads_bits=None):
    """Global decode of workload w, and the merge of `world` rank-local
    decodes built from cp slots."""
    ref = o.run_step(w)
    B = w.block_size
    qb = o.to_bits(w.q, w.dtype)
    seq = np.concatenate([w.hist_seq, w.new_seq])
    pos = np.concatenate([w.hist_pos, w.new_pos])
    key = np.concatenate([o.to_bits(w.hist_key, w.dtype), o.to_bits(w.new_key, w.dtype)])
    val = np.concatenate([o.to_bits(w.hist_value, w.dtype), o.to_bits(w.new_value, w.dtype)])
    # one table for every rank: virtual blocks of B * world tokens
    nvb = max(1, max(-(-int(L) // (B * world)) for L in w.context_lens))
    table = np.full((w.num_seqs, nvb), -1, dtype=np.int32)
    nxt = 0
    for s, L in enumerate(w.context_lens):
        for v in range(-(-int(L) // (B * world))):
            table[s, v] = nxt
            nxt += 1
    outs, lses, pools = [], [], []
    starts = np.arange(w.num_seqs + 1, dtype=np.int32)
    for r in range(world):
        kp, vp = o.new_pools(max(nxt, 1), w.num_kv_heads, B, w.head_dim, w.dtype)
        slots = o.cp_slot_mapping(table, seq, pos, B, world, r, interleave)
        o.write_kv(kp, vp, key, val, slots, B)
        lens = np.array([o.cp_context_len(int(L), B, world, r, interleave)
                         for L in w.context_lens])
        out_r, lse_r = o.prefill_lse(qb, kp, vp, table, lens, starts, w.scale, w.num_kv_heads,
                                     B, w.dtype)
        outs.append(out_r)
        lses.append(lse_r)
        pools.append((kp, vp, slots, lens))
    merged, _ = o.merge_states(np.stack(outs), np.stack(lses))
    return ref["out"], merged, table, pools


def check_cp_merge_equals_unsplit_decode(o):
    for dt, world, inter, B in (("f32", 2, 1, 16), ("f32", 4, 2, 8), ("bf16", 3, 4, 16),
                                ("f32", 4, 16, 16)):
        w = W_.custom([1, 5, 17, 40, 100, 33], 4, 2, 16, B, dt, seed=307_340 + world)
        ref, merged, _, _ = _unsplit_and_ranks(o, w, world, inter)
        assert np.allclose(merged, ref, rtol=0, atol=1e-12), (dt, world, inter)


def check_cp_local_sequences_are_dense(o):
    """A rank's tokens, in position order, fill its blocks' slots 0, 1, 2, ...
    one after another: the rank-local sequence is an ordinary paged sequence
    of cp_context_len tokens; every position has exactly one owner."""
    for B, world, inter in ((16, 2, 1), (8, 4, 2), (16, 3, 16), (32, 2, 8), (16, 1, 1)):
        L = 5 * B * world + 7
        counts = [0] * world
        for p in range(L):
            r = o.cp_owner(p, B, world, inter)
            assert 0 <= r < world
            local = (p // (B * world)) * B + o.cp_local_offset(p, B, world, inter)
            assert local == counts[r], (B, world, inter, p)
            counts[r] += 1
        for r in range(world):
            assert counts[r] == o.cp_context_len(L, B, world, r, inter)
        assert sum(counts) == L


def check_cp_world_one_is_the_plain_mapping(o):
    w = W_.tiny_f32()
    seq, pos = w.hist_seq, w.hist_pos
    assert np.array_equal(o.cp_slot_mapping(w.hist_block_tables, seq, pos, 16, 1, 0, 1),
                          o.slot_mapping(w.hist_block_tables, seq, pos, 16))
    for L in (0, 1, 17, 100):
        assert o.cp_context_len(L, 16, 1, 0) == L


def check_lse_closed_form(o):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 8))
    K = rng.standard_normal((11, 8))
    V = rng.standard_normal((11, 8))
    _, lse = o.attend_lse(q, K, V, 0.3)
    for i in range(3):
        brute = math.log(math.fsum(math.exp(0.3 * float(q[i] @ K[t])) for t in range(11)))
        assert abs(lse[i] - brute) < 1e-12
    o0, l0 = o.attend_lse(q, K[:0], V[:0], 0.3)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def check_merge_closed_forms(o):
    rng = np.random.default_rng(2)
    a = rng.standard_normal((5, 4))
    la = rng.standard_normal(5)
    out, lse = o.merge_states(a[None], la[None])
    assert np.allclose(out, a, atol=1e-15) and np.allclose(lse, la, atol=1e-15)
    out, lse = o.merge_states(np.stack([a, np.full_like(a, 7.0)]),
                              np.stack([la, np.full(5, -np.inf)]))
    assert np.allclose(out, a, atol=1e-15) and np.allclose(lse, la, atol=1e-15)
    out, lse = o.merge_states(np.stack([a, a]), np.stack([la, la]))
    assert np.allclose(out, a, atol=1e-14) and np.allclose(lse, la + math.log(2), atol=1e-14)
    out, lse = o.merge_states(np.zeros((2, 1, 4)), np.full((2, 1), -np.inf))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def check_kernel_tables_address_the_same_slots(o):
    """An allocator block of k kernel blocks: every token's slot number is the
    same through the allocator table at k*B and through the kernel table at
    B, so both address the same memory of a pool laid out in kernel blocks."""
    rng = np.random.default_rng(3)
    for k, Bk in ((2, 8), (4, 16), (1, 16), (2, 16)):
        Bm = k * Bk
        mt = np.full((3, 6), -1, dtype=np.int32)
        ids = rng.permutation(40)[:15]
        mt[0, :6], mt[1, :4], mt[2, :5] = ids[:6], ids[6:10], ids[10:15]
        kt = o.map_to_kernel_blocks(mt, k)
        assert kt.shape == (3, 6 * k)
        for r, nb in ((0, 6), (1, 4), (2, 5)):
            assert np.all(kt[r, nb * k:] == -1)
            for p in range(nb * Bm):
                assert o.slot_of(kt[r], p, Bk) == o.slot_of(mt[r], p, Bm)
        used = kt[kt >= 0]
        assert len(np.unique(used)) == len(used)


ALL_CHECKS = [
    check_cp_merge_equals_unsplit_decode,
    check_cp_local_sequences_are_dense,
    check_cp_world_one_is_the_plain_mapping,
    check_lse_closed_form,
    check_merge_closed_forms,
    check_kernel_tables_address_the_same_slots,
]

"""Checks that pin the oracle's prefill (causal attention of many query rows
per sequence over the paged cache) to what the pages and mathematics fix.

Each ``check_*`` takes the oracle module, so the same checks run against the
real oracle and against copies with a planted mistake
(``test_prefill_oracle.py``).  None restates the oracle's formula: each
compares it with an unpaged scalar-loop causal attention, with the separately
pinned decode, with a closed form, or with an invariant of causal attention.
"""

import numpy as np

import workloads as W


def _tiny(dtype="f32", lengths=(1, 5, 17, 40, 9), qlens=(1, 5, 3, 17, 9), Hq=4, Hkv=2, D=8, B=4,
          seed=307_310):
    return W.prefill(list(lengths), list(qlens), Hq, Hkv, D, B, dtype, seed=seed)


def check_prefill_equals_unpaged_causal_brute(o):
    """Paging moves K/V, the formula stays (P2 comparison table; P3): the
    paged prefill equals textbook causal attention on contiguous arrays."""
    for kw in ({}, {"Hq": 6, "Hkv": 2, "B": 8, "seed": 307_311},
               {"Hq": 2, "Hkv": 2, "B": 16, "lengths": (33, 16, 2), "qlens": (33, 4, 1)}):
        w = _tiny(**kw)
        got = o.run_prefill(w)["out"]
        seqs = o.contiguous_prefill_sequences(w)
        q = o.widen(o.to_bits(w.q, w.dtype), w.dtype)
        for s, (k, v) in enumerate(seqs):
            q0, q1 = int(w.query_start[s]), int(w.query_start[s + 1])
            L, n = int(w.context_lens[s]), q1 - q0
            ref = o.causal_attention_brute(q[q0:q1], k, v, [L - n + i for i in range(n)],
                                           w.scale, w.num_kv_heads)
            assert np.allclose(got[q0:q1], ref, rtol=0, atol=1e-12), f"sequence {s}"


def check_single_rows_are_the_decode(o):
    """n = 1 per sequence is the decode step: equal to the oracle's decode
    (pinned on its own) on the same pools."""
    w = _tiny(qlens=(1, 1, 1, 1, 1))
    r = o.run_prefill(w)
    dec = o.decode(o.to_bits(w.q, w.dtype), r["k_pool"], r["v_pool"], w.block_tables,
                   w.context_lens, w.scale, w.num_kv_heads, w.block_size, w.dtype)
    assert np.allclose(r["out"], dec, rtol=0, atol=1e-13)


def check_each_row_is_a_decode_at_its_position(o):
    """Row i of a chunk is the decode of the sequence cut after its position
    L - n + i (the table unchanged, the length L - n + i + 1)."""
    w = _tiny()
    r = o.run_prefill(w)
    qb = o.to_bits(w.q, w.dtype)
    for s in range(w.num_seqs):
        q0, q1 = int(w.query_start[s]), int(w.query_start[s + 1])
        L, n = int(w.context_lens[s]), q1 - q0
        for i in range(n):
            dec = o.decode(qb[q0 + i:q0 + i + 1], r["k_pool"], r["v_pool"],
                           w.block_tables[s:s + 1], np.array([L - n + i + 1]), w.scale,
                           w.num_kv_heads, w.block_size, w.dtype)
            assert np.allclose(r["out"][q0 + i], dec[0], rtol=0, atol=1e-13), (s, i)


def check_chunks_compose(o):
    """A prompt attended whole equals the same prompt in two chunks: the
    first chunk with only its own tokens cached, the second with all."""
    L, n1 = 37, 20
    whole = _tiny(lengths=(L,), qlens=(L,), seed=307_312)
    r = o.run_prefill(whole)
    qb = o.to_bits(whole.q, whole.dtype)
    part = []
    for Lc, n in ((n1, n1), (L, L - n1)):
        start = np.array([0, n])
        rows = qb[Lc - n:Lc]
        part.append(o.prefill(rows, r["k_pool"], r["v_pool"], whole.block_tables,
                              np.array([Lc]), start, whole.scale, whole.num_kv_heads,
                              whole.block_size, whole.dtype))
    assert np.allclose(np.concatenate(part), r["out"], rtol=0, atol=1e-13)


def check_prefill_block_permutation_invariance(o):
    """Moving blocks and rewriting the table changes nothing (P2 2.1)."""
    w = _tiny()
    r = o.run_prefill(w)
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    kp, vp = np.empty_like(r["k_pool"]), np.empty_like(r["v_pool"])
    kp[perm], vp[perm] = r["k_pool"], r["v_pool"]
    bt = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1)
    got = o.prefill(o.to_bits(w.q, w.dtype), kp, vp, bt, w.context_lens, w.query_start,
                    w.scale, w.num_kv_heads, w.block_size, w.dtype)
    assert np.array_equal(got, r["out"])


def check_closed_forms(o):
    """A one-token prompt returns its own V row exactly; identical keys make
    every row the mean of the V rows it sees."""
    w = _tiny(lengths=(1, 6), qlens=(1, 6), seed=307_313)
    r = o.run_prefill(w)
    vf = o.widen(o.to_bits(w.value, w.dtype), w.dtype)
    G = w.num_heads // w.num_kv_heads
    for h in range(w.num_heads):
        assert np.array_equal(r["out"][0, h], vf[0, h // G])
    key = w.key.copy()
    key[:] = key[0:1]
    w2 = W.PrefillWorkload(**{**w.__dict__, "key": key})
    r2 = o.run_prefill(w2)
    for i in range(6):
        row = 1 + i
        sel = np.nonzero(w.kv_seq == 1)[0][: i + 1]
        for h in range(w.num_heads):
            assert np.allclose(r2["out"][row, h], vf[sel, h // G].mean(axis=0), atol=1e-12)


def check_rows_without_tokens_are_zero(o):
    """More query rows than cached tokens (a broken precondition): rows at
    negative positions see nothing and are zero; the others are unaffected."""
    w = _tiny(lengths=(3,), qlens=(3,), seed=307_314)
    r = o.run_prefill(w)
    qb = o.to_bits(w.q, w.dtype)
    extra = np.concatenate([qb[:2], qb])
    got = o.prefill(extra, r["k_pool"], r["v_pool"], w.block_tables, w.context_lens,
                    np.array([0, 5]), w.scale, w.num_kv_heads, w.block_size, w.dtype)
    assert np.array_equal(got[:2], np.zeros_like(got[:2]))
    assert np.array_equal(got[2:], r["out"])


ALL_CHECKS = [
    check_prefill_equals_unpaged_causal_brute,
    check_single_rows_are_the_decode,
    check_each_row_is_a_decode_at_its_position,
    check_chunks_compose,
    check_prefill_block_permutation_invariance,
    check_closed_forms,
    check_rows_without_tokens_are_zero,
]

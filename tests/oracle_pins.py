"""Checks that pin the CPU oracle to what the pages and mathematics fix.

Each ``check_*`` takes the oracle module as its argument, so the same checks
run against the real oracle (``test_oracle_pins.py``) and against copies with
a planted mistake (``test_oracle_mutants.py``), which must fail at least one.
None of them re-derives the oracle by retyping its formulas: each compares it
with a printed value, an independent brute force, a closed form or an
invariant.
"""

import json
import math
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_step(o):
    w = W.tiny_f32()
    return w, o.run_step(w)


# ---------------------------------------------------------------- indexing

def check_worked_example(o):
    """P3's worked example: L=40, B=16 -> 3 blocks, table 7 -> 2 -> 15."""
    g = _golden("worked_example.json")
    p = g["printed"]
    B, L, row = p["block_size"], p["sequence_length"], p["block_table"]
    assert o.blocks_needed(L, B) == p["num_blocks"]
    for i, (lo, hi) in enumerate(p["logical_token_ranges_inclusive"]):
        assert o.block_token_range(i, L, B) == (lo, hi + 1)
    for lo, hi, phys in p["capacity_ranges_inclusive"]:
        for t in range(lo, min(hi, L - 1) + 1):
            assert o.translate(t, row, B)[2] == phys
    for tok in g["derived"]["tokens"]:
        assert o.translate(tok["t"], row, B) == (tok["logical"], tok["offset"], tok["physical"])
        assert o.slot_of(row, tok["t"], B) == tok["slot"]


def _on_demand_blocks(L, B):
    """Append tokens one at a time; open a block only when the tail is full
    (P1: decode fills the unfilled tail block first)."""
    blocks, fill = 0, B
    for _ in range(L):
        if fill == B:
            blocks, fill = blocks + 1, 0
        fill += 1
    return blocks, (fill if blocks else 0)


def check_block_counts(o):
    """ceil(L/B) equals on-demand allocation; tail waste in [0, B-1]; P3's L=17."""
    for B in (8, 16, 32):
        for L in range(0, 200):
            n, last_fill = _on_demand_blocks(L, B)
            assert o.blocks_needed(L, B) == n
            waste = o.tail_waste([L], B)
            assert waste == (B - last_fill if n else 0)
            assert 0 <= waste <= B - 1
            covered = []
            for i in range(n):
                lo, hi = o.block_token_range(i, L, B)
                covered.extend(range(lo, hi))
            assert covered == list(range(L))
    c = _golden("capacity_numbers.json")
    l17 = c["length17"]
    assert o.blocks_needed(l17["length"], l17["block_size"]) == l17["blocks"]
    lo, hi = o.block_token_range(1, l17["length"], l17["block_size"])
    assert hi - lo == l17["tokens_in_last_block"]
    mx = c["max_tail_waste"]
    assert max(o.tail_waste([L], mx["block_size"]) for L in range(1, 100)) == mx["slots"]
    pre = c["prealloc"]
    assert o.prealloc_waste([pre["used"]], pre["max_len"]) == pre["wasted"]


def check_tiny_closed_form(o):
    """Config {1, 17, 40, 100} at B=16: 1+2+3+7 = 13 blocks, 15+15+8+12 = 50
    tail slots, fragmentation proxy 50 / 208."""
    lengths = [1, 17, 40, 100]
    assert sum(o.blocks_needed(L, 16) for L in lengths) == 13
    assert o.tail_waste(lengths, 16) == 50
    assert abs(o.fragmentation_proxy(lengths, 16) - 50 / 208) < 1e-15
    assert o.fragmentation_proxy([16, 32, 48], 16) == 0.0


def check_slot_roundtrip(o):
    """Write a distinct marker through every (sequence, position) slot, read it
    back through the block table: each sequence sees its markers in order."""
    w = W.tiny_f32()
    B = w.block_size
    seq = np.concatenate([np.full(int(L), s, np.int32) for s, L in enumerate(w.context_lens)])
    pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in w.context_lens])
    slots = o.slot_mapping(w.block_tables, seq, pos, B)
    assert len(set(slots.tolist())) == len(slots)
    assert slots.min() >= 0 and slots.max() < w.num_blocks * B
    k, v = o.new_pools(w.num_blocks, 1, B, 1, "f32")
    marker = np.arange(1, len(seq) + 1, dtype=np.float32).reshape(-1, 1, 1)
    o.write_kv(k, v, marker.view(np.uint32), (marker * 2).view(np.uint32), slots, B)
    at = 0
    for s, L in enumerate(w.context_lens):
        Ks, Vs = o.gather(k, v, w.block_tables[s], int(L), 0, B, "f32")
        want = np.arange(at + 1, at + int(L) + 1, dtype=np.float64)
        assert np.array_equal(Ks[:, 0], want) and np.array_equal(Vs[:, 0], 2 * want)
        at += int(L)
    # -1 rows are skipped and leave the pool untouched
    before_k, before_v = k.copy(), v.copy()
    bad = np.array([-1, -1], np.int64)
    o.write_kv(k, v, np.zeros((2, 1, 1), np.uint32), np.zeros((2, 1, 1), np.uint32), bad, B)
    assert np.array_equal(k, before_k) and np.array_equal(v, before_v)
    neg = o.slot_mapping(w.block_tables, np.array([-1, 0]), np.array([3, -2]), B)
    assert neg.tolist() == [-1, -1]


def check_write_layout(o):
    """A written row lands whole in its block: K at [b, :, off, :], V^T at
    [b, :, :, off], and nothing else changes."""
    B, Hkv, D, NB = 8, 2, 4, 3
    k, v = o.new_pools(NB, Hkv, B, D, "bf16")
    key = np.arange(Hkv * D, dtype=np.uint16).reshape(1, Hkv, D) + 1
    val = key + 100
    o.write_kv(k, v, key, val, np.array([1 * B + 5]), B)
    written_k = np.argwhere(k != o.POISON["bf16"])
    written_v = np.argwhere(v != o.POISON["bf16"])
    assert len(written_k) == Hkv * D and len(written_v) == Hkv * D
    assert set(written_k[:, 0]) == {1} and set(written_k[:, 2]) == {5}
    assert set(written_v[:, 0]) == {1} and set(written_v[:, 3]) == {5}
    assert np.array_equal(k[1, :, 5, :], key[0]) and np.array_equal(v[1, :, :, 5], val[0])


# ---------------------------------------------------------------- attention

def check_paged_equals_unpaged(o):
    """Paging only moves data (P2's comparison table: same formula, different
    access path): the oracle on the paged pool equals textbook attention over
    the contiguous sequences, and equals ``attend`` on the contiguous arrays
    bit for bit."""
    w, r = _tiny_step(o)
    q = o.widen(o.to_bits(w.q, w.dtype), w.dtype)
    G = w.num_heads // w.num_kv_heads
    for s, (k_seq, v_seq) in enumerate(o.contiguous_sequences(w)):
        ref = o.attention_unpaged_brute(q[s], k_seq, v_seq, w.scale, w.num_kv_heads)
        assert np.max(np.abs(r["out"][s] - ref)) < 1e-12
        for g in range(w.num_kv_heads):
            direct = o.attend(q[s, g * G:(g + 1) * G], k_seq[:, g, :], v_seq[:, g, :], w.scale)
            assert np.array_equal(direct, r["out"][s, g * G:(g + 1) * G])


def check_numpy_equals_brute(o):
    """The NumPy path and the scalar-loop path through the same pool agree."""
    w, r = _tiny_step(o)
    brute = o.decode_brute(o.to_bits(w.q, w.dtype), r["k_pool"], r["v_pool"], w.block_tables,
                           w.context_lens, w.scale, w.num_kv_heads, w.block_size, w.dtype)
    assert np.max(np.abs(brute - r["out"])) < 1e-12


def check_permutation_invariance(o):
    """Blocks may sit anywhere (P2: logically contiguous, physically scattered):
    moving every block and rewriting the tables leaves the output bit-identical."""
    w, r = _tiny_step(o)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(w.num_blocks)
    k2 = np.empty_like(r["k_pool"]); v2 = np.empty_like(r["v_pool"])
    k2[perm] = r["k_pool"]; v2[perm] = r["v_pool"]
    t2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    out2 = o.decode(o.to_bits(w.q, w.dtype), k2, v2, t2, w.context_lens, w.scale,
                    w.num_kv_heads, w.block_size, w.dtype)
    assert np.array_equal(out2, r["out"])


def _pool_from_rows(o, k_rows, v_rows, B, dtype="f32"):
    """One sequence, one KV head, rows placed in reversed block order."""
    L, D = k_rows.shape
    nb = o.blocks_needed(L, B)
    k, v = o.new_pools(nb + 1, 1, B, D, dtype)
    row = np.arange(nb, 0, -1, dtype=np.int32)
    slots = o.slot_mapping(row.reshape(1, -1), np.zeros(L, np.int32), np.arange(L), B)
    o.write_kv(k, v, k_rows.astype(np.float32).reshape(L, 1, D).view(np.uint32),
               v_rows.astype(np.float32).reshape(L, 1, D).view(np.uint32), slots, B)
    return k, v, row.reshape(1, -1)


def check_closed_forms(o):
    """Softmax special cases: L=1 returns the V row; q=0 or identical K rows
    return the mean V row; one dominant logit returns its V row; the weight
    ratio of two tokens is exp(scale * (q.k1 - q.k2))."""
    rng = np.random.Generator(np.random.PCG64(11))
    B, D = 8, 4
    def run(qv, krows, vrows, scale=0.5):
        k, v, row = _pool_from_rows(o, krows, vrows, B)
        qb = np.asarray(qv, np.float32).reshape(1, 1, D).view(np.uint32)
        return o.decode(qb, k, v, row, np.array([len(krows)], np.int32), scale, 1, B, "f32")[0, 0]
    kr = rng.standard_normal((1, D)).astype(np.float32)
    vr = rng.standard_normal((1, D)).astype(np.float32)
    assert np.array_equal(run(rng.standard_normal(D), kr, vr), vr[0].astype(np.float64))
    K = rng.standard_normal((21, D)).astype(np.float32)
    V = rng.standard_normal((21, D)).astype(np.float32)
    mean = V.astype(np.float64).mean(axis=0)
    assert np.max(np.abs(run(np.zeros(D), K, V) - mean)) < 1e-12
    same = np.repeat(K[:1], 21, axis=0)
    assert np.max(np.abs(run(rng.standard_normal(D), same, V) - mean)) < 1e-12
    qd = np.zeros(D, np.float32); qd[0] = 1.0
    Kd = np.zeros((21, D), np.float32); Kd[13, 0] = 4000.0
    assert np.array_equal(run(qd, Kd, V), V[13].astype(np.float64))
    # two tokens, V rows e0 and e1: out = (w0, w1) with w0/w1 = exp(scale * (q.k0 - q.k1))
    q2 = np.array([1.0, 0, 0, 0], np.float32)
    K2 = np.array([[3.0, 0, 0, 0], [1.0, 0, 0, 0]], np.float32)
    V2 = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]], np.float32)
    out = run(q2, K2, V2, scale=0.25)
    w0 = 1.0 / (1.0 + math.exp(-0.25 * 2.0))
    assert abs(out[0] - w0) < 1e-15 and abs(out[1] - (1 - w0)) < 1e-15


def check_gqa_grouping(o):
    """Query head h reads KV head h // (Hq / Hkv): with KV head 0's V all 0 and
    KV head 1's all 1, query heads 0,1 give 0 and heads 2,3 give 1."""
    B, D, Hq, Hkv, L = 16, 4, 4, 2, 5
    k, v = o.new_pools(2, Hkv, B, D, "f32")
    rng = np.random.Generator(np.random.PCG64(3))
    keys = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    vals = np.zeros((L, Hkv, D), np.float32); vals[:, 1, :] = 1.0
    row = np.array([[1]], np.int32)
    slots = o.slot_mapping(row, np.zeros(L, np.int32), np.arange(L), B)
    o.write_kv(k, v, keys.view(np.uint32), vals.view(np.uint32), slots, B)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = o.decode(q.view(np.uint32), k, v, row, np.array([L], np.int32), 0.5, Hkv, B, "f32")
    assert np.allclose(out[0, :2], 0.0, atol=1e-14) and np.allclose(out[0, 2:], 1.0, atol=1e-14)


def check_empty_sequence(o):
    """L = 0 attends over nothing and returns zeros without reading the table."""
    k, v = o.new_pools(1, 1, 16, 4, "f32")
    q = np.ones((1, 2, 4), np.float32)
    out = o.decode(q.view(np.uint32), k, v, np.full((1, 1), -1, np.int32),
                   np.array([0], np.int32), 1.0, 1, 16, "f32")
    assert np.array_equal(out, np.zeros((1, 2, 4)))


# ---------------------------------------------------------------- copy-on-write

def check_copy_on_write(o):
    """After the copy, dst equals src bit for bit; src and every other block
    are unchanged; a branch reading a private copy of a shared block gets the
    same output as before (P1: copy-on-write keeps the original for others)."""
    w = W.shared_prefix("fork", num_groups=2, branches=3, prefix_len=32, max_tail=8)
    B = w.block_size
    k, v = o.new_pools(w.num_blocks, w.num_kv_heads, B, w.head_dim, w.dtype)
    hs = o.slot_mapping(w.hist_block_tables, w.hist_seq, w.hist_pos, B)
    o.write_kv(k, v, w.hist_key, w.hist_value, hs, B)
    k0, v0 = k.copy(), v.copy()
    o.copy_blocks(k, v, w.copy_pairs)
    dst = set(int(d) for d in w.copy_pairs[:, 1])
    for src, d in w.copy_pairs:
        assert np.array_equal(k[d], k0[src]) and np.array_equal(v[d], v0[src])
    for b in range(w.num_blocks):
        if b not in dst:
            assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])
    # reading through the pre-copy (shared) or post-copy (private) tables is
    # the same before the step's write
    lens = w.context_lens - 1
    q = o.to_bits(w.q, w.dtype)
    a = o.decode(q, k, v, w.hist_block_tables, lens, w.scale, w.num_kv_heads, B, w.dtype)
    b2 = o.decode(q, k, v, w.block_tables, lens, w.scale, w.num_kv_heads, B, w.dtype)
    assert np.array_equal(a, b2)


def check_bf16_widening(o):
    """bfloat16 bits widen exactly: IEEE values, and torch's own conversion of
    every one of the 65536 patterns (NaNs compared as NaN)."""
    import torch

    known = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x4049: 3.140625, 0x0001: 2.0 ** -133,
             0x7F7F: 3.3895313892515355e38, 0xFF80: -math.inf, 0x0000: 0.0}
    bits = np.array(list(known), np.uint16)
    assert np.array_equal(o.widen(bits, "bf16"), np.array(list(known.values())))
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = o.widen(allbits, "bf16")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    f = np.array([1.0, -0.1, 7e-39, np.inf], np.float32)
    assert np.array_equal(o.widen(f.view(np.uint32), "f32"), f.astype(np.float64))


# ---------------------------------------------------------------- capacity

def check_kv_bytes(o):
    """P3's KV-size estimate (section on why KV becomes a memory problem):
    the bytes must be what the cache really stores.  Pin: write one token
    through ``write_kv`` into fresh pools of one-slot blocks and count the
    bytes that change; that is the size of one token in one layer.  The
    estimate must equal it for K and V rows of both element types, and grow
    linearly in layers and in tokens (the page's two conclusions: linear in
    token count and in concurrent requests).  The page's own example, a
    2048-token prompt with 512 generated tokens, then needs 2560 tokens'
    worth per layer."""
    markers = {"f32": 0x11223344, "bf16": 0x1234}  # every byte differs from the pool poison
    for dtype, elem in (("f32", 4), ("bf16", 2)):
        for Hkv, D in ((1, 4), (2, 64), (8, 128)):
            k, v = o.new_pools(3, Hkv, 1, D, dtype)
            k0, v0 = k.copy(), v.copy()
            sd = k.dtype
            row = np.full((1, Hkv, D), markers[dtype], dtype=sd)
            o.write_kv(k, v, row, row, np.array([1], np.int64), 1)
            changed = int(np.count_nonzero(k.view(np.uint8) != k0.view(np.uint8)) +
                          np.count_nonzero(v.view(np.uint8) != v0.view(np.uint8)))
            assert changed == 2 * Hkv * D * elem  # both rows were written whole
            one = o.kv_bytes(1, 1, Hkv, D, elem)
            assert one == changed
            for layers, tokens in ((1, 7), (32, 1), (32, 2560), (3, 5)):
                assert o.kv_bytes(layers, tokens, Hkv, D, elem) == layers * tokens * changed
    ex = _golden("capacity_numbers.json")["context_example"]
    assert ex["prompt"] + ex["generated"] == ex["context"]
    per_layer = o.kv_bytes(1, ex["context"], 8, 128, 2)
    assert per_layer == o.kv_bytes(1, ex["prompt"], 8, 128, 2) + o.kv_bytes(1, ex["generated"], 8, 128, 2)


ALL_CHECKS = [
    check_bf16_widening,
    check_worked_example, check_block_counts, check_tiny_closed_form, check_slot_roundtrip,
    check_write_layout, check_paged_equals_unpaged, check_numpy_equals_brute,
    check_permutation_invariance, check_closed_forms, check_gqa_grouping,
    check_empty_sequence, check_copy_on_write, check_kv_bytes,
]

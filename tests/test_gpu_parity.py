"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Bit-exact: slot mappings, pools after writes and copies.  Within tolerance
(max abs, fp32 1e-5, bf16 2e-2 with fp32 accumulation): decode outputs element
by element, at small sizes and at the five full workload sizes.
"""

import types

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_307_amd as pa
import workloads as W
from gpu_common import TOL, as_f64, assert_pool_equal, bits, dev, max_err, pools_from_oracle, run_step

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _check_step(w, partition_size, seqs=None, kv_heads=None, check_pool=True, two_phase=False,
                ref=None, append=False, shared_blocks=False):
    _say(f"{w.name} S={w.num_seqs} Hq={w.num_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
         f"B={w.block_size} {w.dtype} P={partition_size}" + (" two-phase" if two_phase else "")
         + (" append" if append else "") + (" shared-blocks" if shared_blocks else ""))
    if ref is None:
        ref = oracle.run_step(w, seqs=seqs, kv_heads=kv_heads)
    r = run_step(w, partition_size, keep=True, two_phase=two_phase, append=append,
                 shared_blocks=shared_blocks)
    assert np.array_equal(bits(r["hist_slots"]), ref["hist_slots"])
    assert np.array_equal(bits(r["new_slots"]), ref["new_slots"])
    if check_pool:
        assert_pool_equal(w, r["k"], r["v"], ref["k_pool"], ref["v_pool"])
    err = max_err(r["out"], ref["out"], seqs, kv_heads, w)
    print(f"[case] max abs err {err:.3e} (tol {TOL[w.dtype]})", flush=True)
    assert err <= TOL[w.dtype]
    return r, ref


# ------------------------------------------------------------- small, exhaustive

@pytest.mark.parametrize("P", [0, 16, 32, 64])
def test_tiny_f32(P):
    w = W.tiny_f32()
    ref = oracle.run_step(w)
    _check_step(w, P, ref=ref)
    _check_step(w, P, ref=ref, append=True)


@pytest.mark.parametrize("P", [0, 16, 48])
def test_tiny_shape_bf16(P):
    w = W.custom([1, 17, 40, 100], 4, 2, 64, 16, "bf16", seed=307_011, name="tiny_bf16")
    ref = oracle.run_step(w)
    _check_step(w, P, ref=ref)
    _check_step(w, P, ref=ref, append=True)


RAGGED = list(range(1, 41)) + [63, 64, 65, 127, 128, 129, 255, 257, 511, 512, 513, 700]

SHAPES = [  # (Hq, Hkv, D, B, dtype)
    (4, 2, 64, 16, "bf16"), (32, 8, 128, 16, "bf16"), (64, 8, 128, 8, "bf16"),
    (64, 8, 128, 32, "bf16"), (16, 1, 128, 16, "bf16"), (8, 8, 64, 16, "bf16"),
    (32, 2, 256, 16, "bf16"), (12, 4, 128, 8, "bf16"),
    (4, 2, 64, 16, "f32"), (32, 8, 128, 8, "f32"), (16, 16, 256, 32, "f32"), (6, 2, 64, 32, "f32"),
]


@pytest.mark.parametrize("shape", [(16, 2, 128), (8, 2, 64), (32, 2, 256)],
                         ids=lambda s: "Hq%d_Hkv%d_D%d" % s)
def test_b32_block_halves(shape):
    """B = 32: a block whose tokens span both halves is decoded as two tiles
    that each take every other group of four tokens (one 16-byte V load
    fetches both tiles' values).  Every length 1..96 three times over, so
    runs start at either half of a block, blocks end in either half, and
    the appended row (token L - 1) lies in either tile; split, single pass,
    two launches, rows appended or written first."""
    Hq, Hkv, D = shape
    lengths = list(range(1, 97)) * 3
    w = W.custom(lengths, Hq, Hkv, D, 32, "bf16", seed=307_060 + Hq + D)
    ref = oracle.run_step(w)
    for P in (0, 32, 512):
        _check_step(w, P, ref=ref)
        _check_step(w, P, ref=ref, append=True)
    _check_step(w, 64, ref=ref, two_phase=True, append=True)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "Hq%d_Hkv%d_D%d_B%d_%s" % s)
def test_ragged_lengths(shape):
    Hq, Hkv, D, B, dt = shape
    w = W.custom(RAGGED, Hq, Hkv, D, B, dt, seed=307_020 + Hq + D + B)
    ref = oracle.run_step(w)
    for P in (0, max(32, B), 512):
        _check_step(w, P, ref=ref)
    _check_step(w, max(32, B), ref=ref, two_phase=True)
    # the appending step: the decode writes each sequence's row itself
    for P in (0, max(32, B)):
        _check_step(w, P, ref=ref, append=True)
    _check_step(w, 512, ref=ref, append=True, two_phase=True)


def test_two_phase_and_one_launch_agree():
    """pa_decode (bf16: one launch, one record per worker share) and
    pa_decode_partials + pa_decode_merge (one record per partition piece)
    fold the same softmax in different orders: both match the oracle, and
    each other to within rounding."""
    w = W.custom([5, 100, 600, 1500], 32, 8, 128, 16, "bf16", seed=307_031)
    r = run_step(w, 0, keep=True)
    ws = pa.alloc_workspace(w.num_seqs, 32, 8, 128, w.max_context_len, 64)
    q = dev(w.q)
    full = pa.decode(q, r["k"], r["v"], r["bt"], r["cl"], w.max_context_len, w.scale,
                     partition_size=64, workspace=ws)
    out = torch.empty_like(q)
    pa.decode_partials(q, r["k"], r["v"], r["bt"], r["cl"], w.max_context_len, w.scale, 64, ws, out)
    pa.decode_merge(out, r["cl"], 8, 16, w.max_blocks_per_seq, w.max_context_len, 64, ws)
    torch.cuda.synchronize()
    ref = oracle.run_step(w)["out"]
    assert np.max(np.abs(as_f64(out) - ref)) <= TOL["bf16"]
    assert np.max(np.abs(as_f64(full) - ref)) <= TOL["bf16"]
    assert np.max(np.abs(as_f64(full) - as_f64(out))) <= TOL["bf16"]


def test_workspace_reused_across_shapes_and_launches():
    """One zero-filled workspace serves decodes of different shapes in turn
    (its counters and records shift with the shape): every launch's stamps
    keep leftovers of the others out, so each result matches the oracle."""
    shapes = [
        W.custom([5, 100, 600, 1500], 32, 8, 128, 16, "bf16", seed=307_032),
        W.custom(list(range(1, 61)), 16, 4, 128, 16, "bf16", seed=307_033),
        W.custom([2000, 3, 77], 8, 8, 64, 32, "bf16", seed=307_034),
    ]
    size = max(pa.decode_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                         w.max_context_len, 64) for w in shapes)
    ws = torch.zeros(size // 4 + 4, dtype=torch.float32, device="cuda")
    state = []
    for w in shapes:
        r = run_step(w, 0, keep=True)
        state.append((w, r, oracle.run_step(w)["out"]))
    for rep in range(3):
        for w, r, ref in state:
            _say(f"workspace reuse rep {rep} {w.name} S={w.num_seqs}")
            out = pa.decode(dev(w.q), r["k"], r["v"], r["bt"], r["cl"], w.max_context_len,
                            w.scale, partition_size=64, workspace=ws)
            torch.cuda.synchronize()
            assert np.max(np.abs(as_f64(out) - ref)) <= TOL["bf16"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_zero_and_short_lengths_decode(dt):
    """Decode only, on the oracle's pool, with some context lengths cut to 0
    and others shortened: L = 0 gives zeros, the rest match the oracle."""
    w = W.custom([30, 70, 1, 200, 16], 8, 2, 64, 16, dt, seed=307_041)
    ref = oracle.run_step(w)
    lens = np.array([0, 33, 0, 129, 16], np.int32)
    want = oracle.decode(oracle.to_bits(w.q, dt), ref["k_pool"], ref["v_pool"], w.block_tables,
                         lens, w.scale, w.num_kv_heads, w.block_size, dt)
    k, v = pools_from_oracle(w, ref["k_pool"], ref["v_pool"])
    for P in (0, 16, 64):
        _say(f"zero/short lengths {dt} P={P}")
        out = pa.decode(dev(w.q), k, v, dev(w.block_tables), dev(lens), int(lens.max()), w.scale,
                        partition_size=P)
        torch.cuda.synchronize()
        got = as_f64(out)
        assert np.all(got[[0, 2]] == 0.0)
        assert np.max(np.abs(got - want)) <= TOL[dt]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_append_with_zero_and_short_lengths(dt):
    """pa_append_decode on the oracle's pool with some lengths cut to 0 and
    others shortened: each sequence with L > 0 gets its row at position
    L - 1 (bit-exact pools), L = 0 writes nothing and gives zeros."""
    w = W.custom([30, 70, 1, 200, 16], 8, 2, 64, 16, dt, seed=307_042)
    base = oracle.run_step(w)
    lens = np.array([0, 33, 0, 129, 16], np.int32)
    live = np.nonzero(lens > 0)[0].astype(np.int32)
    for P in (0, 16, 64):
        _say(f"append zero/short lengths {dt} P={P}")
        kb, vb = base["k_pool"].copy(), base["v_pool"].copy()
        slots = oracle.slot_mapping(w.block_tables, live, lens[live] - 1, w.block_size)
        oracle.write_kv(kb, vb, oracle.to_bits(w.new_key, dt)[live],
                        oracle.to_bits(w.new_value, dt)[live], slots, w.block_size)
        want = oracle.decode(oracle.to_bits(w.q, dt), kb, vb, w.block_tables, lens, w.scale,
                             w.num_kv_heads, w.block_size, dt)
        k, v = pools_from_oracle(w, base["k_pool"], base["v_pool"])
        out = pa.append_decode(dev(w.q), dev(w.new_key), dev(w.new_value), k, v,
                               dev(w.block_tables), dev(lens), int(lens.max()), w.scale,
                               partition_size=P)
        torch.cuda.synchronize()
        assert_pool_equal(w, k, v, kb, vb)
        got = as_f64(out)
        assert np.all(got[[0, 2]] == 0.0)
        assert np.max(np.abs(got - want)) <= TOL[dt]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_context_lens_clamped(dt):
    """context_lens beyond max_context_len, or beyond the table's capacity
    (max_blocks_per_seq * B = 112 here, every row full), are clamped to the
    smaller bound."""
    w = W.custom([112, 112, 112, 112], 8, 2, 64, 16, dt, seed=307_043)
    ref = oracle.run_step(w)
    k, v = pools_from_oracle(w, ref["k_pool"], ref["v_pool"])
    cap = w.max_blocks_per_seq * w.block_size
    assert cap == 112
    lens = np.array([40, 500, 100, 10_000], np.int32)
    for max_len in (80, 200):                       # below and above the capacity
        eff = np.minimum(np.minimum(lens, max_len), cap).astype(np.int32)
        want = oracle.decode(oracle.to_bits(w.q, dt), ref["k_pool"], ref["v_pool"],
                             w.block_tables, eff, w.scale, w.num_kv_heads, w.block_size, dt)
        for P in (0, 32):
            _say(f"clamped lengths {dt} max_len={max_len} P={P}")
            out = pa.decode(dev(w.q), k, v, dev(w.block_tables), dev(lens), max_len, w.scale,
                            partition_size=P)
            torch.cuda.synchronize()
            assert np.max(np.abs(as_f64(out) - want)) <= TOL[dt]


def test_side_stream_and_repeat_are_bit_identical():
    """The ABI runs on the caller's stream: a decode on a side stream gives
    the same bits as on the default stream, and repeating a launch
    reproduces them (the schedule and the merge order are deterministic)."""
    w = W.custom([5, 100, 600, 1500, 17], 32, 8, 128, 16, "bf16", seed=307_044)
    r = run_step(w, 0, keep=True)
    q = dev(w.q)
    args = (q, r["k"], r["v"], r["bt"], r["cl"], w.max_context_len, w.scale)
    base = pa.decode(*args, partition_size=64)
    again = pa.decode(*args, partition_size=64)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = pa.decode(*args, partition_size=64)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(base, again) and torch.equal(base, other)
    ref = oracle.run_step(w)["out"]
    assert np.max(np.abs(as_f64(base) - ref)) <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(8, 2, 64, 8), (32, 8, 128, 16), (16, 4, 128, 32),
                                   (8, 1, 256, 16)])
def test_cache_policies_give_identical_bits(shape):
    """PA_DECODE_SHARED_BLOCKS changes only the cache bits of the K/V loads:
    outputs and pools are bit-identical to the streaming policy's, in single
    pass, split, two-phase and appending launches."""
    Hq, Hkv, D, B = shape
    w = W.custom([1, 16, 17, 200, 700, 1500], Hq, Hkv, D, B, "bf16", seed=307_045 + D + B)
    ref = oracle.run_step(w)["out"]
    for P, two_phase, append in ((0, False, False), (64, False, False), (512, True, False),
                                 (0, False, True), (256, True, True)):
        _say(f"cache policies Hq={Hq} Hkv={Hkv} D={D} B={B} P={P} two_phase={two_phase} "
             f"append={append}")
        a = run_step(w, P, keep=True, two_phase=two_phase, append=append, shared_blocks=False)
        b = run_step(w, P, keep=True, two_phase=two_phase, append=append, shared_blocks=True)
        assert np.array_equal(bits(a["out"]), bits(b["out"]))
        assert torch.equal(a["k"].view(torch.int16), b["k"].view(torch.int16))
        assert torch.equal(a["v"].view(torch.int16), b["v"].view(torch.int16))
        assert np.max(np.abs(as_f64(a["out"]) - ref)) <= TOL["bf16"]


@pytest.mark.parametrize("shape", [
    # (lengths, Hq, Hkv, D): G = 16 at D = 128 stages 3 records per run, G = 16
    # at D = 256 one; G = 4 at D = 128 stages 15, and 20000-token pairs in
    # 16-token partitions give runs of ~28 partitions
    ([6000, 7000, 5000, 30], 32, 2, 128),
    ([6000, 7000, 5000, 30], 16, 1, 256),
    ([20000, 20000, 3000, 17], 32, 8, 128),
])
def test_partition_records_staged_and_drained(shape):
    """Split runs that pass many partition ends stage the partitions'
    records in LDS and store them in bursts, also in mid-run when the
    staging area fills; every record must reach the merge."""
    lengths, Hq, Hkv, D = shape
    w = W.custom(lengths, Hq, Hkv, D, 16, "bf16", seed=307_046 + Hq + D)
    ref = oracle.run_step(w)  # every (sequence, KV head) pair, element by element
    for P in (16, 32):
        _check_step(w, P, check_pool=False, ref=ref)
    _check_step(w, 16, ref=ref, append=True, two_phase=True)


@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (16, 4, 64, 8), (16, 2, 256, 32)])
def test_append_many_short_sequences(shape):
    """Hundreds of 1..40-token sequences: each split worker holds the last
    tile of several pairs, so it keeps two write-back tiles in LDS and
    stores the rest at once; the pools must match the oracle bit for bit."""
    Hq, Hkv, D, B = shape
    rng = np.random.default_rng(307_047 + D)
    lengths = [int(x) for x in rng.integers(1, 41, size=640 if D < 256 else 320)]
    w = W.custom(lengths, Hq, Hkv, D, B, "bf16", seed=307_048 + D + B)
    ref = oracle.run_step(w)
    for P in (0, 16 if B <= 16 else 32, 64):
        _check_step(w, P, ref=ref, append=True, two_phase=P > 0)


def test_single_token_is_exact_copy():
    """L = 1: the output is the token's V row, bit for bit after rounding."""
    w = W.custom([1, 1, 1], 8, 4, 128, 16, "bf16", seed=307_051)
    r = run_step(w, 0)
    G = 2
    want = np.repeat(w.new_value, G, axis=1)  # [S, Hq, D] bf16 bits
    assert np.array_equal(bits(r["out"]), want)


# ------------------------------------------------------------- write / copy / slots

def test_write_skips_negative_and_out_of_range_slots():
    w = W.custom([40, 17], 4, 2, 64, 16, "bf16", seed=307_061)
    ref = oracle.run_step(w)
    k, v = pools_from_oracle(w, ref["k_pool"], ref["v_pool"])
    k0, v0 = bits(k), bits(v)
    cap = w.num_blocks * w.block_size
    slots = torch.tensor([-1, cap, cap + 7, -5], dtype=torch.int64, device="cuda")
    rows = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    pa.write_kv(k, v, rows, rows, slots)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), k0) and np.array_equal(bits(v), v0)


def test_copy_blocks_bit_exact_and_skips_bad_ids():
    w = W.custom([100, 64, 33], 16, 8, 128, 16, "bf16", seed=307_071, pool_factor=2.0)
    ref = oracle.run_step(w)
    k, v = pools_from_oracle(w, ref["k_pool"], ref["v_pool"])
    used = sorted(set(int(b) for b in w.block_tables.ravel() if b >= 0))
    free = [b for b in range(w.num_blocks) if b not in used]
    pairs = np.array([[used[0], free[0]], [used[3], free[1]], [used[5], free[2]],
                      [-1, free[3]], [used[1], w.num_blocks], [w.num_blocks + 2, free[4]]], np.int64)
    pa.copy_blocks(k, v, dev(pairs))
    torch.cuda.synchronize()
    kb, vb = ref["k_pool"].copy(), ref["v_pool"].copy()
    oracle.copy_blocks(kb, vb, pairs[:3])
    assert np.array_equal(bits(k), kb) and np.array_equal(bits(v), vb)


@pytest.mark.parametrize("dt,B,D", [("bf16", 16, 128), ("bf16", 8, 64), ("bf16", 32, 256),
                                    ("f32", 16, 64), ("f32", 32, 128)])
def test_write_orders_bit_exact(dt, B, D):
    """pa_write_kv over rows in prefill order (whole blocks, written as
    tiles), shifted so that blocks straddle the 256-row chunks, reversed,
    shuffled, and with skipped (-1) slots: the pools equal the oracle's bit
    for bit."""
    rng = np.random.default_rng(307_062 + B + D)
    Hkv, NB, T = 4, 96, 700
    blocks = rng.permutation(NB)[:-(-T // B)]
    slots = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1)[:T].astype(np.int64)
    orders = {
        "prefill": slots,
        "shifted": np.concatenate([slots[5:], slots[:5]]),
        "reversed": slots[::-1].copy(),
        "shuffled": rng.permutation(slots),
        "holes": np.where(rng.random(T) < 0.05, -1, slots),
    }
    if dt == "bf16":
        kv = rng.integers(0, 1 << 16, size=(2, T, Hkv, D), dtype=np.uint16)
    else:
        kv = rng.standard_normal((2, T, Hkv, D)).astype(np.float32).view(np.uint32)
    spec = types.SimpleNamespace(dtype=dt)
    for name, sl in orders.items():
        _say(f"write order {name} {dt} B={B} D={D}")
        kb, vb = oracle.new_pools(NB, Hkv, B, D, dt)
        k, v = pools_from_oracle(spec, kb.copy(), vb.copy())
        oracle.write_kv(kb, vb, kv[0], kv[1], sl, B)
        key, val = pools_from_oracle(spec, kv[0], kv[1])
        pa.write_kv(k, v, key, val, dev(sl))
        torch.cuda.synchronize()
        assert_pool_equal(spec, k, v, kb, vb)


def test_slot_mapping_edge_rows():
    bt = np.array([[3, 9, -1], [4, -1, -1]], np.int32)
    seq = np.array([0, 0, 0, 1, 1, -1, 2, 0], np.int32)
    pos = np.array([0, 17, 40, 5, 16, 3, 0, -1], np.int32)
    got = bits(pa.slot_mapping(dev(bt), dev(seq), dev(pos), 16))
    want = oracle.slot_mapping(bt, seq, pos, 16)
    assert want.tolist() == [48, 145, -1, 69, -1, -1, -1, -1]
    assert np.array_equal(got, want)


def test_invalid_block_ids_give_nan_not_faults():
    """A table entry outside [0, num_blocks) inside ceil(L/B) is a broken
    precondition: the kernel's bounds check turns that sequence's output into
    NaN and leaves the others correct."""
    w = W.custom([50, 50, 50], 8, 2, 128, 16, "bf16", seed=307_081)
    ref = oracle.run_step(w)
    k, v = pools_from_oracle(w, ref["k_pool"], ref["v_pool"])
    bt = w.block_tables.copy()
    bt[0, 1] = w.num_blocks + 100
    bt[1, 2] = -1
    for P in (0, 16):
        out = as_f64(pa.decode(dev(w.q), k, v, dev(bt), dev(w.context_lens), w.max_context_len,
                               w.scale, partition_size=P))
        assert np.isnan(out[0]).all() and np.isnan(out[1]).all()
        assert np.max(np.abs(out[2] - ref["out"][2])) <= TOL["bf16"]


# ------------------------------------------------------------- the five workloads at full size

def test_full_llama3_8b_decode():
    w = W.llama3_8b_decode()
    ref = oracle.run_step(w)
    for P in (0, 512, 8192):
        _check_step(w, P, check_pool=(P == 0), ref=ref)
    _check_step(w, 512, check_pool=False, ref=ref, two_phase=True)
    # the benchmark's step: appending partials (4096) + merge, pool checked bit for bit
    _check_step(w, 4096, ref=ref, append=True, two_phase=True)


def test_full_long_context_split():
    """The 8-sequence long-context layer (32K..128K tokens, 512-token
    partitions): every output element of every (sequence, KV head) pair
    against the oracle, in the one-launch, two-launch and appending forms;
    the appending form's pool bit for bit."""
    w = W.long_context()
    ref = oracle.run_step(w)
    for two_phase in (False, True):
        _check_step(w, 512, check_pool=False, two_phase=two_phase, ref=ref)
    _check_step(w, 512, ref=ref, append=True)


@pytest.mark.parametrize("phase", ["fork", "steady", "aligned"])
def test_full_shared_prefix(phase):
    w = W.shared_prefix(phase)
    ref = oracle.run_step(w)
    _check_step(w, 512, ref=ref)
    _check_step(w, 4096, ref=ref, append=True, shared_blocks=True)


def test_full_mixed_lengths_block_sweep():
    outs = {}
    for B in (8, 16, 32):
        w = W.mixed_lengths(B)
        r, _ = _check_step(w, 512, check_pool=(B == 16))
        outs[B] = bits(r["out"])
    # same lengths and token data for every B: the outputs agree
    o8, o16, o32 = (oracle.widen(outs[b], "bf16") for b in (8, 16, 32))
    assert np.max(np.abs(o8 - o16)) <= TOL["bf16"] and np.max(np.abs(o32 - o16)) <= TOL["bf16"]

"""pa_decode_shared_prefix on the GPU against the oracle's plain decode.

Sequences that share the blocks of a common prefix (the pages' parallel
samples of one prompt) are decoded with each shared block streamed once per
KV head for all the group's query heads; the result must equal the plain
definition, element by element within the bf16 tolerance, and the appended
rows must land in the pools bit for bit.  Covered: the full shared-prefix
workloads (fork, steady and aligned steps), ragged groups over many shapes,
groups larger than one prefix unit serves, members shorter than the shared
run, empty groups, shared lengths that are not multiples of 16, bad block
ids, and workspace reuse between grouped and plain launches."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_307_amd as pa
import workloads as W
from gpu_common import TOL, as_f64, assert_pool_equal, bits, dev, pools_from_oracle, torch_dtype

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _history_pools(w):
    """Pools with the history (and copy-on-write copies) written by the HIP path."""
    k, v = pa.empty_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                             torch_dtype(w), "cuda", fill=float("nan"))
    hs = pa.slot_mapping(dev(w.hist_block_tables), dev(w.hist_seq), dev(w.hist_pos), w.block_size)
    pa.write_kv(k, v, dev(w.hist_key), dev(w.hist_value), hs)
    if len(w.copy_pairs):
        pa.copy_blocks(k, v, dev(w.copy_pairs))
    return k, v


def _grouped_step(w, group_start, prefix_lens, P, append, two_phase=False, ws=None):
    """One step through pa_decode_shared_prefix; returns (out, k, v)."""
    k, v = _history_pools(w)
    bt, cl, q = dev(w.block_tables), dev(w.context_lens), dev(w.q)
    gs = dev(np.asarray(group_start, np.int32))
    pl = dev(np.asarray(prefix_lens, np.int32))
    key = value = None
    if append:
        key, value = dev(w.new_key), dev(w.new_value)
    else:
        slots = pa.slot_mapping(bt, dev(w.new_seq), dev(w.new_pos), w.block_size)
        pa.write_kv(k, v, dev(w.new_key), dev(w.new_value), slots)
    out = torch.empty_like(q)
    if ws is None:
        ws = pa.alloc_shared_prefix_workspace(w.num_seqs, w.num_heads, w.num_kv_heads,
                                              w.head_dim, w.max_context_len, P, len(prefix_lens))
    pa.decode_shared_prefix(q, k, v, bt, cl, gs, pl, w.max_context_len, w.scale, P, ws, out,
                            key=key, value=value, partials_only=two_phase)
    if two_phase:
        pa.decode_shared_prefix_merge(out, cl, gs, pl, w.num_kv_heads, w.block_size,
                                      w.max_blocks_per_seq, w.max_context_len, P, ws)
    torch.cuda.synchronize()
    return out, k, v


def _check(w, group_start, prefix_lens, P, append, ref, two_phase=False, check_pool=True):
    _say(f"{w.name} S={w.num_seqs} Hq={w.num_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
         f"B={w.block_size} {w.dtype} P={P} groups={len(prefix_lens)} prefix={list(prefix_lens)[:4]}"
         + (" append" if append else "") + (" two-phase" if two_phase else ""))
    out, k, v = _grouped_step(w, group_start, prefix_lens, P, append, two_phase)
    if check_pool:
        assert_pool_equal(w, k, v, ref["k_pool"], ref["v_pool"])
    err = float(np.max(np.abs(as_f64(out) - ref["out"])))
    print(f"[case] max abs err {err:.3e} (tol {TOL[w.dtype]})", flush=True)
    assert err <= TOL[w.dtype]
    return out


# ------------------------------------------------------------- the full workloads

@pytest.mark.parametrize("phase", ["steady", "fork", "aligned"])
def test_full_shared_prefix_grouped(phase):
    """16 groups of 16 branches sharing a 2048-token prefix: the grouped
    decode equals the oracle on every element, appended rows bit for bit, in
    the benchmark's launch (4096-token partitions, rows appended) and in the
    two-launch and 512-token-partition forms; and it equals pa_decode's
    output within the tolerance."""
    w = W.shared_prefix(phase)
    ref = oracle.run_step(w)
    G, br = w.extra["num_groups"], w.extra["branches"]
    gs = np.arange(0, G * br + 1, br, dtype=np.int32)
    pl = np.full(G, w.extra["prefix_len"], np.int32)
    out = _check(w, gs, pl, 4096, True, ref)
    _check(w, gs, pl, 4096, True, ref, two_phase=True)
    _check(w, gs, pl, 512, False, ref)
    # the same bits whatever the cache hint: the kernel reads identical data
    plain = pa.decode(dev(w.q), *_history_pools_with_step(w), dev(w.block_tables),
                      dev(w.context_lens), w.max_context_len, w.scale, partition_size=4096,
                      shared_blocks=True)
    torch.cuda.synchronize()
    assert float(np.max(np.abs(as_f64(out) - as_f64(plain)))) <= TOL["bf16"]


def _history_pools_with_step(w):
    k, v = _history_pools(w)
    slots = pa.slot_mapping(dev(w.block_tables), dev(w.new_seq), dev(w.new_pos), w.block_size)
    pa.write_kv(k, v, dev(w.new_key), dev(w.new_value), slots)
    return k, v


# ------------------------------------------------------------- ragged groups

GROUP_SHAPES = [  # (Hq, Hkv, D, B)
    (32, 8, 128, 16), (16, 4, 128, 8), (64, 8, 128, 32), (8, 8, 64, 16), (16, 1, 128, 16),
    (32, 2, 256, 16), (12, 4, 64, 8), (6, 2, 256, 32),
]


def _ragged_spec(B, G, D, rng):
    cap = (64 if D <= 128 else 32) // G  # members one prefix unit serves
    sh = lambda n: n * B  # noqa: E731
    return [
        (sh(0), [5]),                                       # a sequence outside any sharing
        (sh(4), [1, 2, 3]),                                 # short prefix, short tails
        (sh(max(1, 48 // B)), list(rng.integers(1, 300, size=min(16, cap)))),  # a full unit
        (sh(max(1, 512 // B)), list(rng.integers(1, 80, size=cap + 3))),      # beyond a unit
        (sh(1), [40]),                                      # a group of one
        (sh(max(1, 700 // B)), list(rng.integers(1, 40, size=2))),
    ]


@pytest.mark.parametrize("shape", GROUP_SHAPES, ids=lambda s: "Hq%d_Hkv%d_D%d_B%d" % s)
def test_ragged_groups(shape):
    Hq, Hkv, D, B = shape
    rng = np.random.default_rng(307_400 + Hq + D + B)
    spec = _ragged_spec(B, Hq // Hkv, D, rng)
    w = W.shared_groups(spec, Hq, Hkv, D, B, "bf16", seed=307_401 + D + B)
    ref = oracle.run_step(w)
    gs, sh = w.extra["group_start"], w.extra["shared_tokens"]
    for P, append in ((512, True), (max(16, B), False), (64, True)):
        _check(w, gs, sh, P, append, ref)
    # a declared shared length below the true one, not a multiple of 16: the
    # rest of the shared tokens are decoded per member
    _check(w, gs, np.maximum(sh - 5, 0), 512, True, ref)
    # no sharing declared at all
    _check(w, gs, np.zeros_like(sh), 512, False, ref)


def test_fp32_ignores_groups():
    """fp32: the groups change nothing (every token is decoded per sequence)."""
    spec = [(32, [1, 9, 17]), (16, [4, 4])]
    w = W.shared_groups(spec, 8, 2, 64, 16, "f32", seed=307_402)
    ref = oracle.run_step(w)
    gs, sh = w.extra["group_start"], w.extra["shared_tokens"]
    _check(w, gs, sh, 32, True, ref)
    _check(w, gs, sh, 512, False, ref)


def test_members_shorter_than_the_shared_run():
    """Decode only, with some members' lengths cut inside the shared tokens
    (the first member's too, which limits what the prefix unit covers) and
    some to 0: each member attends over its own tokens only."""
    spec = [(64, [10, 20, 30, 40, 50]), (128, [7, 7, 7])]
    w = W.shared_groups(spec, 16, 4, 128, 16, "bf16", seed=307_403)
    base = oracle.run_step(w)
    gs, sh = w.extra["group_start"], w.extra["shared_tokens"]
    k, v = pools_from_oracle(w, base["k_pool"], base["v_pool"])
    for lens in ([74, 30, 0, 64, 1, 60, 135, 128], [20, 84, 94, 104, 114, 0, 50, 135]):
        lens = np.array(lens, np.int32)
        want = oracle.decode(oracle.to_bits(w.q, w.dtype), base["k_pool"], base["v_pool"],
                             w.block_tables, lens, w.scale, w.num_kv_heads, w.block_size, w.dtype)
        for P in (16, 512):
            _say(f"short members {lens.tolist()} P={P}")
            out = pa.decode_shared_prefix(dev(w.q), k, v, dev(w.block_tables), dev(lens), dev(gs),
                                          dev(sh), int(lens.max()), w.scale, P)
            torch.cuda.synchronize()
            got = as_f64(out)
            assert np.all(got[lens == 0] == 0.0)
            assert float(np.max(np.abs(got - want))) <= TOL["bf16"]


def test_empty_groups_and_edge_group_arrays():
    """Empty groups (group_start[i] == group_start[i+1]), groups that start
    after sequence 0 and end before the last one, and zero groups."""
    spec = [(0, [3]), (48, [2, 9, 4]), (0, [1]), (32, [6, 6])]
    w = W.shared_groups(spec, 8, 2, 128, 16, "bf16", seed=307_404)
    ref = oracle.run_step(w)
    cases = [
        ([1, 1, 4, 5, 7], [0, 48, 0, 32]),     # an empty first group
        ([1, 4], [48]),                        # one group in the middle of the batch
        ([5, 7, 7], [32, 100]),                # a late group, an empty last group
        ([0, 1, 4, 5, 7], [0, 48, 0, 32]),     # as generated
    ]
    for gs, pl in cases:
        _check(w, np.array(gs, np.int32), np.array(pl, np.int32), 64, True, ref)
    out = torch.empty_like(dev(w.q))
    _, k, v = _grouped_step(w, [0, 1, 4, 5, 7], [0, 48, 0, 32], 64, False)
    # zero groups: the plain split decode
    pa.decode_shared_prefix(dev(w.q), k, v, dev(w.block_tables), dev(w.context_lens),
                            dev(np.zeros(1, np.int32)), dev(np.zeros(0, np.int32)),
                            w.max_context_len, w.scale, 64, out=out)
    torch.cuda.synchronize()
    assert float(np.max(np.abs(as_f64(out) - ref["out"]))) <= TOL["bf16"]


def test_bad_block_in_the_shared_prefix_poisons_its_group():
    """A shared block id outside the pool (in the first member's table, the
    one the prefix unit reads) makes every member of that group NaN and
    leaves the other groups exact."""
    spec = [(64, [3, 5, 7]), (32, [4, 4])]
    w = W.shared_groups(spec, 16, 4, 128, 16, "bf16", seed=307_405)
    base = oracle.run_step(w)
    k, v = pools_from_oracle(w, base["k_pool"], base["v_pool"])
    bt = w.block_tables.copy()
    for s in range(3):
        bt[s, 1] = w.num_blocks + 9
    out = as_f64(pa.decode_shared_prefix(dev(w.q), k, v, dev(bt), dev(w.context_lens),
                                         dev(w.extra["group_start"]),
                                         dev(w.extra["shared_tokens"]), w.max_context_len,
                                         w.scale, 64))
    assert np.isnan(out[:3]).all()
    assert float(np.max(np.abs(out[3:] - base["out"][3:]))) <= TOL["bf16"]


def test_workspace_shared_by_grouped_and_plain_launches():
    """One zero-filled workspace serves grouped and plain decodes in turn:
    the stamps keep each launch's records apart."""
    spec = [(64, [3, 50, 7, 100]), (32, [4, 4, 200])]
    w = W.shared_groups(spec, 32, 8, 128, 16, "bf16", seed=307_406)
    base = oracle.run_step(w)
    k, v = pools_from_oracle(w, base["k_pool"], base["v_pool"])
    gs, sh = dev(w.extra["group_start"]), dev(w.extra["shared_tokens"])
    ws = pa.alloc_shared_prefix_workspace(w.num_seqs, 32, 8, 128, w.max_context_len, 32, 2)
    args = (dev(w.q), k, v, dev(w.block_tables), dev(w.context_lens))
    for rep in range(3):
        _say(f"workspace reuse rep {rep}")
        a = pa.decode_shared_prefix(*args, gs, sh, w.max_context_len, w.scale, 32, ws)
        b = pa.decode(*args, w.max_context_len, w.scale, partition_size=32, workspace=ws)
        torch.cuda.synchronize()
        assert float(np.max(np.abs(as_f64(a) - base["out"]))) <= TOL["bf16"]
        assert float(np.max(np.abs(as_f64(b) - base["out"]))) <= TOL["bf16"]

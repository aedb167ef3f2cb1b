"""Paged prefill / chunked prefill on the GPU (pa_prefill through the C ABI)
against the oracle's prefill: every row of ragged small batches, every row
of the Llama-3-8B-shaped chunked-prefill layer, and the degenerate cases (empty chunks, one-token prompts, rows at negative
positions, bad block ids)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_307_amd as pa
import workloads as W
from gpu_common import TOL, as_f64, dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _to_dev(x, dt):
    return dev(x if dt == "bf16" else np.ascontiguousarray(x, dtype=np.float32))


def run_prefill_gpu(w, table=None, query_start=None, max_query_len=None, out=None):
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    k, v = pa.empty_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, tdt, "cuda",
                             fill=float("nan"))
    bt = dev(w.block_tables)
    if len(w.kv_seq):
        slots = pa.slot_mapping(bt, dev(w.kv_seq), dev(w.kv_pos), w.block_size)
        pa.write_kv(k, v, _to_dev(w.key, w.dtype), _to_dev(w.value, w.dtype), slots)
    if table is not None:
        bt = dev(table)
    qs = dev(w.query_start if query_start is None else query_start)
    mql = w.max_query_len if max_query_len is None else max_query_len
    out = pa.prefill(_to_dev(w.q, w.dtype), k, v, bt, dev(w.context_lens), qs,
                     max(w.max_context_len, 1), mql, w.scale, out=out)
    torch.cuda.synchronize()
    return out


LENS = [(0, 0), (1, 1), (5, 5), (17, 3), (40, 40), (64, 64), (100, 37), (257, 1), (300, 129),
        (33, 16), (50, 0), (16, 16), (31, 31), (520, 200)]

SHAPES = [  # Hq, Hkv, D, B, dtype
    (4, 2, 64, 16, "f32"), (12, 4, 64, 32, "f32"), (8, 2, 256, 8, "f32"),
    (8, 2, 128, 16, "bf16"), (8, 8, 64, 8, "bf16"), (32, 8, 128, 16, "bf16"),
    (16, 1, 128, 32, "bf16"), (6, 2, 256, 8, "bf16"), (64, 8, 128, 16, "bf16"),
    (4, 4, 256, 32, "bf16"), (10, 2, 64, 32, "bf16"), (12, 2, 256, 16, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "Hq%d_Hkv%d_D%d_B%d_%s" % s)
def test_prefill_ragged_batch(shape):
    Hq, Hkv, D, B, dt = shape
    _say(f"prefill ragged {shape}")
    lens, qlens = zip(*LENS)
    w = W.prefill(lens, qlens, Hq, Hkv, D, B, dt, seed=307_320 + D + B + Hq)
    out = run_prefill_gpu(w)
    ref = oracle.run_prefill(w)["out"]
    err = float(np.max(np.abs(as_f64(out) - ref)))
    _say(f"  max abs err {err:.3e}")
    assert err <= TOL[dt]


def test_prefill_whole_prompts_and_single_rows():
    """n = L for every sequence (whole prompts), then n = 1 (decode rows)."""
    for qmode in ("whole", "one"):
        lens = [1, 2, 15, 16, 17, 63, 64, 65, 200, 1000]
        qlens = lens if qmode == "whole" else [1] * len(lens)
        w = W.prefill(lens, qlens, 32, 8, 128, 16, "bf16", seed=307_330)
        out = run_prefill_gpu(w)
        ref = oracle.run_prefill(w)["out"]
        err = float(np.max(np.abs(as_f64(out) - ref)))
        _say(f"prefill {qmode}: max abs err {err:.3e}")
        assert err <= TOL["bf16"]


def test_prefill_work_order_many_pairs_and_ties():
    """The bf16 launch deals (sequence, KV head) pairs to the XCDs and ranks
    each XCD's pairs by length.  More than 64 pairs per XCD (80 sequences x
    8 KV heads) takes the plain order; equal lengths everywhere are ties the
    ranking breaks by index.  Every row must still be computed exactly once."""
    rng = np.random.default_rng(307_366)
    many = [int(x) for x in rng.integers(1, 50, size=80)]
    cases = [("many pairs", many, [min(L, 7) for L in many], 8, 8, 64),
             ("ties", [64] * 20, [64] * 20, 8, 2, 128),
             ("ties, one KV head", [33] * 17 + [5] * 9, [9] * 17 + [5] * 9, 4, 1, 64)]
    for name, lens, qlens, Hq, Hkv, D in cases:
        w = W.prefill(lens, qlens, Hq, Hkv, D, 16, "bf16", seed=307_367)
        out = run_prefill_gpu(w)
        ref = oracle.run_prefill(w)["out"]
        err = float(np.max(np.abs(as_f64(out) - ref)))
        _say(f"prefill work order, {name}: {len(lens)} seqs x {Hkv} KV heads, max abs err {err:.3e}")
        assert err <= TOL["bf16"], name


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_rows_without_tokens_are_zero(dt):
    """Five query rows on three cached tokens: the first two rows sit at
    negative positions and are zero; the rest match the oracle."""
    w = W.prefill([3, 20], [3, 4], 8, 2, 64, 16, dt, seed=307_331)
    q = np.concatenate([w.q[:2], w.q])
    w2 = W.PrefillWorkload(**{**w.__dict__, "q": q, "query_lens": np.array([5, 4], np.int32),
                              "query_start": np.array([0, 5, 9], np.int32)})
    out = as_f64(run_prefill_gpu(w2))
    ref = oracle.run_prefill(w2)["out"]
    assert np.array_equal(out[:2], np.zeros_like(out[:2]))
    assert float(np.max(np.abs(out - ref))) <= TOL[dt]


def test_prefill_bad_block_id_gives_nan_not_fault():
    w = W.prefill([40, 40], [8, 8], 8, 2, 128, 16, "bf16", seed=307_332)
    table = w.block_tables.copy()
    table[0, 1] = w.num_blocks + 7          # sequence 0, tokens 16..31
    out = as_f64(run_prefill_gpu(w, table=table))
    ref = oracle.run_prefill(w)["out"]
    assert np.isnan(out[:8]).all()          # every row of sequence 0 sees tokens 16..31
    assert float(np.max(np.abs(out[8:] - ref[8:]))) <= TOL["bf16"]


@pytest.mark.parametrize("B,bad_block", [(8, 1), (8, 3), (16, 1), (32, 0)])
def test_prefill_bad_block_poisons_exactly_the_rows_that_see_it(B, bad_block):
    """A whole 40-token prompt whose logical block `bad_block` has an id
    outside the pool: rows at positions before that block are exact, rows
    that see it are NaN (B = 8 puts two blocks in one 16-token tile, either
    half of which may be the bad one)."""
    w = W.prefill([40, 40], [40, 40], 8, 2, 128, B, "bf16", seed=307_334 + B)
    table = w.block_tables.copy()
    table[0, bad_block] = w.num_blocks + 3
    out = as_f64(run_prefill_gpu(w, table=table))
    ref = oracle.run_prefill(w)["out"]
    first_bad = bad_block * B
    assert float(np.max(np.abs(out[:first_bad] - ref[:first_bad]), initial=0.0)) <= TOL["bf16"]
    assert np.isnan(out[first_bad:40]).all()
    assert float(np.max(np.abs(out[40:] - ref[40:]))) <= TOL["bf16"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_negative_and_large_scales(dt):
    """The scale is any finite factor: a negative one (the bf16 kernel moves
    its sign into q), large ones (peaked softmax, frequent rescales), zero
    (uniform weights: the rescale threshold is infinite after the first
    tile) and a tiny one, against the oracle."""
    for scale in (-0.09, 0.9, 4.0, 0.0, 1e-30):
        w = W.prefill([5, 40, 130], [5, 7, 64], 8, 2, 64, 16, dt, seed=307_335)
        w = W.PrefillWorkload(**{**w.__dict__, "scale": scale})
        out = as_f64(run_prefill_gpu(w))
        ref = oracle.run_prefill(w)["out"]
        tol = TOL[dt]
        if dt == "f32" and abs(scale) > 1 / np.sqrt(w.head_dim):
            # beyond the usual 1/sqrt(D) scale: fp32 error grows with the
            # logit range (an exponent's relative error is about |logit| x
            # 2^-24), and |scale q.k| <= |scale| max|q| max|k|
            qn = float(np.max(np.linalg.norm(oracle.widen(oracle.to_bits(w.q, dt), dt), axis=-1)))
            kn = float(np.max(np.linalg.norm(np.asarray(w.key, dtype=np.float64), axis=-1)))
            vmax = float(np.max(np.abs(np.asarray(w.value, dtype=np.float64))))
            tol = max(tol, 8 * 2.0 ** -24 * (1 + abs(scale) * qn * kn) * vmax)
        assert float(np.max(np.abs(out - ref))) <= tol, (scale, tol)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_rows_clamped_to_max_query_len(dt):
    """Rows beyond max_query_len are not written: an output pre-filled with a
    sentinel bit pattern keeps it bit for bit in rows 6..9 of each sequence;
    the first 6 rows match the oracle."""
    w = W.prefill([30, 30], [10, 10], 8, 2, 64, 16, dt, seed=307_333)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    itype = torch.int16 if dt == "bf16" else torch.int32
    sentinel = 0x5A5A if dt == "bf16" else 0x5A5A5A5A
    out = torch.full((w.num_query_tokens, w.num_heads, w.head_dim), sentinel, dtype=itype,
                     device="cuda").view(tdt)
    run_prefill_gpu(w, max_query_len=6, out=out)
    ref = oracle.run_prefill(w)["out"]
    got = as_f64(out)
    raw = out.view(itype).cpu().numpy()
    for s in range(2):
        q0 = int(w.query_start[s])
        # rows kept are the first 6 rows (positions L - 10 .. L - 5)
        assert float(np.max(np.abs(got[q0:q0 + 6] - ref[q0:q0 + 6]))) <= TOL[dt]
        assert np.all(raw[q0 + 6:q0 + 10] == sentinel), "a row beyond max_query_len was written"


def test_full_llama3_8b_chunked_prefill():
    """The 16-sequence, 512-token-chunk layer (the benchmark's launch): every
    output element of every (sequence, KV head) against the oracle."""
    w = W.llama3_8b_prefill()
    _say(f"llama3_8b_prefill: {w.num_query_tokens} rows, lengths {w.context_lens.tolist()}")
    out = as_f64(run_prefill_gpu(w))
    ref = oracle.run_prefill(w)["out"]
    assert not np.isnan(ref).any()
    G = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        q0, q1 = int(w.query_start[s]), int(w.query_start[s + 1])
        for g in range(w.num_kv_heads):
            err = float(np.max(np.abs(out[q0:q1, g * G:(g + 1) * G] - ref[q0:q1, g * G:(g + 1) * G])))
            assert err <= TOL["bf16"], (s, g, err)

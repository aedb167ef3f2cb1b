"""Seeded synthetic inputs for one paged decode step.

A :class:`Workload` describes one decode step of a batch over a paged KV
cache, in the shape of the inputs a model runner hands the attention kernel
(page 3, "ModelRunner" section: the current token, each sequence's context
length, its block table, the physical block pool, and the slot for the current
token's K/V).  Because slots and offsets are the method's own arithmetic, a
workload never states them: it states *which* (sequence, position) pairs are
written and with what data, plus the block tables, and each consumer turns
those into slots itself.

Contents of a workload:

* ``context_lens[s]`` -- tokens sequence ``s`` attends over in this step,
  including the token written in this step (its position is ``L - 1``).
* ``block_tables`` -- int32 ``[S, max_blocks_per_seq]``, one row per
  sequence, physical block ids in logical order, padded with -1 (page 2,
  BlockTable section: an int32 table of ``[max_num_reqs,
  max_num_blocks_per_req]``).
* ``hist_*`` -- the history (positions ``0 .. L-2``) written before the step,
  as (sequence, position, key, value) rows, using ``hist_block_tables``.  A
  block shared by several sequences is written once, through the first
  sequence that references it.
* ``copy_pairs`` -- int64 ``[P, 2]`` (src, dst) copy-on-write pairs applied
  after the history and before the step's write; ``block_tables`` is the
  table after those copies (page 1, copy-on-write of a shared partial block:
  only the writer's table row changes).
* ``new_*`` -- the token each sequence writes in this step, at position
  ``L - 1``.
* ``q`` -- ``[S, Hq, D]`` queries of the step's tokens.

Element storage: ``"f32"`` arrays are float32; ``"bf16"`` arrays hold the raw
bfloat16 bit patterns as uint16.

Random streams: one ``numpy.random.SeedSequence(seed)`` is split into
independent child streams (lengths, structure, block permutation, q, history
K/V, new-token K/V), drawn in that order, so a change to one stream's use does
not move the others.  bf16 standard-normal values are drawn by inverse-CDF
sampling: a uniformly random 16-bit index (from PCG64's raw output) selects one
of 65536 equiprobable normal quantiles ``Phi^-1((i + 0.5) / 65536)``, which were
rounded to float32 and then to bfloat16 (round to nearest even).  This is
N(0, 1) at bfloat16 resolution, truncated at +-4.31 sigma (probability 1.6e-5
of the mass beyond it).  float32 values come from ``standard_normal``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "POISON_BITS",
    "tiny_f32",
    "llama3_8b_decode",
    "long_context",
    "shared_prefix",
    "shared_groups",
    "mixed_lengths",
    "custom",
    "PrefillWorkload",
    "prefill",
    "llama3_8b_prefill",
]

# Quiet-NaN bit patterns used to fill every slot no sequence has written.
POISON_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0}

_STREAMS = ("lengths", "structure", "perm", "q", "hist", "new")


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    context_lens: np.ndarray
    block_tables: np.ndarray
    hist_block_tables: np.ndarray
    q: np.ndarray
    hist_seq: np.ndarray
    hist_pos: np.ndarray
    hist_key: np.ndarray
    hist_value: np.ndarray
    copy_pairs: np.ndarray
    new_seq: np.ndarray
    new_pos: np.ndarray
    new_key: np.ndarray
    new_value: np.ndarray
    partition_size: int = 512
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def storage_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# ---------------------------------------------------------------------------
# random draws

_BF16_QUANTILES: Optional[np.ndarray] = None


def _bf16_quantile_table() -> np.ndarray:
    global _BF16_QUANTILES
    if _BF16_QUANTILES is None:
        from scipy.special import ndtri

        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        f = ndtri(p).astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        _BF16_QUANTILES = rounded.astype(np.uint16)
    return _BF16_QUANTILES


def _normal(seedseq: np.random.SeedSequence, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    bitgen = np.random.PCG64(seedseq)
    if dtype == "f32":
        return np.random.Generator(bitgen).standard_normal(n, dtype=np.float32).reshape(shape)
    table = _bf16_quantile_table()
    idx = bitgen.random_raw((n + 3) // 4).view(np.uint16)[:n]
    return table[idx].reshape(shape)


def normal_values(seed: int, shape, dtype: str) -> np.ndarray:
    """Seeded N(0, 1) values in workload storage (float32, or bf16 bits as
    uint16), drawn as described in the module notes."""
    return _normal(np.random.SeedSequence(seed), shape, dtype)


def _streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, children))


# ---------------------------------------------------------------------------
# block allocation (a stand-in for the block manager: hands out ids only)

class _Pool:
    """Free list of physical block ids in a seeded random order."""

    def __init__(self, num_blocks: int, order: np.ndarray):
        self.num_blocks = num_blocks
        self._free = [int(b) for b in order]
        self._next = 0

    def take(self, n: int) -> list:
        if self._next + n > len(self._free):
            raise RuntimeError(
                f"block pool exhausted: need {n} more, {len(self._free) - self._next} free"
            )
        ids = self._free[self._next:self._next + n]
        self._next += n
        return ids

    @property
    def used(self) -> int:
        return self._next


def _blocks_to_hold(tokens: int, block_size: int) -> int:
    """Number of fixed-size blocks a block manager allocates for ``tokens``."""
    return (tokens + block_size - 1) // block_size


def _pool_size(blocks_needed: int, factor: float = 1.25) -> int:
    return int(math.ceil(factor * blocks_needed))


def _contiguous_row(ids: list) -> bool:
    return len(ids) >= 2 and all(b - a == 1 for a, b in zip(ids, ids[1:]))


def _tables_from_rows(rows: list, max_blocks: int) -> np.ndarray:
    table = np.full((len(rows), max_blocks), -1, dtype=np.int32)
    for s, ids in enumerate(rows):
        if len(ids) > max_blocks:
            raise ValueError("row longer than max_blocks_per_seq")
        table[s, :len(ids)] = ids
    return table


def _allocate_private(lengths, block_size, num_blocks, perm_seed, forbid_contiguous=True):
    """Give each sequence its own blocks from a shuffled pool, in (seq, logical) order."""
    rng = np.random.Generator(np.random.PCG64(perm_seed))
    for _attempt in range(64):
        pool = _Pool(num_blocks, rng.permutation(num_blocks))
        rows = [pool.take(_blocks_to_hold(int(L), block_size)) for L in lengths]
        if not forbid_contiguous or not any(_contiguous_row(r) for r in rows):
            return rows
    raise RuntimeError("could not draw a block permutation without contiguous rows")


def _history_rows(lengths):
    """(seq, pos) of every token before the step's token, in sequence order."""
    seq = np.concatenate([np.full(int(L) - 1, s, np.int32) for s, L in enumerate(lengths)]) \
        if len(lengths) else np.zeros(0, np.int32)
    pos = np.concatenate([np.arange(int(L) - 1, dtype=np.int32) for L in lengths]) \
        if len(lengths) else np.zeros(0, np.int32)
    return seq, pos


def _assemble(name, dtype, lengths, rows, hist_rows, Hq, Hkv, D, B, NB, MB, st,
              hist_seq=None, hist_pos=None, copy_pairs=None, partition_size=512,
              extra=None, hist_data=None) -> Workload:
    lengths = np.asarray(lengths, dtype=np.int32)
    S = len(lengths)
    if hist_seq is None:
        hist_seq, hist_pos = _history_rows(lengths)
    Tp = len(hist_seq)
    q = _normal(st["q"], (S, Hq, D), dtype)
    if hist_data is None:
        hist = _normal(st["hist"], (2, Tp, Hkv, D), dtype)
        hist_key, hist_value = hist[0], hist[1]
    else:
        hist_key, hist_value = hist_data
    new = _normal(st["new"], (2, S, Hkv, D), dtype)
    if copy_pairs is None:
        copy_pairs = np.zeros((0, 2), np.int64)
    return Workload(
        name=name, dtype=dtype, num_seqs=S, num_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=B, num_blocks=NB, max_blocks_per_seq=MB,
        scale=1.0 / math.sqrt(D),
        context_lens=lengths,
        block_tables=_tables_from_rows(rows, MB),
        hist_block_tables=_tables_from_rows(hist_rows, MB),
        q=q,
        hist_seq=np.asarray(hist_seq, np.int32), hist_pos=np.asarray(hist_pos, np.int32),
        hist_key=hist_key, hist_value=hist_value,
        copy_pairs=np.asarray(copy_pairs, np.int64).reshape(-1, 2),
        new_seq=np.arange(S, dtype=np.int32), new_pos=(lengths - 1).astype(np.int32),
        new_key=new[0], new_value=new[1],
        partition_size=partition_size, extra=extra or {},
    )


# ---------------------------------------------------------------------------
# the five decode configurations

def tiny_f32(seed: int = 307_001) -> Workload:
    """4 sequences, context lengths {1, 17, 40, 100}, B=16, 4 query / 2 KV heads,
    head_dim 64, fp32, a pool of 32 blocks whose ids are a seeded permutation."""
    st = _streams(seed)
    lengths = [1, 17, 40, 100]
    B, NB = 16, 32
    rows = _allocate_private(lengths, B, NB, st["perm"])
    MB = _blocks_to_hold(max(lengths), B)
    return _assemble("tiny_f32", "f32", lengths, rows, rows, 4, 2, 64, B, NB, MB, st)


def custom(lengths, num_heads, num_kv_heads, head_dim, block_size, dtype="bf16",
           seed=307_100, pool_factor=1.25, max_blocks_per_seq=None, name="custom",
           partition_size=512) -> Workload:
    """Any list of context lengths (each >= 1) over a shuffled pool."""
    st = _streams(seed)
    lengths = [int(x) for x in lengths]
    if any(L < 1 for L in lengths):
        raise ValueError("every context length must be >= 1 (it includes the step's token)")
    need = sum(_blocks_to_hold(L, block_size) for L in lengths)
    NB = max(_pool_size(need, pool_factor), 1)
    rows = _allocate_private(lengths, block_size, NB, st["perm"])
    MB = max_blocks_per_seq or max(1, _blocks_to_hold(max(lengths), block_size))
    return _assemble(name, dtype, lengths, rows, rows, num_heads, num_kv_heads, head_dim,
                     block_size, NB, MB, st, partition_size=partition_size)


def llama3_8b_decode(seed: int = 307_002, num_seqs: int = 64, min_len: int = 512,
                     max_len: int = 4096) -> Workload:
    """Batch of 64, 32 query / 8 KV heads, head_dim 128, bf16, B=16; context
    lengths uniform on the integers [512, 4096]; pool 1.25x the blocks needed,
    shuffled so no sequence's blocks are contiguous."""
    st = _streams(seed)
    B = 16
    lengths = np.random.Generator(np.random.PCG64(st["lengths"])).integers(
        min_len, max_len, size=num_seqs, endpoint=True)
    need = sum(_blocks_to_hold(int(L), B) for L in lengths)
    NB = _pool_size(need)
    rows = _allocate_private(lengths, B, NB, st["perm"])
    MB = _blocks_to_hold(max_len, B)
    return _assemble("llama3_8b_decode", "bf16", lengths, rows, rows, 32, 8, 128, B, NB, MB, st)


def long_context(seed: int = 307_003, num_seqs: int = 8, min_len: int = 32768,
                 max_len: int = 131072, partition_size: int = 512) -> Workload:
    """8 sequences with context lengths uniform on [32768, 131072], 32/8 heads,
    head_dim 128, bf16, B=16, shuffled pool; split into 512-token partitions."""
    st = _streams(seed)
    B = 16
    lengths = np.random.Generator(np.random.PCG64(st["lengths"])).integers(
        min_len, max_len, size=num_seqs, endpoint=True)
    need = sum(_blocks_to_hold(int(L), B) for L in lengths)
    NB = _pool_size(need)
    rows = _allocate_private(lengths, B, NB, st["perm"])
    MB = _blocks_to_hold(max_len, B)
    return _assemble("long_context", "bf16", lengths, rows, rows, 32, 8, 128, B, NB, MB, st,
                     partition_size=partition_size)


def shared_prefix(phase: str = "steady", seed: int = 307_004, num_groups: int = 16,
                  branches: int = 16, prefix_len: int = 2048, max_tail: int = 512) -> Workload:
    """Parallel sampling: ``num_groups`` groups of ``branches`` sequences; every
    branch of a group references the same physical blocks for a
    ``prefix_len``-token prefix (block-aligned at B=16).

    Each group also shares a partially filled *fork* block holding
    ``s_g ~ U{1..15}`` tokens the branches had in common when they forked.

    * ``phase="fork"``: the step in which each branch writes its first own
      token.  The fork block is shared and partial, so every branch but the
      first gets a private copy (copy-on-write pairs in ``copy_pairs``), then
      writes at offset ``s_g``; context = prefix + s_g + 1.
    * ``phase="steady"``: a later step.  Fork blocks are private already;
      each branch has a private tail of ``t ~ U{1..512}`` tokens (including the
      step's token); context = prefix + s_g + t.
    * ``phase="aligned"``: the literal reading with no shared partial block
      (s_g = 0): each branch's first token opens a private block, no copies.
    """
    if phase not in ("fork", "steady", "aligned"):
        raise ValueError(phase)
    st = _streams(seed)
    B, Hq, Hkv, D = 16, 32, 8, 128
    if prefix_len % B:
        raise ValueError("prefix must be block aligned")
    n_prefix_blocks = prefix_len // B
    len_rng = np.random.Generator(np.random.PCG64(st["lengths"]))
    fork_tokens = len_rng.integers(1, B - 1, size=num_groups, endpoint=True)
    tails = len_rng.integers(1, max_tail, size=(num_groups, branches), endpoint=True)
    if phase == "aligned":
        fork_tokens = np.zeros(num_groups, np.int64)
    S = num_groups * branches

    if phase in ("fork", "aligned"):
        lengths = np.array([prefix_len + fork_tokens[g] + 1
                            for g in range(num_groups) for _ in range(branches)])
        if phase == "fork":
            need = num_groups * (n_prefix_blocks + 1 + (branches - 1))
        else:
            need = num_groups * (n_prefix_blocks + branches)
    else:
        lengths = np.array([prefix_len + fork_tokens[g] + tails[g, b]
                            for g in range(num_groups) for b in range(branches)])
        need = num_groups * n_prefix_blocks + sum(
            _blocks_to_hold(int(fork_tokens[g] + tails[g, b]), B)
            for g in range(num_groups) for b in range(branches))
    NB = _pool_size(need)
    MB = _blocks_to_hold(prefix_len + (B - 1) + max_tail, B)
    perm_rng = np.random.Generator(np.random.PCG64(st["perm"]))
    pool = _Pool(NB, perm_rng.permutation(NB))

    hist_rows, rows, copies = [], [], []
    hist_seq, hist_pos, hist_src = [], [], []   # hist_src: (kind, group, branch)
    for g in range(num_groups):
        prefix_ids = pool.take(n_prefix_blocks)
        s_g = int(fork_tokens[g])
        first = g * branches
        # the shared prefix is written once, through the group's first branch
        hist_seq.append(np.full(prefix_len, first, np.int32))
        hist_pos.append(np.arange(prefix_len, dtype=np.int32))
        hist_src.append(("prefix", g, 0, prefix_len))
        if phase == "fork":
            fork_id = pool.take(1)
            if s_g:
                hist_seq.append(np.full(s_g, first, np.int32))
                hist_pos.append(np.arange(prefix_len, prefix_len + s_g, dtype=np.int32))
                hist_src.append(("fork", g, 0, s_g))
            for b in range(branches):
                hist_rows.append(prefix_ids + fork_id)
                if b == 0:
                    rows.append(prefix_ids + fork_id)   # last referrer writes in place
                else:
                    private = pool.take(1)
                    copies.append((fork_id[0], private[0]))
                    rows.append(prefix_ids + private)
        elif phase == "aligned":
            for b in range(branches):
                private = pool.take(1)
                hist_rows.append(prefix_ids + private)
                rows.append(prefix_ids + private)
        else:
            for b in range(branches):
                n_own = s_g + int(tails[g, b])
                own = pool.take(_blocks_to_hold(n_own, B))
                hist_rows.append(prefix_ids + own)
                rows.append(prefix_ids + own)
                seq = first + b
                if s_g:
                    hist_seq.append(np.full(s_g, seq, np.int32))
                    hist_pos.append(np.arange(prefix_len, prefix_len + s_g, dtype=np.int32))
                    hist_src.append(("fork", g, b, s_g))
                t_hist = int(tails[g, b]) - 1
                if t_hist:
                    hist_seq.append(np.full(t_hist, seq, np.int32))
                    hist_pos.append(np.arange(prefix_len + s_g, prefix_len + s_g + t_hist,
                                              dtype=np.int32))
                    hist_src.append(("tail", g, b, t_hist))

    # history data: one prefix and one fork run per group (identical for every
    # branch of the group), private data for each tail
    hist_gen = st["hist"].spawn(3)
    prefix_data = _normal(hist_gen[0], (num_groups, 2, prefix_len, Hkv, D), "bf16")
    fork_data = _normal(hist_gen[1], (num_groups, 2, B, Hkv, D), "bf16")
    n_tail = sum(n for kind, _g, _b, n in hist_src if kind == "tail")
    tail_data = _normal(hist_gen[2], (2, max(n_tail, 0), Hkv, D), "bf16")
    keys, values, tail_at = [], [], 0
    for kind, g, _b, n in hist_src:
        if kind == "prefix":
            keys.append(prefix_data[g, 0]); values.append(prefix_data[g, 1])
        elif kind == "fork":
            keys.append(fork_data[g, 0, :n]); values.append(fork_data[g, 1, :n])
        else:
            keys.append(tail_data[0, tail_at:tail_at + n])
            values.append(tail_data[1, tail_at:tail_at + n])
            tail_at += n
    hist_key = np.concatenate(keys) if keys else np.zeros((0, Hkv, D), np.uint16)
    hist_value = np.concatenate(values) if values else np.zeros((0, Hkv, D), np.uint16)

    extra = {"phase": phase, "num_groups": num_groups, "branches": branches,
             "prefix_len": prefix_len, "fork_tokens": fork_tokens.astype(np.int32),
             "tails": tails.astype(np.int32), "blocks_used": pool.used}
    return _assemble(f"shared_prefix_{phase}", "bf16", lengths, rows, hist_rows,
                     Hq, Hkv, D, B, NB, MB, st,
                     hist_seq=np.concatenate(hist_seq), hist_pos=np.concatenate(hist_pos),
                     copy_pairs=np.array(copies, np.int64).reshape(-1, 2), extra=extra,
                     hist_data=(hist_key, hist_value))


def shared_groups(spec, num_heads, num_kv_heads, head_dim, block_size, dtype="bf16",
                  seed=307_120, pool_factor=1.25, name="shared_groups") -> Workload:
    """Sequences that share the blocks of a common prefix, group by group.

    ``spec`` is a list of ``(shared_tokens, tails)``: one group per entry,
    whose ``len(tails)`` members are consecutive in the batch and share the
    physical blocks of their first ``shared_tokens`` tokens (a multiple of
    the block size; 0 = no sharing), member ``i`` then owning ``tails[i] >= 1``
    more tokens (the step's token among them) in private blocks.  The shared
    tokens are written once, through the group's first member.  ``extra``
    holds ``group_start`` (int32 ``[groups + 1]``) and ``shared_tokens``
    (int32 ``[groups]``)."""
    st = _streams(seed)
    B = int(block_size)
    lengths, group_start, shared = [], [0], []
    for sh, tails in spec:
        if sh % B:
            raise ValueError("shared tokens must fill whole blocks")
        if any(int(t) < 1 for t in tails):
            raise ValueError("every member owns at least the step's token")
        lengths += [sh + int(t) for t in tails]
        group_start.append(len(lengths))
        shared.append(sh)
    need = sum(sh // B + sum(_blocks_to_hold(int(t), B) for t in tails) for sh, tails in spec)
    NB = max(_pool_size(need, pool_factor), 1)
    pool = _Pool(NB, np.random.Generator(np.random.PCG64(st["perm"])).permutation(NB))
    rows, hist_seq, hist_pos, src = [], [], [], []
    s = 0
    for gi, (sh, tails) in enumerate(spec):
        common = pool.take(sh // B)
        if sh:  # written once, through the first member
            hist_seq.append(np.full(sh, s, np.int32))
            hist_pos.append(np.arange(sh, dtype=np.int32))
            src.append(("shared", gi, sh))
        for t in tails:
            rows.append(common + pool.take(_blocks_to_hold(int(t), B)))
            if int(t) > 1:
                hist_seq.append(np.full(int(t) - 1, s, np.int32))
                hist_pos.append(np.arange(sh, sh + int(t) - 1, dtype=np.int32))
                src.append(("own", s, int(t) - 1))
            s += 1
    Hkv, D = num_kv_heads, head_dim
    n_hist = sum(x[2] for x in src)
    hist = _normal(st["hist"], (2, n_hist, Hkv, D), dtype)
    MB = max(1, max(len(r) for r in rows))
    extra = {"group_start": np.array(group_start, np.int32),
             "shared_tokens": np.array(shared, np.int32)}
    return _assemble(name, dtype, lengths, rows, rows, num_heads, num_kv_heads, head_dim, B, NB,
                     MB, st,
                     hist_seq=np.concatenate(hist_seq) if hist_seq else np.zeros(0, np.int32),
                     hist_pos=np.concatenate(hist_pos) if hist_pos else np.zeros(0, np.int32),
                     extra=extra, hist_data=(hist[0], hist[1]))


def mixed_lengths(block_size: int = 16, seed: int = 307_005, num_seqs: int = 256,
                  median: float = 1024.0, sigma: float = 1.0, min_len: int = 16,
                  max_len: int = 8192) -> Workload:
    """256 sequences, lognormal context lengths (median 1024, sigma 1, clipped to
    [16, 8192]), 64 query / 8 KV heads, head_dim 128, bf16.  Lengths and token
    data do not depend on ``block_size``; only the pool and its permutation
    (seeded by 307_050 + B) do, so outputs are identical across B."""
    st = _streams(seed)
    B = int(block_size)
    z = np.random.Generator(np.random.PCG64(st["lengths"])).standard_normal(num_seqs)
    lengths = np.clip(np.rint(np.exp(np.log(median) + sigma * z)), min_len, max_len).astype(np.int64)
    need = sum(_blocks_to_hold(int(L), B) for L in lengths)
    NB = _pool_size(need)
    rows = _allocate_private(lengths, B, NB, np.random.SeedSequence(307_050 + B))
    MB = _blocks_to_hold(max_len, B)
    return _assemble(f"mixed_lengths_B{B}", "bf16", lengths, rows, rows, 64, 8, 128, B, NB, MB, st)


# ---------------------------------------------------------------------------
# prefill / chunked prefill

@dataclasses.dataclass
class PrefillWorkload:
    """One prefill step: sequence s holds ``context_lens[s]`` tokens in the
    cache and brings its last ``query_lens[s]`` positions as query rows
    ``query_start[s] .. query_start[s+1] - 1``.  ``kv_seq`` / ``kv_pos`` /
    ``key`` / ``value`` are the rows of every cached token (the chunk's own
    included), written before the attention."""
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    context_lens: np.ndarray
    query_lens: np.ndarray
    query_start: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    kv_seq: np.ndarray
    kv_pos: np.ndarray
    key: np.ndarray
    value: np.ndarray

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def num_query_tokens(self) -> int:
        return int(self.query_start[-1])


def prefill(lengths, query_lens, num_heads, num_kv_heads, head_dim, block_size, dtype="bf16",
            seed=307_300, pool_factor=1.25, name="prefill") -> PrefillWorkload:
    """Sequences of the given cached lengths (>= 0), each with its last
    ``query_lens[s]`` positions as query rows, over a shuffled pool."""
    st = _streams(seed)
    lengths = np.asarray([int(x) for x in lengths], dtype=np.int32)
    qlens = np.asarray([int(x) for x in query_lens], dtype=np.int32)
    if lengths.shape != qlens.shape or (lengths < 0).any() or (qlens < 0).any():
        raise ValueError("lengths and query_lens: same count, non-negative")
    B = block_size
    need = sum(_blocks_to_hold(int(L), B) for L in lengths)
    NB = max(_pool_size(need, pool_factor), 1)
    rows = _allocate_private(lengths, B, NB, st["perm"])
    MB = max(1, max((_blocks_to_hold(int(L), B) for L in lengths), default=1))
    starts = np.zeros(len(lengths) + 1, dtype=np.int32)
    starts[1:] = np.cumsum(qlens)
    T = int(starts[-1])
    kv_seq = np.concatenate([np.full(int(L), s, np.int32) for s, L in enumerate(lengths)]) \
        if len(lengths) else np.zeros(0, np.int32)
    kv_pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in lengths]) \
        if len(lengths) else np.zeros(0, np.int32)
    kv = _normal(st["hist"], (2, len(kv_seq), num_kv_heads, head_dim), dtype)
    q = _normal(st["q"], (T, num_heads, head_dim), dtype)
    return PrefillWorkload(
        name=name, dtype=dtype, num_seqs=len(lengths), num_heads=num_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B, num_blocks=NB,
        max_blocks_per_seq=MB, scale=1.0 / math.sqrt(head_dim), context_lens=lengths,
        query_lens=qlens, query_start=starts, block_tables=_tables_from_rows(rows, MB), q=q,
        kv_seq=kv_seq, kv_pos=kv_pos, key=kv[0], value=kv[1])


def llama3_8b_prefill(seed: int = 307_301, num_seqs: int = 16, chunk: int = 512,
                      min_len: int = 512, max_len: int = 4096) -> PrefillWorkload:
    """Chunked prefill of a Llama-3-8B-shaped layer: 16 sequences whose cached
    lengths are uniform on [512, 4096], each bringing its last 512 positions
    as one chunk of query rows; 32 query / 8 KV heads, head_dim 128, bf16,
    B=16, pool 1.25x the blocks needed, shuffled."""
    st = _streams(seed)
    lengths = np.random.Generator(np.random.PCG64(st["lengths"])).integers(
        min_len, max_len, size=num_seqs, endpoint=True)
    return prefill(lengths, [min(chunk, int(L)) for L in lengths], 32, 8, 128, 16, "bf16",
                   seed=seed + 1, name="llama3_8b_prefill")

"""Plain fp64 CPU oracle of paged decode attention.  TEST INFRASTRUCTURE ONLY.

This module is the checker, not the product: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it.
It shares no code with the HIP library; the two meet only in the seeded inputs
of ``workloads``.

Sources (three web pages on PagedAttention):

* [P1] "什么是 PagedAttention？" (qubittool glossary) -- sections 映射逻辑块与物理块
  (mapping logical to physical blocks) and 共享但不污染状态 (sharing without
  corrupting state).
* [P2] "PagedAttention学习笔记" (juejin) -- section 2.1 核心原理 (core principle),
  the table comparing it with FlashAttention, section 三 (algorithm flow:
  sequence diagram), and the BlockTable walkthrough (块表与槽位映射).
* [P3] "KV cache 显存管理：为什么 PagedAttention 是 vLLM 的核心" (mini-vLLM blog) --
  sections 分页思想 (the paging idea, worked example), 为什么固定大小 block
  可以减少浪费 (why fixed blocks cut waste), PagedAttention 改变了什么 (what
  PagedAttention changes: the index formulas) and 对 ModelRunner 的影响 (the
  kernel's inputs).

What is computed has a plain definition: paging changes where K/V live, not
the attention formula ([P2] comparison table: the formula is unchanged, only
the access path differs; [P3] "what PagedAttention changes").  So ``decode``
gathers each sequence's K/V through its block table into contiguous fp64
arrays and evaluates softmax(q K^T * scale) V directly.

Readings where the pages are silent (each also listed in the design notes):

* Pool layout (the pages call layouts versioned implementation details):
  K pool ``[num_blocks, Hkv, B, D]``, V pool ``[num_blocks, Hkv, D, B]``.
  Slot ``s`` names block ``s // B``, offset ``s % B`` in both.  The attention
  result does not depend on this choice; bit-exact pool comparisons do.
* ``context_lens[s]`` counts the step's own token, which the step writes at
  position ``L - 1`` before attending, so the query attends to itself.
* Grouped-query heads: query head ``h`` reads KV head ``h // (Hq // Hkv)``.
* ``scale`` multiplies q.k (the pages print softmax(QK^T)V without one).
* A sequence with ``L == 0`` attends over nothing: its output is zero.
* Slot -1 means "not this rank's entry": the write skips it ([P2] section 三
  and the BlockTable walkthrough).
* Copy-on-write copies whole blocks; slots past the valid entries are unused
  and never read, so the valid entries come out identical ([P1] sharing).

Storage: pools hold raw bits (uint16 for bfloat16, uint32 for float32) so
writes and copies are pure bit moves; ``widen`` turns bits into fp64 exactly.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "blocks_needed", "block_token_range", "translate", "slot_of", "slot_mapping",
    "storage_dtype", "to_bits", "widen", "new_pools", "write_kv", "copy_blocks",
    "gather", "attend", "decode", "decode_brute", "attention_unpaged_brute",
    "contiguous_sequences", "run_step", "prefill", "causal_attention_brute",
    "contiguous_prefill_sequences", "run_prefill", "attend_lse", "prefill_lse", "merge_states",
    "cp_owner", "cp_local_offset", "cp_slot_mapping", "cp_context_len",
    "map_to_kernel_blocks", "tail_waste", "fragmentation_proxy",
    "prealloc_waste", "kv_bytes", "POISON",
]

POISON = {"f32": 0x7FC00000, "bf16": 0x7FC0}


# --------------------------------------------------------------------------
# blocking and address translation

def blocks_needed(L: int, B: int) -> int:
    """Logical blocks a length-L sequence needs: ceil(L / B).  [P2 2.1]"""
    return (L + B - 1) // B


def block_token_range(i: int, L: int, B: int):
    """Token interval [iB, min((i+1)B, L)) held by logical block i.  [P2 2.1]"""
    return i * B, min((i + 1) * B, L)


def translate(t: int, table_row, B: int):
    """Logical token t -> (logical block, offset in block, physical block).

    [P3 "what PagedAttention changes"]: logical_block_id = t // B,
    block_offset = t % B, physical_block_id = block_table[logical_block_id].
    """
    lb = t // B
    off = t % B
    pb = int(table_row[lb])
    return lb, off, pb


def slot_of(table_row, pos: int, B: int) -> int:
    """Flat slot of (request, position): block_id * B + pos % B.  [P2 BlockTable]"""
    _lb, off, pb = translate(pos, table_row, B)
    return pb * B + off


def slot_mapping(block_tables, seq_idx, positions, B: int) -> np.ndarray:
    """One slot per (sequence, position) row, int64.  A sequence id outside
    the table, a negative position, or a table entry of -1 gives -1 (skip)."""
    out = np.empty(len(seq_idx), dtype=np.int64)
    for i, (s, p) in enumerate(zip(seq_idx, positions)):
        s, p = int(s), int(p)
        if s < 0 or s >= block_tables.shape[0] or p < 0:
            out[i] = -1
            continue
        lb = p // B
        if lb >= block_tables.shape[1] or int(block_tables[s, lb]) < 0:
            out[i] = -1
            continue
        out[i] = slot_of(block_tables[s], p, B)
    return out


# --------------------------------------------------------------------------
# storage

def storage_dtype(dtype: str):
    return np.uint32 if dtype == "f32" else np.uint16


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Workload storage (float32 or bf16 bits as uint16) -> raw bits."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return np.ascontiguousarray(x, dtype=np.uint16)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw bits -> exact fp64 values."""
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def new_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: str):
    """NaN-filled K pool [NB, Hkv, B, D] and V pool [NB, Hkv, D, B] of raw bits."""
    sd = storage_dtype(dtype)
    k = np.full((num_blocks, num_kv_heads, block_size, head_dim), POISON[dtype], dtype=sd)
    v = np.full((num_blocks, num_kv_heads, head_dim, block_size), POISON[dtype], dtype=sd)
    return k, v


def write_kv(k_pool, v_pool, key_bits, value_bits, slots, B: int) -> None:
    """Write token i's K/V rows to slot[i], in list order; slot -1 is skipped.

    [P3 "ModelRunner"]: the slot tells where the current token's K/V go;
    [P2 section 三]: -1 marks an entry this rank does not own.
    """
    for i, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        b, o = slot // B, slot % B
        k_pool[b, :, o, :] = key_bits[i]
        v_pool[b, :, :, o] = value_bits[i]


def copy_blocks(k_pool, v_pool, pairs) -> None:
    """Copy-on-write: for each (src, dst), block dst becomes a copy of src.  [P1]"""
    for src, dst in pairs:
        k_pool[int(dst)] = k_pool[int(src)]
        v_pool[int(dst)] = v_pool[int(src)]


# --------------------------------------------------------------------------
# attention

def gather(k_pool, v_pool, table_row, L: int, kv_head: int, B: int, dtype: str):
    """Contiguous fp64 K [L, D] and V [L, D] of one sequence and KV head,
    collected block by block through the table row.  [P2 2.1, P3]"""
    D = k_pool.shape[3]
    Ks = np.empty((L, D), dtype=np.float64)
    Vs = np.empty((L, D), dtype=np.float64)
    for i in range(blocks_needed(L, B)):
        lo, hi = block_token_range(i, L, B)
        pb = int(table_row[i])
        n = hi - lo
        Ks[lo:hi] = widen(k_pool[pb, kv_head, :n, :], dtype)
        Vs[lo:hi] = widen(v_pool[pb, kv_head, :, :n], dtype).T
    return Ks, Vs


def attend(q_rows: np.ndarray, Ks: np.ndarray, Vs: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for each row of q, in fp64.  Empty K -> zeros."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    if Ks.shape[0] == 0:
        return np.zeros((q_rows.shape[0], Vs.shape[1]), dtype=np.float64)
    logits = (q_rows @ Ks.T) * scale
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    return (w @ Vs) / w.sum(axis=1, keepdims=True)


def decode(q_bits, k_pool, v_pool, block_tables, context_lens, scale: float,
           num_kv_heads: int, B: int, dtype: str, seqs=None, kv_heads=None) -> np.ndarray:
    """Decode attention for every (sequence, query head), fp64 [S, Hq, D].

    ``seqs`` / ``kv_heads`` restrict the work to a sample; other rows stay NaN.
    """
    S, Hq, D = q_bits.shape
    G = Hq // num_kv_heads
    q = widen(q_bits, dtype)
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        for g in (range(num_kv_heads) if kv_heads is None else kv_heads):
            Ks, Vs = gather(k_pool, v_pool, block_tables[s], L, g, B, dtype)
            out[s, g * G:(g + 1) * G] = attend(q[s, g * G:(g + 1) * G], Ks, Vs, scale)
    return out


def decode_brute(q_bits, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads,
                 B, dtype):
    """The same result with pure-Python scalar loops (tiny inputs only)."""
    S, Hq, D = q_bits.shape
    G = Hq // num_kv_heads
    q = widen(q_bits, dtype)
    kf = widen(k_pool, dtype)
    vf = widen(v_pool, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        for h in range(Hq):
            g = h // G
            logits = []
            for t in range(L):
                _lb, off, pb = translate(t, block_tables[s], B)
                acc = 0.0
                for d in range(D):
                    acc += float(q[s, h, d]) * float(kf[pb, g, off, d])
                logits.append(acc * scale)
            if not logits:
                continue
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            den = sum(w)
            for d in range(D):
                num = 0.0
                for t in range(L):
                    _lb, off, pb = translate(t, block_tables[s], B)
                    num += w[t] * float(vf[pb, g, d, off])
                out[s, h, d] = num / den
    return out


def attention_unpaged_brute(q, k_seq, v_seq, scale, num_kv_heads):
    """Textbook decode attention over contiguous per-sequence K/V (no paging):
    q [Hq, D] fp64, k_seq/v_seq [L, Hkv, D] fp64; pure-Python loops."""
    Hq, D = q.shape
    G = Hq // num_kv_heads
    L = k_seq.shape[0]
    out = np.zeros((Hq, D))
    for h in range(Hq):
        g = h // G
        logits = [scale * sum(float(q[h, d]) * float(k_seq[t, g, d]) for d in range(D))
                  for t in range(L)]
        if not logits:
            continue
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        den = sum(w)
        for d in range(D):
            out[h, d] = sum(w[t] * float(v_seq[t, g, d]) for t in range(L)) / den
    return out


def contiguous_sequences(w):
    """Per-sequence contiguous fp64 K/V [L, Hkv, D] straight from a workload's
    (sequence, position) rows -- no block table involved.  Only valid for
    workloads without shared blocks (every position written by its own
    sequence)."""
    out = []
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        k = np.full((L, w.num_kv_heads, w.head_dim), np.nan)
        v = np.full((L, w.num_kv_heads, w.head_dim), np.nan)
        sel = np.nonzero(w.hist_seq == s)[0]
        k[w.hist_pos[sel]] = widen(to_bits(w.hist_key[sel], w.dtype), w.dtype)
        v[w.hist_pos[sel]] = widen(to_bits(w.hist_value[sel], w.dtype), w.dtype)
        sel = np.nonzero(w.new_seq == s)[0]
        k[w.new_pos[sel]] = widen(to_bits(w.new_key[sel], w.dtype), w.dtype)
        v[w.new_pos[sel]] = widen(to_bits(w.new_value[sel], w.dtype), w.dtype)
        out.append((k, v))
    return out


def run_step(w, seqs=None, kv_heads=None):
    """One decode step on a workload: write the history, apply copy-on-write,
    write the step's token, attend.  Returns a dict with the pools (raw bits),
    both slot mappings and the fp64 output."""
    B = w.block_size
    k_pool, v_pool = new_pools(w.num_blocks, w.num_kv_heads, B, w.head_dim, w.dtype)
    hist_slots = slot_mapping(w.hist_block_tables, w.hist_seq, w.hist_pos, B)
    write_kv(k_pool, v_pool, to_bits(w.hist_key, w.dtype), to_bits(w.hist_value, w.dtype),
             hist_slots, B)
    copy_blocks(k_pool, v_pool, w.copy_pairs)
    new_slots = slot_mapping(w.block_tables, w.new_seq, w.new_pos, B)
    write_kv(k_pool, v_pool, to_bits(w.new_key, w.dtype), to_bits(w.new_value, w.dtype),
             new_slots, B)
    out = decode(to_bits(w.q, w.dtype), k_pool, v_pool, w.block_tables, w.context_lens,
                 w.scale, w.num_kv_heads, B, w.dtype, seqs=seqs, kv_heads=kv_heads)
    return {"k_pool": k_pool, "v_pool": v_pool, "hist_slots": hist_slots,
            "new_slots": new_slots, "out": out}


# --------------------------------------------------------------------------
# prefill / chunked prefill

def prefill(q_bits, k_pool, v_pool, block_tables, context_lens, query_start, scale: float,
            num_kv_heads: int, B: int, dtype: str, seqs=None, kv_heads=None) -> np.ndarray:
    """Causal attention of many query rows per sequence over its paged K/V,
    fp64 [T, Hq, D].

    Sequence s holds L = context_lens[s] tokens and owns query rows
    query_start[s] .. query_start[s+1]-1; those n rows are its last n
    positions, so row i sits at position L - n + i and sees tokens
    0 .. L - n + i.  [P1 映射逻辑块与物理块: prefill asks for blocks by input
    length; P2 comparison with FlashAttention and P3 "what PagedAttention
    changes": paging moves K/V, the formula stays.]  A row whose position is
    negative sees nothing and gets zeros.  ``seqs`` / ``kv_heads`` restrict
    the work to a sample; other rows stay NaN.
    """
    T, Hq, D = q_bits.shape
    G = Hq // num_kv_heads
    q = widen(q_bits, dtype)
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    S = len(context_lens)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        n = q1 - q0
        for g in (range(num_kv_heads) if kv_heads is None else kv_heads):
            Ks, Vs = gather(k_pool, v_pool, block_tables[s], L, g, B, dtype)
            for i in range(n):
                visible = max(L - n + i + 1, 0)
                out[q0 + i, g * G:(g + 1) * G] = attend(q[q0 + i, g * G:(g + 1) * G],
                                                        Ks[:visible], Vs[:visible], scale)
    return out


def causal_attention_brute(q, k_seq, v_seq, positions, scale, num_kv_heads):
    """Textbook causal attention over contiguous K/V, no paging: row i of q
    [n, Hq, D] sees tokens 0 .. positions[i] of k_seq/v_seq [L, Hkv, D];
    pure-Python loops through the unpaged brute force."""
    out = np.zeros(q.shape, dtype=np.float64)
    for i, p in enumerate(positions):
        p = int(p)
        if p < 0:
            continue
        out[i] = attention_unpaged_brute(q[i], k_seq[:p + 1], v_seq[:p + 1], scale, num_kv_heads)
    return out


def contiguous_prefill_sequences(w):
    """Per-sequence contiguous fp64 K/V [L, Hkv, D] from a prefill workload's
    (sequence, position) rows, no block table involved."""
    out = []
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        k = np.full((L, w.num_kv_heads, w.head_dim), np.nan)
        v = np.full((L, w.num_kv_heads, w.head_dim), np.nan)
        sel = np.nonzero(w.kv_seq == s)[0]
        k[w.kv_pos[sel]] = widen(to_bits(w.key[sel], w.dtype), w.dtype)
        v[w.kv_pos[sel]] = widen(to_bits(w.value[sel], w.dtype), w.dtype)
        out.append((k, v))
    return out


def run_prefill(w, seqs=None, kv_heads=None):
    """One prefill step on a prefill workload: write every cached row at its
    slot, then attend.  Returns the pools (raw bits), the slots and the fp64
    output."""
    B = w.block_size
    k_pool, v_pool = new_pools(w.num_blocks, w.num_kv_heads, B, w.head_dim, w.dtype)
    slots = slot_mapping(w.block_tables, w.kv_seq, w.kv_pos, B)
    write_kv(k_pool, v_pool, to_bits(w.key, w.dtype), to_bits(w.value, w.dtype), slots, B)
    out = prefill(to_bits(w.q, w.dtype), k_pool, v_pool, w.block_tables, w.context_lens,
                  w.query_start, w.scale, w.num_kv_heads, B, w.dtype, seqs=seqs,
                  kv_heads=kv_heads)
    return {"k_pool": k_pool, "v_pool": v_pool, "slots": slots, "out": out}


# --------------------------------------------------------------------------
# context parallelism: rank-interleaved tokens, per-rank partials, merge
#
# [P2 BlockTable walkthrough]: under decode / prefill context parallelism the
# slot mapping uses a virtual block size and a mask, writing -1 for entries a
# rank does not own; when the allocator's block size differs from the one
# the kernel needs, each allocator block is split into several kernel
# blocks.  The pages give no formula for ownership.  Reading taken: W ranks
# share one block table; a virtual block of B * W tokens maps to table entry
# table[p // (B * W)] on every rank (each rank has its own pool); inside it,
# runs of I tokens (the interleave, I dividing B) go to the ranks in turn,
# and a rank packs the runs it owns in order into its B slots of the block.

def cp_owner(p: int, B: int, W: int, I: int) -> int:
    """Rank owning logical token p."""
    return (p % (B * W)) // I % W


def cp_local_offset(p: int, B: int, W: int, I: int) -> int:
    """Offset of token p inside its owner's block."""
    vo = p % (B * W)
    return vo // (I * W) * I + vo % I


def cp_slot_mapping(block_tables, seq_idx, positions, B: int, W: int, rank: int,
                    I: int = 1) -> np.ndarray:
    """Slots of rank ``rank``: table[p // (B W)] * B + local offset for the
    tokens it owns, -1 for the others."""
    out = np.full(len(positions), -1, dtype=np.int64)
    for i, (s, p) in enumerate(zip(seq_idx, positions)):
        s, p = int(s), int(p)
        if cp_owner(p, B, W, I) != rank:
            continue
        out[i] = int(block_tables[s][p // (B * W)]) * B + cp_local_offset(p, B, W, I)
    return out


def cp_context_len(L: int, B: int, W: int, rank: int, I: int = 1) -> int:
    """Tokens of a length-L sequence that rank ``rank`` holds (counted one
    by one)."""
    return sum(1 for p in range(L) if cp_owner(p, B, W, I) == rank)


def attend_lse(q_rows, Ks, Vs, scale):
    """softmax(q K^T scale) V and the natural log of sum_t exp(q.k_t scale)
    per row; an empty K gives zeros and -inf."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    if Ks.shape[0] == 0:
        return (np.zeros((q_rows.shape[0], Vs.shape[1])),
                np.full(q_rows.shape[0], -np.inf))
    logits = (q_rows @ Ks.T) * scale
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    den = w.sum(axis=1, keepdims=True)
    return (w @ Vs) / den, (m + np.log(den))[:, 0]


def prefill_lse(q_bits, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                num_kv_heads, B, dtype):
    """``prefill`` plus each row's log-sum-exp, fp64 [T, Hq, D] and [T, Hq]."""
    T, Hq, D = q_bits.shape
    G = Hq // num_kv_heads
    q = widen(q_bits, dtype)
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        n = q1 - q0
        for g in range(num_kv_heads):
            Ks, Vs = gather(k_pool, v_pool, block_tables[s], L, g, B, dtype)
            for i in range(n):
                visible = max(L - n + i + 1, 0)
                o, l = attend_lse(q[q0 + i, g * G:(g + 1) * G], Ks[:visible], Vs[:visible], scale)
                out[q0 + i, g * G:(g + 1) * G] = o
                lse[q0 + i, g * G:(g + 1) * G] = l
    return out, lse


def merge_states(outs, lses):
    """Combine partial attentions over disjoint token sets: with M the largest
    log-sum-exp, out = sum_w e^(lse_w - M) o_w / sum_w e^(lse_w - M) (the
    log-sum-exp identity).  outs [W, ..., D], lses [W, ...]; rows whose every
    lse is -inf give zeros and -inf."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    Ms = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lses - Ms[None])
    den = w.sum(axis=0)
    num = (w[..., None] * outs).sum(axis=0)
    safe = np.where(den > 0, den, 1.0)
    out = np.where((den > 0)[..., None], num / safe[..., None], 0.0)
    lse = np.where(den > 0, Ms + np.log(safe), -np.inf)
    return out, lse


def map_to_kernel_blocks(manager_tables, k: int) -> np.ndarray:
    """Allocator block b of k * B_kernel tokens is kernel blocks b*k .. b*k+k-1:
    row [i] -> row [i*k + j] = table[i] * k + j (-1 stays -1)."""
    mt = np.asarray(manager_tables)
    rows, mb = mt.shape
    kt = np.full((rows, mb * k), -1, dtype=np.int32)
    for r in range(rows):
        for i in range(mb):
            if mt[r, i] < 0:
                continue
            for j in range(k):
                kt[r, i * k + j] = mt[r, i] * k + j
    return kt


# --------------------------------------------------------------------------
# capacity arithmetic

def tail_waste(lengths, B: int) -> int:
    """Unused slots in the last block of every sequence.  [P3 "why fixed blocks"]"""
    return int(sum(blocks_needed(int(L), B) * B - int(L) for L in lengths))


def fragmentation_proxy(lengths, B: int) -> float:
    """1 - used slots / (allocated blocks * B).  [P2 experiments section]"""
    used = sum(int(L) for L in lengths)
    alloc = sum(blocks_needed(int(L), B) for L in lengths) * B
    return 1.0 - used / alloc if alloc else 0.0


def prealloc_waste(lengths, max_len: int) -> int:
    """Slots never used when every request reserves max_len contiguous slots.
    [P3 "the most direct approach"]"""
    return int(sum(max_len - int(L) for L in lengths))


def kv_bytes(layers: int, tokens: int, kv_heads: int, head_dim: int, dtype_size: int) -> int:
    """KV cache bytes = layers x tokens x KV heads x head_dim x 2 x dtype_size.
    [P3 "why KV becomes a memory problem"]"""
    return layers * tokens * kv_heads * head_dim * 2 * dtype_size

/*
 * pa.h -- C ABI of the paged KV-cache decode library (libpa.so, gfx950).
 *
 * The hot path of PagedAttention: each sequence's K/V live in fixed-size
 * physical blocks of B tokens that need not be adjacent; a per-sequence block
 * table maps logical block i to a physical block id, so logical token t sits
 * in block block_table[t / B] at offset t % B.  Pages this follows:
 *
 *   [P1] "什么是 PagedAttention？" (qubittool glossary): 映射逻辑块与物理块
 *        (logical -> physical block mapping), 共享但不污染状态 (sharing and
 *        copy-on-write of a shared partial block).
 *   [P2] "PagedAttention学习笔记" (juejin): section 2.1 (ceil(L/B) blocks,
 *        block i holds tokens [iB, min((i+1)B, L))), section 三 (the kernel
 *        reads Q and the block table, gathers K/V by block, computes
 *        softmax(QK^T)V), and the BlockTable walkthrough (int32 table of
 *        [max_num_reqs, max_num_blocks_per_req]; slot = block_id * B +
 *        pos % B; -1 marks an entry this rank does not own).
 *   [P3] "KV cache 显存管理：为什么 PagedAttention 是 vLLM 的核心" (mini-vLLM
 *        blog): PagedAttention 改变了什么 (logical_block = t // B, offset =
 *        t % B, physical = block_table[logical]) and 对 ModelRunner 的影响
 *        (the kernel is given the current token, each sequence's context
 *        length and block table, the physical block pool, and the slot of the
 *        current token's K/V).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every pointer argument is a device pointer to memory the caller
 *           owns (hipMalloc'ed or a torch tensor's storage).  The library
 *           allocates nothing and keeps no state apart from the fixed scratch
 *           array of pa_decode_scratch (one per device, part of the loaded
 *           code); calls are thread-safe except overlapping pa_decode_scratch
 *           calls on one device.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *           stream).  Every call only enqueues work on it and returns; results
 *           are visible after the stream is synchronised.  Device-side faults
 *           surface at that synchronisation.
 * Errors.   Every argument is checked on the host before anything is
 *           launched; a failing check returns a negative PA_ERR_* and enqueues
 *           nothing.  A call whose work is empty (zero tokens, sequences or
 *           pairs) returns PA_OK without launching.  A failed launch returns
 *           PA_ERR_HIP.  pa_status_string() names a status.
 * Element types.
 *           PA_DTYPE_F32 (IEEE binary32) or PA_DTYPE_BF16 (bfloat16).  q, the
 *           K/V pools, key/value and out of one call share the dtype.
 *           Accumulation is always fp32; outputs are rounded to the dtype with
 *           round-to-nearest-even.
 * Cache layout (both pools, row-major, element offsets):
 *           k_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *           v_cache [num_blocks][num_kv_heads][head_dim][block_size]
 *           Slot s names block s / block_size, offset s % block_size in both.
 *           The pages leave the layout to the implementation; this one makes
 *           each (block, KV head) tile of K and of V one contiguous run of
 *           block_size * head_dim elements, with V's tokens innermost so the
 *           P.V contraction reads them directly as matrix-core operands.
 * Supported shapes.
 *           head_dim in {64, 128, 256}; block_size in {8, 16, 32};
 *           num_heads % num_kv_heads == 0 and num_heads / num_kv_heads <= 16.
 * Grouped-query attention.
 *           Query head h reads KV head h / (num_heads / num_kv_heads).
 * Memory safety.
 *           Kernels never access memory outside the documented extents even
 *           when a precondition is broken: an out-of-range block id or slot
 *           is skipped by writes and copies, and makes the affected decode
 *           outputs NaN.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent sizes      */
  PA_ERR_UNSUPPORTED = -2, /* a head_dim / block_size / dtype / group size not built */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required            */
  PA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed            */
  PA_ERR_NO_BLOCKS = -5,   /* block manager: not enough free blocks (nothing changed) */
  PA_ERR_STATE = -6,       /* block manager: sequence live/idle state does not allow it */
  PA_ERR_TOO_LARGE = -7    /* pa_decode_scratch: the call needs more than its fixed scratch */
};

enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 };

/*
 * Decode flags (the `flags` argument of the decode entry points; other bits
 * are rejected with PA_ERR_INVALID_ARG).
 *
 * PA_DECODE_SHARED_BLOCKS -- the launch reads some physical blocks from more
 *   than one sequence (a shared prompt prefix, parallel samples or beams that
 *   have not diverged; the pages' copy-on-write sharing).  The bf16 kernel
 *   then reads K/V with the default cache policy, so that repeated reads of a
 *   shared block can hit in the L2 or the last-level cache.  Without the flag
 *   it reads K/V tiles as streamed, read-once data (the nontemporal policy;
 *   block sizes 8 and 16), which is faster when every block is read once per
 *   launch and slower when blocks are shared.  Results are identical either
 *   way; the fp32 kernel ignores the flag.
 */
enum { PA_DECODE_SHARED_BLOCKS = 1 };

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_string(int status);

/*
 * pa_slot_mapping -- flat cache slot of each (sequence, position) row.
 * [P2 BlockTable walkthrough: block_id = block_table[req, pos // B],
 *  slot = block_id * B + pos % B; -1 = not written by this rank.]
 *
 *   slot_mapping  out  int64 [num_tokens]
 *   block_tables  in   int32 [num_seqs][max_blocks_per_seq]
 *   seq_ids       in   int32 [num_tokens]  sequence of each row
 *   positions     in   int32 [num_tokens]  logical token position of each row
 *
 * A row gets -1 when its sequence id is outside [0, num_seqs), when its
 * position is negative, when the position's logical block is >=
 * max_blocks_per_seq, or when the table entry there is negative.  Returns PA_ERR_INVALID_ARG for null pointers (with
 * num_tokens > 0), negative sizes, or block_size < 1.
 */
int pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables, const int32_t* seq_ids,
                    const int32_t* positions, int32_t num_tokens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t block_size, void* stream);

/*
 * pa_write_kv -- store each token's K and V rows at its slot.
 * [P3 对 ModelRunner 的影响: the slot is where the current token's K/V go;
 *  P2 section 三: slot -1 is skipped.]
 *
 *   k_cache, v_cache  in/out  pools in the layout above, num_blocks blocks
 *   key, value        in      [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping      in      int64 [num_tokens]
 *
 * Row i is written to block slot_mapping[i] / block_size, offset
 * slot_mapping[i] % block_size.  Rows with a negative slot, or a slot
 * >= num_blocks * block_size, are skipped.  Non-negative slots must be
 * distinct within one call (two rows for one slot leave either row there).
 * The result is bit-exact: the stored bits are the input bits.
 */
int pa_write_kv(void* k_cache, void* v_cache, const void* key, const void* value,
                const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                void* stream);

/*
 * pa_copy_blocks -- copy-on-write of whole blocks.
 * [P1 共享但不污染状态: a sequence about to write into a shared partial block
 *  gets a private block holding a copy of the valid entries; only that
 *  sequence's table changes, the original keeps its other references.]
 *
 *   k_cache, v_cache  in/out  pools in the layout above
 *   block_mapping     in      int64 [num_pairs][2] = (src, dst)
 *
 * For each pair, K block dst and V block dst (all KV heads, all slots)
 * become bit-exact copies of block src.  Pairs with an id outside
 * [0, num_blocks) are skipped.  The dst ids must be distinct and disjoint
 * from the src ids of the same call.  Updating block tables is the
 * caller's part (host-side block management).
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t dtype, void* stream);

/*
 * Split-KV workspace.  With partition_size > 0 the decode work is split and
 * merged with a log-sum-exp reduction.  The 16-token tiles of all (sequence,
 * KV head) pairs form one line that is cut into equal slices, one per worker
 * (a single-wave workgroup; as many workers as fit on the device at once, at
 * most 4096).  A slice is cut further at pair boundaries and at partition
 * boundaries (every partition_size tokens of a pair), and each piece yields
 * one record
 *   float o[G][head_dim], m[G], l[G]; uint32 stamp      (G = heads per KV head)
 * where, over the piece's tokens t and with x_t = scale * log2(e) * q.k_t,
 *   m = max_t x_t,  l = sum_t 2^(x_t - m),  o = sum_t 2^(x_t - m) v_t.
 * A piece that is a whole pair writes its output directly instead.  The
 * workspace holds a small block of per-launch metadata and room for
 * num_seqs * num_kv_heads * (4 + ceil(max_context_len / partition_size))
 * + 4096 records (the first four records of each pair in slots of their
 * own, so the merge finds them without a lookup); it must be 16-byte
 * aligned and at least pa_decode_workspace_bytes() long.
 * Allocate it zero-filled once and reuse it: each launch stamps its records,
 * so records left by earlier launches are ignored (zero is never a stamp).
 * pa_decode_workspace_bytes returns 0 when partition_size == 0 (single pass,
 * no workspace) or an argument is invalid.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size);

/*
 * pa_decode -- one decode step of attention over the paged cache.
 * [P2 section 三 and section 2.1; P3 PagedAttention 改变了什么: the attention
 *  formula is unchanged, only the K/V access path goes through the table.]
 *
 *   out           out [num_seqs][num_heads][head_dim]
 *   q             in  [num_seqs][num_heads][head_dim]
 *   k_cache, v_cache  in  pools in the layout above
 *   block_tables  in  int32 [num_seqs][max_blocks_per_seq], -1 padded
 *   context_lens  in  int32 [num_seqs]: tokens attended by sequence s,
 *                     including the one written this step (position L - 1)
 *   max_context_len   host-side upper bound of context_lens (sizes the grid)
 *   scale             multiplies q.k before the softmax (typically 1/sqrt(D))
 *   partition_size    0: single pass, no workspace needed.  Otherwise split
 *                     the context into partitions of this many tokens (a
 *                     multiple of 16 and of block_size) and merge them with a
 *                     log-sum-exp reduction.
 *   workspace, workspace_bytes  >= pa_decode_workspace_bytes(...) when
 *                     partition_size > 0; may be NULL/0 otherwise.
 *   flags             0 or PA_DECODE_SHARED_BLOCKS (a cache hint, above)
 *
 * out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) V_t over t < L_s, with
 * K_t, V_t read from block block_tables[s][t / B] at offset t % B and KV head
 * h / G.  A sequence with L_s == 0 gets zeros; context_lens[s] larger than
 * max_context_len or max_blocks_per_seq * block_size is clamped to the
 * smaller.  Table entries at or past ceil(L_s / B) are never read.  Slots of
 * the last block past L_s are never used (they may hold anything, NaN
 * included).  Returns PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED /
 * PA_ERR_WORKSPACE on a failed check; with partition_size > 0,
 * PA_ERR_UNSUPPORTED also when num_seqs * (4 * ceil(max_context_len / 16)
 * + 12) exceeds 2^31 - 1 or, times num_kv_heads, reaches 2^40 (the split
 * schedule places each 16-token tile at 4 line positions and each
 * (sequence, KV head) run start at 12, counts positions per KV head in
 * 32-bit integers and divides them in doubles).
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
              int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
              int32_t flags, void* stream);

/*
 * pa_decode_partials / pa_decode_merge -- the two phases pa_decode runs when
 * partition_size > 0, callable one by one with the same arguments and
 * workspace, partials first.  pa_decode_partials writes the records (and the
 * outputs of pairs that are a single piece); pa_decode_merge combines each
 * remaining pair's records, M = max_p m_p, w_p = 2^(m_p - M),
 * out = sum_p w_p o_p / sum_p w_p l_p, and writes zeros for sequences of
 * length 0.
 */
int pa_decode_partials(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_context_len, float scale, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, int32_t dtype, int32_t flags,
                       void* stream);

int pa_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int32_t block_size, int32_t max_context_len, int32_t partition_size,
                    const void* workspace, size_t workspace_bytes, int32_t dtype, void* stream);

/*
 * pa_append_decode / pa_append_decode_partials -- a decode step that also
 * stores the step's own K/V row.
 * [P3 对 ModelRunner 的影响: the current token's K/V go to its slot and the
 *  kernel attends over the context through the block table; P2 BlockTable
 *  walkthrough: slot = block_table[s][pos // B] * B + pos % B.]
 *
 *   key, value        in      [num_seqs][num_kv_heads][head_dim], 16-byte
 *                             aligned: row s is the K/V of sequence s's
 *                             token at position L_s - 1
 *   k_cache, v_cache  in/out  pools in the layout above
 *   every other argument as pa_decode / pa_decode_partials
 *
 * The result equals pa_write_kv of row s at the slot of position L_s - 1
 * (L_s the clamped context length; nothing is written for L_s == 0 or a
 * table entry outside [0, num_blocks)) followed by pa_decode (respectively
 * pa_decode_partials, to be followed by pa_decode_merge).  For bf16 the
 * write is part of the decode launch: the worker that owns the last tile of
 * each (sequence, KV head) stores that head's row and uses it in its tile,
 * so no other launch or wave touches the slot.  For fp32 a write launch
 * precedes the decode.  Errors as pa_decode, plus PA_ERR_INVALID_ARG for a
 * missing or misaligned key/value (with num_seqs > 0).
 */
int pa_append_decode(void* out, const void* q, const void* key, const void* value, void* k_cache,
                     void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                     int32_t max_context_len, float scale, int32_t partition_size,
                     void* workspace, size_t workspace_bytes, int32_t dtype, int32_t flags,
                     void* stream);

int pa_append_decode_partials(void* out, const void* q, const void* key, const void* value,
                              void* k_cache, void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, int32_t dtype,
                              int32_t flags, void* stream);

/*
 * pa_prefill -- paged prefill / chunked-prefill attention: many query tokens
 * per sequence, causal, over the same paged cache the decode reads.
 * [P1 映射逻辑块与物理块: prefill asks for blocks by input length and reads
 *  them through the block table; P2 section 2.1 and section 三: the kernel
 *  gathers K/V by block and computes softmax(QK^T)V, the formula unchanged
 *  by paging; P3 PagedAttention 改变了什么: logical_block = t // B, offset =
 *  t % B.]
 *
 *   out           out  [num_query_tokens][num_heads][head_dim], dtype of q
 *   lse           out  fp32 [num_query_tokens][num_heads], or NULL: the natural
 *                      log of sum_t exp(scale * q . K_t) over the tokens the
 *                      row sees (-inf for a row that sees none) -- what
 *                      pa_merge_states needs to combine partial results
 *   q             in   [num_query_tokens][num_heads][head_dim]
 *   k_cache, v_cache in pools in the layout above
 *   block_tables  in   int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  in   int32 [num_seqs]: L_s, tokens of sequence s in the
 *                      cache, the query tokens included
 *   query_start   in   int32 [num_seqs + 1]: sequence s owns query rows
 *                      query_start[s] .. query_start[s+1] - 1 (n_s rows)
 *
 * The n_s query rows of sequence s are its last n_s positions,
 * L_s - n_s .. L_s - 1, whose K/V the caller has already written (pa_write_kv
 * at their slots).  Row i attends to tokens 0 .. L_s - n_s + i:
 *   out[query_start[s] + i][h] = softmax_t(scale * q . K_t) V_t over those
 * tokens, with query head h reading KV head h / (num_heads / num_kv_heads).
 * n_s = L_s is a whole prompt, n_s < L_s a chunk after earlier chunks, and
 * n_s = 1 the decode step.  L_s is clamped as in pa_decode and n_s to the
 * rows of q.  Only the first max_query_len rows of a sequence are computed
 * (their positions still count all n_s rows); rows beyond are not written.  A row
 * whose position is negative (n_s > L_s, a broken precondition) sees no token
 * and gets zeros.  Any group size is supported.  bf16 runs on matrix cores
 * (16x16 tiles of (position, head) rows x tokens); fp32 runs one wave per row.
 * No workspace.  Errors as pa_decode; PA_ERR_UNSUPPORTED when the launch
 * would exceed the grid limits.
 */
int pa_prefill(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, int32_t num_seqs, int32_t num_query_tokens,
               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
               int32_t max_query_len, float scale, int32_t dtype, void* stream);

/*
 * pa_decode_lse -- pa_decode that also writes, for every (sequence, query
 * head), the natural log of sum_t exp(scale * q . K_t) over its context:
 *   lse  out  fp32 [num_seqs][num_heads] (-inf for a sequence of length 0)
 * Other arguments, results and errors as pa_decode; PA_ERR_INVALID_ARG for a
 * NULL lse when num_seqs > 0.  This is what pa_merge_states needs to combine
 * decodes over disjoint token sets, e.g. the context-parallel ranks below.
 */
int pa_decode_lse(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                  float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                  int32_t dtype, int32_t flags, void* stream);

/*
 * Shared-prefix decode.
 * [P1 共享但不污染状态: branches sampled from one prompt reference the same
 *  physical blocks for their common tokens (reference counted, immutable)
 *  until a branch writes into a shared block, which copy-on-write first
 *  makes private; P2 section 2.1 (共享与写时复制): physical blocks are shared
 *  across sequences through their block tables.]
 *
 * pa_decode_shared_prefix computes exactly what pa_decode (with key/value:
 * pa_append_decode) computes, and is told which sequences share blocks so
 * that each shared block is read once per KV head for all the sharers'
 * query heads instead of once per sequence:
 *
 *   group_start  in  int32 [num_groups + 1], device: group i is sequences
 *                    group_start[i] .. group_start[i+1] - 1 (consecutive in
 *                    the batch; groups in increasing order, disjoint)
 *   prefix_lens  in  int32 [num_groups], device: the first prefix_lens[i]
 *                    tokens of every member of group i lie in the same
 *                    physical blocks (the members' tables agree on those
 *                    entries)
 *   key, value   in  as pa_append_decode, or both NULL (no row appended)
 *   other arguments as pa_decode; partition_size must be > 0, and the
 *   workspace at least pa_decode_shared_prefix_workspace_bytes(...) long
 *   (16-byte aligned, zero-filled once, reusable as pa_decode's).
 *
 * Each group's shared tokens, rounded down to a multiple of 16 and to the
 * first member's length, are streamed once per KV head through the first
 * member's table, with the query heads of up to 64 / G members (32 / G at
 * head_dim 256) as matrix-core columns; the members' other tokens are
 * decoded as pa_decode does, and a log-sum-exp merge combines the two.
 * Members beyond that count decode all their tokens themselves, so any
 * group size is correct.  Preconditions: the tables agree as stated (the
 * shared tokens are read through the first member's table), and with
 * key/value a member's row position L - 1 lies past its shared tokens
 * (copy-on-write has made the block it is written into private); a row
 * whose position lies inside them is not written.  Broken preconditions
 * give wrong values, never out-of-bounds accesses.  The fp32 kernel ignores
 * the groups (it decodes every sequence's tokens; same results).
 * pa_decode_shared_prefix_partials and pa_decode_shared_prefix_merge are
 * its two launches, callable one by one.  Errors as pa_decode, plus
 * PA_ERR_INVALID_ARG for num_groups < 0, partition_size <= 0, NULL group
 * arrays (num_groups > 0), or only one of key / value, and
 * PA_ERR_UNSUPPORTED for num_groups > 512.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t partition_size,
                                               int32_t num_groups);

int pa_decode_shared_prefix(void* out, const void* q, const void* key, const void* value,
                            void* k_cache, void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* group_start,
                            const int32_t* prefix_lens, int32_t num_groups, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, float scale, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, int32_t dtype,
                            int32_t flags, void* stream);

int pa_decode_shared_prefix_partials(void* out, const void* q, const void* key, const void* value,
                                     void* k_cache, void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* group_start,
                                     const int32_t* prefix_lens, int32_t num_groups,
                                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, int32_t dtype, int32_t flags,
                                     void* stream);

int pa_decode_shared_prefix_merge(void* out, const int32_t* context_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int32_t num_groups, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t block_size,
                                  int32_t max_context_len, int32_t partition_size,
                                  const void* workspace, size_t workspace_bytes, int32_t dtype,
                                  void* stream);

/*
 * pa_decode_scratch -- pa_decode with no workspace argument, for callers
 * that cannot allocate device memory (code being recorded into a HIP graph,
 * tight serving loops, hosts that forbid hipMalloc): it allocates nothing
 * itself either.
 *
 * Arguments, results and errors as pa_decode without workspace and
 * workspace_bytes.  With partition_size > 0 the split-KV records go to a
 * scratch buffer the library holds: a fixed 64 MiB array in device memory,
 * one per device, present from the library's load until the process ends.
 * A call whose workspace would exceed it (pa_decode_workspace_bytes with the
 * same sizes > 64 MiB) returns PA_ERR_TOO_LARGE before anything is enqueued.
 * The first call on a device also enqueues one kernel that zeroes that
 * device's buffer.  Every call on a device shares its buffer: calls that
 * overlap in time on one device (on different streams, or from different
 * threads without ordering) race and may return wrong results; calls
 * ordered on one stream do not.  partition_size == 0 runs the single pass,
 * which needs no buffer.
 */
int pa_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_context_len, float scale, int32_t partition_size,
                      int32_t dtype, int32_t flags, void* stream);

/*
 * Context parallelism.
 * [P2 BlockTable walkthrough: under decode / prefill context parallelism the
 *  slot mapping uses a virtual block size and a mask, and writes -1 for the
 *  entries a rank does not own.]
 *
 * The pages give no ownership formula; the one used here: cp_world ranks
 * share one block table and each has its own pool.  Token p lies in virtual
 * block p / (block_size * cp_world), i.e. table entry
 * block_tables[s][p / (block_size * cp_world)] on every rank.  Inside the
 * virtual block, runs of `interleave` tokens (a divisor of block_size) go to
 * ranks 0 .. cp_world-1 in turn, and a rank packs the runs it owns into the
 * block_size slots of its copy of the block, in order.  A rank's tokens thus
 * form an ordinary paged sequence in its own pool, whose length
 * pa_cp_context_lens gives: pa_decode_lse (or pa_prefill with lse) attends
 * over it, and pa_merge_states combines the ranks' results.
 * cp_world = 1 is the plain mapping.  Exchanging the partial results between
 * GPUs is the caller's (one all-gather of out and lse per step).
 */

/*
 * pa_cp_slot_mapping -- rank cp_rank's slot of each (sequence, position)
 * row: block_tables[s][p / (B * W)] * B + local offset for tokens the rank
 * owns, -1 for the others and for rows outside the table (as
 * pa_slot_mapping).  Arguments as pa_slot_mapping plus cp_world >= 1,
 * 0 <= cp_rank < cp_world, interleave >= 1 dividing block_size.
 */
int pa_cp_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                       const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                       int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t cp_world, int32_t cp_rank, int32_t interleave, void* stream);

/*
 * pa_cp_context_lens -- tokens rank cp_rank holds of each sequence:
 *   local_lens  out  int32 [num_seqs]
 *   context_lens in  int32 [num_seqs] (negative counts as 0)
 */
int pa_cp_context_lens(int32_t* local_lens, const int32_t* context_lens, int32_t num_seqs,
                       int32_t block_size, int32_t cp_world, int32_t cp_rank, int32_t interleave,
                       void* stream);

/*
 * pa_merge_states -- combine partial attention results over disjoint token
 * sets (context-parallel ranks, or any split of a sequence's tokens) with
 * the log-sum-exp identity:
 *   out[r] = sum_w e^(lse_w[r] - M) states_w[r] / sum_w e^(lse_w[r] - M),
 *   out_lse[r] = M + ln sum_w e^(lse_w[r] - M),  M = max_w lse_w[r].
 *   out         out  [num_rows][head_dim], dtype
 *   out_lse     out  fp32 [num_rows], or NULL
 *   states      in   [num_states][num_rows][head_dim], dtype
 *   state_lses  in   fp32 [num_states][num_rows]
 * A row of a decode or prefill output is one (token, head): num_rows =
 * tokens * heads.  A state whose lse is -inf (no tokens) is ignored; a row
 * whose every lse is -inf gets zeros and -inf; a NaN lse makes the row NaN.
 * head_dim must be a multiple of 4; out and states aligned to 4 elements.
 */
int pa_merge_states(void* out, float* out_lse, const void* states, const float* state_lses,
                    int32_t num_states, int32_t num_rows, int32_t head_dim, int32_t dtype,
                    void* stream);

/*
 * pa_map_to_kernel_blocks -- tables for the kernel when the allocator's
 * block holds k = kernel_blocks_per_block kernel blocks.
 * [P2 BlockTable walkthrough: when the allocator's block size differs from
 *  the one the kernel needs, each allocator block is split into several
 *  kernel blocks.]
 *   kernel_tables  out int32 [num_rows][max_blocks_per_row * k]
 *   manager_tables in  int32 [num_rows][max_blocks_per_row]
 * Entry i * k + j = manager_tables[i] * k + j (-1 stays -1, and so does an id
 * whose product overflows int32): the pool is laid out in kernel blocks, and
 * allocator block b is kernel blocks b*k .. b*k+k-1.  Every token then has
 * the same slot number through either table (at block sizes k*B and B).
 */
int pa_map_to_kernel_blocks(int32_t* kernel_tables, const int32_t* manager_tables,
                            int32_t num_rows, int32_t max_blocks_per_row,
                            int32_t kernel_blocks_per_block, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

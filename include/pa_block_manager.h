/*
 * pa_block_manager.h -- host-side KV block manager of libpa.so.
 *
 * The allocator that the paged decode path presupposes: it owns the free
 * physical blocks of one K/V pool, keeps every sequence's block table, and
 * hands out what the device calls of pa.h consume -- int64 slots for
 * pa_write_kv, int64 (src, dst) pairs for pa_copy_blocks, and int32 table
 * rows plus context lengths for the decode entry points.  It runs on the
 * host only and never touches device memory.  Pages this follows:
 *
 *   [P3] "KV cache 显存管理：为什么 PagedAttention 是 vLLM 的核心", section
 *        "Block manager 是 PagedAttention 的前置条件": the block manager keeps
 *        the free blocks, allocates for new requests, adds blocks during
 *        decode, keeps each sequence's table, frees at the end, and says
 *        whether memory can take a new request; section "对 Scheduler 的影响":
 *        prefill needs blocks for every prompt token, decode a new block only
 *        when the current one is full, and a batch whose new blocks exceed the
 *        free ones cannot run as a whole.
 *   [P1] "什么是 PagedAttention？", 映射逻辑块与物理块: decode fills the tail
 *        block before taking a new one; a failed allocation is reported and
 *        never served by overwriting another sequence's state.
 *        共享但不污染状态: sequences share immutable blocks under a reference
 *        count; writing into a shared partial block first gives the writer a
 *        private copy and changes only the writer's table.
 *   [P2] "PagedAttention学习笔记", section 2.1 and its state diagram: ceil(L/B)
 *        blocks per sequence, ref_cnt per block, a block returns to the free
 *        pool when its count drops to zero.
 *
 * Policy where the pages leave a choice:
 *   - the free queue is first-in first-out (allocation takes the head; a
 *     block whose count reaches zero joins the tail; a finished sequence
 *     releases its blocks in logical order); its initial order is the
 *     caller's `free_order`, or ascending ids;
 *   - a decode batch is served in list order, and is all or nothing: on a
 *     shortage the call returns PA_ERR_NO_BLOCKS and changes nothing, so the
 *     caller can preempt (pa_bm_free) or shrink the batch and retry;
 *   - copy-on-write copies whole blocks; of k sequences that share one
 *     partial tail block and append in one batch, the first k-1 get private
 *     copies and the last writes in place.
 *
 * Sequences are rows [0, max_seqs) of the block table.  Status codes are
 * those of pa.h: PA_OK, PA_ERR_INVALID_ARG (null pointer, id out of range,
 * negative size, a sequence listed twice, a table row that would overflow),
 * PA_ERR_NO_BLOCKS (not enough free blocks; nothing changed), PA_ERR_STATE
 * (a sequence that must be live is not, or one that must be idle is live).
 * Every failing call leaves the manager unchanged.  A handle is not
 * thread-safe: one caller at a time.  The handle owns its host memory; the
 * caller owns every array it passes.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/*
 * pa_bm_create -- a manager of num_blocks blocks of block_size tokens, for
 * up to max_seqs sequences of up to max_blocks_per_seq blocks each.
 *   free_order  in   int32 [num_blocks], a permutation of 0..num_blocks-1
 *                    giving the initial free-queue order, or NULL (ascending)
 *   out         out  the new handle (NULL on failure)
 * PA_ERR_INVALID_ARG for non-positive sizes or a free_order that is not a
 * permutation; PA_ERR_HIP is never returned.
 */
int pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                 int32_t max_blocks_per_seq, const int32_t* free_order, pa_block_manager** out);

/* Release the handle and its memory (NULL is ignored). */
void pa_bm_destroy(pa_block_manager* bm);

/* Free blocks (reference count zero). */
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/* Reference count of a block: the number of live tables holding it; -1 for an
 * id outside [0, num_blocks). */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block);

/* Tokens held by a sequence; -1 if it is not live or out of range. */
int32_t pa_bm_context_len(const pa_block_manager* bm, int32_t seq);

/*
 * pa_bm_can_allocate -- admission test [P3 对 Scheduler 的影响]: 1 if a new
 * sequence of num_tokens tokens fits (ceil(num_tokens / B) blocks free and
 * within a table row), 0 if not, PA_ERR_INVALID_ARG for num_tokens < 0.
 */
int pa_bm_can_allocate(const pa_block_manager* bm, int32_t num_tokens);

/*
 * pa_bm_allocate -- prefill: make idle sequence `seq` live with num_tokens
 * tokens in ceil(num_tokens / B) blocks taken from the free queue
 * [P1 映射逻辑块与物理块: prefill asks for blocks by input length].
 *   slots  out  int64 [num_tokens] host: the slot of positions 0..num_tokens-1
 *               (table[pos / B] * B + pos % B), ready for pa_write_kv; may be
 *               NULL when num_tokens == 0
 * Zero tokens make a live sequence with an empty table.
 */
int pa_bm_allocate(pa_block_manager* bm, int32_t seq, int32_t num_tokens, int64_t* slots);

/*
 * pa_bm_fork -- idle sequence `child` shares every block of live `parent`
 * (parallel sampling, beams) [P1 共享但不污染状态; P2 2.1]: same table and
 * length, every count raised by one.  Takes no block.
 */
int pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t child);

/*
 * pa_bm_blocks_needed_to_append -- the free blocks pa_bm_append would take
 * for this batch (new tail blocks plus copy-on-write copies), or a negative
 * status for arguments pa_bm_append would reject (other than a shortage).
 */
int pa_bm_blocks_needed_to_append(const pa_block_manager* bm, const int32_t* seqs, int32_t n);

/*
 * pa_bm_append -- decode: one more token for each of the n distinct live
 * sequences in `seqs`, in list order [P1 映射逻辑块与物理块; P1
 * 共享但不污染状态; P3 对 Scheduler 的影响].  A sequence whose length is a
 * multiple of B takes a new block; one whose partial tail block is shared
 * takes a private block and a copy pair; otherwise it writes in place.
 *   slots       out  int64 [n] host: slot of each sequence's new token
 *   copy_pairs  out  int64 [n][2] host: (src, dst) blocks for pa_copy_blocks,
 *                    to run before the write; the first *num_copies rows are set
 *   num_copies  out  number of pairs
 * PA_ERR_NO_BLOCKS if the batch needs more blocks than are free (nothing
 * changes); PA_ERR_INVALID_ARG if a row would exceed max_blocks_per_seq.
 */
int pa_bm_append(pa_block_manager* bm, const int32_t* seqs, int32_t n, int64_t* slots,
                 int64_t* copy_pairs, int32_t* num_copies);

/*
 * pa_bm_free -- the sequence ends (or is preempted): every count of its
 * blocks drops by one and blocks reaching zero join the free queue's tail
 * [P3 Block manager section; P2 state diagram].
 */
int pa_bm_free(pa_block_manager* bm, int32_t seq);

/*
 * pa_bm_block_tables -- export table rows for the decode entry points.
 *   seqs          in   int32 [n] host rows to export, or NULL for rows 0..n-1
 *   block_tables  out  int32 [n][max_blocks_per_seq] host, padded with -1
 *   context_lens  out  int32 [n] host (0 for an idle sequence); may be NULL
 */
int pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t n,
                       int32_t* block_tables, int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */

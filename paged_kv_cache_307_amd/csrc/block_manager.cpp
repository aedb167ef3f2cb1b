// Host-side KV block manager: free queue, reference counts, block tables.
//
// What it does follows the pages' account of the block manager ("KV cache
// 显存管理：为什么 PagedAttention 是 vLLM 的核心", sections on the block
// manager and on the scheduler; "什么是 PagedAttention？", sections 映射逻辑块与
// 物理块 and 共享但不污染状态; "PagedAttention学习笔记", section 2.1 and its
// block state diagram).  The policy choices the pages leave open are stated in
// include/pa_block_manager.h.
//
// Layout: every array is sized once at creation, so no call allocates.  The
// free queue is a ring of num_blocks ids; tables are one flat
// [max_seqs][max_blocks_per_seq] int32 array, -1 past each row's blocks, which
// is exactly the row format the decode entry points read.  A decode batch is
// planned before anything changes (so a shortage leaves no trace): the plan
// walks the batch in order with a per-block "count as earlier members left
// it" kept in a scratch array and reset afterwards.

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "pa_block_manager.h"

namespace {

enum Step : int8_t { kInPlace = 0, kNewBlock = 1, kCopyOnWrite = 2 };

}  // namespace

struct pa_block_manager {
  int32_t num_blocks, block_size, max_seqs, max_blocks;
  std::vector<int32_t> ring;     // free queue: ring[(head + i) % num_blocks], i < free_count
  int32_t head = 0, free_count = 0;
  std::vector<int32_t> ref;      // per block
  std::vector<int32_t> table;    // [max_seqs][max_blocks], -1 padded
  std::vector<int32_t> nblk;     // blocks in each row
  std::vector<int32_t> len;      // tokens per sequence, -1 = idle
  // scratch for planning a batch
  std::vector<int32_t> pending;  // per block: count as earlier batch members left it, -1 = untouched
  std::vector<int32_t> touched;  // blocks whose `pending` entry is set
  std::vector<int8_t> plan;      // per batch member
  std::vector<uint8_t> listed;   // per sequence: seen in this batch

  int32_t* row(int32_t s) { return table.data() + int64_t(s) * max_blocks; }
  const int32_t* row(int32_t s) const { return table.data() + int64_t(s) * max_blocks; }
  int64_t capacity_tokens() const { return int64_t(max_blocks) * block_size; }

  int32_t pop_free() {
    int32_t b = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --free_count;
    return b;
  }
  void push_free(int32_t b) {
    int64_t tail = int64_t(head) + free_count;
    ring[tail % num_blocks] = b;
    ++free_count;
  }

  // Argument checks shared by append and its block count; same order as the
  // status precedence documented in the header.
  int check_batch(const int32_t* seqs, int32_t n) {
    if (n < 0 || (n > 0 && !seqs)) return PA_ERR_INVALID_ARG;
    int st = PA_OK;
    int32_t i = 0;
    for (; i < n; ++i) {
      int32_t s = seqs[i];
      if (s < 0 || s >= max_seqs || listed[s]) { st = PA_ERR_INVALID_ARG; break; }
      listed[s] = 1;
    }
    for (int32_t j = 0; j < i; ++j) listed[seqs[j]] = 0;
    if (st != PA_OK) return st;
    for (i = 0; i < n; ++i)
      if (len[seqs[i]] < 0) return PA_ERR_STATE;
    for (i = 0; i < n; ++i)
      if (len[seqs[i]] >= capacity_tokens()) return PA_ERR_INVALID_ARG;
    return PA_OK;
  }

  // Fill plan[0..n) and return the number of fresh blocks the batch takes.
  int32_t make_plan(const int32_t* seqs, int32_t n) {
    int32_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      int32_t s = seqs[i], pos = len[s];
      if (pos % block_size == 0) {
        plan[i] = kNewBlock;
        ++need;
        continue;
      }
      int32_t tail = row(s)[pos / block_size];
      int32_t count = pending[tail] >= 0 ? pending[tail] : ref[tail];
      if (count > 1) {
        if (pending[tail] < 0) touched.push_back(tail);
        pending[tail] = count - 1;
        plan[i] = kCopyOnWrite;
        ++need;
      } else {
        plan[i] = kInPlace;
      }
    }
    for (int32_t b : touched) pending[b] = -1;
    touched.clear();
    return need;
  }
};

extern "C" {

int pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                 int32_t max_blocks_per_seq, const int32_t* free_order, pa_block_manager** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1 || max_seqs < 1 || max_blocks_per_seq < 1)
    return PA_ERR_INVALID_ARG;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return PA_ERR_INVALID_ARG;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_seqs = max_seqs;
    bm->max_blocks = max_blocks_per_seq;
    bm->ring.resize(num_blocks);
    bm->ref.assign(num_blocks, 0);
    bm->table.assign(size_t(max_seqs) * size_t(max_blocks_per_seq), -1);
    bm->nblk.assign(max_seqs, 0);
    bm->len.assign(max_seqs, -1);
    bm->pending.assign(num_blocks, -1);
    bm->touched.reserve(max_seqs);
    bm->plan.assign(max_seqs, kInPlace);
    bm->listed.assign(max_seqs, 0);
  } catch (...) {
    delete bm;
    return PA_ERR_INVALID_ARG;
  }
  if (free_order) {
    // must be a permutation: mark each id once
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PA_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      bm->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->ring[i] = i;
  }
  bm->head = 0;
  bm->free_count = num_blocks;
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) { return bm ? bm->free_count : -1; }

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pa_bm_context_len(const pa_block_manager* bm, int32_t seq) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return -1;
  return bm->len[seq];
}

int pa_bm_can_allocate(const pa_block_manager* bm, int32_t num_tokens) {
  if (!bm || num_tokens < 0) return PA_ERR_INVALID_ARG;
  int64_t need = (int64_t(num_tokens) + bm->block_size - 1) / bm->block_size;
  return need <= bm->max_blocks && need <= bm->free_count ? 1 : 0;
}

int pa_bm_allocate(pa_block_manager* bm, int32_t seq, int32_t num_tokens, int64_t* slots) {
  if (!bm || seq < 0 || seq >= bm->max_seqs || num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens > 0 && !slots) return PA_ERR_INVALID_ARG;
  if (bm->len[seq] >= 0) return PA_ERR_STATE;
  const int32_t B = bm->block_size;
  int64_t need = (int64_t(num_tokens) + B - 1) / B;
  if (need > bm->max_blocks) return PA_ERR_INVALID_ARG;
  if (need > bm->free_count) return PA_ERR_NO_BLOCKS;
  int32_t* r = bm->row(seq);
  for (int32_t i = 0; i < int32_t(need); ++i) {
    int32_t b = bm->pop_free();
    bm->ref[b] = 1;
    r[i] = b;
  }
  bm->nblk[seq] = int32_t(need);
  bm->len[seq] = num_tokens;
  for (int32_t t = 0; t < num_tokens; ++t) slots[t] = int64_t(r[t / B]) * B + t % B;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t child) {
  if (!bm || parent < 0 || parent >= bm->max_seqs || child < 0 || child >= bm->max_seqs)
    return PA_ERR_INVALID_ARG;
  if (bm->len[parent] < 0 || bm->len[child] >= 0) return PA_ERR_STATE;
  const int32_t n = bm->nblk[parent];
  std::memcpy(bm->row(child), bm->row(parent), sizeof(int32_t) * size_t(n));
  for (int32_t i = 0; i < n; ++i) ++bm->ref[bm->row(parent)[i]];
  bm->nblk[child] = n;
  bm->len[child] = bm->len[parent];
  return PA_OK;
}

int pa_bm_blocks_needed_to_append(const pa_block_manager* cbm, const int32_t* seqs, int32_t n) {
  if (!cbm) return PA_ERR_INVALID_ARG;
  // planning only touches scratch arrays, which it restores
  pa_block_manager* bm = const_cast<pa_block_manager*>(cbm);
  int st = bm->check_batch(seqs, n);
  if (st != PA_OK) return st;
  return bm->make_plan(seqs, n);
}

int pa_bm_append(pa_block_manager* bm, const int32_t* seqs, int32_t n, int64_t* slots,
                 int64_t* copy_pairs, int32_t* num_copies) {
  if (!bm || !num_copies) return PA_ERR_INVALID_ARG;
  *num_copies = 0;
  if (n > 0 && (!slots || !copy_pairs)) return PA_ERR_INVALID_ARG;
  int st = bm->check_batch(seqs, n);
  if (st != PA_OK) return st;
  if (bm->make_plan(seqs, n) > bm->free_count) return PA_ERR_NO_BLOCKS;
  const int32_t B = bm->block_size;
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t s = seqs[i], pos = bm->len[s];
    int32_t* r = bm->row(s);
    if (bm->plan[i] == kNewBlock) {
      int32_t b = bm->pop_free();
      bm->ref[b] = 1;
      r[bm->nblk[s]++] = b;
    } else if (bm->plan[i] == kCopyOnWrite) {
      int32_t tail = r[pos / B];
      int32_t b = bm->pop_free();
      bm->ref[b] = 1;
      --bm->ref[tail];
      r[pos / B] = b;
      copy_pairs[2 * copies] = tail;
      copy_pairs[2 * copies + 1] = b;
      ++copies;
    }
    slots[i] = int64_t(r[pos / B]) * B + pos % B;
    bm->len[s] = pos + 1;
  }
  *num_copies = copies;
  return PA_OK;
}

int pa_bm_free(pa_block_manager* bm, int32_t seq) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return PA_ERR_INVALID_ARG;
  if (bm->len[seq] < 0) return PA_ERR_STATE;
  int32_t* r = bm->row(seq);
  for (int32_t i = 0; i < bm->nblk[seq]; ++i) {
    int32_t b = r[i];
    if (--bm->ref[b] == 0) bm->push_free(b);
    r[i] = -1;
  }
  bm->nblk[seq] = 0;
  bm->len[seq] = -1;
  return PA_OK;
}

int pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t n,
                       int32_t* block_tables, int32_t* context_lens) {
  if (!bm || n < 0 || (n > 0 && !block_tables)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    int32_t s = seqs ? seqs[i] : i;
    if (s < 0 || s >= bm->max_seqs) return PA_ERR_INVALID_ARG;
  }
  const size_t row_bytes = sizeof(int32_t) * size_t(bm->max_blocks);
  for (int32_t i = 0; i < n; ++i) {
    int32_t s = seqs ? seqs[i] : i;
    std::memcpy(block_tables + int64_t(i) * bm->max_blocks, bm->row(s), row_bytes);
    if (context_lens) context_lens[i] = bm->len[s] < 0 ? 0 : bm->len[s];
  }
  return PA_OK;
}

}  // extern "C"

// Slot mapping, KV write and copy-on-write block copy kernels.
//
// [P2 "PagedAttention学习笔记", BlockTable walkthrough] slot = block_id * B +
// pos % B with block_id = block_table[req, pos // B]; -1 = not this rank's row.
// [P3 "KV cache 显存管理", 对 ModelRunner 的影响] the current token's K/V are
// written at its slot.  [P1 "什么是 PagedAttention？", 共享但不污染状态] a
// writer to a shared partial block first gets a private copy.
//
// The appending form of the write takes the slot of each sequence's last
// position from its block table (the decode step's own token).
//
// All of them are HBM-bound byte movers; each 64-lane wave moves whole 16-byte
// vectors where the layout is contiguous (K rows, whole blocks) and single
// elements where it is strided (V's token-innermost rows).

#include "device_common.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void slot_mapping_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, int num_tokens,
    int num_seqs, int max_blocks_per_seq, int block_size) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_tokens) return;
  const int s = seq_ids[i];
  const int pos = positions[i];
  int64_t slot = -1;
  if (s >= 0 && s < num_seqs && pos >= 0) {
    const int logical = pos / block_size;
    if (logical < max_blocks_per_seq) {
      const int32_t block = block_tables[int64_t(s) * max_blocks_per_seq + logical];
      if (block >= 0) slot = int64_t(block) * block_size + pos % block_size;
    }
  }
  slots[i] = slot;
}

// Store one token row (all KV heads) at (block, off): K rows are contiguous
// (head_dim elements per KV head) and move as 16-byte vectors; V stores each
// element at stride block_size (tokens innermost).  One workgroup.
template <typename Elem>
__device__ __forceinline__ void store_row(Elem* __restrict__ k_cache, Elem* __restrict__ v_cache,
                                          const Elem* __restrict__ key_row,
                                          const Elem* __restrict__ value_row, int64_t block,
                                          int off, int num_kv_heads, int head_dim,
                                          int block_size) {
  const int row = num_kv_heads * head_dim;            // elements per token row
  const int64_t block_elems = int64_t(row) * block_size;
  constexpr int kVec = 16 / sizeof(Elem);
  const int row_vecs = row / kVec;
  const int dim_vecs = head_dim / kVec;
  const uint4* src_k = reinterpret_cast<const uint4*>(key_row);
  for (int v = threadIdx.x; v < row_vecs; v += kThreads) {
    const int h = v / dim_vecs;
    const int dv = v % dim_vecs;
    Elem* dst = k_cache + block * block_elems + (int64_t(h) * block_size + off) * head_dim;
    reinterpret_cast<uint4*>(dst)[dv] = src_k[v];
  }
  Elem* vblk = v_cache + block * block_elems + off;
  for (int e = threadIdx.x; e < row; e += kThreads) {
    // e = h * head_dim + d  ->  v_cache[block][h][d][off]
    vblk[int64_t(e) * block_size] = value_row[e];
  }
}

// One workgroup per token row i, stored at slot_mapping[i].
template <typename Elem>
__global__ __launch_bounds__(kThreads) void write_kv_kernel(
    Elem* __restrict__ k_cache, Elem* __restrict__ v_cache, const Elem* __restrict__ key,
    const Elem* __restrict__ value, const int64_t* __restrict__ slots, int num_kv_heads,
    int head_dim, int block_size, int num_blocks) {
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= int64_t(num_blocks) * block_size) return;
  const int64_t row = int64_t(i) * num_kv_heads * head_dim;
  store_row(k_cache, v_cache, key + row, value + row, slot / block_size, int(slot % block_size),
            num_kv_heads, head_dim, block_size);
}

// One workgroup per sequence s: its row goes to position L_s - 1 (L_s the
// clamped context length) through the block table; nothing for L_s = 0 or
// a table entry outside [0, num_blocks).
template <typename Elem>
__global__ __launch_bounds__(kThreads) void append_kv_kernel(DecodeArgs a, int head_dim,
                                                             int block_size) {
  const int s = blockIdx.x;
  const int L = effective_len(a, s, block_size);
  if (L == 0) return;
  const int p = L - 1;
  const int32_t block = a.block_tables[int64_t(s) * a.max_blocks_per_seq + p / block_size];
  if (block < 0 || block >= a.num_blocks) return;
  const int64_t row = int64_t(s) * a.num_kv_heads * head_dim;
  // the pools are writable when a row is appended (the API takes them non-const)
  store_row(static_cast<Elem*>(const_cast<void*>(a.k_cache)),
            static_cast<Elem*>(const_cast<void*>(a.v_cache)),
            static_cast<const Elem*>(a.new_k) + row, static_cast<const Elem*>(a.new_v) + row,
            block, p % block_size, a.num_kv_heads, head_dim, block_size);
}

// One workgroup per (pair, pool): copies a whole block of one pool.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const int64_t* __restrict__ pairs,
    int64_t block_vecs, int num_blocks) {
  const int pair = blockIdx.x >> 1;
  uint4* pool = (blockIdx.x & 1) ? v_cache : k_cache;
  const int64_t src = pairs[2 * int64_t(pair)];
  const int64_t dst = pairs[2 * int64_t(pair) + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* from = pool + src * block_vecs;
  uint4* to = pool + dst * block_vecs;
  for (int64_t v = threadIdx.x; v < block_vecs; v += kThreads) to[v] = from[v];
}

}  // namespace

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* block_tables, const int32_t* seq_ids,
                               const int32_t* positions, int num_tokens, int num_seqs,
                               int max_blocks_per_seq, int block_size, hipStream_t stream) {
  return launch(slot_mapping_kernel, dim3(ceil_div(num_tokens, kThreads)), dim3(kThreads), 0,
                stream, slots, block_tables, seq_ids, positions, num_tokens, num_seqs,
                max_blocks_per_seq, block_size);
}

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* key, const void* value,
                           const int64_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int elem_bytes, hipStream_t stream) {
  if (elem_bytes == 4) {
    return launch(write_kv_kernel<uint32_t>, dim3(num_tokens), dim3(kThreads), 0, stream,
                  static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                  static_cast<const uint32_t*>(key), static_cast<const uint32_t*>(value), slots,
                  num_kv_heads, head_dim, block_size, num_blocks);
  }
  return launch(write_kv_kernel<uint16_t>, dim3(num_tokens), dim3(kThreads), 0, stream,
                static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value), slots,
                num_kv_heads, head_dim, block_size, num_blocks);
}

hipError_t launch_append_kv(const DecodeArgs& a, int head_dim, int block_size, int elem_bytes,
                            hipStream_t stream) {
  if (elem_bytes == 4)
    return launch(append_kv_kernel<uint32_t>, dim3(a.num_seqs), dim3(kThreads), 0, stream, a,
                  head_dim, block_size);
  return launch(append_kv_kernel<uint16_t>, dim3(a.num_seqs), dim3(kThreads), 0, stream, a,
                head_dim, block_size);
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              int elem_bytes, hipStream_t stream) {
  const int64_t block_vecs = int64_t(num_kv_heads) * block_size * head_dim * elem_bytes / 16;
  return launch(copy_blocks_kernel, dim3(2 * num_pairs), dim3(kThreads), 0, stream,
                static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs, block_vecs,
                num_blocks);
}

}  // namespace pa

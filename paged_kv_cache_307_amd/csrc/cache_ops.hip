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
// All of them are HBM-bound byte movers.  They move whole 16-byte vectors
// where the layout is contiguous (K rows, whole blocks, and V rows of blocks
// the write fills, transposed through LDS) and single elements where it is
// strided (V's token-innermost rows of a lone token).

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

// Rows per workgroup of the write (the LDS arrays are sized for it, one row
// per thread).  Writes with few chunks take 64 rows per workgroup and split
// the KV heads over workgroups: a prefill chunk's 8192 rows of 8 heads in
// 1024 workgroups, 25.9 us, against 30.8 us at 128 rows and 47 us at 256.
// A whole history keeps 256 rows and one pass over all heads of a chunk:
// 331 us for 131,759 rows, against 369 us in 64-row split chunks.
constexpr int kWriteChunk = 256;
constexpr int kSmallWriteChunk = 64;
// Below this many chunks the write also splits KV heads over workgroups.
constexpr int kSplitHeadsBelowChunks = 512;
// Largest (block, KV head) V tile the write transposes through LDS.
constexpr int kTileLdsBytes = 32768;

// One wave stores KV head h of one token row at (block, off): the K row as
// 16-byte vectors, V one element per dim at stride block_size.
template <typename Elem>
__device__ __forceinline__ void store_head_wave(Elem* __restrict__ k_cache,
                                                Elem* __restrict__ v_cache,
                                                const Elem* __restrict__ key_row,
                                                const Elem* __restrict__ value_row, int64_t block,
                                                int off, int h, int num_kv_heads, int head_dim,
                                                int block_size, int lane) {
  const int64_t tile = (block * num_kv_heads + h) * int64_t(block_size) * head_dim;
  constexpr int kVec = 16 / sizeof(Elem);
  const uint4* src_k = reinterpret_cast<const uint4*>(key_row + int64_t(h) * head_dim);
  uint4* dst_k = reinterpret_cast<uint4*>(k_cache + tile + int64_t(off) * head_dim);
  for (int v = lane; v < head_dim / kVec; v += 64) dst_k[v] = src_k[v];
  const Elem* src_v = value_row + int64_t(h) * head_dim;
  Elem* vt = v_cache + tile + off;
  for (int d = lane; d < head_dim; d += 64) vt[int64_t(d) * block_size] = src_v[d];  // [d][off]
}

// The write of rows [c0, c0 + n) of a slot mapping, n <= CHUNK <= kWriteChunk.
//
// Rows usually come sequence by sequence with ascending positions, so most
// blocks receive all B of their slots, in order, from B consecutive rows.
// Such a block is written as whole (block, KV head) tiles: K rows as 16-byte
// vectors, and V transposed through LDS so that each dim's row of B tokens
// leaves as full 16-byte vectors.  Storing a V column one element at a time
// (token-innermost layout) writes 2 of every 2 * B bytes of each row
// segment, a partial write of a memory sector per element.  Rows of blocks
// this chunk does not fill (and every row when the tile path does not
// apply) take the element path, one wave per row.  Slots are distinct (the
// API's precondition), so a block filled here gets no other row anywhere.
// The grid's second dimension splits the KV heads: workgroup (c, y) writes
// heads y, y + gridDim.y, ... of chunk c, so a chunk's blocks are written by
// as many workgroups as there are heads.
template <typename Elem, int CHUNK>
__global__ __launch_bounds__(kThreads) void write_kv_kernel(
    Elem* __restrict__ k_cache, Elem* __restrict__ v_cache, const Elem* __restrict__ key,
    const Elem* __restrict__ value, const int64_t* __restrict__ slots, int num_tokens,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, int tile_path) {
  __shared__ int64_t s_slot[kWriteChunk];
  __shared__ int s_start[kWriteChunk];  // row r starts a block this chunk fills
  __shared__ __align__(16) Elem v_tile[kTileLdsBytes / sizeof(Elem)];
  static_assert(CHUNK <= kWriteChunk && kWriteChunk == kThreads, "one slot per thread");
  const int64_t c0 = int64_t(blockIdx.x) * CHUNK;
  const int n = int(min<int64_t>(CHUNK, num_tokens - c0));
  const int t = threadIdx.x;
  const int64_t limit = int64_t(num_blocks) * block_size;
  {
    int64_t sl = -1;
    if (t < n) {
      sl = slots[c0 + t];
      if (sl < 0 || sl >= limit) sl = -1;  // skipped
    }
    s_slot[t] = sl;
  }
  __syncthreads();
  const int B = block_size;
  {
    bool start = false;
    if (tile_path && t < n && t + B <= n && s_slot[t] >= 0 && s_slot[t] % B == 0) {
      start = true;
      for (int j = 1; j < B && start; ++j) start = s_slot[t + j] == s_slot[t] + j;
    }
    s_start[t] = start;
  }
  __syncthreads();

  const int row_elems = num_kv_heads * head_dim;
  constexpr int kVec = 16 / sizeof(Elem);
  // Whole blocks: the (block, KV head) tiles of this workgroup (blocks that
  // start at a listed row, heads y, y + gridDim.y, ...) go in rounds of as
  // many tiles as the LDS area holds, so that a round's loads and stores are
  // all in flight together: K rows straight to the tile, V rows into LDS as
  // [token][dim], then out as [dim][token].
  __shared__ int s_list[kWriteChunk];
  __shared__ int s_count;
  if (t == 0) s_count = 0;
  __syncthreads();
  if (s_start[t]) s_list[atomicAdd(&s_count, 1)] = t;
  __syncthreads();
  const int nstart = s_count;
  const int dvecs = head_dim / kVec;
  const int jvecs = B / kVec;
  const int heads_here = (num_kv_heads - int(blockIdx.y) + int(gridDim.y) - 1) / int(gridDim.y);
  const int units = nstart * heads_here;
  const int tile_elems = B * head_dim;
  const int per_round = max(1, int(kTileLdsBytes / (int64_t(tile_elems) * sizeof(Elem))));
  for (int u0 = 0; u0 < units; u0 += per_round) {
    const int nb = min(per_round, units - u0);
#pragma unroll 4
    for (int v = t; v < nb * B * dvecs; v += kThreads) {
      const int ui = v / (B * dvecs);
      const int w = v % (B * dvecs);
      const int j = w / dvecs;
      const int dv = w % dvecs;
      const int unit = u0 + ui;
      const int r = s_list[unit / heads_here];
      const int h = int(blockIdx.y) + (unit % heads_here) * int(gridDim.y);
      const int64_t tile = (s_slot[r] / B * num_kv_heads + h) * int64_t(tile_elems);
      const int64_t src = (c0 + r + j) * row_elems + int64_t(h) * head_dim;
      reinterpret_cast<uint4*>(k_cache + tile + int64_t(j) * head_dim)[dv] =
          reinterpret_cast<const uint4*>(key + src)[dv];
      reinterpret_cast<uint4*>(v_tile + (ui * B + j) * head_dim)[dv] =
          reinterpret_cast<const uint4*>(value + src)[dv];
    }
    __syncthreads();
    for (int v = t; v < nb * head_dim * jvecs; v += kThreads) {
      const int ui = v / (head_dim * jvecs);
      const int w = v % (head_dim * jvecs);
      const int d = w / jvecs;
      const int j0 = (w % jvecs) * kVec;
      const int unit = u0 + ui;
      const int r = s_list[unit / heads_here];
      const int h = int(blockIdx.y) + (unit % heads_here) * int(gridDim.y);
      const int64_t tile = (s_slot[r] / B * num_kv_heads + h) * int64_t(tile_elems);
      Elem e[kVec];
#pragma unroll
      for (int u = 0; u < kVec; ++u) e[u] = v_tile[(ui * B + j0 + u) * head_dim + d];
      uint4 q;
      __builtin_memcpy(&q, e, 16);
      *reinterpret_cast<uint4*>(v_cache + tile + int64_t(d) * B + j0) = q;
    }
    __syncthreads();
  }

  // the other rows, one wave per row
  const int wave = t / 64;
  const int lane = t % 64;
  for (int i = wave; i < n; i += kThreads / 64) {
    const int64_t sl = s_slot[i];
    if (sl < 0) continue;
    bool in_tile = false;  // covered by a block written above
    if (tile_path) {
      const int first = i - int(sl % B);
      in_tile = first >= 0 && s_start[first];
    }
    if (in_tile) continue;
    const int64_t row = (c0 + i) * row_elems;
    for (int h = blockIdx.y; h < num_kv_heads; h += gridDim.y)
      store_head_wave(k_cache, v_cache, key + row, value + row, sl / B, int(sl % B), h,
                      num_kv_heads, head_dim, B, lane);
  }
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
  // whole-block tiles when a V row of B tokens is whole 16-byte vectors, the
  // V pool and rows are 16-byte aligned (the ABI asks only element
  // alignment of them), and one head's V tile fits the LDS buffer
  const bool v_aligned = (reinterpret_cast<uintptr_t>(v_cache) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(value) % 16 == 0);
  const int tile_path = v_aligned && (int64_t(block_size) * elem_bytes % 16 == 0) &&
                        int64_t(block_size) * head_dim * elem_bytes <= kTileLdsBytes &&
                        block_size <= kSmallWriteChunk;
  // Few chunks (a prefill chunk, a decode step): split each chunk's heads
  // over workgroups so the write has enough of them; 8192 rows of 8 heads
  // took 240 us as 32 workgroups and 71 us as 256, then 47.5 us once
  // each workgroup moved its tiles in rounds, 25.9 us in 64-row chunks.
  // Many chunks (a whole history) fill the device already, and one pass
  // over all heads of a chunk measured faster there.
  const bool many = ceil_div(num_tokens, kWriteChunk) >= kSplitHeadsBelowChunks;
  const int chunk = many ? kWriteChunk : kSmallWriteChunk;
  const int chunks = ceil_div(num_tokens, chunk);
  const int split = many ? 1 : (num_kv_heads < 65535 ? num_kv_heads : 65535);
  const dim3 grid{unsigned(chunks), unsigned(split)};
  if (elem_bytes == 4) {
    auto k = many ? write_kv_kernel<uint32_t, kWriteChunk> : write_kv_kernel<uint32_t, kSmallWriteChunk>;
    return launch(k, grid, dim3(kThreads), 0, stream,
                  static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                  static_cast<const uint32_t*>(key), static_cast<const uint32_t*>(value), slots,
                  num_tokens, num_kv_heads, head_dim, block_size, num_blocks, tile_path);
  }
  auto k = many ? write_kv_kernel<uint16_t, kWriteChunk> : write_kv_kernel<uint16_t, kSmallWriteChunk>;
  return launch(k, grid, dim3(kThreads), 0, stream,
                static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value), slots,
                num_tokens, num_kv_heads, head_dim, block_size, num_blocks, tile_path);
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

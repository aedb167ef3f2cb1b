// Internal declarations shared by the HIP sources of libpa (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace pa {

// Arguments of one decode launch (partials or single pass) and of the merge.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* new_k;          // append: K row [S][Hkv][D] of each sequence's token L - 1, or null
  const void* new_v;          // append: V row, same shape
  float* lse;                 // [S][Hq] log-sum-exp of each (sequence, head), or null
  float* ws;                  // split-KV records (see schedule.h), nullptr in single pass
  void* ws_meta;              // split-KV meta block: prefT, prefP, N
  int32_t workers;            // split-KV worker grid
  uint32_t epoch;             // split-KV launch stamp (marks this launch's records)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;              // num_heads / num_kv_heads
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;    // clamp for context_lens
  int32_t partition_size;     // tokens per partition (multiple of 16 and of B)
  int32_t max_partitions;     // ceil(max_context_len / partition_size), >= 1
  int32_t split;              // 1: balanced split-KV workers; 0: one wave per (seq, KV head)
  int32_t shared_blocks;      // 1: blocks may be read by several sequences (default-cached loads)
  float scale_log2e;          // scale * log2(e)
  // Shared-prefix groups (split launches only; num_groups == 0 otherwise).
  // Group i is sequences group_start[i] .. group_start[i+1] - 1, whose first
  // prefix_lens[i] tokens sit in the same physical blocks.  The line then
  // starts with one prefix unit per group (its shared tokens, read once per
  // KV head for all members' query heads), followed by each sequence's
  // remaining tokens (schedule.h).
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int32_t num_groups;
  int32_t prefix_members;     // members of a group a prefix unit serves (its columns / group)
  float* ws_wide;             // records of prefix pieces: prefix_members records each
  // Line positions a pair of a grouped line takes beyond its tiles (its run
  // start: table window, queries, first loads), and per tile of a prefix
  // unit (whose tiles also feed all members' columns): the balanced cut then
  // gives every worker about the same time, not the same tile count.
  int32_t tail_lead;
  int32_t tail_wt;
  int32_t prefix_lead;
  int32_t prefix_wt;
};

// Arguments of one prefill launch.
struct PrefillArgs {
  void* out;
  float* lse;                  // [num_query_tokens][num_heads] log-sum-exp per row, or null
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [num_seqs + 1] first query row of each sequence
  int32_t num_seqs;
  int32_t num_query_tokens;    // rows of q and out
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;               // num_heads / num_kv_heads
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;     // clamp for context_lens
  int32_t max_query_len;       // clamp for query rows per sequence
  int32_t row_groups;          // bf16: ceil(max_query_len * group / rows of one workgroup)
  float scale;
  float scale_log2e;
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Floats in one split-KV record: o[G][D], m[G], l[G], the launch epoch
// (uint32 bits), padded so every record starts on a 16-byte boundary.
__host__ __device__ inline int64_t record_floats(int group, int head_dim) {
  return int64_t(group) * head_dim + (2 * group + 1 + 3) / 4 * 4;
}

// Launch `kernel` and return hipLaunchKernel's own status (never a stale
// error left by an earlier call).  Arguments are converted to the kernel's
// parameter types first.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                  hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
  std::tuple<KArgs...> values(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, values);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
}

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_slot_mapping(int64_t* slots, const int32_t* block_tables, const int32_t* seq_ids,
                               const int32_t* positions, int num_tokens, int num_seqs,
                               int max_blocks_per_seq, int block_size, hipStream_t stream);
hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* key, const void* value,
                           const int64_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int elem_bytes, hipStream_t stream);
// Write key/value row s at position context_lens[s] - 1 (clamped as in the
// decode) of sequence s, through its block table.
hipError_t launch_append_kv(const DecodeArgs& a, int head_dim, int block_size, int elem_bytes,
                            hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              int elem_bytes, hipStream_t stream);

// Decode partials / single pass.  Returns hipErrorInvalidValue for a shape
// with no compiled kernel (the API checks shapes first).
hipError_t launch_decode_bf16_mfma(const DecodeArgs& a, int head_dim, int block_size,
                                   hipStream_t stream);
// Number of split-KV workers a decode kernel should use on the current
// device: compute units x min(resident workgroups per compute unit, 3),
// capped at the workspace's worker bound.  0 on failure.  Cached per kernel
// and device.
int resident_workers(const void* kernel, int block_threads);
// groups: the grouped (shared-prefix) kernel, at most kMaxGroupWorkers.
int decode_workers_bf16_mfma(int head_dim, int block_size, bool groups = false);
int decode_workers_simt(int head_dim, bool bf16);
hipError_t launch_decode_simt(const DecodeArgs& a, int head_dim, int block_size, bool bf16,
                              hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, bool bf16,
                          hipStream_t stream);
hipError_t launch_cp_slot_mapping(int64_t* slots, const int32_t* block_tables,
                                  const int32_t* seq_ids, const int32_t* positions,
                                  int num_tokens, int num_seqs, int max_blocks_per_seq,
                                  int block_size, int world, int rank, int interleave,
                                  hipStream_t stream);
hipError_t launch_cp_context_lens(int32_t* local_lens, const int32_t* context_lens, int num_seqs,
                                  int block_size, int world, int rank, int interleave,
                                  hipStream_t stream);
hipError_t launch_merge_states(void* out, float* out_lse, const void* states, const float* lses,
                               int num_states, int64_t num_rows, int head_dim, bool bf16,
                               hipStream_t stream);
hipError_t launch_map_to_kernel_blocks(int32_t* kernel_tables, const int32_t* manager_tables,
                                       int num_rows, int max_blocks, int k, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, int block_size, bool bf16,
                               hipStream_t stream);

}  // namespace pa

// Context parallelism and allocator/kernel block tables.
//
// "PagedAttention学习笔记", BlockTable walkthrough: under decode / prefill
// context parallelism the slot mapping works with a virtual block size and
// a mask, writing -1 for the entries a rank does not own; when the block
// size of the allocator differs from the one the kernel needs, each
// allocator block is split into several kernel blocks.
//
// Ownership (the pages give no formula; this is the reading the library
// takes): W ranks share one block table and each holds its own pool.  Token
// p lies in virtual block p / (B W), table entry table[p / (B W)] on every
// rank; inside the virtual block, runs of I tokens (the interleave, a
// divisor of B) go to ranks 0, 1, ..., W-1 in turn, and a rank packs the
// runs it owns into its B slots of that block in order.  A rank's tokens thus
// form an ordinary paged sequence in its own pool, of the length
// pa_cp_context_lens gives, which any decode or prefill call attends over;
// the ranks' partial results, each with its log-sum-exp, are combined by
// pa_merge_states with the log-sum-exp identity.

#include <math.h>

#include "device_common.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void cp_slot_mapping_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, int num_tokens,
    int num_seqs, int max_blocks_per_seq, int block_size, int world, int rank, int interleave) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_tokens) return;
  const int s = seq_ids[i];
  const int pos = positions[i];
  int64_t slot = -1;
  if (s >= 0 && s < num_seqs && pos >= 0) {
    const int64_t vbs = int64_t(block_size) * world;  // virtual block size
    const int64_t vb = pos / vbs;
    const int vo = int(pos % vbs);
    const int owner = (vo / interleave) % world;
    if (vb < max_blocks_per_seq && owner == rank) {
      const int32_t block = block_tables[int64_t(s) * max_blocks_per_seq + vb];
      const int local = vo / (interleave * world) * interleave + vo % interleave;
      if (block >= 0) slot = int64_t(block) * block_size + local;
    }
  }
  slots[i] = slot;
}

// Tokens of a length-L sequence that rank r holds: B per full virtual block,
// then the runs of the last, partial virtual block that fall to r.
__global__ __launch_bounds__(kThreads) void cp_context_lens_kernel(
    int32_t* __restrict__ local_lens, const int32_t* __restrict__ context_lens, int num_seqs,
    int block_size, int world, int rank, int interleave) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= num_seqs) return;
  const int L = max(context_lens[s], 0);
  const int vbs = block_size * world;
  const int full = L / vbs, rem = L % vbs;
  const int runs = rem / interleave, part = rem % interleave;
  int n = full * block_size + interleave * ((runs + world - 1 - rank) / world);
  if (runs % world == rank) n += part;
  local_lens[s] = n;
}

template <typename Elem>
struct Vec4;
template <>
struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  static __device__ __forceinline__ void store(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
  }
};
template <>
struct Vec4<uint16_t> {
  static __device__ __forceinline__ float4 load(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
  }
  static __device__ __forceinline__ void store(uint16_t* p, float4 v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
};

// out[r] = sum_w e^(lse_w[r] - M) o_w[r] / sum_w e^(lse_w[r] - M), M the
// largest lse of row r; a row whose every lse is -inf gets zeros and -inf.
// One thread per four dims of a row.
template <typename Elem>
__global__ __launch_bounds__(kThreads) void merge_states_kernel(
    Elem* __restrict__ out, float* __restrict__ out_lse, const Elem* __restrict__ states,
    const float* __restrict__ lses, int num_states, int64_t num_rows, int head_dim) {
  const int q = head_dim / 4;
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= num_rows * q) return;
  const int64_t row = idx / q;
  const int c = int(idx % q);
  float M = -INFINITY;
  bool nan = false;
  for (int w = 0; w < num_states; ++w) {
    const float l = lses[int64_t(w) * num_rows + row];
    nan |= l != l;
    M = fmaxf(M, l);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (M > -INFINITY) {
    for (int w = 0; w < num_states; ++w) {
      const float l = lses[int64_t(w) * num_rows + row];
      if (l == -INFINITY) continue;
      const float e = expf(l - M);
      const float4 o = Vec4<Elem>::load(states + (int64_t(w) * num_rows + row) * head_dim + 4 * c);
      acc.x += e * o.x;
      acc.y += e * o.y;
      acc.z += e * o.z;
      acc.w += e * o.w;
      den += e;
    }
  }
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = -INFINITY;
  if (den > 0.f) {
    const float inv = 1.0f / den;
    r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    lse = M + logf(den);
  }
  if (nan) {
    const float qn = __builtin_nanf("");
    r = make_float4(qn, qn, qn, qn);
    lse = qn;
  }
  Vec4<Elem>::store(out + row * head_dim + 4 * c, r);
  if (out_lse && c == 0) out_lse[row] = lse;
}

__global__ __launch_bounds__(kThreads) void map_to_kernel_blocks_kernel(
    int32_t* __restrict__ kernel_tables, const int32_t* __restrict__ manager_tables,
    int64_t num_entries, int max_blocks, int k) {
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= num_entries) return;
  const int64_t row = idx / (int64_t(max_blocks) * k);
  const int e = int(idx % (int64_t(max_blocks) * k));
  const int32_t m = manager_tables[row * max_blocks + e / k];
  const int64_t b = int64_t(m) * k + e % k;
  kernel_tables[idx] = (m < 0 || b > 0x7FFFFFFF) ? -1 : int32_t(b);
}

}  // namespace

hipError_t launch_cp_slot_mapping(int64_t* slots, const int32_t* block_tables,
                                  const int32_t* seq_ids, const int32_t* positions,
                                  int num_tokens, int num_seqs, int max_blocks_per_seq,
                                  int block_size, int world, int rank, int interleave,
                                  hipStream_t stream) {
  return launch(cp_slot_mapping_kernel, dim3(ceil_div(num_tokens, kThreads)), dim3(kThreads), 0,
                stream, slots, block_tables, seq_ids, positions, num_tokens, num_seqs,
                max_blocks_per_seq, block_size, world, rank, interleave);
}

hipError_t launch_cp_context_lens(int32_t* local_lens, const int32_t* context_lens, int num_seqs,
                                  int block_size, int world, int rank, int interleave,
                                  hipStream_t stream) {
  return launch(cp_context_lens_kernel, dim3(ceil_div(num_seqs, kThreads)), dim3(kThreads), 0,
                stream, local_lens, context_lens, num_seqs, block_size, world, rank, interleave);
}

hipError_t launch_merge_states(void* out, float* out_lse, const void* states, const float* lses,
                               int num_states, int64_t num_rows, int head_dim, bool bf16,
                               hipStream_t stream) {
  const int64_t threads = num_rows * (head_dim / 4);
  const dim3 grid(unsigned((threads + kThreads - 1) / kThreads));
  if (bf16)
    return launch(merge_states_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                  static_cast<uint16_t*>(out), out_lse, static_cast<const uint16_t*>(states), lses,
                  num_states, num_rows, head_dim);
  return launch(merge_states_kernel<float>, grid, dim3(kThreads), 0, stream,
                static_cast<float*>(out), out_lse, static_cast<const float*>(states), lses,
                num_states, num_rows, head_dim);
}

hipError_t launch_map_to_kernel_blocks(int32_t* kernel_tables, const int32_t* manager_tables,
                                       int num_rows, int max_blocks, int k, hipStream_t stream) {
  const int64_t n = int64_t(num_rows) * max_blocks * k;
  return launch(map_to_kernel_blocks_kernel, dim3(unsigned((n + kThreads - 1) / kThreads)),
                dim3(kThreads), 0, stream, kernel_tables, manager_tables, n, max_blocks, k);
}

}  // namespace pa

// C ABI of libpa: host-side argument checks, launch geometry, dispatch.
// Every check runs before anything is enqueued; see include/pa.h for the
// contract of each entry point.

#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <tuple>
#include <vector>

#include "internal.h"
#include "pa.h"
#include "schedule.h"

namespace pa {

constexpr int kWorkersPerCu = 3;

int resident_workers(const void* kernel, int block_threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::vector<std::tuple<const void*, int, int>> cache;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : cache)
      if (std::get<0>(e) == kernel && std::get<1>(e) == dev) return std::get<2>(e);
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess)
    return 0;
  // Three single-wave workers per compute unit: enough loads in flight to
  // keep HBM busy, and the fewer the workers, the fewer the piece starts
  // (each costs dependent memory round trips) per byte streamed.
  const int workers = std::min(kMaxWorkers, std::max(1, cus * std::min(per_cu, kWorkersPerCu)));
  std::lock_guard<std::mutex> lock(mu);
  cache.emplace_back(kernel, dev, workers);
  return workers;
}

}  // namespace pa

namespace {

using pa::DecodeArgs;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes_of(int32_t dtype) {
  switch (dtype) {
    case PA_DTYPE_F32: return 4;
    case PA_DTYPE_BF16: return 2;
    default: return 0;
  }
}

int status_of(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

bool supported_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }
bool supported_block_size(int32_t b) { return b == 8 || b == 16 || b == 32; }

// Shape checks common to pa_write_kv / pa_copy_blocks.
int check_cache_shape(int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, int32_t dtype) {
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if ((int64_t(head_dim) * eb) % 16 != 0) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

struct DecodePlan {
  DecodeArgs args;
  int head_dim;
  int block_size;
  bool bf16;
  bool split;  // records + merge needed
};

int64_t effective_max_len(int32_t max_context_len, int32_t max_blocks_per_seq, int32_t block_size) {
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  return max_context_len < cap ? max_context_len : cap;
}

// Sizes the split schedule handles: S * ceil(L_max / 16) tiles per KV head
// within 31 bits, and a line of fewer than 2^40 tiles in all.
bool split_line_fits(int32_t num_seqs, int32_t num_kv_heads, int64_t max_len) {
  const int64_t tiles = int64_t(num_seqs) * ((max_len + 15) / 16);
  return tiles <= 0x7FFFFFFF && tiles * num_kv_heads < (int64_t(1) << 40);
}

int64_t max_parts_for(int64_t max_len, int32_t partition_size) {
  const int64_t parts = (max_len + partition_size - 1) / partition_size;
  return parts > 1 ? parts : 1;
}

int64_t workspace_bytes_for(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t head_dim,
                            int64_t max_parts) {
  return pa::meta_bytes(num_seqs) + pa::max_records(num_seqs, num_kv_heads, max_parts) *
                                        pa::record_floats(group, head_dim) * int64_t(sizeof(float));
}

// Stamp of a split-KV launch: records written by the launch carry it, so the
// merge can tell them from records left in the workspace by earlier launches.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0x1234567u};
  uint32_t e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return e == 0 ? 1u : e;
}

int decode_workers(bool bf16, int head_dim, int block_size, bool groups = false) {
  return bf16 ? pa::decode_workers_bf16_mfma(head_dim, block_size, groups)
              : pa::decode_workers_simt(head_dim, false);
}

// Line weights of a grouped launch (schedule.h), in quarter tiles of
// streaming time, fitted to per-worker timelines of the shared-prefix batch
// on MI355X: a tail tile 4; a prefix tile (which also feeds 64 query
// columns) 6; a tail run's start (table window, queries, then the first
// tile: two dependent memory round trips) 23; a prefix run's start and end
// (queries of 64 columns, and one record per member stored) 52.
constexpr int kTailWt = 4;
constexpr int kTailLead = 23;
constexpr int kPrefixWt = 6;
constexpr int kPrefixLead = 52;

// Line weights of a plain split launch, in the same quarter tiles: a tile
// 4, a run's start 12.  At B = 32 a run's start and end cost about 1.2 us
// more (per-worker timelines of the mixed-length batch: its first tile may be
// a block's second half, whose V the run loads on its own, and a run that
// ends on a block's first tile also fetches the second's V), and the fitted
// start is 20: the balanced cut at 12 left the workers with many short runs
// finishing last.
constexpr int kPlainWt = 4;
constexpr int kPlainLead = 12;
constexpr int kPlainLeadB32 = 20;

void set_line_weights(DecodeArgs& a, bool groups, int block_size) {
  a.tail_lead = groups ? kTailLead : (block_size >= 32 ? kPlainLeadB32 : kPlainLead);
  a.tail_wt = groups ? kTailWt : kPlainWt;
  a.prefix_lead = kPrefixLead;
  a.prefix_wt = kPrefixWt;
}

// Longest context the split-schedule size check should assume: a pair's
// positions are its tiles times the heaviest weight plus a lead.
int64_t weighted_len(int64_t max_len, bool groups) {
  if (!groups) return max_len * kPlainWt + 16 * int64_t(kPlainLeadB32);
  const int wt = kPrefixWt > kTailWt ? kPrefixWt : kTailWt;
  const int lead = kTailLead > kPrefixLead ? kTailLead : kPrefixLead;
  return max_len * wt + 16 * int64_t(lead);
}

// Query columns of a prefix unit (bf16 kernel): 64 at head_dim <= 128, 32
// at 256; the members a unit serves are those columns / group size.
int prefix_members_for(int32_t head_dim, int32_t group) {
  return (head_dim <= 128 ? 64 : 32) / group;
}

// Workspace of a grouped (shared-prefix) launch: the meta block over
// num_groups + S units, the tail records (as a plain launch's), then the
// wide records of the prefix pieces.
int64_t group_workspace_bytes_for(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                                  int32_t head_dim, int64_t max_parts, int32_t num_groups) {
  const int64_t rec = pa::record_floats(group, head_dim) * int64_t(sizeof(float));
  return pa::meta_bytes_units(num_seqs + num_groups) +
         pa::max_records(num_seqs, num_kv_heads, max_parts) * rec +
         pa::max_wide_records(num_groups, num_kv_heads) * prefix_members_for(head_dim, group) * rec;
}

// Validate the decode arguments and fill the launch plan.  Returns PA_OK with
// plan->args.num_seqs == 0 when there is nothing to do.
int plan_decode(DecodePlan* plan, void* out, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                size_t workspace_bytes, int32_t dtype, int32_t flags,
                const int32_t* group_start = nullptr, const int32_t* prefix_lens = nullptr,
                int32_t num_groups = 0) {
  if (num_groups < 0) return PA_ERR_INVALID_ARG;
  if (num_groups > pa::kMaxGroups) return PA_ERR_UNSUPPORTED;
  if (num_groups > 0 && partition_size <= 0) return PA_ERR_INVALID_ARG;  // grouped: split only
  if (num_groups > 0 && num_seqs > 0 && (!group_start || !prefix_lens)) return PA_ERR_INVALID_ARG;
  if (int64_t(num_seqs) + num_groups > 0x3FFFFFFF) return PA_ERR_UNSUPPORTED;
  if ((flags & ~int32_t(PA_DECODE_SHARED_BLOCKS)) != 0) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || partition_size < 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (elem_bytes_of(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  const int32_t group = num_heads / num_kv_heads;
  if (group > 16) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  plan->args = DecodeArgs{};
  plan->args.num_seqs = 0;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARG;
  if (int64_t(num_seqs) * num_heads > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;

  const int64_t max_len = effective_max_len(max_context_len, max_blocks_per_seq, block_size);
  // the split schedule sums 16-token tiles over sequences (and prefix units)
  // in 32-bit integers and divides line positions (tiles x KV heads) times
  // workers in doubles
  if (partition_size > 0 &&
      !split_line_fits(num_seqs + num_groups, num_kv_heads, weighted_len(max_len, num_groups > 0)))
    return PA_ERR_UNSUPPORTED;
  DecodeArgs& a = plan->args;
  plan->split = partition_size > 0;
  if (plan->split) {
    const int64_t parts = max_parts_for(max_len, partition_size);
    // the fp32 kernel has no prefix units: it decodes every token of every
    // sequence (the same result), in a plain layout that fits the grouped one
    const bool groups = num_groups > 0 && dtype == PA_DTYPE_BF16;
    const int64_t need =
        num_groups > 0
            ? group_workspace_bytes_for(num_seqs, num_kv_heads, group, head_dim, parts, num_groups)
            : workspace_bytes_for(num_seqs, num_kv_heads, group, head_dim, parts);
    if (!workspace || int64_t(workspace_bytes) < need || !aligned16(workspace))
      return PA_ERR_WORKSPACE;
    const int workers = decode_workers(dtype == PA_DTYPE_BF16, head_dim, block_size, groups);
    if (workers <= 0) return PA_ERR_HIP;
    a.ws_meta = workspace;
    a.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    (groups ? pa::meta_bytes_units(num_seqs + num_groups)
                                            : pa::meta_bytes(num_seqs)));
    if (groups) {
      a.ws_wide = a.ws + pa::max_records(num_seqs, num_kv_heads, parts) *
                             pa::record_floats(group, head_dim);
      a.group_start = group_start;
      a.prefix_lens = prefix_lens;
      a.num_groups = num_groups;
      a.prefix_members = prefix_members_for(head_dim, group);
    }
    set_line_weights(a, groups, block_size);
    a.workers = workers;
    a.partition_size = partition_size;
    a.max_partitions = int32_t(parts);
    a.split = 1;
    a.epoch = next_epoch();
  } else {
    if (int64_t(num_seqs) * num_kv_heads > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    a.partition_size = int32_t(std::max<int64_t>(16, (max_len + 15) / 16 * 16));
    a.max_partitions = 1;
    a.split = 0;
  }
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = int32_t(max_len);
  a.scale_log2e = scale * 1.4426950408889634f;
  a.shared_blocks = (flags & PA_DECODE_SHARED_BLOCKS) ? 1 : 0;
  plan->head_dim = head_dim;
  plan->block_size = block_size;
  plan->bf16 = dtype == PA_DTYPE_BF16;
  return PA_OK;
}

// The decode launch of a plan.  With an appended row (plan.args.new_k set)
// the matrix-core kernel writes and uses the row itself; the fp32 kernel
// runs after a separate append launch.
hipError_t launch_partials(const DecodePlan& plan, hipStream_t stream) {
  if (plan.bf16) return pa::launch_decode_bf16_mfma(plan.args, plan.head_dim, plan.block_size, stream);
  DecodeArgs a = plan.args;
  if (a.new_k) {
    const hipError_t e = pa::launch_append_kv(a, plan.head_dim, plan.block_size, 4, stream);
    if (e != hipSuccess) return e;
    a.new_k = a.new_v = nullptr;
  }
  return pa::launch_decode_simt(a, plan.head_dim, plan.block_size, false, stream);
}

// Checks of the appended rows (after plan_decode accepted the rest).
int check_append(const void* key, const void* value, int32_t num_seqs) {
  if (num_seqs == 0) return PA_OK;
  if (!key || !value) return PA_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// The merge launch of a split decode (plain, or grouped with num_groups > 0),
// rebuilt from its sizes: the same schedule and workspace layout as the
// partials launch.
int merge_call(void* out, const int32_t* context_lens, const int32_t* group_start,
               const int32_t* prefix_lens, int32_t num_groups, int32_t num_seqs,
               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t max_blocks_per_seq, int32_t block_size, int32_t max_context_len,
               int32_t partition_size, const void* workspace, size_t workspace_bytes,
               int32_t dtype, void* stream) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 0 ||
      max_context_len < 0 || partition_size < 0 || num_heads % num_kv_heads != 0 ||
      num_groups < 0)
    return PA_ERR_INVALID_ARG;
  if (elem_bytes_of(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
    return PA_ERR_INVALID_ARG;
  if (num_groups > 0 && partition_size == 0) return PA_ERR_INVALID_ARG;
  if (num_groups > pa::kMaxGroups) return PA_ERR_UNSUPPORTED;
  if (int64_t(num_seqs) + num_groups > 0x3FFFFFFF) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || partition_size == 0) return PA_OK;
  if (!out || !context_lens) return PA_ERR_INVALID_ARG;
  if (num_groups > 0 && (!group_start || !prefix_lens)) return PA_ERR_INVALID_ARG;
  if (!aligned16(out)) return PA_ERR_INVALID_ARG;
  const int64_t max_len = effective_max_len(max_context_len, max_blocks_per_seq, block_size);
  const int64_t parts = max_parts_for(max_len, partition_size);
  const int32_t group = num_heads / num_kv_heads;
  const int64_t need =
      num_groups > 0
          ? group_workspace_bytes_for(num_seqs, num_kv_heads, group, head_dim, parts, num_groups)
          : workspace_bytes_for(num_seqs, num_kv_heads, group, head_dim, parts);
  if (!workspace || !aligned16(workspace) || int64_t(workspace_bytes) < need)
    return PA_ERR_WORKSPACE;
  if (int64_t(num_seqs) * num_heads > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
  if (!split_line_fits(num_seqs + num_groups, num_kv_heads, weighted_len(max_len, num_groups > 0)))
    return PA_ERR_UNSUPPORTED;
  const bool bf16 = dtype == PA_DTYPE_BF16;
  const bool groups = num_groups > 0 && bf16;
  const int workers = decode_workers(bf16, head_dim, block_size, groups);
  if (workers <= 0) return PA_ERR_HIP;
  DecodeArgs a{};
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a.out = out;
  a.context_lens = context_lens;
  a.ws_meta = ws;
  a.ws = reinterpret_cast<float*>(ws + (groups ? pa::meta_bytes_units(num_seqs + num_groups)
                                               : pa::meta_bytes(num_seqs)));
  if (groups) {
    a.ws_wide = a.ws + pa::max_records(num_seqs, num_kv_heads, parts) *
                           pa::record_floats(group, head_dim);
    a.group_start = group_start;
    a.prefix_lens = prefix_lens;
    a.num_groups = num_groups;
    a.prefix_members = prefix_members_for(head_dim, group);
  }
  set_line_weights(a, groups, block_size);
  a.workers = workers;
  a.split = 1;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = int32_t(max_len);
  a.partition_size = partition_size;
  a.max_partitions = int32_t(parts);
  return status_of(pa::launch_decode_merge(a, head_dim, block_size, bf16,
                                           static_cast<hipStream_t>(stream)));
}

// A grouped decode: partials (with the step's rows appended when key and
// value are given), then the merge unless partials_only.
int shared_prefix_call(void* out, const void* q, const void* key, const void* value,
                       void* k_cache, void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* group_start,
                       const int32_t* prefix_lens, int32_t num_groups, int32_t num_seqs,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_context_len, float scale, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, int32_t dtype, int32_t flags,
                       void* stream, bool partials_only) {
  if ((key == nullptr) != (value == nullptr)) return PA_ERR_INVALID_ARG;
  if (partition_size <= 0) return PA_ERR_INVALID_ARG;
  DecodePlan plan;
  int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                       workspace_bytes, dtype, flags, group_start, prefix_lens, num_groups);
  if (st != PA_OK) return st;
  if (key) {
    st = check_append(key, value, num_seqs);
    if (st != PA_OK) return st;
  }
  if (plan.args.num_seqs == 0) return PA_OK;
  plan.args.new_k = key;
  plan.args.new_v = value;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_partials(plan, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (!partials_only)
    e = pa::launch_decode_merge(plan.args, plan.head_dim, plan.block_size, plan.bf16, s);
  return status_of(e);
}

// ---------------------------------------------------------------------------
// Library-owned scratch for pa_decode_scratch: the split-KV workspace of
// callers that cannot allocate device memory.  One copy per device, held
// until the process ends; every pa_decode_scratch call on a device shares
// it, so calls that overlap on one device race.

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zeroes n16 16-byte words (a fill kernel rather than a memset node, so the
// first call may be recorded in a graph).
__global__ void scratch_zero_kernel(uint4* p, int64_t n16) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxScratchDevices = 64;

// The device address of the current device's copy of `scratch`, found once
// per device with that device current (the array's name is a host-side
// stand-in, not a device address).  The first call on a device also zeroes
// the copy on `stream`: the workspace contract wants zeros before the first
// launch (a stamp of 0 is never used).
hipError_t scratch_address(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    e = pa::launch(scratch_zero_kernel, dim3(1024), dim3(256), 0, stream,
                   static_cast<uint4*>(p), int64_t(kScratchBytes / 16));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP launch failed";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free KV blocks";
    case PA_ERR_STATE: return "PA_ERR_STATE: sequence is not in the required live/idle state";
    case PA_ERR_TOO_LARGE:
      return "PA_ERR_TOO_LARGE: the call needs more than the library's fixed scratch buffer";
    default: return "unknown status";
  }
}

int pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables, const int32_t* seq_ids,
                    const int32_t* positions, int32_t num_tokens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t block_size, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || block_size < 1)
    return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || !seq_ids || !positions) return PA_ERR_INVALID_ARG;
  if (!block_tables && int64_t(num_seqs) * max_blocks_per_seq > 0) return PA_ERR_INVALID_ARG;
  return status_of(pa::launch_slot_mapping(slot_mapping, block_tables, seq_ids, positions,
                                           num_tokens, num_seqs, max_blocks_per_seq, block_size,
                                           static_cast<hipStream_t>(stream)));
}

int pa_write_kv(void* k_cache, void* v_cache, const void* key, const void* value,
                const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                void* stream) {
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  const int st = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !key || !value || !slot_mapping) return PA_ERR_INVALID_ARG;
  const int eb = elem_bytes_of(dtype);
  if (!aligned16(k_cache) || !aligned16(key) ||
      (reinterpret_cast<uintptr_t>(v_cache) % eb) || (reinterpret_cast<uintptr_t>(value) % eb))
    return PA_ERR_INVALID_ARG;
  return status_of(pa::launch_write_kv(k_cache, v_cache, key, value, slot_mapping, num_tokens,
                                       num_kv_heads, head_dim, block_size, num_blocks, eb,
                                       static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t dtype, void* stream) {
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  const int st = check_cache_shape(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;
  if (int64_t(num_pairs) * 2 > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
  return status_of(pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, num_kv_heads,
                                          head_dim, block_size, num_blocks, elem_bytes_of(dtype),
                                          static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || partition_size <= 0 || num_heads % num_kv_heads != 0)
    return 0;
  const int64_t parts = max_parts_for(max_context_len, partition_size);
  return size_t(workspace_bytes_for(num_seqs, num_kv_heads, num_heads / num_kv_heads, head_dim, parts));
}

int pa_decode_partials(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_context_len, float scale, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, int32_t dtype, int32_t flags,
                       void* stream) {
  DecodePlan plan;
  const int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                             workspace_bytes, dtype, flags);
  if (st != PA_OK || plan.args.num_seqs == 0) return st;
  return status_of(launch_partials(plan, static_cast<hipStream_t>(stream)));
}

int pa_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int32_t block_size, int32_t max_context_len, int32_t partition_size,
                    const void* workspace, size_t workspace_bytes, int32_t dtype, void* stream) {
  return merge_call(out, context_lens, nullptr, nullptr, 0, num_seqs, num_heads, num_kv_heads,
                    head_dim, max_blocks_per_seq, block_size, max_context_len, partition_size,
                    workspace, workspace_bytes, dtype, stream);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
              int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
              int32_t flags, void* stream) {
  DecodePlan plan;
  const int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                             workspace_bytes, dtype, flags);
  if (st != PA_OK || plan.args.num_seqs == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_partials(plan, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (plan.split) e = pa::launch_decode_merge(plan.args, plan.head_dim, plan.block_size, plan.bf16, s);
  return status_of(e);
}

int pa_prefill(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, int32_t num_seqs, int32_t num_query_tokens,
               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
               int32_t max_query_len, float scale, int32_t dtype, void* stream) {
  if (num_seqs < 0 || num_query_tokens < 0 || num_heads < 1 || num_kv_heads < 1 ||
      num_blocks < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || max_query_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (elem_bytes_of(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARG;
  const int32_t group = num_heads / num_kv_heads;
  const bool bf16 = dtype == PA_DTYPE_BF16;
  pa::PrefillArgs a{};
  if (bf16) {
    // the launch's workgroups at the smallest row group (32 rows, D = 256),
    // the pairs rounded up to the 8 XCDs
    const int64_t row_groups = (int64_t(max_query_len) * group + 31) / 32;
    if ((int64_t(num_kv_heads) * num_seqs + 7) * row_groups > 0x7FFFFFF8) return PA_ERR_UNSUPPORTED;
  } else if (num_heads > 65535 || num_seqs > 65535) {
    return PA_ERR_UNSUPPORTED;
  }
  if (int64_t(num_query_tokens) * num_heads * head_dim > (int64_t(1) << 40)) return PA_ERR_UNSUPPORTED;
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_query_tokens = num_query_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = int32_t(effective_max_len(max_context_len, max_blocks_per_seq, block_size));
  a.max_query_len = max_query_len;
  a.scale = scale;
  a.scale_log2e = scale * 1.4426950408889634f;
  return status_of(pa::launch_prefill(a, head_dim, block_size, bf16, static_cast<hipStream_t>(stream)));
}

int pa_cp_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                       const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                       int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t cp_world, int32_t cp_rank, int32_t interleave, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || block_size < 1)
    return PA_ERR_INVALID_ARG;
  if (cp_world < 1 || cp_rank < 0 || cp_rank >= cp_world || interleave < 1 ||
      block_size % interleave != 0 || int64_t(block_size) * cp_world > 0x7FFFFFFF)
    return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || !seq_ids || !positions) return PA_ERR_INVALID_ARG;
  if (!block_tables && int64_t(num_seqs) * max_blocks_per_seq > 0) return PA_ERR_INVALID_ARG;
  return status_of(pa::launch_cp_slot_mapping(slot_mapping, block_tables, seq_ids, positions,
                                              num_tokens, num_seqs, max_blocks_per_seq, block_size,
                                              cp_world, cp_rank, interleave,
                                              static_cast<hipStream_t>(stream)));
}

int pa_cp_context_lens(int32_t* local_lens, const int32_t* context_lens, int32_t num_seqs,
                       int32_t block_size, int32_t cp_world, int32_t cp_rank, int32_t interleave,
                       void* stream) {
  if (num_seqs < 0 || block_size < 1 || cp_world < 1 || cp_rank < 0 || cp_rank >= cp_world ||
      interleave < 1 || block_size % interleave != 0 || int64_t(block_size) * cp_world > 0x7FFFFFFF)
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!local_lens || !context_lens) return PA_ERR_INVALID_ARG;
  return status_of(pa::launch_cp_context_lens(local_lens, context_lens, num_seqs, block_size,
                                              cp_world, cp_rank, interleave,
                                              static_cast<hipStream_t>(stream)));
}

int pa_merge_states(void* out, float* out_lse, const void* states, const float* state_lses,
                    int32_t num_states, int32_t num_rows, int32_t head_dim, int32_t dtype,
                    void* stream) {
  if (num_states < 1 || num_rows < 0 || head_dim < 4 || head_dim % 4 != 0)
    return PA_ERR_INVALID_ARG;
  if (elem_bytes_of(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (num_rows == 0) return PA_OK;
  if (!out || !states || !state_lses) return PA_ERR_INVALID_ARG;
  const uintptr_t align = dtype == PA_DTYPE_BF16 ? 8 : 16;
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(states)) % align != 0)
    return PA_ERR_INVALID_ARG;
  if (int64_t(num_rows) * (head_dim / 4) / 256 >= 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
  return status_of(pa::launch_merge_states(out, out_lse, states, state_lses, num_states, num_rows,
                                           head_dim, dtype == PA_DTYPE_BF16,
                                           static_cast<hipStream_t>(stream)));
}

int pa_map_to_kernel_blocks(int32_t* kernel_tables, const int32_t* manager_tables,
                            int32_t num_rows, int32_t max_blocks_per_row,
                            int32_t kernel_blocks_per_block, void* stream) {
  if (num_rows < 0 || max_blocks_per_row < 0 || kernel_blocks_per_block < 1)
    return PA_ERR_INVALID_ARG;
  const int64_t n = int64_t(num_rows) * max_blocks_per_row * kernel_blocks_per_block;
  if (n == 0) return PA_OK;
  if (!kernel_tables || !manager_tables) return PA_ERR_INVALID_ARG;
  if (int64_t(max_blocks_per_row) * kernel_blocks_per_block > 0x7FFFFFFF ||
      (n + 255) / 256 > 0x7FFFFFFF)
    return PA_ERR_UNSUPPORTED;
  return status_of(pa::launch_map_to_kernel_blocks(kernel_tables, manager_tables, num_rows,
                                                   max_blocks_per_row, kernel_blocks_per_block,
                                                   static_cast<hipStream_t>(stream)));
}

int pa_decode_lse(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                  float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                  int32_t dtype, int32_t flags, void* stream) {
  DecodePlan plan;
  const int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                             workspace_bytes, dtype, flags);
  if (st != PA_OK || plan.args.num_seqs == 0) return st;
  if (!lse) return PA_ERR_INVALID_ARG;
  plan.args.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_partials(plan, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (plan.split) e = pa::launch_decode_merge(plan.args, plan.head_dim, plan.block_size, plan.bf16, s);
  return status_of(e);
}

int pa_append_decode_partials(void* out, const void* q, const void* key, const void* value,
                              void* k_cache, void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, int32_t dtype,
                              int32_t flags, void* stream) {
  DecodePlan plan;
  int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                       workspace_bytes, dtype, flags);
  if (st != PA_OK) return st;
  st = check_append(key, value, num_seqs);
  if (st != PA_OK || plan.args.num_seqs == 0) return st;
  plan.args.new_k = key;
  plan.args.new_v = value;
  return status_of(launch_partials(plan, static_cast<hipStream_t>(stream)));
}

int pa_append_decode(void* out, const void* q, const void* key, const void* value, void* k_cache,
                     void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                     int32_t max_context_len, float scale, int32_t partition_size,
                     void* workspace, size_t workspace_bytes, int32_t dtype, int32_t flags,
                     void* stream) {
  DecodePlan plan;
  int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                       workspace_bytes, dtype, flags);
  if (st != PA_OK) return st;
  st = check_append(key, value, num_seqs);
  if (st != PA_OK || plan.args.num_seqs == 0) return st;
  plan.args.new_k = key;
  plan.args.new_v = value;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_partials(plan, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (plan.split) e = pa::launch_decode_merge(plan.args, plan.head_dim, plan.block_size, plan.bf16, s);
  return status_of(e);
}

int pa_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_context_len, float scale, int32_t partition_size,
                      int32_t dtype, int32_t flags, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (partition_size > 0 && num_seqs > 0 && num_heads > 0 && num_kv_heads > 0 &&
      head_dim > 0 && num_heads % num_kv_heads == 0 && max_context_len >= 0 &&
      max_blocks_per_seq >= 0 && block_size > 0) {
    // the size the split needs, before any launch (the other arguments are
    // checked by plan_decode below)
    const int64_t max_len = effective_max_len(max_context_len, max_blocks_per_seq, block_size);
    const int64_t need = workspace_bytes_for(num_seqs, num_kv_heads, num_heads / num_kv_heads,
                                             head_dim, max_parts_for(max_len, partition_size));
    if (need > int64_t(kScratchBytes)) return PA_ERR_TOO_LARGE;
    // checks that need no device first, so a bad call touches nothing
    DecodePlan probe;
    const int st = plan_decode(&probe, out, q, k_cache, v_cache, block_tables, context_lens,
                               num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, max_blocks_per_seq, max_context_len, scale,
                               partition_size, nullptr, 0, dtype, flags);
    if (st != PA_OK && st != PA_ERR_WORKSPACE) return st;
    if (scratch_address(s, &ws) != hipSuccess) return PA_ERR_HIP;
    ws_bytes = kScratchBytes;
  }
  DecodePlan plan;
  const int st = plan_decode(&plan, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len, scale, partition_size, ws,
                             ws_bytes, dtype, flags);
  if (st != PA_OK || plan.args.num_seqs == 0) return st;
  hipError_t e = launch_partials(plan, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (plan.split) e = pa::launch_decode_merge(plan.args, plan.head_dim, plan.block_size, plan.bf16, s);
  return status_of(e);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t partition_size,
                                               int32_t num_groups) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || partition_size <= 0 || num_groups < 0 ||
      num_groups > pa::kMaxGroups ||
      num_heads % num_kv_heads != 0 || num_heads / num_kv_heads > 16)
    return 0;
  const int64_t parts = max_parts_for(max_context_len, partition_size);
  return size_t(group_workspace_bytes_for(num_seqs, num_kv_heads, num_heads / num_kv_heads,
                                          head_dim, parts, num_groups));
}

int pa_decode_shared_prefix(void* out, const void* q, const void* key, const void* value,
                            void* k_cache, void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* group_start,
                            const int32_t* prefix_lens, int32_t num_groups, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, float scale, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, int32_t dtype,
                            int32_t flags, void* stream) {
  return shared_prefix_call(out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                            group_start, prefix_lens, num_groups, num_seqs, num_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                            max_context_len, scale, partition_size, workspace, workspace_bytes,
                            dtype, flags, stream, false);
}

int pa_decode_shared_prefix_partials(void* out, const void* q, const void* key, const void* value,
                                     void* k_cache, void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* group_start,
                                     const int32_t* prefix_lens, int32_t num_groups,
                                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, int32_t dtype, int32_t flags,
                                     void* stream) {
  return shared_prefix_call(out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                            group_start, prefix_lens, num_groups, num_seqs, num_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                            max_context_len, scale, partition_size, workspace, workspace_bytes,
                            dtype, flags, stream, true);
}

int pa_decode_shared_prefix_merge(void* out, const int32_t* context_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int32_t num_groups, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t block_size,
                                  int32_t max_context_len, int32_t partition_size,
                                  const void* workspace, size_t workspace_bytes, int32_t dtype,
                                  void* stream) {
  if (partition_size <= 0) return PA_ERR_INVALID_ARG;
  return merge_call(out, context_lens, group_start, prefix_lens, num_groups, num_seqs, num_heads,
                    num_kv_heads, head_dim, max_blocks_per_seq, block_size, max_context_len,
                    partition_size, workspace, workspace_bytes, dtype, stream);
}

}  // extern "C"

// Work schedule of the split-KV decode: a balanced cut of all KV tiles over
// a fixed number of single-wave workers.
//
// Every (sequence s, KV head g) owns T_s = ceil(L_s / 16) tiles of 16 tokens.
// The tiles of all pairs are laid on one line in (s, g, tile) order; pair
// (s, g) starts at Hkv * prefT[s] + g * T_s, prefT being the exclusive prefix
// sum of T_s.  Worker b of W owns the line slice [start(b), start(b+1)) with
// start(b) = floor(N * b / W), N the line length, so every worker streams the
// same number of tiles and all finish together.
//
// A worker cuts its slice into pieces at pair boundaries and at partition
// boundaries (every partition_size tokens of a pair).  Each piece yields one
// log-sum-exp record with line index  gp + b,  gp being the global index of
// the partition the piece lies in (partitions numbered along the line, pair
// (s, g) starting at Hkv * prefP[s] + g * nparts_s, prefP the exclusive
// prefix of nparts_s = ceil(L_s / partition_size)).  Along the line every
// cut raises gp or b (or both), so indices are distinct and below
// total_partitions + W, and a pair's records have consecutive indices
// k = 0, 1, ... from its first.  The first few of them are stored at slots
// indexed by the pair instead (PairSlots below).  A piece that is a whole
// pair writes the final output instead of a record.  The merge walks the
// same cuts per pair.
// (A worker may stream one pair's pieces back to back as a single run,
// writing each partition's record as it passes the partition's end.)
#pragma once

#include "device_common.h"

namespace pa {

// Largest worker grid the workspace is sized for.
constexpr int kMaxWorkers = 4096;

// A pair's records are numbered k = 0, 1, ... in line order (k = partition
// + worker - the worker of the pair's first tile).  The first kPairSlots of
// them have slots of their own, indexed by the pair, so the merge can load
// them without first finding where the pair's records start; the others sit
// in an overflow region at their line index (global partition + worker).
constexpr int kPairSlots = 4;

// Workspace layout (bytes): int32 prefT[S], int32 prefP[S], int64 N and
// uint32 epoch (at an 8-aligned offset), padding to 256, then the records:
// S * Hkv * kPairSlots pair slots, then the overflow region.
__host__ __device__ inline int64_t meta_bytes(int num_seqs) {
  const int64_t n_off = (int64_t(num_seqs) * 8 + 7) / 8 * 8;
  return (n_off + 16 + 255) / 256 * 256;
}
__host__ __device__ inline int64_t max_records(int num_seqs, int num_kv_heads, int64_t max_parts) {
  return int64_t(num_seqs) * num_kv_heads * (kPairSlots + max_parts) + kMaxWorkers;
}

// Where the records of one pair live.
struct PairSlots {
  int64_t fixed;     // slot of record 0 among the pair slots: pair index * kPairSlots
  int64_t overflow;  // overflow slot of record 0: S * Hkv * kPairSlots + line index of record 0
};
__device__ __forceinline__ int64_t record_slot(const PairSlots& p, int k) {
  return k < kPairSlots ? p.fixed + k : p.overflow + k;
}

// floor(p / q) for 0 <= p < 2^53 and 1 <= q < 2^53, through one double
// division instead of a 64-bit integer division (which the GPU runs as a
// long software sequence).  Exact: p and q are exact in double and the
// quotient is rounded once, with an error below (p / q) * 2^-53 < 1 / q;
// an integer quotient is exact, and any other lies at least 1 / q from the
// next integer, so the rounding never crosses one.  The line length N is
// kept below 2^40 by the host, so N * W < 2^52 here.
__device__ __forceinline__ int64_t floor_div_small(int64_t p, int64_t q) {
  return int64_t(floor(double(p) / double(q)));
}

__device__ __forceinline__ int64_t slice_start(int64_t n, int workers, int b) {
  return floor_div_small(n * b, workers);
}
// The worker whose slice holds line position x (0 <= x < n).
__device__ __forceinline__ int owner_of(int64_t n, int workers, int64_t x) {
  return int(floor_div_small((x + 1) * workers - 1, n));
}

// A pair's place on the line: `span` positions, `lead` of them for its run
// start, then `wt` per tile (tile t at lead + t * wt from the pair's start),
// so that the equal cut of positions gives workers equal time rather than
// equal tiles (a run's start costs dependent memory round trips).  The
// weights come from the launch (DecodeArgs::tail_lead, tail_wt).
struct PairShape {
  int tiles;   // T_s
  int parts;   // nparts_s
  int span;    // positions of one pair: tail_lead + tiles * tail_wt, or 0
};

__device__ __forceinline__ PairShape shape_of_len(const DecodeArgs& a, int L) {
  PairShape p;
  p.tiles = (L + 15) / 16;
  p.parts = (L + a.partition_size - 1) / a.partition_size;
  p.span = p.tiles > 0 ? a.tail_lead + p.tiles * a.tail_wt : 0;
  return p;
}

__device__ __forceinline__ PairShape pair_shape(const DecodeArgs& a, int s, int block_size) {
  return shape_of_len(a, effective_len(a, s, block_size));
}

// Inclusive wave-wide prefix sum of a 32-bit value.
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// One wave locates worker b's slice: N (the line length), [x0, x1), and the
// sequence holding x0 with its prefixes.  Worker 0 also publishes prefT,
// prefP and N in the workspace meta block for the merge.
struct Slice {
  int64_t n, x0, x1;
  int seq;          // sequence holding x0 (valid when x0 < x1)
  int len;          // its effective length
  int64_t pref_t;   // prefT[seq]
  int64_t pref_p;   // prefP[seq]
};

__device__ __forceinline__ int64_t* meta_n(const DecodeArgs& a) {
  return reinterpret_cast<int64_t*>(reinterpret_cast<char*>(a.ws_meta) +
                                    (int64_t(a.num_seqs) * 8 + 7) / 8 * 8);
}

__device__ __forceinline__ Slice locate_slice(const DecodeArgs& a, int block_size, int lane, int b) {
  const int S = a.num_seqs;
  const int per = (S + 63) / 64;  // consecutive sequences per lane
  const int first = min(S, lane * per);
  const int last = min(S, first + per);
  int lt = 0, lp = 0;
  for (int s = first; s < last; ++s) {
    const PairShape ps = pair_shape(a, s, block_size);
    lt += ps.span;
    lp += ps.parts;
  }
  const int it = wave_inclusive_scan(lt, lane);
  const int ip = wave_inclusive_scan(lp, lane);
  Slice r;
  r.n = int64_t(wave_uniform(__shfl(it, 63))) * a.num_kv_heads;
  r.x0 = r.n > 0 ? slice_start(r.n, a.workers, b) : 0;
  r.x1 = r.n > 0 ? slice_start(r.n, a.workers, b + 1) : 0;
  const bool publish = b == 0;
  int32_t* meta = reinterpret_cast<int32_t*>(a.ws_meta);
  int found_s = -1, found_len = 0;
  int64_t found_t = 0, found_p = 0;
  int64_t ct = it - lt, cp = ip - lp;
  for (int s = first; s < last; ++s) {
    const int len = effective_len(a, s, block_size);
    const PairShape ps = shape_of_len(a, len);
    if (publish) {
      meta[s] = int32_t(ct);
      meta[S + s] = int32_t(cp);
    }
    if (ps.span > 0 && r.x0 >= ct * a.num_kv_heads && r.x0 < (ct + ps.span) * a.num_kv_heads) {
      found_s = s;
      found_len = len;
      found_t = ct;
      found_p = cp;
    }
    ct += ps.span;
    cp += ps.parts;
  }
  if (publish && lane == 0) {
    *meta_n(a) = r.n;
    *reinterpret_cast<uint32_t*>(meta_n(a) + 1) = a.epoch;
  }
  const unsigned long long owner = __ballot(found_s >= 0);
  const int src = owner ? int(__builtin_ctzll(owner)) : 0;
  r.seq = wave_uniform(__shfl(found_s, src));
  r.len = wave_uniform(__shfl(found_len, src));
  r.pref_t = wave_uniform64(__shfl(found_t, src));
  r.pref_p = wave_uniform64(__shfl(found_p, src));
  return r;
}

// Calls run(s, g, L, first_tile, num_tiles, whole, slots, k0) for every run
// of consecutive tiles of one pair in worker b's slice, in line order.  A
// run ends only at a pair boundary or at the slice's end; it may span
// several partitions, and the tiles of the pair's partition p (p = tile *
// 16 / partition_size) make the pair's record k0 + p, stored at
// record_slot(slots, k0 + p).  whole: the run is the entire pair and the
// pair has one partition, so the output is written directly and no record
// is made.
template <typename RunFn>
__device__ __forceinline__ void walk_slice_runs(const DecodeArgs& a, int block_size, int lane,
                                                int b, RunFn&& run) {
  const Slice sl = locate_slice(a, block_size, lane, b);
  if (sl.x0 >= sl.x1) return;
  const int Hkv = a.num_kv_heads;
  int s = sl.seq;
  int64_t sbase = sl.pref_t * Hkv;        // line start of sequence s
  int64_t gpb = sl.pref_p * Hkv;          // first partition index of sequence s
  // the current sequence's length comes from the scan; the next one's is
  // fetched a sequence ahead
  int len = sl.len;
  int len_next = s + 1 < a.num_seqs ? effective_len(a, s + 1, block_size) : 0;
  PairShape ps = shape_of_len(a, len);
  const int lead = a.tail_lead, wt = a.tail_wt;
  int64_t cur = sl.x0;
  while (cur < sl.x1) {
    if (cur >= sbase + int64_t(Hkv) * ps.span) {
      sbase += int64_t(Hkv) * ps.span;
      gpb += int64_t(Hkv) * ps.parts;
      ++s;
      len = len_next;
      len_next = s + 1 < a.num_seqs ? effective_len(a, s + 1, block_size) : 0;
      ps = shape_of_len(a, len);
      continue;
    }
    const int64_t off = cur - sbase;
    const int g = int(off / ps.span);
    const int64_t pair_base = sbase + int64_t(g) * ps.span;
    const int64_t end = min(pair_base + ps.span, sl.x1);
    // tiles whose positions pair_base + lead + t * wt lie in [cur, end)
    const int64_t first_pos = pair_base + lead;
    const int tin = cur <= first_pos ? 0 : int((cur - first_pos + wt - 1) / wt);
    const int tend = end <= first_pos ? 0 : min(ps.tiles, int((end - first_pos + wt - 1) / wt));
    cur = end;
    if (tend <= tin) continue;  // only the pair's lead (or between tiles) in this slice
    const int ntile = tend - tin;
    const bool whole = tin == 0 && ntile == ps.tiles && ps.parts == 1;
    const int b_first = owner_of(sl.n, a.workers, first_pos);
    PairSlots slots;
    slots.fixed = (int64_t(s) * Hkv + g) * kPairSlots;
    slots.overflow = int64_t(a.num_seqs) * Hkv * kPairSlots + gpb + int64_t(g) * ps.parts + b_first;
    run(s, g, len, tin, ntile, whole, slots, b - b_first);
  }
}

// Calls piece(s, g, L, first_tile, num_tiles, whole, record_slot) for
// every piece of worker b's slice, in line order: the runs above, cut
// further at partition boundaries.
template <typename PieceFn>
__device__ __forceinline__ void walk_slice(const DecodeArgs& a, int block_size, int lane, int b,
                                           PieceFn&& piece) {
  const int tpp = a.partition_size / 16;  // tiles per partition
  walk_slice_runs(a, block_size, lane, b,
                  [&](int s, int g, int len, int tin, int ntile, bool whole,
                      const PairSlots& slots, int k0) {
                    if (whole) {
                      piece(s, g, len, tin, ntile, true, int64_t(0));
                      return;
                    }
                    const int end = tin + ntile;
                    for (int t = tin; t < end;) {
                      const int part = t / tpp;
                      const int e = min(end, (part + 1) * tpp);
                      piece(s, g, len, t, e - t, false, record_slot(slots, k0 + part));
                      t = e;
                    }
                  });
}

// The records of pair (s, g): records 0 .. count - 1, at
// record_slot(slots, k).  Some k in that range belong to no piece (a worker
// cut falling on a partition cut skips one); their slots hold records of
// older launches, whose epoch differs.  Needs the meta block written by
// worker 0.  Returns false when the pair has no tiles.
struct PairRecords {
  PairSlots slots;
  int count;
  bool whole;      // one piece: its worker wrote the output directly
  uint32_t epoch;  // stamp of the launch that wrote the meta block
};

// Slots of pair (s, g) that need no meta block (pair slots only).
__device__ __forceinline__ int64_t pair_fixed_slot(const DecodeArgs& a, int s, int g) {
  return (int64_t(s) * a.num_kv_heads + g) * kPairSlots;
}

__device__ __forceinline__ bool pair_records(const DecodeArgs& a, int block_size, int s, int g,
                                             PairRecords* pr) {
  // the meta loads go out with the length's, not after it
  const int32_t* meta = reinterpret_cast<const int32_t*>(a.ws_meta);
  const int64_t n = *meta_n(a);
  const int32_t pref_t = meta[s];
  const int32_t pref_p = meta[a.num_seqs + s];
  const uint32_t epoch = *reinterpret_cast<const uint32_t*>(meta_n(a) + 1);
  asm volatile("" ::: "memory");
  const PairShape ps = pair_shape(a, s, block_size);
  if (ps.tiles == 0) return false;
  const int Hkv = a.num_kv_heads;
  const int64_t base = int64_t(pref_t) * Hkv + int64_t(g) * ps.span + a.tail_lead;
  const int64_t gp0 = int64_t(pref_p) * Hkv + int64_t(g) * ps.parts;
  const int b_first = owner_of(n, a.workers, base);
  const int b_last = owner_of(n, a.workers, base + int64_t(ps.tiles - 1) * a.tail_wt);
  pr->slots.fixed = pair_fixed_slot(a, s, g);
  pr->slots.overflow = int64_t(a.num_seqs) * Hkv * kPairSlots + gp0 + b_first;
  pr->count = ps.parts + b_last - b_first;
  pr->whole = b_first == b_last && ps.parts == 1;
  pr->epoch = epoch;
  return true;
}

// ---------------------------------------------------------------------------
// Shared-prefix groups.  Sequences group_start[i] .. group_start[i+1] - 1 of
// a launch share the physical blocks of their first prefix_lens[i] tokens
// (the pages' reference-counted sharing: parallel samples of one prompt).
// The line then holds U = num_groups + S units: first one prefix unit per
// group, then one tail unit per sequence.  A prefix unit streams the shared
// tokens once per KV head, for the query heads of up to prefix_members
// members at once (the matrix-core columns), reading the blocks through the
// first member's table; a member's tail unit holds its other tokens.  Only
// whole 16-token tiles are shared, so the prefix length a unit covers is
// rounded down to a multiple of 16 and clamped to the first member's
// length; a member beyond prefix_members, or outside every group, has a
// tail unit holding all its tokens.
//
// Records: a prefix unit has one partition; the piece of prefix pair p =
// i * Hkv + g (group i, KV head g) that worker b streams writes one record
// per member into wide slot p + b of the wide region.  Along the line every
// cut raises p or b, so the slots are distinct and below
// num_groups * Hkv + W.  Tail units number their partitions and records
// exactly as plain launches number sequences'.
//
// Each worker first stages the group table in LDS (two coalesced rounds of
// loads, issued after the loads of its lanes' unit lengths), so that a
// sequence's group is a lookup in LDS rather than a chain of dependent
// memory loads.  Worker 0 also publishes, per unit,
// what the merge needs (its line and partition prefixes, its first token or
// length, its group and member), so the merge reads no group arrays.

// Groups a grouped launch may have (the LDS group table's capacity).
constexpr int kMaxGroups = 512;

// Workers a grouped launch may use: the wide region is sized for them.
constexpr int kMaxGroupWorkers = 1024;

// Wide records of a grouped launch (each prefix_members member records).
__host__ __device__ inline int64_t max_wide_records(int num_groups, int num_kv_heads) {
  return int64_t(num_groups) * num_kv_heads + kMaxGroupWorkers;
}

// Meta block of a grouped launch: int32 prefT[U], prefP[U], aux0[U],
// aux1[U], then int64 N and uint32 epoch, padded to 256 bytes.
__host__ __device__ inline int64_t meta_bytes_units(int units) {
  const int64_t n_off = (int64_t(units) * 16 + 7) / 8 * 8;
  return (n_off + 16 + 255) / 256 * 256;
}

// The group table in LDS, one 16-byte entry per group i:
// {start_i, start_{i+1}, plen_i, 0}, the starts clamped to [0, S] and plen_i
// the tokens prefix unit i covers.
struct GroupTable {
  int4* rec;  // [num_groups]
};

template <int B>
__device__ __forceinline__ void stage_group_table(const DecodeArgs& a, GroupTable gt, int lane) {
  const int n = a.num_groups;
  const int S = a.num_seqs;
  auto clamp_start = [&](int i) {
    const int x = load_ro(a.group_start, i);
    return x < 0 ? 0 : (x > S ? S : x);
  };
  for (int i = lane; i < n; i += 64) {
    const int s0 = clamp_start(i);
    const int s1 = clamp_start(i + 1);
    const int p = max(load_ro(a.prefix_lens, i), 0);
    const int members = max(0, min(s1 - s0, a.prefix_members));
    const int plen = members > 0 ? min(p, effective_len(a, s0, B)) / 16 * 16 : 0;
    gt.rec[i] = make_int4(s0, s1, plen, 0);
  }
  __syncthreads();  // one wave: orders the LDS writes before the reads
}

struct GroupInfo {
  int first;    // first member sequence
  int members;  // members the prefix unit serves
  int plen;     // tokens the prefix unit covers (a multiple of 16)
};

__device__ __forceinline__ GroupInfo group_info(const DecodeArgs& a, const int4& r) {
  GroupInfo gi;
  gi.first = r.x;
  gi.members = max(0, min(r.y - r.x, a.prefix_members));
  gi.plen = r.z;
  return gi;
}

__device__ __forceinline__ GroupInfo group_info(const DecodeArgs& a, const GroupTable& gt, int i) {
  return group_info(a, gt.rec[i]);
}

// The group of sequence s: the last group starting at or before it, or -1.
// Sequences are looked up in increasing order along a cursor that keeps the
// current group's entry in registers: a binary search in the LDS table for
// the first, then a step to the next entry only when s passes the group's
// end.
struct GroupCursor {
  int g = -1;
  int4 r;
};

__device__ __forceinline__ int group_at(const DecodeArgs& a, const GroupTable& gt, int s,
                                        GroupCursor& c) {
  const int n = a.num_groups;
  if (c.g < 0 || c.r.x > s) {
    if (n <= 0 || gt.rec[0].x > s) return -1;
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gt.rec[mid].x <= s) lo = mid; else hi = mid - 1;
    }
    c.g = lo;
    c.r = gt.rec[lo];
  }
  while (s >= c.r.y && c.g + 1 < n) {
    const int4 nx = gt.rec[c.g + 1];
    if (nx.x > s) break;
    ++c.g;
    c.r = nx;
  }
  return c.g;
}

// Tokens of sequence s (effective length L) that its group's prefix unit
// covers: 0 unless s is one of the members the unit serves.
__device__ __forceinline__ int seq_prefix_tokens(const DecodeArgs& a, const GroupTable& gt, int s,
                                                 int L, GroupCursor& c, int* group, int* member) {
  *group = -1;
  *member = -1;
  const int g = group_at(a, gt, s, c);
  if (g < 0) return 0;
  const GroupInfo gi = group_info(a, c.r);
  const int m = s - gi.first;
  if (m < 0 || m >= gi.members) return 0;
  *group = g;
  *member = m;
  return min(gi.plen, L);
}

// Shape of unit u of a grouped line.  Each of its Hkv pairs takes `span`
// line positions: `lead` positions for the run start, then `wt` per tile
// (tile t of the pair sits at position lead + t * wt from the pair's start;
// a worker owns the tiles whose positions fall in its slice).
struct UnitShape {
  int tiles;   // 16-token tiles
  int parts;   // partitions (0 for a prefix unit: its records are wide)
  int tok0;    // first token of the unit within its sequence
  int len;     // tail unit: the sequence's effective length; prefix unit: plen
  int aux;     // tail unit of a served member: group << 8 | member; else -1
  int lead, wt, span;
};

__device__ __forceinline__ void set_span(UnitShape& us, int lead, int wt) {
  us.lead = lead;
  us.wt = wt;
  us.span = us.tiles > 0 ? lead + us.tiles * wt : 0;
}

// Unit u's shape; for a tail unit L is its sequence's effective length.
__device__ __forceinline__ UnitShape unit_shape_len(const DecodeArgs& a, const GroupTable& gt,
                                                    int u, int L, GroupCursor& c) {
  UnitShape us;
  if (u < a.num_groups) {
    us.len = gt.rec[u].z;
    us.tiles = us.len / 16;
    us.parts = 0;
    us.tok0 = 0;
    us.aux = -1;
    set_span(us, a.prefix_lead, a.prefix_wt);
    return us;
  }
  int grp, mem;
  const int s = u - a.num_groups;
  const int t0 = seq_prefix_tokens(a, gt, s, L, c, &grp, &mem);
  const int n = L - t0;
  us.tiles = (n + 15) / 16;
  us.parts = (n + a.partition_size - 1) / a.partition_size;
  us.tok0 = t0;
  us.len = L;
  us.aux = grp >= 0 ? (grp << 8) | mem : -1;
  set_span(us, a.tail_lead, a.tail_wt);
  return us;
}

// Effective length of unit u's sequence (0 for a prefix unit or past the end).
__device__ __forceinline__ int unit_len(const DecodeArgs& a, int u, int block_size) {
  const int s = u - a.num_groups;
  return s >= 0 && s < a.num_seqs ? effective_len(a, s, block_size) : 0;
}

// Worker b's slice of a grouped line: as locate_slice, over units.  Worker
// 0 publishes the meta block for the merge.
struct UnitSlice {
  int64_t n, x0, x1;
  int unit;        // unit holding x0 (valid when x0 < x1)
  UnitShape shape; // its shape
  int64_t pref_t;  // prefT[unit]
  int64_t pref_p;  // prefP[unit]
};

__device__ __forceinline__ int64_t* meta_n_units(const DecodeArgs& a) {
  const int U = a.num_groups + a.num_seqs;
  return reinterpret_cast<int64_t*>(reinterpret_cast<char*>(a.ws_meta) +
                                    (int64_t(U) * 16 + 7) / 8 * 8);
}

// A lane's units are consecutive.  Their lengths are loaded kPrefetch at a
// time, all issued before any is used, and the shapes of the first
// kPrefetch units are kept in registers between the two passes (the line
// total, then the slice search and the published meta), so a lane holding
// at most kPrefetch units (launches of up to 64 * kPrefetch units) computes
// each shape once.
constexpr int kPrefetch = 8;

__device__ __forceinline__ void load_unit_lens(const DecodeArgs& a, int c0, int last,
                                               int block_size, int (&len)[kPrefetch]) {
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) len[i] = c0 + i < last ? unit_len(a, c0 + i, block_size) : 0;
}

__device__ __forceinline__ UnitSlice locate_unit_slice(const DecodeArgs& a, const GroupTable& gt,
                                                       int block_size, int lane, int b) {
  const int U = a.num_groups + a.num_seqs;
  const int per = (U + 63) / 64;  // consecutive units per lane
  const int first = min(U, lane * per);
  const int last = min(U, first + per);
  UnitShape kept[kPrefetch];
  int lt = 0, lp = 0;
  {
    GroupCursor c;
    int len[kPrefetch];
    // the lengths' loads go out first, the group table's after them
    load_unit_lens(a, first, last, block_size, len);
    if (block_size == 8) stage_group_table<8>(a, gt, lane);
    else if (block_size == 16) stage_group_table<16>(a, gt, lane);
    else stage_group_table<32>(a, gt, lane);
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
      kept[i] = UnitShape{};
      if (first + i < last) {
        kept[i] = unit_shape_len(a, gt, first + i, len[i], c);
        lt += kept[i].span;
        lp += kept[i].parts;
      }
    }
    for (int c0 = first + kPrefetch; c0 < last; c0 += kPrefetch) {
      load_unit_lens(a, c0, last, block_size, len);
#pragma unroll
      for (int i = 0; i < kPrefetch; ++i) {
        if (c0 + i < last) {
          const UnitShape us = unit_shape_len(a, gt, c0 + i, len[i], c);
          lt += us.span;
          lp += us.parts;
        }
      }
    }
  }
  const int it = wave_inclusive_scan(lt, lane);
  const int ip = wave_inclusive_scan(lp, lane);
  UnitSlice r;
  r.n = int64_t(wave_uniform(__shfl(it, 63))) * a.num_kv_heads;
  r.x0 = r.n > 0 ? slice_start(r.n, a.workers, b) : 0;
  r.x1 = r.n > 0 ? slice_start(r.n, a.workers, b + 1) : 0;
  const bool publish = b == 0;
  int32_t* meta = reinterpret_cast<int32_t*>(a.ws_meta);
  int found_u = -1;
  UnitShape found{};
  int64_t found_t = 0, found_p = 0;
  int64_t ct = it - lt, cp = ip - lp;
  auto visit = [&](int u, const UnitShape& us) {
    if (publish) {
      meta[u] = int32_t(ct);
      meta[U + u] = int32_t(cp);
      meta[2 * U + u] = u < a.num_groups ? us.len : us.tok0;
      meta[3 * U + u] = us.aux;
    }
    if (us.span > 0 && r.x0 >= ct * a.num_kv_heads && r.x0 < (ct + us.span) * a.num_kv_heads) {
      found_u = u;
      found = us;
      found_t = ct;
      found_p = cp;
    }
    ct += us.span;
    cp += us.parts;
  };
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i)
    if (first + i < last) visit(first + i, kept[i]);
  if (first + kPrefetch < last) {
    GroupCursor c;
    int len[kPrefetch];
    for (int c0 = first + kPrefetch; c0 < last; c0 += kPrefetch) {
      load_unit_lens(a, c0, last, block_size, len);
#pragma unroll
      for (int i = 0; i < kPrefetch; ++i)
        if (c0 + i < last) visit(c0 + i, unit_shape_len(a, gt, c0 + i, len[i], c));
    }
  }
  if (publish && lane == 0) {
    *meta_n_units(a) = r.n;
    *reinterpret_cast<uint32_t*>(meta_n_units(a) + 1) = a.epoch;
  }
  const unsigned long long owner = __ballot(found_u >= 0);
  const int src = owner ? int(__builtin_ctzll(owner)) : 0;
  r.unit = wave_uniform(__shfl(found_u, src));
  r.shape.tiles = wave_uniform(__shfl(found.tiles, src));
  r.shape.parts = wave_uniform(__shfl(found.parts, src));
  r.shape.tok0 = wave_uniform(__shfl(found.tok0, src));
  r.shape.len = wave_uniform(__shfl(found.len, src));
  r.shape.aux = wave_uniform(__shfl(found.aux, src));
  r.shape.lead = wave_uniform(__shfl(found.lead, src));
  r.shape.wt = wave_uniform(__shfl(found.wt, src));
  r.shape.span = wave_uniform(__shfl(found.span, src));
  r.pref_t = wave_uniform64(__shfl(found_t, src));
  r.pref_p = wave_uniform64(__shfl(found_p, src));
  return r;
}

// One run of a grouped line: tiles [tin, tin + ntile) of unit `unit`, KV
// head kvh.  A prefix run (prefix) is group `seq`'s shared tokens; a tail
// run is sequence `seq`'s tokens from tok0 on.
struct UnitRun {
  int unit, seq, kvh;
  bool prefix;
  UnitShape shape;
  int tin, ntile;
  bool whole;       // tail runs only: the whole pair, one partition, no prefix
  PairSlots slots;  // tail runs: record slots
  int64_t wide;     // prefix runs: the wide slot of this piece
  int k0;
};

// Calls run(UnitRun) for every run of worker b's slice of a grouped line,
// in line order (as walk_slice_runs does for a plain line).  The next
// sequence's length is loaded a unit ahead.
template <typename RunFn>
__device__ __forceinline__ void walk_unit_runs(const DecodeArgs& a, const GroupTable& gt,
                                               int block_size, int lane, int b, RunFn&& run) {
  const UnitSlice sl = locate_unit_slice(a, gt, block_size, lane, b);
  if (sl.x0 >= sl.x1) return;
  const int Hkv = a.num_kv_heads;
  const int U = a.num_groups + a.num_seqs;
  int u = sl.unit;
  UnitShape us = sl.shape;
  int64_t ubase = sl.pref_t * Hkv;  // line start of unit u
  int64_t gpb = sl.pref_p * Hkv;    // first tail partition index of unit u
  GroupCursor c;
  int len_next = unit_len(a, u + 1, block_size);
  int64_t cur = sl.x0;
  while (cur < sl.x1) {
    if (cur >= ubase + int64_t(Hkv) * us.span) {
      ubase += int64_t(Hkv) * us.span;
      gpb += int64_t(Hkv) * us.parts;
      ++u;
      if (u >= U) break;  // cannot happen: the slice ends inside the line
      us = unit_shape_len(a, gt, u, len_next, c);
      len_next = unit_len(a, u + 1, block_size);
      continue;
    }
    const int64_t off = cur - ubase;
    const int g = int(off / us.span);
    const int64_t pair_base = ubase + int64_t(g) * us.span;
    const int64_t pair_end = pair_base + us.span;
    const int64_t end = min(pair_end, sl.x1);
    // tiles whose positions pair_base + lead + t * wt lie in [cur, end)
    const int64_t first_pos = pair_base + us.lead;
    const int tin = cur <= first_pos ? 0 : int((cur - first_pos + us.wt - 1) / us.wt);
    const int tend = end <= first_pos ? 0 : min(us.tiles, int((end - first_pos + us.wt - 1) / us.wt));
    cur = end;
    if (tend <= tin) continue;  // only the pair's lead (or between tiles) in this slice
    UnitRun r;
    r.unit = u;
    r.kvh = g;
    r.prefix = u < a.num_groups;
    r.seq = r.prefix ? u : u - a.num_groups;
    r.shape = us;
    r.tin = tin;
    r.ntile = tend - tin;
    const int b_first = owner_of(sl.n, a.workers, first_pos);
    r.wide = 0;
    if (r.prefix) {
      r.whole = false;
      r.slots = PairSlots{0, 0};
      r.wide = int64_t(u) * Hkv + g + b;
    } else {
      r.whole = tin == 0 && r.ntile == us.tiles && us.parts == 1 && us.tok0 == 0;
      r.slots.fixed = (int64_t(r.seq) * Hkv + g) * kPairSlots;
      r.slots.overflow = int64_t(a.num_seqs) * Hkv * kPairSlots + gpb + int64_t(g) * us.parts + b_first;
    }
    r.k0 = b - b_first;
    run(r);
  }
}

// The records the merge of sequence s, KV head g folds in a grouped launch:
// its tail pair's (as pair_records) and, for a member of a prefix unit, the
// pieces of the prefix pair (wide slots, one record per member).  Read
// from the meta block worker 0 published: two rounds of loads.
struct UnitRecords {
  PairRecords tail;   // tail.count == 0 when the tail has no tiles
  bool prefix;        // a member served by a prefix unit
  int64_t wide;       // wide slot of the prefix pair's first piece
  int wide_count;     // its pieces (slots wide .. wide + wide_count - 1)
  int member;         // the sequence's member index (record within a wide slot)
  int len;            // the sequence's effective length
};

__device__ __forceinline__ void unit_records(const DecodeArgs& a, int block_size, int s, int g,
                                             UnitRecords* ur) {
  const int U = a.num_groups + a.num_seqs;
  const int32_t* meta = reinterpret_cast<const int32_t*>(a.ws_meta);
  const int u = a.num_groups + s;
  const int64_t n = *meta_n_units(a);
  const uint32_t epoch = *reinterpret_cast<const uint32_t*>(meta_n_units(a) + 1);
  const int32_t pref_t = meta[u];
  const int32_t pref_p = meta[U + u];
  const int32_t tok0 = meta[2 * U + u];
  const int32_t aux = meta[3 * U + u];
  const int L = effective_len(a, s, block_size);
  asm volatile("" ::: "memory");
  const int Hkv = a.num_kv_heads;
  const int nt = L - tok0;
  const int tiles = (nt + 15) / 16;
  const int parts = (nt + a.partition_size - 1) / a.partition_size;
  const int span = tiles > 0 ? a.tail_lead + tiles * a.tail_wt : 0;
  ur->len = L;
  ur->tail.epoch = epoch;
  ur->tail.slots.fixed = pair_fixed_slot(a, s, g);
  ur->tail.slots.overflow = 0;
  ur->tail.count = 0;
  ur->tail.whole = false;
  if (tiles > 0) {
    const int64_t base = int64_t(pref_t) * Hkv + int64_t(g) * span + a.tail_lead;
    const int64_t gp0 = int64_t(pref_p) * Hkv + int64_t(g) * parts;
    const int b_first = owner_of(n, a.workers, base);
    const int b_last = owner_of(n, a.workers, base + int64_t(tiles - 1) * a.tail_wt);
    ur->tail.slots.overflow = int64_t(a.num_seqs) * Hkv * kPairSlots + gp0 + b_first;
    ur->tail.count = parts + b_last - b_first;
    ur->tail.whole = b_first == b_last && parts == 1 && tok0 == 0;
  }
  ur->prefix = false;
  ur->wide = 0;
  ur->wide_count = 0;
  ur->member = 0;
  if (tok0 > 0 && aux >= 0) {
    const int grp = aux >> 8;
    const int64_t pbase = int64_t(meta[grp]) * Hkv;
    const int ptiles = meta[2 * U + grp] / 16;
    const int pspan = a.prefix_lead + ptiles * a.prefix_wt;
    const int64_t base = pbase + int64_t(g) * pspan + a.prefix_lead;
    const int b_first = owner_of(n, a.workers, base);
    const int b_last = owner_of(n, a.workers, base + int64_t(ptiles - 1) * a.prefix_wt);
    ur->prefix = true;
    ur->wide = int64_t(grp) * Hkv + g + b_first;
    ur->wide_count = b_last - b_first + 1;
    ur->member = aux & 0xFF;
  }
}

}  // namespace pa

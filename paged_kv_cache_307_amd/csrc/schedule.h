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

struct PairShape {
  int tiles;   // T_s
  int parts;   // nparts_s
};

__device__ __forceinline__ PairShape shape_of_len(const DecodeArgs& a, int L) {
  PairShape p;
  p.tiles = (L + 15) / 16;
  p.parts = (L + a.partition_size - 1) / a.partition_size;
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
    lt += ps.tiles;
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
    if (ps.tiles > 0 && r.x0 >= ct * a.num_kv_heads && r.x0 < (ct + ps.tiles) * a.num_kv_heads) {
      found_s = s;
      found_len = len;
      found_t = ct;
      found_p = cp;
    }
    ct += ps.tiles;
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
  int64_t cur = sl.x0;
  while (cur < sl.x1) {
    if (cur >= sbase + int64_t(Hkv) * ps.tiles) {
      sbase += int64_t(Hkv) * ps.tiles;
      gpb += int64_t(Hkv) * ps.parts;
      ++s;
      len = len_next;
      len_next = s + 1 < a.num_seqs ? effective_len(a, s + 1, block_size) : 0;
      ps = shape_of_len(a, len);
      continue;
    }
    const int64_t off = cur - sbase;
    const int g = int(off / ps.tiles);
    const int tin = int(off - int64_t(g) * ps.tiles);
    const int64_t end = min(sbase + int64_t(g + 1) * ps.tiles, sl.x1);
    const int ntile = int(end - cur);
    const bool whole = tin == 0 && ntile == ps.tiles && ps.parts == 1;
    const int64_t pair_base = sbase + int64_t(g) * ps.tiles;
    const int b_first = owner_of(sl.n, a.workers, pair_base);
    PairSlots slots;
    slots.fixed = (int64_t(s) * Hkv + g) * kPairSlots;
    slots.overflow = int64_t(a.num_seqs) * Hkv * kPairSlots + gpb + int64_t(g) * ps.parts + b_first;
    run(s, g, len, tin, ntile, whole, slots, b - b_first);
    cur = end;
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
  const int64_t base = int64_t(pref_t) * Hkv + int64_t(g) * ps.tiles;
  const int64_t gp0 = int64_t(pref_p) * Hkv + int64_t(g) * ps.parts;
  const int b_first = owner_of(n, a.workers, base);
  const int b_last = owner_of(n, a.workers, base + ps.tiles - 1);
  pr->slots.fixed = pair_fixed_slot(a, s, g);
  pr->slots.overflow = int64_t(a.num_seqs) * Hkv * kPairSlots + gp0 + b_first;
  pr->count = ps.parts + b_last - b_first;
  pr->whole = b_first == b_last && ps.parts == 1;
  pr->epoch = epoch;
  return true;
}

}  // namespace pa

// Split-KV merge: combine the records of each (sequence, query head) into
// the final output with a log-sum-exp reduction.
//
// With piece records (m_p, l_p, o_p) as written by the decode workers (m_p
// the piece's maximum of scale * log2(e) * q.k, l_p = sum of 2^(x - m_p),
// o_p = sum of 2^(x - m_p) v), the exact softmax result is
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p l_p.
// A pair's records are numbered from 0 in line order; the first few sit in
// slots indexed by the pair, the rest in an overflow region (schedule.h).
// Records of this launch carry its epoch stamp.  Pairs written whole by one worker are left
// alone; pairs of length 0 get zeros.
//
// One workgroup of one, four or sixteen waves per (sequence, query head).
// In each wave, lane t handles the 16-byte dim chunk t % (D/4) of every
// (256/D)-th record, so each load is a coalesced float4; the lane groups'
// partial sums meet through lane shuffles, and the waves' through LDS.

#include <math.h>

#include "device_common.h"
#include "schedule.h"

namespace pa {

namespace {

constexpr int kThreads = 64;  // lanes per wave

template <typename Elem>
__device__ __forceinline__ Elem from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float f) { return f32_to_bf16(f); }

template <typename Elem>
__device__ __forceinline__ void store4(Elem* dst, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, float4 v) {
  *reinterpret_cast<float4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, float4 v) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// Running log-sum-exp state of a lane: max, denominator, numerator chunks.
template <int CPL>
struct Fold {
  float m, den;
  float4 num[CPL];
};

// a <- a (+) b.  A state that saw no record has den == 0 (a record has
// l >= 1, or NaN when a broken block id poisoned it, which must propagate).
template <int CPL>
__device__ __forceinline__ void fold_into(Fold<CPL>& a, const Fold<CPL>& b) {
  if (b.den == 0.f) return;
  if (a.den == 0.f) {
    a = b;
    return;
  }
  const float M = fmaxf(a.m, b.m);
  const float wa = exp2f(a.m - M), wb = exp2f(b.m - M);
  a.den = wa * a.den + wb * b.den;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    a.num[i].x = wa * a.num[i].x + wb * b.num[i].x;
    a.num[i].y = wa * a.num[i].y + wb * b.num[i].y;
    a.num[i].z = wa * a.num[i].z + wb * b.num[i].z;
    a.num[i].w = wa * a.num[i].w + wb * b.num[i].w;
  }
  a.m = M;
}

// NW waves per (sequence, query head): one wave for pairs with few records,
// more when partitions are many.  kGroups: a grouped launch (shared-prefix
// groups, schedule.h): a member also folds its prefix pair's records.
template <typename Elem, int D, int NW, bool kGroups>
__global__ __launch_bounds__(kThreads * NW) void merge_kernel(DecodeArgs a, int B) {
  constexpr int CH = D / 4 < kThreads ? D / 4 : kThreads;  // float4 chunks per lane group
  constexpr int CPL = D / 4 / CH;                          // chunks per lane (1 up to D = 256)
  constexpr int GPW = kThreads / CH;                       // record groups per wave
  constexpr int PG = GPW * NW;                             // record groups in the workgroup
  const int sh = blockIdx.x;
  const int h = sh % a.num_heads;
  const int s = sh / a.num_heads;
  const int G = a.group;
  const int kvh = h / G;
  const int hl = h % G;
  const int lane = threadIdx.x % kThreads;
  const int wave = threadIdx.x / kThreads;
  Elem* out = static_cast<Elem*>(a.out) + (int64_t(s) * a.num_heads + h) * D;
  const int64_t R = record_floats(G, D);
  const int c = lane % CH;
  const int pg = wave * GPW + lane / CH;

  // Lane (pg, c) folds records pg, pg + PG, ... into a running (max,
  // denominator, numerator chunks c, c + CH, ...), rescaling when the max
  // grows.  A stamp from another launch drops a record.
  Fold<CPL> f;
  f.m = -INFINITY;
  f.den = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) f.num[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold_record = [&](float mq, float lq, const float4* oq) {
    if (mq > f.m) {
      const float r = exp2f(f.m - mq);  // 0 on the first record
      f.den *= r;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        f.num[i].x *= r; f.num[i].y *= r; f.num[i].z *= r; f.num[i].w *= r;
      }
      f.m = mq;
    }
    const float w = exp2f(mq - f.m);
    f.den += w * lq;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      f.num[i].x += w * oq[i].x;
      f.num[i].y += w * oq[i].y;
      f.num[i].z += w * oq[i].z;
      f.num[i].w += w * oq[i].w;
    }
  };
  struct Loaded {
    uint32_t st;
    float m, l;
    float4 o[CPL];
  };
  auto load_record = [&](int64_t slot) {
    const float* rec = a.ws + slot * R;
    Loaded r;
    r.st = __float_as_uint(rec[G * D + 2 * G]);
    r.m = rec[G * D + hl];
    r.l = rec[G * D + G + hl];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      r.o[i] = *reinterpret_cast<const float4*>(rec + hl * D + 4 * (c + CH * i));
    return r;
  };

  // Records 0 .. kPairSlots - 1 sit in slots indexed by the pair, so in a
  // plain launch their loads go out together with the meta block's, before
  // the pair's record count is known; most pairs have no others.  A grouped
  // launch needs the meta block before its prefix records anyway, so there
  // the pair slots are loaded with those, only as many as hold records
  // (a member's tail often has one): the fork step's merge read 52 MB, about
  // 15 MB of them stale slots.
  constexpr int KF = (kPairSlots + PG - 1) / PG;  // pair slots per lane
  const int64_t fixed0 = pair_fixed_slot(a, s, kvh);
  Loaded fr[KF];
  if constexpr (!kGroups) {
#pragma unroll
    for (int u = 0; u < KF; ++u) fr[u] = load_record(fixed0 + min(pg + u * PG, kPairSlots - 1));
    // keep them ahead of the length and meta loads below: the compiler would
    // otherwise sink them past the empty-sequence exit, after its wait
    asm volatile("" ::: "memory");
  }

  PairRecords pr;
  UnitRecords ur;
  bool empty;
  if constexpr (kGroups) {
    unit_records(a, B, s, kvh, &ur);
    pr = ur.tail;
    empty = ur.len == 0;
  } else {
    empty = !pair_records(a, B, s, kvh, &pr);
  }
  if (empty) {  // empty sequence
    for (int i = lane + wave * kThreads; i < D; i += kThreads * NW) out[i] = from_f32<Elem>(0.f);
    if (a.lse && threadIdx.x == 0) a.lse[int64_t(s) * a.num_heads + h] = -INFINITY;
    return;
  }
  if (pr.whole) return;  // written whole by its worker
  if constexpr (kGroups) {
    // the live pair slots (clamped loads of a slot past the count re-read
    // the last live one, which the cache serves)
    const int live_last = max(min(pr.count, kPairSlots) - 1, 0);
#pragma unroll
    for (int u = 0; u < KF; ++u) fr[u] = load_record(fixed0 + min(pg + u * PG, live_last));
    // the prefix pieces: one wide slot per worker that streamed part of the
    // group's shared tokens for this KV head, this member's record in it.
    // A member shorter than a piece's tokens has l = 0 there: skipped.
    // The loads of kWideUnroll records per lane go out together (clamped to
    // the last piece), so a member costs one more round trip to memory.
    if (ur.prefix) {
      constexpr int kWideUnroll = 4;
      const int64_t mslot = int64_t(ur.member);
      for (int k0 = pg; k0 < ur.wide_count; k0 += PG * kWideUnroll) {
        Loaded r[kWideUnroll];
#pragma unroll
        for (int u = 0; u < kWideUnroll; ++u) {
          const int64_t k = min(k0 + u * PG, ur.wide_count - 1);
          const float* rec = a.ws_wide + ((ur.wide + k) * a.prefix_members + mslot) * R;
          r[u].st = __float_as_uint(rec[G * D + 2 * G]);
          r[u].m = rec[G * D + hl];
          r[u].l = rec[G * D + G + hl];
#pragma unroll
          for (int i = 0; i < CPL; ++i)
            r[u].o[i] = *reinterpret_cast<const float4*>(rec + hl * D + 4 * (c + CH * i));
        }
#pragma unroll
        for (int u = 0; u < kWideUnroll; ++u)
          if (k0 + u * PG < ur.wide_count && r[u].st == pr.epoch && !(r[u].l == 0.f))
            fold_record(r[u].m, r[u].l, r[u].o);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < KF; ++u) {
    const int k = pg + u * PG;
    if (k < kPairSlots && k < pr.count && fr[u].st == pr.epoch)
      fold_record(fr[u].m, fr[u].l, fr[u].o);
  }

  // The rest, from the overflow region: the loads of kUnroll records are
  // issued together and unconditionally (clamped to the last record), so a
  // pair costs one more round trip to memory per kUnroll records per lane.
  constexpr int kUnroll = 2;
  for (int q0 = kPairSlots + pg; q0 < pr.count; q0 += PG * kUnroll) {
    Loaded r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      r[u] = load_record(pr.slots.overflow + min(q0 + u * PG, pr.count - 1));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (q0 + u * PG < pr.count && r[u].st == pr.epoch) fold_record(r[u].m, r[u].l, r[u].o);
  }
  // Fold the wave's record groups (lanes c, c + CH, ...) together through
  // lane shuffles; every lane of a chunk ends with the wave's state.
#pragma unroll
  for (int off = CH; off < kThreads; off <<= 1) {
    Fold<CPL> o;
    o.m = __shfl_xor(f.m, off);
    o.den = __shfl_xor(f.den, off);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      o.num[i].x = __shfl_xor(f.num[i].x, off);
      o.num[i].y = __shfl_xor(f.num[i].y, off);
      o.num[i].z = __shfl_xor(f.num[i].z, off);
      o.num[i].w = __shfl_xor(f.num[i].w, off);
    }
    fold_into(f, o);
  }
  if constexpr (NW > 1) {  // then the waves' states through LDS
    __shared__ Fold<CPL> part[NW][CH];
    if (lane < CH) part[wave][lane] = f;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < NW; ++w)
      if (lane < CH) fold_into(f, part[w][lane]);
  }
  if (a.lse && lane == 0)  // ln sum e^(scale q.k) = (m + log2 den) ln 2
    a.lse[int64_t(s) * a.num_heads + h] = (f.m + __log2f(f.den)) * 0.6931471805599453f;
  if (lane < CH) {
    const float inv = 1.0f / f.den;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float4 t = f.num[i];
      t.x *= inv; t.y *= inv; t.z *= inv; t.w *= inv;
      store4<Elem>(out + 4 * (c + CH * i), t);
    }
  }
}

// Waves per (sequence, query head) in the merge: one while a pair's records
// fit in a couple of rounds of loads, four for longer runs of partitions,
// sixteen for very long ones (a 128K-token context has 256 partitions of
// 512 tokens), so that each wave folds only a few rounds of records.
constexpr int kWideMergeParts = 8;
constexpr int kWiderMergeParts = 32;

template <typename Elem, int D, bool kGroups>
hipError_t launch_merge_g(const DecodeArgs& a, int block_size, hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_heads));
  if (a.max_partitions > kWiderMergeParts)
    return launch(merge_kernel<Elem, D, 16, kGroups>, grid, dim3(16 * kThreads), 0, stream, a,
                  block_size);
  if (a.max_partitions > kWideMergeParts)
    return launch(merge_kernel<Elem, D, 4, kGroups>, grid, dim3(4 * kThreads), 0, stream, a,
                  block_size);
  return launch(merge_kernel<Elem, D, 1, kGroups>, grid, dim3(kThreads), 0, stream, a, block_size);
}

template <typename Elem, int D>
hipError_t launch_merge_d(const DecodeArgs& a, int block_size, hipStream_t stream) {
  if constexpr (sizeof(Elem) == 2) {  // groups are a bf16 decode path
    if (a.num_groups > 0) return launch_merge_g<Elem, D, true>(a, block_size, stream);
  }
  return launch_merge_g<Elem, D, false>(a, block_size, stream);
}

template <typename Elem>
hipError_t launch_merge_elem(const DecodeArgs& a, int head_dim, int block_size, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_merge_d<Elem, 64>(a, block_size, stream);
    case 128: return launch_merge_d<Elem, 128>(a, block_size, stream);
    case 256: return launch_merge_d<Elem, 256>(a, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, int block_size, bool bf16,
                               hipStream_t stream) {
  return bf16 ? launch_merge_elem<uint16_t>(a, head_dim, block_size, stream)
              : launch_merge_elem<float>(a, head_dim, block_size, stream);
}

}  // namespace pa

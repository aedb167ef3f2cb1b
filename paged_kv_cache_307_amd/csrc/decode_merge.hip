// Split-KV merge: combine the records of each (sequence, query head) into
// the final output with a log-sum-exp reduction.
//
// With piece records (m_p, l_p, o_p) as written by the decode workers (m_p
// the piece's maximum of scale * log2(e) * q.k, l_p = sum of 2^(x - m_p),
// o_p = sum of 2^(x - m_p) v), the exact softmax result is
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p l_p.
// A pair's records lie in a short index range (schedule.h); records of this
// launch carry its epoch stamp.  Pairs written whole by one worker are left
// alone; pairs of length 0 get zeros.
//
// One wave per (sequence, query head).  Lane t handles the 16-byte dim
// chunk t % (D/4) of every (256/D)-th record, so each load is a coalesced
// float4; the lane groups' partial sums meet through lane shuffles.

#include <math.h>

#include "device_common.h"
#include "schedule.h"

namespace pa {

namespace {

constexpr int kThreads = 64;  // one wave per (sequence, query head)

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

template <typename Elem, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeArgs a, int B) {
  constexpr int CH = D / 4 < kThreads ? D / 4 : kThreads;  // float4 chunks per lane group
  constexpr int CPL = D / 4 / CH;                          // chunks per lane (1 up to D = 256)
  constexpr int PG = kThreads / CH;                        // record groups in the wave
  const int sh = blockIdx.x;
  const int h = sh % a.num_heads;
  const int s = sh / a.num_heads;
  const int G = a.group;
  const int kvh = h / G;
  const int hl = h % G;
  const int lane = threadIdx.x;
  Elem* out = static_cast<Elem*>(a.out) + (int64_t(s) * a.num_heads + h) * D;
  PairRecords pr;
  if (!pair_records(a, B, s, kvh, &pr)) {  // empty sequence
    for (int i = lane; i < D; i += kThreads) out[i] = from_f32<Elem>(0.f);
    return;
  }
  if (pr.whole) return;  // written whole by its worker
  const int64_t R = record_floats(G, D);
  const float* base = a.ws + pr.first * R;
  const int count = int(pr.last - pr.first + 1);

  // One pass: lane (pg, c) folds records pg, pg + PG, ... into a running
  // (max, denominator, numerator chunks c, c + CH, ...), rescaling when the
  // max grows.  The loads of kUnroll records are issued together and
  // unconditionally (a stamp from another launch only drops the record
  // afterwards), so a pair costs one round trip to memory per kUnroll
  // records per lane.
  constexpr int kUnroll = 2;
  const int c = lane % CH;
  const int pg = lane / CH;
  float m_t = -INFINITY, den_t = 0.f;
  float4 num[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) num[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q0 = pg; q0 < count; q0 += PG * kUnroll) {
    uint32_t st[kUnroll];
    float mq[kUnroll], lq[kUnroll];
    float4 oq[kUnroll][CPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float* rec = base + int64_t(min(q0 + u * PG, count - 1)) * R;
      st[u] = __float_as_uint(rec[G * D + 2 * G]);
      mq[u] = rec[G * D + hl];
      lq[u] = rec[G * D + G + hl];
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        oq[u][i] = *reinterpret_cast<const float4*>(rec + hl * D + 4 * (c + CH * i));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (q0 + u * PG >= count || st[u] != pr.epoch) continue;
      if (mq[u] > m_t) {
        const float r = exp2f(m_t - mq[u]);  // 0 on the first record
        den_t *= r;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          num[i].x *= r; num[i].y *= r; num[i].z *= r; num[i].w *= r;
        }
        m_t = mq[u];
      }
      const float w = exp2f(mq[u] - m_t);
      den_t += w * lq[u];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        num[i].x += w * oq[u][i].x;
        num[i].y += w * oq[u][i].y;
        num[i].z += w * oq[u][i].z;
        num[i].w += w * oq[u][i].w;
      }
    }
  }
  // Fold the record groups (lanes c, c + CH, ...) into group 0.  A group
  // that saw no record has den == 0 (a record has l >= 1, or NaN when a
  // broken block id poisoned it, which must propagate).
#pragma unroll
  for (int off = CH; off < kThreads; off <<= 1) {
    const float m_o = __shfl_xor(m_t, off);
    const float den_o = __shfl_xor(den_t, off);
    float4 num_o[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      num_o[i].x = __shfl_xor(num[i].x, off);
      num_o[i].y = __shfl_xor(num[i].y, off);
      num_o[i].z = __shfl_xor(num[i].z, off);
      num_o[i].w = __shfl_xor(num[i].w, off);
    }
    if (den_o == 0.f) continue;  // same decision in every lane of the pair of groups
    if (den_t == 0.f) {
      m_t = m_o;
      den_t = den_o;
#pragma unroll
      for (int i = 0; i < CPL; ++i) num[i] = num_o[i];
      continue;
    }
    const float M = fmaxf(m_t, m_o);
    const float w = exp2f(m_t - M), wo = exp2f(m_o - M);
    den_t = w * den_t + wo * den_o;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      num[i].x = w * num[i].x + wo * num_o[i].x;
      num[i].y = w * num[i].y + wo * num_o[i].y;
      num[i].z = w * num[i].z + wo * num_o[i].z;
      num[i].w = w * num[i].w + wo * num_o[i].w;
    }
    m_t = M;
  }
  if (pg == 0) {
    const float inv = 1.0f / den_t;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float4 t = num[i];
      t.x *= inv; t.y *= inv; t.z *= inv; t.w *= inv;
      store4<Elem>(out + 4 * (c + CH * i), t);
    }
  }
}

template <typename Elem>
hipError_t launch_merge_elem(const DecodeArgs& a, int head_dim, int block_size, hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_heads));
  switch (head_dim) {
    case 64: return launch(merge_kernel<Elem, 64>, grid, dim3(kThreads), 0, stream, a, block_size);
    case 128: return launch(merge_kernel<Elem, 128>, grid, dim3(kThreads), 0, stream, a, block_size);
    case 256: return launch(merge_kernel<Elem, 256>, grid, dim3(kThreads), 0, stream, a, block_size);
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

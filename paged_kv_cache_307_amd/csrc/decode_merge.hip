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
// One 256-thread workgroup per (sequence, query head).  Thread t handles the
// 16-byte dim chunk t % (D/4) of every (1024/D)-th record, so each load is a
// coalesced float4; the partial sums meet in LDS.

#include <math.h>

#include "device_common.h"
#include "schedule.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

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
  constexpr int CH = D / 4;             // float4 chunks per head
  constexpr int PG = kThreads / CH;     // record groups
  const int sh = blockIdx.x;
  const int h = sh % a.num_heads;
  const int s = sh / a.num_heads;
  const int G = a.group;
  const int kvh = h / G;
  const int hl = h % G;
  Elem* out = static_cast<Elem*>(a.out) + (int64_t(s) * a.num_heads + h) * D;
  PairRecords pr;
  if (!pair_records(a, B, s, kvh, &pr)) {  // empty sequence
    for (int i = threadIdx.x; i < D; i += kThreads) out[i] = from_f32<Elem>(0.f);
    return;
  }
  if (pr.whole) return;  // written whole by its worker
  const int64_t R = record_floats(G, D);
  const float* base = a.ws + pr.first * R;
  const int count = int(pr.last - pr.first + 1);

  // One pass: thread (pg, c) folds records pg, pg + PG, ... into a running
  // (max, denominator, numerator chunk c), rescaling when the max grows.
  // The loads of kUnroll records are issued together and unconditionally
  // (a stamp from another launch only drops the record afterwards), so a
  // pair costs one round trip to memory per kUnroll records per thread.
  constexpr int kUnroll = 2;
  const int c = threadIdx.x % CH;
  const int pg = threadIdx.x / CH;
  float m_t = -INFINITY, den_t = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q0 = pg; q0 < count; q0 += PG * kUnroll) {
    uint32_t st[kUnroll];
    float mq[kUnroll], lq[kUnroll];
    float4 oq[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float* rec = base + int64_t(min(q0 + u * PG, count - 1)) * R;
      st[u] = __float_as_uint(rec[G * D + 2 * G]);
      mq[u] = rec[G * D + hl];
      lq[u] = rec[G * D + G + hl];
      oq[u] = *reinterpret_cast<const float4*>(rec + hl * D + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (q0 + u * PG >= count || st[u] != pr.epoch) continue;
      if (mq[u] > m_t) {
        const float r = exp2f(m_t - mq[u]);  // 0 on the first record
        den_t *= r;
        num.x *= r; num.y *= r; num.z *= r; num.w *= r;
        m_t = mq[u];
      }
      const float w = exp2f(mq[u] - m_t);
      den_t += w * lq[u];
      num.x += w * oq[u].x;
      num.y += w * oq[u].y;
      num.z += w * oq[u].z;
      num.w += w * oq[u].w;
    }
  }
  __shared__ float sm_m[PG];
  __shared__ float sm_den[PG];
  __shared__ float4 sm_num[PG][CH];
  if (c == 0) {
    sm_m[pg] = m_t;
    sm_den[pg] = den_t;
  }
  sm_num[pg][c] = num;
  __syncthreads();
  if (threadIdx.x < CH) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < PG; ++g) M = fmaxf(M, sm_m[g]);
    float den = 0.f;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < PG; ++g) {
      // a group that saw no record has den == 0 (a record has l >= 1, or
      // NaN when a broken block id poisoned it, which must propagate)
      if (sm_den[g] == 0.f) continue;
      const float w = exp2f(sm_m[g] - M);
      den += w * sm_den[g];
      const float4 u = sm_num[g][c];
      t.x += w * u.x; t.y += w * u.y; t.z += w * u.z; t.w += w * u.w;
    }
    const float inv = 1.0f / den;
    t.x *= inv; t.y *= inv; t.z *= inv; t.w *= inv;
    store4<Elem>(out + 4 * c, t);
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

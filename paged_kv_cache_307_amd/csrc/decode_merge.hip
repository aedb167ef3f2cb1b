// Split-KV merge: combine the records of each (sequence, query head) into
// the final output with a log-sum-exp reduction.
//
// With piece records (m_p, l_p, o_p) as written by the decode workers (m_p
// the piece's maximum of scale * log2(e) * q.k, l_p = sum of 2^(x - m_p),
// o_p = sum of 2^(x - m_p) v), the exact softmax result is
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p l_p.
// The pieces of a pair are found by walking the same cuts the workers made
// (schedule.h).  Pairs written whole by one worker are left alone; pairs of
// length 0 get zeros.
//
// One 256-thread workgroup per (sequence, query head).  Thread t handles the
// 16-byte dim chunk t % (D/4) of every (1024/D)-th piece, so each load is a
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

__device__ __forceinline__ float block_reduce(float x, float* sm, bool is_max) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float y = __shfl_xor(x, m);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[wave] = x;
  __syncthreads();
  float r = sm[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, sm[w]) : r + sm[w];
  return r;
}

template <typename Elem, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeArgs a, int B) {
  constexpr int CH = D / 4;             // float4 chunks per head
  constexpr int PG = kThreads / CH;     // piece groups
  const int sh = blockIdx.x;
  const int h = sh % a.num_heads;
  const int s = sh / a.num_heads;
  const int G = a.group;
  const int kvh = h / G;
  const int hl = h % G;
  Elem* out = static_cast<Elem*>(a.out) + (int64_t(s) * a.num_heads + h) * D;
  if (effective_len(a, s, B) == 0) {
    for (int i = threadIdx.x; i < D; i += kThreads) out[i] = from_f32<Elem>(0.f);
    return;
  }
  const int npieces = for_each_piece(a, B, s, kvh, [](int64_t) {});
  if (npieces <= 1) return;  // written whole by its worker
  const int64_t R = record_floats(G, D);
  const float* recs = a.ws;

  __shared__ float sm_red[kThreads / 64];
  __shared__ float4 sm_num[PG][CH];

  float mloc = -INFINITY;
  {
    int q = 0;
    for_each_piece(a, B, s, kvh, [&](int64_t idx) {
      if (q % kThreads == int(threadIdx.x)) mloc = fmaxf(mloc, recs[idx * R + G * D + hl]);
      ++q;
    });
  }
  const float M = block_reduce(mloc, sm_red, true);
  float dloc = 0.f;
  const int c = threadIdx.x % CH;
  const int pg = threadIdx.x / CH;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    int q = 0;
    for_each_piece(a, B, s, kvh, [&](int64_t idx) {
      const float* rec = recs + idx * R;
      if (q % kThreads == int(threadIdx.x)) dloc += exp2f(rec[G * D + hl] - M) * rec[G * D + G + hl];
      if (q % PG == pg) {
        const float w = exp2f(rec[G * D + hl] - M);
        const float4 o = *reinterpret_cast<const float4*>(rec + hl * D + 4 * c);
        num.x += w * o.x;
        num.y += w * o.y;
        num.z += w * o.z;
        num.w += w * o.w;
      }
      ++q;
    });
  }
  const float den = block_reduce(dloc, sm_red, false);
  sm_num[pg][c] = num;
  __syncthreads();
  if (threadIdx.x < CH) {
    float4 t = sm_num[0][c];
#pragma unroll
    for (int g = 1; g < PG; ++g) {
      const float4 u = sm_num[g][c];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
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

// Paged decode attention on the vector ALUs, for float32 caches (and bf16
// shapes the matrix-core kernel does not take).
//
// Same result as the matrix-core kernel: out[s][h] = softmax_t(scale *
// q.k_t) v_t over the L_s tokens of sequence s, token t read from block
// block_table[s][t / B] at offset t % B, KV head h / G.  [P2
// "PagedAttention学习笔记", section 2.1 and section 三; P3 "KV cache 显存管理",
// PagedAttention 改变了什么.]
//
// One wave per (sequence, KV head, partition).  The partition is walked in
// chunks of 64 tokens: lane j owns token c0 + j for the q.k phase (its K row
// read with 16-byte loads, dotted with the G queries held in LDS), the chunk
// maximum updates an online softmax (exact fp32 exp2), and for the p.v phase
// lanes switch to head dims, each accumulating dims lane, lane + 64, ... over
// the chunk's tokens.

#include <math.h>

#include "device_common.h"

namespace pa {

namespace {

constexpr int kGMax = 16;

template <typename Elem>
__device__ __forceinline__ float to_f32(Elem e);
template <>
__device__ __forceinline__ float to_f32<float>(float e) { return e; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t e) { return bf16_to_f32(e); }

template <typename Elem>
__device__ __forceinline__ Elem from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float f) { return f32_to_bf16(f); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <typename Elem, int D>
__global__ __launch_bounds__(64) void decode_simt_kernel(DecodeArgs a, int B) {
  constexpr int DPL = D / 64;                 // dims per lane in the p.v phase
  constexpr int VEC = 16 / sizeof(Elem);      // elements per 16-byte K load

  const int bid = blockIdx.x;
  const int p = bid % a.max_partitions;
  const int sg = bid / a.max_partitions;
  const int kvh = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  const int G = a.group;
  const int L = effective_len(a, s, B);
  const int P = a.partition_size;
  const int nparts = (L + P - 1) / P;
  const int lane = threadIdx.x;
  Elem* out = static_cast<Elem*>(a.out);

  if (L == 0) {
    if (p == 0) {
      Elem* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
      for (int i = lane; i < G * D; i += 64) o[i] = from_f32<Elem>(0.f);
    }
    return;
  }
  if (p >= nparts) return;

  const int t_begin = p * P;
  const int t_end = min(L, t_begin + P);
  const int32_t* row = a.block_tables + int64_t(s) * a.max_blocks_per_seq;
  const Elem* kc = static_cast<const Elem*>(a.k_cache);
  const Elem* vc = static_cast<const Elem*>(a.v_cache);

  __shared__ float q_s[kGMax][D];
  __shared__ float p_s[kGMax][64];
  __shared__ int64_t vbase_s[64];

  const Elem* qg = static_cast<const Elem*>(a.q) + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
  for (int i = lane; i < G * D; i += 64) q_s[i / D][i % D] = to_f32<Elem>(qg[i]) * a.scale_log2e;
  __syncthreads();

  float acc[kGMax][DPL];
  float m_run[kGMax], l_part[kGMax];
#pragma unroll
  for (int h = 0; h < kGMax; ++h) {
    m_run[h] = -INFINITY;
    l_part[h] = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[h][k] = 0.f;
  }

  const int64_t tile_elems = int64_t(B) * D;
  for (int c0 = t_begin; c0 < t_end; c0 += 64) {
    const int t = c0 + lane;
    const bool valid = t < t_end;
    bool bad = false;
    int64_t kbase = 0, vbase = 0;
    if (valid) {
      int pb = row[t / B];
      const int off = t % B;
      bad = unsigned(pb) >= unsigned(a.num_blocks);
      pb = bad ? 0 : pb;
      const int64_t tile = (int64_t(pb) * a.num_kv_heads + kvh) * tile_elems;
      kbase = tile + int64_t(off) * D;
      vbase = tile + off;
    }
    float x[kGMax];
#pragma unroll
    for (int h = 0; h < kGMax; ++h) x[h] = 0.f;
    if (valid) {
      for (int d = 0; d < D; d += VEC) {
        const uint4 raw = *reinterpret_cast<const uint4*>(kc + kbase + d);
        Elem e[VEC];
        __builtin_memcpy(e, &raw, 16);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float kv = to_f32<Elem>(e[v]);
#pragma unroll
          for (int h = 0; h < kGMax; ++h)
            if (h < G) x[h] += q_s[h][d + v] * kv;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kGMax; ++h) {
      if (h < G) {
        float xh = valid ? (bad ? __builtin_nanf("") : x[h]) : -INFINITY;
        const float cmax = wave_max(xh);
        const float m_new = fmaxf(m_run[h], cmax);
        const float alpha = (m_run[h] == -INFINITY) ? 0.f : exp2f(m_run[h] - m_new);
        const float pw = exp2f(xh - m_new);
        m_run[h] = m_new;
        l_part[h] = l_part[h] * alpha + pw;
        p_s[h][lane] = pw;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[h][k] *= alpha;
      }
    }
    vbase_s[lane] = vbase;
    __syncthreads();
    const int nvalid = min(64, t_end - c0);
    for (int j = 0; j < nvalid; ++j) {
      const int64_t vb = vbase_s[j];
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const float vv = to_f32<Elem>(vc[vb + int64_t(lane + 64 * k) * B]);
#pragma unroll
        for (int h = 0; h < kGMax; ++h)
          if (h < G) acc[h][k] += p_s[h][j] * vv;
      }
    }
    __syncthreads();
  }

  const bool single = nparts == 1;
  float* rec = nullptr;
  if (!single)
    rec = a.ws + ((int64_t(s) * a.num_kv_heads + kvh) * a.max_partitions + p) * record_floats(G, D);
#pragma unroll
  for (int h = 0; h < kGMax; ++h) {
    if (h >= G) continue;
    const float l_tot = wave_sum(l_part[h]);
    if (single) {
      Elem* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G + h) * D;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[lane + 64 * k] = from_f32<Elem>(acc[h][k] / l_tot);
    } else {
#pragma unroll
      for (int k = 0; k < DPL; ++k) rec[h * D + lane + 64 * k] = acc[h][k];
      if (lane == 0) {
        rec[G * D + h] = m_run[h];
        rec[G * D + G + h] = l_tot;
      }
    }
  }
}

template <typename Elem>
hipError_t launch_elem(const DecodeArgs& a, int head_dim, int block_size, hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_kv_heads * a.max_partitions));
  switch (head_dim) {
    case 64: return launch(decode_simt_kernel<Elem, 64>, grid, dim3(64), 0, stream, a, block_size);
    case 128: return launch(decode_simt_kernel<Elem, 128>, grid, dim3(64), 0, stream, a, block_size);
    case 256: return launch(decode_simt_kernel<Elem, 256>, grid, dim3(64), 0, stream, a, block_size);
    default: return hipErrorInvalidValue;
  }
}

// Split-KV merge: one workgroup per (sequence, KV head); thread i handles
// (head i / D, dim i % D) of the group.  M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p o_p / sum_p w_p l_p.
template <typename Elem, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int B) {
  const int sg = blockIdx.x;
  const int kvh = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  const int G = a.group;
  const int L = effective_len(a, s, B);
  const int nparts = (L + a.partition_size - 1) / a.partition_size;
  if (nparts <= 1) return;
  const int64_t R = record_floats(G, D);
  const float* recs = a.ws + (int64_t(s) * a.num_kv_heads + kvh) * a.max_partitions * R;
  Elem* out = static_cast<Elem*>(a.out) + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int h = i / D;
    float M = -INFINITY;
    for (int q = 0; q < nparts; ++q) M = fmaxf(M, recs[q * R + G * D + h]);
    float num = 0.f, den = 0.f;
    for (int q = 0; q < nparts; ++q) {
      const float w = exp2f(recs[q * R + G * D + h] - M);
      den += w * recs[q * R + G * D + G + h];
      num += w * recs[q * R + i];
    }
    out[i] = from_f32<Elem>(num / den);
  }
}

template <typename Elem>
hipError_t launch_merge_elem(const DecodeArgs& a, int head_dim, int block_size, hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_kv_heads));
  switch (head_dim) {
    case 64: return launch(merge_kernel<Elem, 64>, grid, dim3(256), 0, stream, a, block_size);
    case 128: return launch(merge_kernel<Elem, 128>, grid, dim3(256), 0, stream, a, block_size);
    case 256: return launch(merge_kernel<Elem, 256>, grid, dim3(256), 0, stream, a, block_size);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_simt(const DecodeArgs& a, int head_dim, int block_size, bool bf16,
                              hipStream_t stream) {
  return bf16 ? launch_elem<uint16_t>(a, head_dim, block_size, stream)
              : launch_elem<float>(a, head_dim, block_size, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, int block_size, bool bf16,
                               hipStream_t stream) {
  return bf16 ? launch_merge_elem<uint16_t>(a, head_dim, block_size, stream)
              : launch_merge_elem<float>(a, head_dim, block_size, stream);
}

}  // namespace pa

// Paged decode attention on the vector ALUs, for float32 caches (and bf16
// shapes the matrix-core kernel does not take).
//
// Same result as the matrix-core kernel: out[s][h] = softmax_t(scale *
// q.k_t) v_t over the L_s tokens of sequence s, token t read from block
// block_table[s][t / B] at offset t % B, KV head h / G.  [P2
// "PagedAttention学习笔记", section 2.1 and section 三; P3 "KV cache 显存管理",
// PagedAttention 改变了什么.]
//
// One wave per worker (see schedule.h) or, in single pass, per (sequence, KV
// head).  Each piece's token range is walked in chunks of 64 tokens: lane j owns token c0 + j for the q.k phase (its K row
// read with 16-byte loads, dotted with the G queries held in LDS), the chunk
// maximum updates an online softmax (exact fp32 exp2), and for the p.v phase
// lanes switch to head dims, each accumulating dims lane, lane + 64, ... over
// the chunk's tokens.

#include <math.h>

#include "device_common.h"
#include "schedule.h"

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

template <typename Elem, int D, bool kSplit>
__global__ __launch_bounds__(64) void decode_simt_kernel(DecodeArgs a, int B) {
  constexpr int DPL = D / 64;                 // dims per lane in the p.v phase
  constexpr int VEC = 16 / sizeof(Elem);      // elements per 16-byte K load
  const int G = a.group;
  const int lane = threadIdx.x;
  Elem* out = static_cast<Elem*>(a.out);
  const Elem* kc = static_cast<const Elem*>(a.k_cache);
  const Elem* vc = static_cast<const Elem*>(a.v_cache);

  __shared__ float q_s[kGMax][D];
  __shared__ float p_s[kGMax][64];
  __shared__ int64_t vbase_s[64];

  auto piece = [&](int s, int kvh, int L, int tin, int ntile, bool whole, int64_t rec_slot) {
    // Every argument is the same in all lanes; say so, so that addresses
    // built from them stay in scalar registers.
    s = wave_uniform(s);
    kvh = wave_uniform(kvh);
    L = wave_uniform(L);
    tin = wave_uniform(tin);
    ntile = wave_uniform(ntile);
    whole = wave_uniform(int(whole)) != 0;
    rec_slot = wave_uniform64(rec_slot);
    const int t_begin = 16 * tin;
    const int t_end = min(L, 16 * (tin + ntile));
    const int32_t* row = a.block_tables + int64_t(s) * a.max_blocks_per_seq;
    const Elem* qg = static_cast<const Elem*>(a.q) + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
    __syncthreads();
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
        int pb = load_ro(row, t / B);
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

    float* rec = whole ? nullptr : a.ws + rec_slot * record_floats(G, D);
#pragma unroll
    for (int h = 0; h < kGMax; ++h) {
      if (h >= G) continue;
      const float l_tot = wave_sum(l_part[h]);
      if (whole) {
        if (a.lse && lane == 0)  // ln sum e^(scale q.k) = (m + log2 l) ln 2
          a.lse[int64_t(s) * a.num_heads + int64_t(kvh) * G + h] =
              (m_run[h] + __log2f(l_tot)) * 0.6931471805599453f;
        Elem* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G + h) * D;
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[lane + 64 * k] = from_f32<Elem>(acc[h][k] / l_tot);
      } else {
#pragma unroll
        for (int k = 0; k < DPL; ++k) rec[h * D + lane + 64 * k] = acc[h][k];
        if (lane == 0) {
          rec[G * D + h] = m_run[h];
          rec[G * D + G + h] = l_tot;
          if (h == 0) rec[G * D + 2 * G] = __uint_as_float(a.epoch);
        }
      }
    }
  };

  if constexpr (kSplit) {
    walk_slice(a, B, lane, blockIdx.x, piece);
  } else {
    const int kvh = blockIdx.x % a.num_kv_heads;
    const int s = blockIdx.x / a.num_kv_heads;
    const int L = effective_len(a, s, B);
    if (L == 0) {
      Elem* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
      for (int i = lane; i < G * D; i += 64) o[i] = from_f32<Elem>(0.f);
      if (a.lse && lane < G) a.lse[int64_t(s) * a.num_heads + int64_t(kvh) * G + lane] = -INFINITY;
      return;
    }
    piece(s, kvh, L, 0, (L + 15) / 16, true, 0);
  }
}

template <typename Elem, int D>
hipError_t launch_ed(const DecodeArgs& a, int block_size, hipStream_t stream) {
  if (a.split)
    return launch(decode_simt_kernel<Elem, D, true>, dim3(unsigned(a.workers)), dim3(64), 0,
                  stream, a, block_size);
  const dim3 grid(unsigned(int64_t(a.num_seqs) * a.num_kv_heads));
  return launch(decode_simt_kernel<Elem, D, false>, grid, dim3(64), 0, stream, a, block_size);
}

template <typename Elem>
hipError_t launch_elem(const DecodeArgs& a, int head_dim, int block_size, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_ed<Elem, 64>(a, block_size, stream);
    case 128: return launch_ed<Elem, 128>(a, block_size, stream);
    case 256: return launch_ed<Elem, 256>(a, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename Elem>
int workers_elem(int head_dim) {
  switch (head_dim) {
    case 64: return resident_workers(reinterpret_cast<const void*>(decode_simt_kernel<Elem, 64, true>), 64);
    case 128: return resident_workers(reinterpret_cast<const void*>(decode_simt_kernel<Elem, 128, true>), 64);
    case 256: return resident_workers(reinterpret_cast<const void*>(decode_simt_kernel<Elem, 256, true>), 64);
    default: return 0;
  }
}

}  // namespace

hipError_t launch_decode_simt(const DecodeArgs& a, int head_dim, int block_size, bool bf16,
                              hipStream_t stream) {
  return bf16 ? launch_elem<uint16_t>(a, head_dim, block_size, stream)
              : launch_elem<float>(a, head_dim, block_size, stream);
}

int decode_workers_simt(int head_dim, bool bf16) {
  return bf16 ? workers_elem<uint16_t>(head_dim) : workers_elem<float>(head_dim);
}

}  // namespace pa

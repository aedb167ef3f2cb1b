// Paged decode attention for bfloat16 caches on gfx950 matrix cores.
//
// What is computed: for sequence s and query head h, softmax over the L_s
// context tokens of scale * q.k_t, applied to v_t, where token t's K/V are
// read from physical block block_table[s][t / B] at offset t % B and KV head
// h / G.  [P2 "PagedAttention学习笔记", section 2.1 and section 三; P3 "KV cache
// 显存管理", PagedAttention 改变了什么: logical_block = t // B, offset = t % B,
// physical = block_table[logical].]  The online-softmax tiling is the
// FlashAttention technique the pages say composes with paged storage (P2,
// comparison with FlashAttention).
//
// Work decomposition.  One workgroup of 4 waves per (sequence, KV head,
// partition).  The partition's tokens are cut into 16-token tiles; wave w
// takes tiles w, w+4, ...  A tile is the unit of both matrix-core products:
//
//   S^T[16 tok x 16 col] = K_tile[16 tok x D] . Q^T[D x 16 col]  (16x16x32 bf16, D/32 steps)
//   O^T[D x 16 col]     += V^T_tile[D x 16 tok] . P^T[16 tok x 16 col] (16x16x16 bf16, D/16)
//
// where the 16 columns are the G <= 16 query heads sharing the KV head
// (columns >= G hold zero queries and are never stored), so every K/V byte
// is read once per KV head for all G heads.  Operand layouts (lane l, row
// r = l & 15, group k = l >> 4):
//   K operand   lane holds token r, dims 32j + 8k .. +7  -> one 16-byte load
//               per step from the [B][D] K tile;
//   Q operand   lane holds head column r, the same dims;
//   S^T result  lane holds tokens 4k .. 4k+3 of column r;
//   P^T operand lane holds tokens 4k .. 4k+3 of column r -- exactly the S^T
//               result, so the softmax weights never leave the lane;
//   V operand   lane holds dim 16c + r, tokens 4k .. 4k+3 -> one 8-byte load
//               from the token-innermost [D][B] V tile;
//   O^T result  lane holds dims 16c + 4k .. +3 of column r.
// Each 16-byte K load of a wave covers 16 tokens x 64 contiguous bytes and
// each 8-byte V load covers 16 dims x 16 tokens = 512 contiguous bytes.
//
// Softmax runs in the log2 domain (q.k * scale * log2 e) with a lazily
// updated running maximum: the accumulator is rescaled only when a tile's
// maximum exceeds the maximum in use by more than 8 (a factor 256), which
// keeps every weight <= 2^8 and is exact because the final division uses the
// same maximum.  The block-table entry of a tile is wave-uniform and lives in
// a scalar register; K/V addresses are a scalar 64-bit tile base plus a
// per-lane 32-bit offset, so no vector ALU is spent on address arithmetic.
// The next tile's loads are issued before the current tile is consumed.

#include <math.h>

#include "device_common.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct Tile {
  uint4 k[D / 32];
  uint2 v[D / 16];
};

// Physical placement of one 16-token tile for this lane.
struct TilePlace {
  const char* k_base;  // wave-uniform when B >= 16
  const char* v_base;
  bool bad;            // a block id outside [0, num_blocks): results become NaN
};

__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int D, int B>
__device__ __forceinline__ TilePlace place_tile(const DecodeArgs& a, const int32_t* row, int kvh,
                                                int t0, int nblk, int lane) {
  constexpr int64_t kTileBytes = int64_t(B) * D * 2;  // one (block, KV head) tile
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  TilePlace tp;
  if constexpr (B >= kTile) {
    const int lb = t0 / B;
    int pb = row[lb];
    tp.bad = unsigned(pb) >= unsigned(a.num_blocks);
    pb = tp.bad ? 0 : pb;
    const int64_t tile = int64_t(pb) * a.num_kv_heads + kvh;
    const int in_block = t0 % B;  // 0, or 16 when B == 32
    tp.k_base = kc + tile * kTileBytes + int64_t(in_block) * D * 2;
    tp.v_base = vc + tile * kTileBytes + int64_t(in_block) * 2;
  } else {
    // B == 8: the tile spans two blocks; the second may not exist.
    const int lb0 = t0 / B;
    int pb0 = row[lb0];
    int pb1 = (lb0 + 1 < nblk) ? row[lb0 + 1] : pb0;
    const bool bad0 = unsigned(pb0) >= unsigned(a.num_blocks);
    const bool bad1 = unsigned(pb1) >= unsigned(a.num_blocks);
    pb0 = bad0 ? 0 : pb0;
    pb1 = bad1 ? 0 : pb1;
    // K: this lane's token is (lane & 15); V: its tokens are 4*(lane >> 4) ..
    const bool k_second = (lane & 15) >= B;
    const bool v_second = (lane >> 4) >= 2;
    const int64_t tk = int64_t(k_second ? pb1 : pb0) * a.num_kv_heads + kvh;
    const int64_t tv = int64_t(v_second ? pb1 : pb0) * a.num_kv_heads + kvh;
    tp.k_base = kc + tk * kTileBytes - (k_second ? int64_t(B) * D * 2 : 0);
    tp.v_base = vc + tv * kTileBytes - (v_second ? int64_t(B) * 2 : 0);
    tp.bad = (lane >> 4) >= 2 ? bad1 : bad0;  // the S^T rows this lane owns
  }
  return tp;
}

template <int D, int B>
__device__ __forceinline__ void load_tile(Tile<D>& r, const TilePlace& tp, uint32_t k_off,
                                          uint32_t v_off) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    r.k[j] = *reinterpret_cast<const uint4*>(tp.k_base + k_off + 64 * j);
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    r.v[c] = *reinterpret_cast<const uint2*>(tp.v_base + v_off + 32 * B * c);
}

template <int D, int B>
__global__ __launch_bounds__(kThreads) void decode_bf16_mfma_kernel(DecodeArgs a) {
  constexpr int KSTEPS = D / 32;
  constexpr int DCH = D / 16;

  const int bid = blockIdx.x;
  const int p = bid % a.max_partitions;
  const int sg = bid / a.max_partitions;
  const int kvh = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  const int G = a.group;
  const int L = effective_len(a, s, B);
  const int P = a.partition_size;
  const int nparts = (L + P - 1) / P;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  uint16_t* out = static_cast<uint16_t*>(a.out);

  if (L == 0) {
    if (p == 0) {
      uint16_t* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
      for (int i = tid; i < G * D; i += kThreads) o[i] = 0;
    }
    return;
  }
  if (p >= nparts) return;

  const int t_begin = p * P;
  const int t_end = min(L, t_begin + P);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
  const int nblk = (L + B - 1) / B;
  const int32_t* row = a.block_tables + int64_t(s) * a.max_blocks_per_seq;

  // Q^T operand: column col = query head kvh*G + col (zero beyond G).
  bf16x8_t qop[KSTEPS];
  {
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                         (int64_t(s) * a.num_heads + int64_t(kvh) * G + col) * D + 8 * grp;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < G) v = *reinterpret_cast<const uint4*>(qh + 32 * j);
      qop[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Per-lane byte offsets inside a tile.
  const uint32_t k_off = uint32_t(col) * D * 2 + uint32_t(grp) * 16;
  const uint32_t v_off = uint32_t(col) * B * 2 + uint32_t(grp) * 8;

  floatx4_t acc[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) acc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  auto consume = [&](Tile<D>& r, int tile, bool bad) {
    const int t0 = t_begin + tile * kTile;
    const int valid = t_end - t0;  // >= 1
    floatx4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[j]), qop[j],
                                                     sacc, 0, 0, 0);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sacc[i] * a.scale_log2e;
    if (valid < kTile) {  // last, partial tile: drop tokens >= t_end
      const int first = 4 * grp;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (first + i < valid) ? x[i] : -INFINITY;
      const int n = min(max(valid - first, 0), 4);
      const uint32_t mx = (n >= 1 ? 0x0000FFFFu : 0u) | (n >= 2 ? 0xFFFF0000u : 0u);
      const uint32_t my = (n >= 3 ? 0x0000FFFFu : 0u) | (n >= 4 ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        r.v[c].x &= mx;
        r.v[c].y &= my;
      }
    }
    if (bad) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_nanf("");
    }
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (__any(tmax > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < DCH; ++c) acc[c] *= alpha;
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const uint2 pp = make_uint2(pack_bf16x2_rne(pr[0], pr[1]), pack_bf16x2_rne(pr[2], pr[3]));
    const short4_t pop = __builtin_bit_cast(short4_t, pp);
#pragma unroll
    for (int c = 0; c < DCH; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, r.v[c]), pop,
                                                         acc[c], 0, 0, 0);
  };

  // Software pipeline: tile i+4's loads are in flight while tile i is used.
  Tile<D> r0, r1;
  int tile = wave;
  bool bad0 = false, bad1 = false;
  if (tile < ntiles) {
    TilePlace tp = place_tile<D, B>(a, row, kvh, t_begin + tile * kTile, nblk, lane);
    bad0 = tp.bad;
    load_tile<D, B>(r0, tp, k_off, v_off);
  }
  while (tile < ntiles) {
    int next = tile + kWaves;
    if (next < ntiles) {
      TilePlace tp = place_tile<D, B>(a, row, kvh, t_begin + next * kTile, nblk, lane);
      bad1 = tp.bad;
      load_tile<D, B>(r1, tp, k_off, v_off);
    }
    consume(r0, tile, bad0);
    tile = next;
    if (tile >= ntiles) break;
    next = tile + kWaves;
    if (next < ntiles) {
      TilePlace tp = place_tile<D, B>(a, row, kvh, t_begin + next * kTile, nblk, lane);
      bad0 = tp.bad;
      load_tile<D, B>(r0, tp, k_off, v_off);
    }
    consume(r1, tile, bad1);
    tile = next;
  }

  // Wave totals: l over the four row groups of each column.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // Combine the 4 waves in LDS.
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ floatx4_t sm_acc[kWaves][DCH][64];
  if (grp == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_run;
  }
#pragma unroll
  for (int c = 0; c < DCH; ++c) sm_acc[wave][c][lane] = acc[c];
  __syncthreads();

  float M = sm_m[0][col];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][col]);
  float wgt[kWaves];
  float l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm_m[w][col];
    wgt[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    l_tot += wgt[w] * sm_l[w][col];
  }

  const bool single = nparts == 1;
  const int h = kvh * G + col;
  float* rec = nullptr;
  if (!single)
    rec = a.ws + ((int64_t(s) * a.num_kv_heads + kvh) * a.max_partitions + p) * record_floats(G, D);
  if (!single && wave == 0 && grp == 0 && col < G) {
    rec[G * D + col] = M;
    rec[G * D + G + col] = l_tot;
  }
  const float inv_l = 1.0f / l_tot;
  for (int c = wave; c < DCH; c += kWaves) {
    floatx4_t o = wgt[0] * sm_acc[0][c][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) o += wgt[w] * sm_acc[w][c][lane];
    if (col < G) {
      const int d0 = 16 * c + 4 * grp;
      if (single) {
        const uint2 ob = make_uint2(pack_bf16x2_rne(o[0] * inv_l, o[1] * inv_l),
                                    pack_bf16x2_rne(o[2] * inv_l, o[3] * inv_l));
        *reinterpret_cast<uint2*>(out + (int64_t(s) * a.num_heads + h) * D + d0) = ob;
      } else {
        *reinterpret_cast<floatx4_t*>(rec + col * D + d0) = o;
      }
    }
  }
}

template <int D, int B>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  const int64_t grid = int64_t(a.num_seqs) * a.num_kv_heads * a.max_partitions;
  return launch(decode_bf16_mfma_kernel<D, B>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, a);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int block_size, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_one<D, 8>(a, stream);
    case 16: return launch_one<D, 16>(a, stream);
    case 32: return launch_one<D, 32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_bf16_mfma(const DecodeArgs& a, int head_dim, int block_size,
                                   hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(a, block_size, stream);
    case 128: return launch_d<128>(a, block_size, stream);
    case 256: return launch_d<256>(a, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa

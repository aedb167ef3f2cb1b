// Paged prefill / chunked-prefill attention on gfx950.
//
// What is computed: sequence s holds L_s tokens in its paged K/V (token t in
// physical block block_table[s][t / B] at offset t % B -- "PagedAttention学习笔记"
// section 2.1; "KV cache 显存管理", PagedAttention 改变了什么) and brings n_s
// query tokens, its last n_s positions L_s - n_s .. L_s - 1, whose K/V are
// already in the cache (written through their slots first).  Query row i of
// the sequence attends causally: softmax over tokens 0 .. L_s - n_s + i of
// scale * q.k_t, applied to v_t.  A whole prompt is n_s = L_s; a chunk of a
// long prompt, or several tokens verified at once, is n_s < L_s; n_s = 1 is
// the decode step.  The pages' prefill asks for blocks by input length
// ("什么是 PagedAttention？", 映射逻辑块与物理块) and reads history through the
// same table as decode; only the number of query rows differs.
//
// bf16 kernel.  For one (sequence, KV head) the query rows are the pairs
// (position i, head of the group) in order, i * G + head; a wave takes NC
// tiles of 16 of them (64 rows at NC = 4) as the columns of the matrix-core
// tiles
//
//   S^T[16 tok x 16 col] = K_tile[16 tok x D] . Q^T[D x 16 col]   (16x16x32 bf16)
//   O^T[32 dim x 32 col] += V^T_tile[32 dim x 16 tok] . P^T[16 tok x 32 col]
//                                   (32x32x16 bf16, column tiles taken in pairs)
//
// S^T has the operand layout of the decode kernel (lane l: row/column l & 15,
// group l >> 4; K rows are 16-byte loads from the [B][D] tile); P^T of two
// column tiles is rearranged by one lane swap into the 32x32 product's
// operand, whose V^T rows are 16-byte loads from the token-innermost [D][B]
// tile.  Each K/V tile thus feeds NC products of each kind.  Column c sees
// tokens below its own limit lim_c = L - n + i_c + 1; tiles below the
// smallest limit of the wave need no mask.  Block ids are scalar loads
// fetched one tile ahead of the tile loads.  A workgroup is one wave; the
// launch order keeps all row groups of one (sequence, KV head) on one XCD
// (workgroup i runs on XCD i % 8), latest positions first, so the re-reads
// of a tile by other row groups hit that XCD's L2.
//
// fp32 kernel.  One wave per (query row, head): lanes hold D / 64 dims each;
// each token's dot product is reduced across the wave.  It exists for the
// tight-tolerance parity of the causal logic, not for speed.

#include <math.h>

#include "device_common.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 1;  // waves per workgroup: 1, 2, 4 -> 445, 442, 438 us on the chunked layer, 470, 483, 496 on whole 2048-token prompts
constexpr int kTile = 16;
constexpr float kRescale = 8.0f;  // lazy maximum: weights stay <= 2^8
constexpr int kXcds = 8;
// The Q operands of a wave's column tiles (NC x D/32 16-byte pieces per
// lane) wait in LDS, read just before each product, instead of in
// registers: with them resident, accumulators + Q + load ring exceed the
// 256 vector registers and the compiler parks Q in accumulation registers,
// copying it back before every product.
constexpr bool kQInLds = true;
constexpr uint32_t kNanPair = 0x7FC07FC0u;  // two bfloat16 quiet NaNs
// Word 3 of a raw buffer descriptor on gfx9-family parts: 32-bit data
// format, no swizzle (the loads are untyped 16- and 8-byte fetches).
constexpr int kRawWord3 = 0x00020000;

__device__ __forceinline__ uint32_t pack2_rne(float lo, float hi) {
  float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// IEEE maximum (a NaN operand gives NaN).  It maps to one v_maximum3_f32,
// where fmaxf (maxNum, which drops a NaN operand) first quiets each operand
// that is not known to be canonical with an extra v_max_f32 -- every lane
// swap result and matrix-core output here.  Only tile maxima use it: a
// column that sees a NaN logit is NaN through its exponentials either way.
__device__ __forceinline__ float max_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// max / sum of x over the four row groups of an MFMA result column (lanes
// l, l ^ 16, l ^ 32, l ^ 48), via gfx950 lane swaps.
__device__ __forceinline__ float col_max(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nan(__uint_as_float(s[0]), __uint_as_float(s[1]));
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nan(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Sequence s of the launch: clamped length L, its n query rows (positions
// L - n .. L - 1), the first `rows` of them computed (at most max_query_len),
// and the index q0 of its first query row.
struct SeqRows {
  int L, n, rows, q0;
};

__device__ __forceinline__ SeqRows seq_rows(const PrefillArgs& a, int s, int B) {
  SeqRows r;
  int L = load_ro(a.context_lens, s);
  L = L < 0 ? 0 : L;
  L = L > a.max_context_len ? a.max_context_len : L;
  const int cap = a.max_blocks_per_seq * B;
  r.L = L > cap ? cap : L;
  // rows stay inside q / out even if query_start is not a valid prefix sum
  int q0 = load_ro(a.query_start, s);
  q0 = q0 < 0 ? 0 : (q0 > a.num_query_tokens ? a.num_query_tokens : q0);
  int n = load_ro(a.query_start, s + 1) - q0;
  n = n < 0 ? 0 : n;
  r.n = n > a.num_query_tokens - q0 ? a.num_query_tokens - q0 : n;
  r.rows = r.n > a.max_query_len ? a.max_query_len : r.n;
  r.q0 = q0;
  return r;
}

// K as the QK product's operand (lane: token l % 16, dims 32j + 8 (l / 16)
// .. +7); V as the 32 x 32 PV product's operand: lane l holds dim 32b + l %
// 32 and tokens 8 (l / 32) .. +7 of the tile, one 16-byte load per block.
template <int D>
struct KVTile {
  uint4 k[D / 32];
  uint4 v[D / 32];
};

// Loads of the 16-token tile at t0 of KV head kvh (ids of its block(s) in
// pb0 / pb1; pb1 is the second block of a B = 8 tile).  Out-of-range ids
// read block 0, and the K rows of their tokens become NaN, so every logit
// of those tokens and every output that sees them is NaN.
template <int D, int B>
__device__ __forceinline__ void load_kv_tile(KVTile<D>& r, const PrefillArgs& a, int pb0, int pb1,
                                             int kvh, int t0, int lane) {
  constexpr int64_t kTileBytes = int64_t(B) * D * 2;
  const int col = lane & 15, grp = lane >> 4;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const bool bad0 = unsigned(pb0) >= unsigned(a.num_blocks);
  const bool bad1 = unsigned(pb1) >= unsigned(a.num_blocks);
  pb0 = bad0 ? 0 : pb0;
  pb1 = bad1 ? 0 : pb1;
  if constexpr (B >= kTile) {
    // The tile's K and V bases are wave-uniform (one block): scalar buffer
    // descriptors, and each lane adds the same 32-bit offset to every tile,
    // instead of a 64-bit address per lane and load.
    const int in_block = t0 % B;
    const int64_t tile = (int64_t(pb0) * a.num_kv_heads + kvh) * kTileBytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kc + tile + int64_t(in_block) * D * 2), 0, int(kTileBytes), kRawWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vc + tile + in_block * 2), 0, int(kTileBytes), kRawWord3);
    const int k_off = col * D * 2 + grp * 16;
    const int v_off = (lane & 31) * B * 2 + (lane >> 5) * 16;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
      r.k[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off, 64 * j, 0));
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
      r.v[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off, 64 * B * b, 0));
    // A bad block id poisons the tile's K with NaN, so the products carry
    // it into every logit of the tile (rare; the branch is wave-uniform).
    if (__builtin_amdgcn_readfirstlane(int(bad0))) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) r.k[j] = make_uint4(kNanPair, kNanPair, kNanPair, kNanPair);
    }
  } else {
    // K row `col` and V tokens 8 (l / 32) .. +7 (a whole 8-token dim row)
    // come from the tile's first or second block
    const bool k_second = col >= B;
    const bool v_second = (lane >> 5) != 0;
    const int kr = k_second ? col - B : col;
    const char* kb = kc + (int64_t(k_second ? pb1 : pb0) * a.num_kv_heads + kvh) * kTileBytes +
                     int64_t(kr) * D * 2 + grp * 16;
    const char* vb = vc + (int64_t(v_second ? pb1 : pb0) * a.num_kv_heads + kvh) * kTileBytes +
                     int64_t(lane & 31) * B * 2;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) r.k[j] = *reinterpret_cast<const uint4*>(kb + 64 * j);
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
      r.v[b] = *reinterpret_cast<const uint4*>(vb + int64_t(64) * B * b);
    // K row `col` comes from the block of token `col`; a bad id there
    // poisons that token's logits in every column
    if (k_second ? bad1 : bad0) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) r.k[j] = make_uint4(kNanPair, kNanPair, kNanPair, kNanPair);
    }
    (void)v_second;
  }
}

// a for lanes 0-15 and 32-47, b for lanes 16-31 and 48-63.  The empty asm
// hands the compiler two register values, so that the choice stays a lane
// select; picking between two elements of a register array by lane was
// otherwise turned into a load through a lane-dependent address, which put
// the array in scratch memory.
__device__ __forceinline__ float pick_half(int lane, float a, float b) {
  asm("" : "+v"(a), "+v"(b));
  return (lane & 16) ? b : a;
}

// NC: 16-row column tiles per wave (each K/V tile feeds NC products of each
// kind); RING: register tiles in flight (tile k + RING - 1 loads while tile
// k is consumed).
template <int D, int B, int NC, int RING>
__global__ __launch_bounds__(kWaves * 64) void prefill_bf16_mfma_kernel(PrefillArgs a) {
  constexpr int KSTEPS = D / 32;
  constexpr int kWaveRows = kTile * NC;
  const int G = a.group;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  // XCD-aware work index.  Workgroup i runs on XCD i % 8 and is that XCD's
  // j-th, j = i / 8.  The (sequence, KV head) pairs are dealt to the XCDs in
  // turn (pair p to XCD p % 8), and an XCD takes the row groups of its pairs
  // one pair after another: every row group of a pair reads the pair's tiles
  // through one L2, and the XCDs' shares are alike whatever the sequences'
  // lengths (with 8 KV heads, XCD x takes KV head x of every sequence).
  // Longest first: when an XCD holds at most 64 pairs, its k-th pair is the
  // one of rank k by context length (descending, ties by index), so the
  // longest waves start first and short ones fill the end.  Every workgroup
  // ranks the same lengths, so each pair is taken exactly once.
  const int xcd = blockIdx.x % kXcds;
  const int j = blockIdx.x / kXcds;
  const int pairs = a.num_seqs * a.num_kv_heads;
  const int k = j / a.row_groups;                         // slot among the XCD's pairs
  const int px = (pairs - xcd + kXcds - 1) / kXcds;       // pairs on this XCD
  if (k >= px) return;
  int pair = xcd + kXcds * k;
  if (px <= 64) {
    const int mine = xcd + kXcds * min(lane, px - 1);
    const int key = load_ro(a.context_lens, mine / a.num_kv_heads);
    int rank = 0;
    for (int m = 0; m < px; ++m) {
      const int km = __builtin_amdgcn_readlane(key, m);
      rank += (km > key || (km == key && m < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < px && rank == k);
    if (hit) pair = xcd + kXcds * int(__builtin_ctzll(hit));
  }
  const int rg = a.row_groups - 1 - j % a.row_groups;  // latest positions first
  const int kvh = pair % a.num_kv_heads;
  const int s = pair / a.num_kv_heads;
  const SeqRows sr = seq_rows(a, s, B);
  const int L = wave_uniform(sr.L), n = wave_uniform(sr.n), q0 = wave_uniform(sr.q0);
  const int nrows = wave_uniform(sr.rows) * G;
  const int r0 = (rg * kWaves + wave) * kWaveRows;  // first row of this wave
  if (r0 >= nrows) return;                           // wave-uniform: no barrier below
  const int r_last = min(r0 + kWaveRows, nrows) - 1;
  // visible-token limits: row r (position i = r / G) sees tokens
  // [0, L - n + i + 1); the wave's range and its unmasked prefix
  const int base = L - n + 1;
  const int t_end = min(L, max(base + r_last / G, 0));
  const int lim_min = max(base + r0 / G, 0);
  int lim[NC], qi[NC], qh[NC];
  bool col_ok[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int row = r0 + c * kTile + col;
    col_ok[c] = row < nrows;
    lim[c] = col_ok[c] ? max(base + row / G, 0) : 0;
    qi[c] = row / G;
    qh[c] = kvh * G + row % G;
  }

  // O^T accumulators of the 32 x 32 PV products: column pair p holds column
  // tiles 2p and 2p + 1; lane l's column is tile 2p + (l / 16) % 2, row
  // l % 16; element e is dim 32b + 8 (e / 4) + 4 (l / 32) + e % 4.
  static_assert(NC % 2 == 0, "column tiles go in pairs");
  floatx16_t acc[NC / 2][D / 32];
  // m_run: the maximum in use (of c q.k, c = |scale| log2 e, see cpos).  Kept beside
  // it, since they change only when m_run does: neg_m = -m_run, or 0 while
  // the column has seen nothing (m_run = -inf), the exponent's offset; and
  // thr = (m_run + kRescale) / c, the raw q.k a tile's maximum must exceed
  // for a rescale.
  float m_run[NC], l_run[NC], neg_m[NC], thr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
      if (c < NC / 2) acc[c][b] = floatx16_t{};
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
    neg_m[c] = 0.f;
    thr[c] = -INFINITY;
  }

  if (t_end > 0) {
    // c = |scale| log2 e; for a negative scale the sign goes into q (exact:
    // a sign-bit flip of each bf16 element)
    // Masked logits are -inf and meet c in the exponent's fused multiply-add,
    // so c is kept at least FLT_MIN: a zero scale would give -inf * 0 = NaN.
    // At |scale log2 e| < FLT_MIN every weight is then 2^(q.k FLT_MIN - m)
    // instead of 2^(q.k scale log2 e - m), both 1 to fp32 precision.
    const float cpos = fmaxf(fabsf(a.scale_log2e), 1.17549435e-38f);
    const float inv_c = 1.0f / cpos;
    const uint32_t qsign = a.scale_log2e < 0.f ? 0x80008000u : 0u;
    __shared__ __align__(16) u32x4_t q_lds[kQInLds ? kWaves * NC * KSTEPS * 64 : 1];
    bf16x8_t qop[kQInLds ? 1 : NC][KSTEPS];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           (int64_t(q0 + qi[c]) * a.num_heads + qh[c]) * D + 8 * grp;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (col_ok[c]) v = *reinterpret_cast<const uint4*>(qp + 32 * j);
        v.x ^= qsign;
        v.y ^= qsign;
        v.z ^= qsign;
        v.w ^= qsign;
        if constexpr (kQInLds)
          q_lds[((wave * NC + c) * KSTEPS + j) * 64 + lane] = u32x4_t{v.x, v.y, v.z, v.w};
        else
          qop[c][j] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    const int32_t* trow = a.block_tables + int64_t(s) * a.max_blocks_per_seq;
    const int nblk = (L + B - 1) / B;
    const int ntile = (t_end + kTile - 1) / kTile;
    const int last = ntile - 1;

    // Q^T operand of column tile c, step j.  The LDS read is volatile so that
    // it stays in the loop, next to its product, instead of being hoisted
    // out of it into registers.
    auto q_operand = [&](int c, int j) -> bf16x8_t {
      if constexpr (kQInLds) {
        typedef __attribute__((address_space(3))) const volatile u32x4_t lds_q_t;
        const lds_q_t* p =
            (const lds_q_t*)(&q_lds[((wave * NC + c) * KSTEPS + j) * 64 + lane]);
        return __builtin_bit_cast(bf16x8_t, u32x4_t(*p));
      } else {
        return qop[c][j];
      }
    };

    auto consume = [&](KVTile<D>& r, int k) {
      const int t0 = k * kTile;
      const int tb = t0 + 4 * grp;
      if (t0 + kTile > t_end) {  // tokens past the wave's range may be unused slots
        const int nv = min(max(t_end - (t0 + 8 * (lane >> 5)), 0), 8);  // this lane's V tokens
        uint32_t m4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          m4[q] = (nv > 2 * q ? 0x0000FFFFu : 0u) | (nv > 2 * q + 1 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          r.v[b].x &= m4[0];
          r.v[b].y &= m4[1];
          r.v[b].z &= m4[2];
          r.v[b].w &= m4[3];
        }
      }
      // wave-uniform: a scalar branch skips the masks on interior tiles
      const bool edge = __builtin_amdgcn_readfirstlane(int(t0 + kTile > lim_min)) != 0;
      // The NC column tiles are independent; each phase runs over all of them
      // so that their products and softmax chains interleave in one basic
      // block (a branch per column tile would fence each chain off).
      floatx4_t sacc[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[j]),
                                                            q_operand(c, j), sacc[c], 0, 0, 0);
      }
      // raw q.k (q's sign carries the sign of the scale, so the scale
      // factor c = |scale| log2 e is positive and max(c x) = c max(x)); the
      // factor is applied inside the exponent's fused multiply-add
      float x[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[c][i] = sacc[c][i];
      if (edge) {  // causal edge (and the tail): per-column limit
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[c][i] = tb + i < lim[c] ? x[c][i] : -INFINITY;
      }
      float tmax[NC];  // raw q.k
      bool grow = false;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        tmax[c] = col_max(max_nan(max_nan(x[c][0], x[c][1]), max_nan(x[c][2], x[c][3])));
        grow |= tmax[c] > thr[c];
      }
      if (__any(grow)) {  // rare: one branch for all column tiles
        float alpha[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float m_new = fmaxf(m_run[c], tmax[c] * cpos);
          alpha[c] = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[c] - m_new);
          l_run[c] *= alpha[c];
          m_run[c] = m_new;
          neg_m[c] = m_new == -INFINITY ? 0.f : -m_new;
          thr[c] = (m_new + kRescale) * inv_c;
        }
#pragma unroll
        for (int p = 0; p < NC / 2; ++p) {
          const float al = pick_half(lane, alpha[2 * p], alpha[2 * p + 1]);
#pragma unroll
          for (int b = 0; b < D / 32; ++b) acc[p][b] *= al;
        }
      }
      short4_t pop[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[c][i], cpos, neg_m[c]));
        l_run[c] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        pop[c] = __builtin_bit_cast(short4_t,
                                    make_uint2(pack2_rne(pr[0], pr[1]), pack2_rne(pr[2], pr[3])));
      }
      // P^T of column tiles 2p, 2p + 1 as the 32 x 32 product's operand:
      // lane l needs tokens 8 (l / 32) .. +7 of its column, which sit in
      // lanes l and l + 16 (first tile) or l - 16 and l (second tile); one
      // lane swap between 16-lane rows per 32-bit word brings them there.
#pragma unroll
      for (int p = 0; p < NC / 2; ++p) {
        const uint2 pa = __builtin_bit_cast(uint2, pop[2 * p]);
        const uint2 pb = __builtin_bit_cast(uint2, pop[2 * p + 1]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(pa.x, pb.x, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(pa.y, pb.y, false, false);
        const bf16x8_t pp = __builtin_bit_cast(bf16x8_t, u32x4_t{s0[0], s1[0], s0[1], s1[1]});
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
          acc[p][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, r.v[b]), pp,
                                                              acc[p][b], 0, 0, 0);
      }
    };

    // Ring of RING register tiles; every load is issued unconditionally (the
    // index clamped to the last tile) so each wait covers exactly the loads
    // before it.
    KVTile<D> ring[RING];
    // Block ids are scalar loads fetched one issue ahead: a tile's vector
    // loads then wait only for its own ids (the scalar counter), never for
    // the tiles still in flight (a vector-register table window would make
    // every issue wait for all outstanding vector loads).
    auto fetch_ids = [&](int k, int& p0, int& p1) {
      k = wave_uniform(min(k, last));  // a scalar index: a scalar load
      const int lb = k * kTile / B;
      p0 = load_ro(trow, lb);
      p1 = p0;
      if constexpr (B < kTile) p1 = lb + 1 < nblk ? load_ro(trow, lb + 1) : p0;
    };
    int next0, next1;
    fetch_ids(0, next0, next1);
    auto issue = [&](KVTile<D>& r, int k) {
      const int pb0 = wave_uniform(next0), pb1 = wave_uniform(next1);
      load_kv_tile<D, B>(r, a, pb0, pb1, kvh, min(k, last) * kTile, lane);
      fetch_ids(k + 1, next0, next1);
    };
#pragma unroll
    for (int d = 0; d < RING - 1; ++d) issue(ring[d], d);
    for (int k = 0; k < ntile; k += RING) {
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        issue(ring[(d + RING - 1) % RING], k + d + RING - 1);
        if (k + d < ntile) consume(ring[d], k + d);
      }
    }
  }

  float l_tot[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) l_tot[c] = col_sum(l_run[c]);
  // lane l writes row r0 + 32p + l % 32 (column tile 2p + (l / 16) % 2),
  // dims 32b + 8i + 4 (l / 32) .. +3
#pragma unroll
  for (int p = 0; p < NC / 2; ++p) {
    const float lt = pick_half(lane, l_tot[2 * p], l_tot[2 * p + 1]);
    const float mr = pick_half(lane, m_run[2 * p], m_run[2 * p + 1]);
    const int row = r0 + 32 * p + (lane & 31);
    if (row < nrows) {
      const int64_t orow = int64_t(q0 + row / G) * a.num_heads + kvh * G + row % G;
      if (a.lse && lane < 32)
        // ln sum_t e^(scale q.k_t) = (m + log2 l) ln 2, m and l in the log2 domain;
        // -inf for a row that sees no token (l == 0), NaN for a row poisoned
        // by a bad block id (l is NaN), so a merge of ranks propagates it
        a.lse[orow] = lt > 0.f ? (mr + __log2f(lt)) * 0.6931471805599453f
                               : (lt == 0.f ? -INFINITY : __builtin_nanf(""));
      const float inv_l = lt > 0.f ? 1.0f / lt : 0.f;  // a row that sees no token: zeros
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow * D + 4 * (lane >> 5);
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint2*>(o + 32 * b + 8 * i) =
              make_uint2(pack2_rne(acc[p][b][4 * i] * inv_l, acc[p][b][4 * i + 1] * inv_l),
                         pack2_rne(acc[p][b][4 * i + 2] * inv_l, acc[p][b][4 * i + 3] * inv_l));
    }
  }
}

// fp32: one wave per (query row, query head), grid over all rows.
template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a, int B) {
  constexpr int E = D / 64;  // dims per lane: lane + 64 e
  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int i = blockIdx.x;
  const SeqRows sr = seq_rows(a, s, B);
  if (i >= sr.rows) return;
  const int kvh = h / a.group;
  const int lim = min(max(sr.L - sr.n + i + 1, 0), sr.L);
  const float* qp = static_cast<const float*>(a.q) + (int64_t(sr.q0 + i) * a.num_heads + h) * D;
  float q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = qp[lane + 64 * e];
    acc[e] = 0.f;
  }
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* trow = a.block_tables + int64_t(s) * a.max_blocks_per_seq;
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < lim; ++t) {
    int pb = load_ro(trow, t / B);
    const bool bad = unsigned(pb) >= unsigned(a.num_blocks);
    pb = bad ? 0 : pb;
    const int off = t % B;
    const int64_t tile = (int64_t(pb) * a.num_kv_heads + kvh) * B * D;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) dot += q[e] * kc[tile + int64_t(off) * D + lane + 64 * e];
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) dot += __shfl_xor(dot, sh);
    float x = bad ? __builtin_nanf("") : dot * a.scale;
    const float m_new = fmaxf(m, x);
    const float alpha = m_new == -INFINITY ? 1.f : expf(m - m_new);
    const float p = expf(x - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e)
      acc[e] = acc[e] * alpha + p * vc[tile + int64_t(lane + 64 * e) * B + off];
    m = m_new;
  }
  float* o = static_cast<float*>(a.out) + (int64_t(sr.q0 + i) * a.num_heads + h) * D;
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  if (a.lse && lane == 0)
    a.lse[int64_t(sr.q0 + i) * a.num_heads + h] =
        l > 0.f ? m + logf(l) : (l == 0.f ? -INFINITY : __builtin_nanf(""));  // NaN: bad block id
#pragma unroll
  for (int e = 0; e < E; ++e) o[lane + 64 * e] = acc[e] * inv_l;
}

// Column tiles per wave of the bf16 kernel for head_dim D (the larger D, the
// more registers a column tile holds).  Measured on the 16-sequence,
// 512-token-chunk layer at D = 128 (accumulators in VGPRs, see build.py):
// 1 tile per wave ~2.0 ms, 2 tiles 1.04-1.08 ms (also at two waves per SIMD),
// 4 tiles 0.82-0.85 ms.  Two register tiles in the load ring: with Q in LDS
// the kernel then needs 246 vector registers and no accumulation registers,
// so two waves share each SIMD (446 us on that layer, against 645 with a
// third ring tile, 282 registers, one wave per SIMD, and 511 with Q in
// registers and three ring tiles).
template <int D>
constexpr int prefill_nc() { return D >= 256 ? 2 : 4; }
constexpr int kPrefillRing = 2;

template <int D>
hipError_t launch_bf16_d(PrefillArgs a, int block_size, hipStream_t stream) {
  constexpr int NC = prefill_nc<D>();
  constexpr int RING = kPrefillRing;
  const int64_t pairs = int64_t(a.num_seqs) * a.num_kv_heads;
  const int64_t groups = (pairs + kXcds - 1) / kXcds * kXcds * a.row_groups;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid{unsigned(groups)}, block{unsigned(kWaves * 64)};
  switch (block_size) {
    case 8: return launch(prefill_bf16_mfma_kernel<D, 8, NC, RING>, grid, block, 0, stream, a);
    case 16: return launch(prefill_bf16_mfma_kernel<D, 16, NC, RING>, grid, block, 0, stream, a);
    case 32: return launch(prefill_bf16_mfma_kernel<D, 32, NC, RING>, grid, block, 0, stream, a);
    default: return hipErrorInvalidValue;
  }
}

// Rows of one workgroup of the bf16 kernel.
int prefill_group_rows(int head_dim) {
  switch (head_dim) {
    case 64: return kWaves * kTile * prefill_nc<64>();
    case 128: return kWaves * kTile * prefill_nc<128>();
    default: return kWaves * kTile * prefill_nc<256>();
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a0, int head_dim, int block_size, bool bf16,
                          hipStream_t stream) {
  PrefillArgs a = a0;
  if (bf16) {
    const int64_t rows = prefill_group_rows(head_dim);
    a.row_groups = int32_t((int64_t(a.max_query_len) * a.group + rows - 1) / rows);
    switch (head_dim) {
      case 64: return launch_bf16_d<64>(a, block_size, stream);
      case 128: return launch_bf16_d<128>(a, block_size, stream);
      case 256: return launch_bf16_d<256>(a, block_size, stream);
      default: return hipErrorInvalidValue;
    }
  }
  const dim3 grid(unsigned(a.max_query_len), unsigned(a.num_heads), unsigned(a.num_seqs));
  switch (head_dim) {
    case 64: return launch(prefill_f32_kernel<64>, grid, dim3(64), 0, stream, a, block_size);
    case 128: return launch(prefill_f32_kernel<128>, grid, dim3(64), 0, stream, a, block_size);
    case 256: return launch(prefill_f32_kernel<256>, grid, dim3(64), 0, stream, a, block_size);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa

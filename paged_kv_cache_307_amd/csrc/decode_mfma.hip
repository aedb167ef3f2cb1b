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
// Work decomposition.  Each (sequence, KV head) pair's tokens are cut into
// 16-token tiles.  Split launches run a fixed set of single-wave workers
// that share the tiles of all pairs equally (schedule.h); each streams its
// share pair by pair and leaves log-sum-exp records for the merge.  Single
// pass runs one wave per pair.  A tile is the unit of both matrix-core
// products:
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
// same maximum.  A run's block-table entries are staged 64 at a time in a
// vector register (one load per window, the next window loaded a window
// ahead); a tile's entry is read from it into a scalar register.  K/V
// addresses are a scalar 64-bit tile base plus a per-lane 32-bit offset, so
// no vector ALU is spent on address arithmetic.
// The next tile's loads are issued before the current tile is consumed, also
// across partition ends, where a split run writes a record and goes on.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "schedule.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 64;  // one wave per worker
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;
constexpr int kRing = 2;  // register tiles in the load ring

template <int D>
struct Tile {
  uint4 k[D / 32];
  uint2 v[D / 16];
  uint2 v2[D / 16];  // B = 32, a block's first tile: the second tile's V (see load_tile_b32)
  bool bad;  // a block id outside [0, num_blocks): the tile's results become NaN
};

// Physical block ids of one tile (wave-uniform scalars).  A tile is one
// block when B >= 16 and two consecutive blocks when B == 8.
struct TileIds {
  int pb0;
  int pb1;
};

// Block-table window: lane i holds the table entry of logical block b0 + i
// (clamped to the sequence's last block, so every read stays in its row).
// One vector load fetches the ids of up to 64 blocks; tiles then take their
// ids from it with a lane read, off the memory path.
__device__ __forceinline__ int load_window(const int32_t* row, int b0, int nblk, int lane) {
  return row[min(b0 + lane, nblk - 1)];
}

// Tiles one window serves: their blocks must fit in 64 entries (with B = 32
// a tile run may start in the middle of a block, costing one entry).
template <int B>
constexpr int window_tiles() {
  return B < kTile ? 64 * B / kTile : (B == kTile ? 64 : 63 * B / kTile);
}

// Ids of the tile starting at token t0 from the window based at block wb.
template <int B>
__device__ __forceinline__ TileIds window_ids(int win, int wb, int t0, int nblk) {
  const int lb = t0 / B;
  TileIds id;
  id.pb0 = __builtin_amdgcn_readlane(win, lb - wb);
  if constexpr (B < kTile) {
    id.pb1 = (lb + 1 < nblk) ? __builtin_amdgcn_readlane(win, lb + 1 - wb) : id.pb0;
  } else {
    id.pb1 = id.pb0;
  }
  return id;
}

__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Word 3 of a raw buffer descriptor on gfx9-family parts: 32-bit data
// format, no swizzle; the loads below are untyped 16- and 8-byte fetches.
constexpr int kRawBufferWord3 = 0x00020000;

// Cache-policy operand of the tile loads.  When every block is read once per
// launch, the tiles are streamed with the nontemporal (nt) bit: on MI355X
// this raises the rate of the decode's random 4 KiB tile reads from ~5.7 to
// ~6.4 TB/s.  When blocks are shared between sequences the default policy
// keeps them in the caches for their other readers.  With B = 32 a 16-token
// V tile in token order covers half of each 128-byte line and the next tile
// reads the other half from the L2, so such tiles (grouped launches) keep
// the default policy; plain runs number a block's two tiles so that one
// load fetches whole V lines (load_tile_b32), and stream them.
constexpr int kStreamOnce = 2;

template <int B, bool kStream>
constexpr int tile_policy() { return kStream && B <= 16 ? kStreamOnce : 0; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kRawBufferWord3);
}

// Issue the loads of one tile.  B >= 16: the tile lies in one block; its K
// and V bases are scalars and each lane adds a fixed 32-bit offset (buffer
// loads, bounds-checked against the tile).  B == 8: each lane picks the
// block its rows fall in and uses a 64-bit address.
template <int D, int B, bool kStream>
__device__ __forceinline__ void load_tile(Tile<D>& r, const DecodeArgs& a, const TileIds& id,
                                          int kvh, int t0, int lane, uint32_t k_off,
                                          uint32_t v_off) {
  constexpr int kTileBytes = B * D * 2;  // one (block, KV head) tile of K or of V
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  if constexpr (B >= kTile) {
    const bool bad = unsigned(id.pb0) >= unsigned(a.num_blocks);
    const int pb = bad ? 0 : id.pb0;
    const int64_t tile = (int64_t(pb) * a.num_kv_heads + kvh) * kTileBytes;
    const int in_block = t0 % B;  // 0, or 16 when B == 32
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + tile + in_block * D * 2, kTileBytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + tile + in_block * 2, kTileBytes);
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
      r.k[j] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off, 64 * j, tile_policy<B, kStream>()));
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      r.v[c] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, 32 * B * c, tile_policy<B, kStream>()));
    r.bad = bad;
  } else {
    const bool bad0 = unsigned(id.pb0) >= unsigned(a.num_blocks);
    const bool bad1 = unsigned(id.pb1) >= unsigned(a.num_blocks);
    const int pb0 = bad0 ? 0 : id.pb0;
    const int pb1 = bad1 ? 0 : id.pb1;
    // K: this lane's token is (lane & 15); V: its tokens are 4*(lane >> 4) ..
    const bool k_second = (lane & 15) >= B;
    const bool v_second = (lane >> 4) >= 2;
    const int64_t tk = (int64_t(k_second ? pb1 : pb0) * a.num_kv_heads + kvh) * kTileBytes;
    const int64_t tv = (int64_t(v_second ? pb1 : pb0) * a.num_kv_heads + kvh) * kTileBytes;
    const char* kb = kc + tk - (k_second ? B * D * 2 : 0) + k_off;
    const char* vb = vc + tv - (v_second ? B * 2 : 0) + v_off;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(kb + 64 * j);
      const u32x4_t t = kStream ? __builtin_nontemporal_load(p) : *p;
      r.k[j] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x2_t* p = reinterpret_cast<const u32x2_t*>(vb + 32 * B * c);
      const u32x2_t t = kStream ? __builtin_nontemporal_load(p) : *p;
      r.v[c] = make_uint2(t.x, t.y);
    }
    r.bad = v_second ? bad1 : bad0;  // the S^T rows this lane owns
  }
}

// B = 32 in plain runs: the two 16-token tiles of a block whose tokens span
// both halves (32 blk + 16 < L) take the tokens {0-3, 8-11, 16-19, 24-27}
// and {4-7, 12-15, 20-23, 28-31} of the block, in that order (a matrix
// product sums over its k index in any order, as long as P^T and V^T agree;
// the masks and the appended row follow the same numbering).  Row r of the
// first tile is block token 8 (r / 4) + r % 4, of the second that + 4, so
// lane group g's V tokens of both tiles, 8g .. 8g + 7, are one 16-byte piece
// of each dim row: the first tile's load fetches whole 64-byte dim rows
// (whole 128-byte lines), keeping the second tile's half in v2, and the
// second tile loads only its K rows.  A last block of at most 16 tokens is
// one tile in plain order.  What a load site fetches of V is fixed at
// compile time (the run's parity fixes which tiles come where), so each
// wait covers exactly the loads it needs.
enum VLoad { kVWide = 0, kVHalf = 1, kVNone = 2 };

template <int D, int kV, bool kStream>
__device__ __forceinline__ void load_tile_b32(Tile<D>& r, const DecodeArgs& a, const TileIds& id,
                                              int kvh, int t0, int L, int lane, uint32_t k_off,
                                              uint32_t k_off_pair) {
  constexpr int B = 32;
  constexpr int kTileBytes = B * D * 2;
  constexpr int kPol = kStream ? kStreamOnce : 0;
  const int col = lane & 15, grp = lane >> 4;
  const bool bad = unsigned(id.pb0) >= unsigned(a.num_blocks);
  const int pb = bad ? 0 : id.pb0;
  const int64_t tile = (int64_t(pb) * a.num_kv_heads + kvh) * kTileBytes;
  const int blk0 = t0 & ~(B - 1);
  const int half = (t0 / kTile) & 1;
  const bool paired = blk0 + kTile < L;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const __amdgpu_buffer_rsrc_t rk =
      tile_rsrc(kc + tile + (paired ? half * 4 * D * 2 : half * kTile * D * 2), kTileBytes);
  const uint32_t ko = paired ? k_off_pair : k_off;
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    r.k[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 64 * j, kPol));
  if constexpr (kV != kVNone) {
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + tile, kTileBytes);
    const uint32_t vrow = uint32_t(col) * B * 2;
    if constexpr (kV == kVWide) {
      // paired: tokens 8g .. 8g + 7; a one-tile block: tokens 4g .. 4g + 3 (low half)
      const uint32_t vo = vrow + uint32_t(grp) * (paired ? 16 : 8);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4_t t = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 32 * B * c, kPol));
        r.v[c] = make_uint2(t.x, t.y);
        r.v2[c] = make_uint2(t.z, t.w);
      }
    } else {  // a block's second tile on its own (its run starts there)
      const uint32_t vo = vrow + uint32_t(grp) * 16 + 8;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        r.v[c] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, vo, 32 * B * c, kPol));
    }
  }
  r.bad = bad;
}

// IEEE maximum (a NaN operand gives NaN): one v_maximum3_f32, where fmaxf
// first quiets every operand not known to be canonical (lane swap results,
// matrix-core outputs) with an extra v_max_f32.  Only tile maxima use it; a
// column with a NaN logit is NaN through its exponentials either way.
__device__ __forceinline__ float max_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// x and its values in lanes l ^ 16, l ^ 32, l ^ 48 (the four row groups of
// an MFMA result column), combined with max or +, via gfx950 lane swaps.
__device__ __forceinline__ float colmax4(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nan(__uint_as_float(s[0]), __uint_as_float(s[1]));
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nan(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float colsum4(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Appending decode: the step's own K/V row (token L - 1) of a (sequence, KV
// head) is read from the caller's key/value arrays and held spread over the
// wave, E = kRowElems dims per lane (lane m holds dims [mE, mE + E)).
template <int D>
struct NewRow {
  static constexpr int kElems = D >= 256 ? 4 : 2;  // dims per lane
  static constexpr int kDwords = kElems / 2;
  static constexpr int kLanes = D / kElems;        // lanes holding data
  uint32_t k[kDwords];
  uint32_t v[kDwords];
};

template <int D>
__device__ __forceinline__ NewRow<D> load_new_row(const DecodeArgs& a, int s, int kvh, int lane) {
  NewRow<D> nr;
  const int64_t row = (int64_t(s) * a.num_kv_heads + kvh) * (D / 2);  // in dwords
  const int m = min(lane, NewRow<D>::kLanes - 1);
  const uint32_t* kr = static_cast<const uint32_t*>(a.new_k) + row + m * NewRow<D>::kDwords;
  const uint32_t* vr = static_cast<const uint32_t*>(a.new_v) + row + m * NewRow<D>::kDwords;
#pragma unroll
  for (int i = 0; i < NewRow<D>::kDwords; ++i) {
    nr.k[i] = kr[i];
    nr.v[i] = vr[i];
  }
  return nr;
}

// Stage the new row in the wave's LDS buffer (K row, then V row).
template <int D>
__device__ __forceinline__ void stage_new_row(const NewRow<D>& nr, uint32_t* lds, int lane) {
  if (lane < NewRow<D>::kLanes) {
#pragma unroll
    for (int i = 0; i < NewRow<D>::kDwords; ++i) {
      lds[lane * NewRow<D>::kDwords + i] = nr.k[i];
      lds[D / 2 + lane * NewRow<D>::kDwords + i] = nr.v[i];
    }
  }
  __syncthreads();  // one wave: orders the LDS writes before later reads
}

// Put the staged row into the operand registers of the tile holding token
// rt (0..15 within the tile): the K operand lanes of row rt read their
// 16-byte chunks straight into place, and the V operand lanes holding token
// rt insert one value per dim chunk.
template <int D>
__device__ __forceinline__ void put_new_row(Tile<D>& r, const uint32_t* lds, int rt, int col,
                                            int grp) {
  const uint16_t* kl = reinterpret_cast<const uint16_t*>(lds);
  const uint16_t* vl = kl + D;
  if (col == rt) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) r.k[j] = *reinterpret_cast<const uint4*>(kl + 32 * j + 8 * grp);
  }
  if (grp == rt / 4) {
    const int half = 16 * (rt % 2);
    const uint32_t keep = ~(0xFFFFu << half);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const uint32_t val = vl[16 * c + col];
      if (rt % 4 < 2)
        r.v[c].x = (r.v[c].x & keep) | (val << half);
      else
        r.v[c].y = (r.v[c].y & keep) | (val << half);
    }
  }
}

// Appending decode: write the tile holding the step's token back to the
// cache once the token's row is in its registers (before the tile is masked
// for consumption): the token's K row from the lanes of row rt, and the
// tile's V rows whole, every lane's 8 bytes, the other tokens' values being
// the ones just read.  The token's V column thus leaves as full 32-byte row
// segments (2 KiB of 4 KiB tile rows at D = 128) instead of D two-byte
// stores at a 32-byte stride, each of which HBM has to merge into its
// sector.  Only lanes whose rows lie in the token's block pb store (a B = 8
// tile spans two blocks).  Only this wave touches that block in this launch.
template <int D, int B>
__device__ __forceinline__ void store_tile_back(const Tile<D>& r, const DecodeArgs& a, int pb,
                                                int kvh, int t0, int rt, int lane,
                                                uint32_t k_off, uint32_t v_off,
                                                bool paired = false) {
  constexpr int kTileBytes = B * D * 2;
  // the pools are writable when a row is appended (the API takes them non-const)
  char* kc = static_cast<char*>(const_cast<void*>(a.k_cache));
  char* vc = static_cast<char*>(const_cast<void*>(a.v_cache));
  const int64_t tile = (int64_t(pb) * a.num_kv_heads + kvh) * kTileBytes;
  const int col = lane & 15;
  const int grp = lane >> 4;
  bool v_here = true;
  int64_t k_shift = 0, v_shift = 0;
  if constexpr (B == 32) {
    const int half = (t0 / kTile) & 1;
    if (paired) {  // the numbering of load_tile_b32: row rt is block token 8 (rt / 4) + rt % 4 + 4 half
      k_shift = (int64_t(8 * (rt / 4) + rt % 4 + 4 * half) - rt) * D * 2;  // from row rt (k_off)
      v_shift = int64_t(grp) * 8 + half * 8;                              // 16 g + 8 half from 8 g (v_off)
    } else {
      k_shift = half * kTile * D * 2;
      v_shift = half * kTile * 2;
    }
  } else if constexpr (B >= kTile) {
    const int in_block = t0 % B;  // 0
    k_shift = in_block * D * 2;
    v_shift = in_block * 2;
  } else {  // the tile's second block holds tokens B .. 15
    const bool second = rt >= B;
    k_shift = second ? -int64_t(B) * D * 2 : 0;
    v_shift = second ? -int64_t(B) * 2 : 0;
    v_here = (grp >= 2) == second;
  }
  if (col == rt) {
    char* kb = kc + tile + k_shift + k_off;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) *reinterpret_cast<uint4*>(kb + 64 * j) = r.k[j];
  }
  if (v_here) {
    char* vb = vc + tile + v_shift + v_off;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) *reinterpret_cast<uint2*>(vb + 32 * B * c) = r.v[c];
  }
}

// Column tiles of a prefix run: 64 query columns (members x heads) at
// D <= 128, 32 at D = 256 (their accumulators take D/4 registers each).
template <int D>
constexpr int prefix_col_tiles() { return D <= 128 ? 4 : 2; }

// A prefix run: tiles [tin, tin + ntile) of a group's shared tokens, for KV
// head kvh and the query heads of all the group's served members at once.
// [P1 共享但不污染状态 and P2 section 2.1: branches of one prompt reference the
// same physical blocks for their common tokens.]  The shared blocks are read
// once, through the first member's table, and feed NC column tiles:
//
//   S^T[16 tok x 16 col] = K_tile . Q^T     per column tile (16x16x32 bf16)
//   O^T[D x 16 col]     += V^T_tile . P^T   per column tile (16x16x16 bf16)
//
// column c = 16 * ct + (lane & 15) is member c / G, query head c % G of the
// KV head.  Each column stops at its member's own length (a member shorter
// than the shared run reads only its tokens).  At the end the run's state is
// one record per member (o, m, l in the record format of the tail runs) in
// wide slot `wide`.
template <int D, int B, bool kStream>
__device__ __forceinline__ void run_prefix(const DecodeArgs& a, GroupInfo gi, int kvh, int tin,
                                        int ntile, int64_t wide, int lane, uint32_t k_off,
                                        uint32_t v_off) {
  constexpr int NC = prefix_col_tiles<D>();
  constexpr int KSTEPS = D / 32;
  constexpr int DCH = D / 16;
  const int G = a.group;
  const int col = lane & 15;
  const int grp = lane >> 4;
  gi.first = wave_uniform(gi.first);
  gi.members = wave_uniform(gi.members);
  gi.plen = wave_uniform(gi.plen);
  kvh = wave_uniform(kvh);
  tin = wave_uniform(tin);
  ntile = wave_uniform(ntile);
  wide = wave_uniform64(wide);
  const int ncols = gi.members * G;
  const int t_begin = tin * kTile;
  const int nblk = (gi.plen + B - 1) / B;
  const int32_t* row = a.block_tables + int64_t(gi.first) * a.max_blocks_per_seq;

  // Q^T operands and column limits.  Columns past the members hold zero
  // queries and the run's length (never stored).
  bf16x8_t qop[NC][KSTEPS];
  int lim[NC];
  int lane_min = gi.plen;
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const int c = ct * 16 + col;
    const bool used = c < ncols;
    const int m = used ? c / G : 0;
    const int hh = used ? c - m * G : 0;
    const int s = gi.first + m;
    lim[ct] = used ? min(gi.plen, effective_len(a, s, B)) : gi.plen;
    lane_min = min(lane_min, lim[ct]);
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                         (int64_t(s) * a.num_heads + int64_t(kvh) * G + hh) * D + 8 * grp;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (used) v = *reinterpret_cast<const uint4*>(qh + 32 * j);
      qop[ct][j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // tiles below every column's limit need no mask
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) lane_min = min(lane_min, __shfl_xor(lane_min, d));
  const int all_lim = wave_uniform(lane_min);

  floatx4_t acc[NC][DCH];
  float m_run[NC], l_run[NC];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
#pragma unroll
    for (int c = 0; c < DCH; ++c) acc[ct][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
  }

  auto t0_of = [&](int k) { return t_begin + k * kTile; };

  auto consume = [&](const Tile<D>& r, int k) {
    const int t0 = t0_of(k);
    floatx4_t sacc[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      sacc[ct] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        sacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[j]),
                                                           qop[ct][j], sacc[ct], 0, 0, 0);
    }
    short4_t pop[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sacc[ct][i] * a.scale_log2e;
      if (t0 + kTile > all_lim) {  // some column stops inside this tile
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (t0 + 4 * grp + i < lim[ct]) ? x[i] : -INFINITY;
      }
      if (r.bad) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __builtin_nanf("");
      }
      const float tmax = colmax4(max_nan(max_nan(x[0], x[1]), max_nan(x[2], x[3])));
      if (__any(tmax > m_run[ct] + kRescaleThreshold)) {
        const float m_new = fmaxf(m_run[ct], tmax);
        // a column that has seen no token yet keeps m = -inf and weight 1
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[ct] - m_new);
        l_run[ct] *= alpha;
#pragma unroll
        for (int c = 0; c < DCH; ++c) acc[ct][c] *= alpha;
        m_run[ct] = m_new;
      }
      const float m_use = m_run[ct] == -INFINITY ? 0.f : m_run[ct];
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
      l_run[ct] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      const uint2 pp = make_uint2(pack_bf16x2_rne(pr[0], pr[1]), pack_bf16x2_rne(pr[2], pr[3]));
      pop[ct] = __builtin_bit_cast(short4_t, pp);
    }
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const short4_t vop = __builtin_bit_cast(short4_t, r.v[c]);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
        acc[ct][c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop[ct], acc[ct][c], 0, 0, 0);
    }
  };

  // The tile pipeline of the tail runs (a ring of kRing register tiles, the
  // block ids from a window of the first member's table), with every tile
  // whole: the run covers a multiple of 16 tokens.
  {
    constexpr int kWin = window_tiles<B>();
    Tile<D> ring[kRing];
    int win = load_window(row, t_begin / B, nblk, lane);
    for (int k0 = 0; k0 < ntile; k0 += kWin) {
      const int k1 = min(ntile, k0 + kWin);
      const int wb = t0_of(k0) / B;
      const int last = k1 - 1;
      TileIds id;
#pragma unroll
      for (int d = 0; d < kRing - 1; ++d) {
        const int kd = min(k0 + d, last);
        id = window_ids<B>(win, wb, t0_of(kd), nblk);
        load_tile<D, B, kStream>(ring[d], a, id, kvh, t0_of(kd), lane, k_off, v_off);
      }
      id = window_ids<B>(win, wb, t0_of(min(k0 + kRing - 1, last)), nblk);
      int nxt = win;
      if (k1 < ntile) nxt = load_window(row, t0_of(k1) / B, nblk, lane);
      for (int k = k0; k < k1; k += kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
          const int kl = min(k + d + kRing - 1, last);
          load_tile<D, B, kStream>(ring[(d + kRing - 1) % kRing], a, id, kvh, t0_of(kl), lane,
                                   k_off, v_off);
          id = window_ids<B>(win, wb, t0_of(min(k + d + kRing, last)), nblk);
          if (k + d < k1) consume(ring[d], k + d);
        }
      }
      win = nxt;
    }
  }

  // One record per member: o[G][D], m[G], l[G], the stamp.
  const int rec_f = int(record_floats(G, D));
  float* wrec = a.ws_wide + wide * a.prefix_members * rec_f;
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const float l_tot = colsum4(l_run[ct]);
    const int c = ct * 16 + col;
    if (c < ncols) {
      const int m = c / G;
      const int hh = c - m * G;
      float* rec = wrec + int64_t(m) * rec_f;
#pragma unroll
      for (int cc = 0; cc < DCH; ++cc)
        *reinterpret_cast<floatx4_t*>(rec + hh * D + 16 * cc + 4 * grp) = acc[ct][cc];
      if (grp == 0) {
        rec[G * D + hh] = m_run[ct];
        rec[G * D + G + hh] = l_tot;
        if (hh == 0) rec[G * D + 2 * G] = __uint_as_float(a.epoch);
      }
    }
  }
}

// kParts: some pair has more than one partition, so a run may pass
// partition ends (split launches only).  kGroups: a grouped line (split
// launches with shared-prefix groups, schedule.h).
template <int D, int B, bool kSplit, bool kStream, bool kParts, bool kGroups>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D > 128 || kSplit ? 1 : 2)))
void decode_bf16_mfma_kernel(DecodeArgs a) {
  constexpr int KSTEPS = D / 32;
  constexpr int DCH = D / 16;
  const int G = a.group;
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  __shared__ uint32_t new_row_lds[D];  // appending decode: the new K row, then the V row
  // A split worker's records wait here, with their workspace indices, and
  // go out in bursts: when the area is full and after the worker's last
  // run.  A global store in mid-stream would hold up the worker's next
  // loads, because the wait for a load also waits for every store issued
  // before it; a store's acknowledgement under full load takes a long
  // round trip.  32 KiB holds 15 records at G = 4, D = 128 (a 128K-token
  // context in 512-token partitions puts ~14 partitions in a worker's
  // slice) and at least one at G = 16, D = 256.  Four such workgroups fit
  // on a compute unit, one per SIMD, as many as the decode runs.
  constexpr int kRecLdsFloats = kSplit ? 8192 : 4;
  constexpr int kMaxStaged = kSplit ? 16 : 1;
  __shared__ __align__(16) float rec_lds[kRecLdsFloats];
  __shared__ int64_t rec_dst[kMaxStaged];
  // Appending split workers keep their write-back tiles here too (the V rows
  // of every lane and the token's K row) and store them after their last
  // run, for the same reason: stored in mid-stream they held up the next
  // run's first loads.  Two tiles, 4.25 KiB each at D = 128; a worker with
  // more appending runs stores the others at once.
  constexpr int kTbSlots = kSplit ? 2 : 0;
  constexpr int kTbDwords = D * 8 + D / 2;  // V: D/16 x 64 lanes x 2; K: D/32 x 4 lanes x 4
  __shared__ __align__(16) uint32_t tb_lds[kTbSlots > 0 ? kTbSlots * kTbDwords : 1];
  __shared__ int tb_info[kTbSlots > 0 ? kTbSlots * 4 : 1];  // block, kvh, tile start, row
  int tb_used = 0;
  const int rec_f = int(record_floats(G, D));
  const int stage_slots = min(kMaxStaged, kRecLdsFloats / rec_f);
  int staged = 0;  // records waiting in LDS

  // Copies the staged records to their places in the workspace, eight
  // 16-byte chunks per lane in flight at a time.
  auto drain = [&]() {
    __syncthreads();  // one wave: orders the LDS writes before the reads
    const int q4 = rec_f / 4;
    constexpr int kBurst = 8;
    for (int sl = 0; sl < staged; ++sl) {
      const floatx4_t* src = reinterpret_cast<const floatx4_t*>(rec_lds + sl * rec_f);
      floatx4_t* dst = reinterpret_cast<floatx4_t*>(a.ws + wave_uniform64(rec_dst[sl]) * rec_f);
      for (int i0 = 0; i0 < q4; i0 += kBurst * kThreads) {
        floatx4_t v[kBurst];
#pragma unroll
        for (int u = 0; u < kBurst; ++u) {
          const int i = i0 + u * kThreads + lane;
          if (i < q4) v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < kBurst; ++u) {
          const int i = i0 + u * kThreads + lane;
          if (i < q4) dst[i] = v[u];
        }
      }
    }
    __syncthreads();  // and the reads before the slots are written again
    staged = 0;
  };

  // Per-lane byte offsets inside a tile (k_off_pair: K row col of a paired
  // B = 32 tile, see load_tile_b32).
  const uint32_t k_off = uint32_t(col) * D * 2 + uint32_t(grp) * 16;
  const uint32_t v_off = uint32_t(col) * B * 2 + uint32_t(grp) * 8;
  const uint32_t k_off_pair = uint32_t(8 * (col / 4) + col % 4) * D * 2 + uint32_t(grp) * 16;
  // B = 32 plain runs use the paired numbering of load_tile_b32; grouped
  // launches (whose tail runs may start inside a block's first tile) do not.
  constexpr bool kPair = B == 32 && !kGroups;

  // Keeps an appending tile's write-back for later (see tb_lds), or stores
  // it now when both slots are taken.
  auto write_back = [&](const Tile<D>& r, int pb, int kvh, int t0, int rt, bool paired) {
    if (tb_used == kTbSlots) {
      store_tile_back<D, B>(r, a, pb, kvh, t0, rt, lane, k_off, v_off, paired);
      return;
    }
    uint32_t* slot = tb_lds + tb_used * kTbDwords;
#pragma unroll
    for (int c = 0; c < DCH; ++c)
      *reinterpret_cast<uint2*>(slot + (c * kThreads + lane) * 2) = r.v[c];
    if (col == rt) {
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        *reinterpret_cast<uint4*>(slot + D * 8 + (j * 4 + grp) * 4) = r.k[j];
    }
    if (lane == 0) {
      tb_info[tb_used * 4 + 0] = pb;
      tb_info[tb_used * 4 + 1] = kvh;
      tb_info[tb_used * 4 + 2] = t0;
      tb_info[tb_used * 4 + 3] = rt | (paired ? 0x100 : 0);
    }
    ++tb_used;
  };
  // Stores the kept write-backs.
  auto flush_write_backs = [&]() {
    __syncthreads();  // one wave: orders the LDS writes before the reads
    for (int i = 0; i < tb_used; ++i) {
      const uint32_t* slot = tb_lds + i * kTbDwords;
      const int pb = wave_uniform(tb_info[i * 4 + 0]);
      const int kvh = wave_uniform(tb_info[i * 4 + 1]);
      const int t0 = wave_uniform(tb_info[i * 4 + 2]);
      const int rtp = wave_uniform(tb_info[i * 4 + 3]);
      const int rt = rtp & 0xFF;
      Tile<D> r;
#pragma unroll
      for (int c = 0; c < DCH; ++c)
        r.v[c] = *reinterpret_cast<const uint2*>(slot + (c * kThreads + lane) * 2);
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        r.k[j] = *reinterpret_cast<const uint4*>(slot + D * 8 + (j * 4 + grp) * 4);
      r.bad = false;
      store_tile_back<D, B>(r, a, pb, kvh, t0, rt, lane, k_off, v_off, (rtp & 0x100) != 0);
    }
    tb_used = 0;
  };

  // One run: tiles [tin, tin + ntile) of pair (s, kvh), counted from token
  // tok0 (0, or the tokens of a shared prefix that a prefix unit streams).
  // The tiles of the pair's partition p make its record k_first + p (stored
  // at record_slot(slots, k_first + p)), or, when the run is the whole pair
  // (one partition), go straight to the output.
  auto run = [&](int s, int kvh, int L, int tok0, int tin, int ntile, bool whole,
                 PairSlots slots, int k_first) {
    // Every argument is the same in all lanes; say so, so that addresses
    // built from them stay in scalar registers.
    s = wave_uniform(s);
    kvh = wave_uniform(kvh);
    L = wave_uniform(L);
    tok0 = wave_uniform(tok0);
    tin = wave_uniform(tin);
    ntile = wave_uniform(ntile);
    whole = wave_uniform(int(whole)) != 0;
    slots.fixed = wave_uniform64(slots.fixed);
    slots.overflow = wave_uniform64(slots.overflow);
    k_first = wave_uniform(k_first);
    const int t_begin = tok0 + tin * kTile;
    const int t_end = min(L, tok0 + (tin + ntile) * kTile);
    const int nblk = (L + B - 1) / B;
    const int32_t* row = a.block_tables + int64_t(s) * a.max_blocks_per_seq;

    // Appending decode: the run holding the pair's last tile uses the step's
    // row (token L - 1) in that tile and writes the tile back with the row
    // in its slot.
    // The tile holding token L - 1 (counted from tok0) and its row there:
    // the last tile, or with the paired B = 32 numbering whichever half of
    // the last block holds it.
    int tile_new = (L - tok0 + kTile - 1) / kTile - 1;
    int rt_new = L - 1 - tok0 - tile_new * kTile;
    bool paired_new = false;
    if constexpr (kPair) {
      const int blk0 = (L - 1) & ~(B - 1);
      const int off = L - 1 - blk0;
      if (blk0 + kTile < L) {
        paired_new = true;
        tile_new = blk0 / kTile + ((off >> 2) & 1);
        rt_new = 4 * (off >> 3) + (off & 3);
      }
    }
    const bool append = a.new_k != nullptr && tile_new >= tin && tile_new < tin + ntile;
    NewRow<D> nr{};
    int pb_new = 0;
    if (append) {  // issued first: its wait below overlaps the table window's
      nr = load_new_row<D>(a, s, kvh, lane);
      pb_new = load_ro(row, (L - 1) / B);
    }

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

    floatx4_t acc[DCH];
#pragma unroll
    for (int c = 0; c < DCH; ++c) acc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // Partition bookkeeping: the run passes partition ends without draining
    // its loads; at each one the partition's state becomes a record (staged
    // like every record) and the state starts afresh.  (Without kParts
    // every pair is a single partition and no end is passed.)
    const int tpp = a.partition_size / kTile;
    int part = kParts ? tin / tpp : 0;
    int part_left = (part + 1) * tpp - tin;  // tiles of partition `part` still to consume

    // Stages the state as the record of partition p: o[col][dims], m[col],
    // l[col], the stamp.  l is summed over the four row groups of each
    // column first, so every lane of a column holds its (m, l).
    auto stage = [&](int p) {
      const float l_tot = colsum4(l_run);
      if (col < G) {
        const int base = staged * rec_f;
#pragma unroll
        for (int c = 0; c < DCH; ++c)
          *reinterpret_cast<floatx4_t*>(&rec_lds[base + col * D + 16 * c + 4 * grp]) = acc[c];
        if (grp == 0) {
          rec_lds[base + G * D + col] = m_run;
          rec_lds[base + G * D + G + col] = l_tot;
          if (col == 0) rec_lds[base + G * D + 2 * G] = __uint_as_float(a.epoch);
        }
      }
      if (lane == 0) rec_dst[staged] = record_slot(slots, k_first + p);
      if (++staged == stage_slots) drain();
    };
    // The run's end: the output itself for a whole pair, else the last
    // partition's record.
    auto finish = [&]() {
      if (whole) {
        const float l_tot = colsum4(l_run);
        if (a.lse && col < G && grp == 0)  // ln sum e^(scale q.k) = (m + log2 l) ln 2
          a.lse[int64_t(s) * a.num_heads + int64_t(kvh) * G + col] =
              (m_run + __log2f(l_tot)) * 0.6931471805599453f;
        if (col < G) {
          const float inv_l = 1.0f / l_tot;
          uint16_t* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G + col) * D + 4 * grp;
#pragma unroll
          for (int c = 0; c < DCH; ++c)
            *reinterpret_cast<uint2*>(o + 16 * c) =
                make_uint2(pack_bf16x2_rne(acc[c][0] * inv_l, acc[c][1] * inv_l),
                           pack_bf16x2_rne(acc[c][2] * inv_l, acc[c][3] * inv_l));
        }
      } else {
        stage(part);
      }
    };

    auto t0_of = [&](int k) { return t_begin + k * kTile; };

    auto consume = [&](Tile<D>& r, int k) {
      // this lane's first token (of 4) in the tile, and the end of the tokens
      // the tile may hold: tokens from `limit` on are dropped
      const int t0 = t0_of(k);
      int first = t0 + 4 * grp, span_end = t0 + kTile, limit = t_end;
      if constexpr (kPair) {
        const int blk0 = t0 & ~(B - 1);
        if (blk0 + kTile < L) {
          first = blk0 + 8 * grp + 4 * ((t0 / kTile) & 1);
          span_end = blk0 + B;
        }
        limit = L;
      }
      floatx4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[j]),
                                                       qop[j], sacc, 0, 0, 0);
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sacc[i] * a.scale_log2e;
      if (span_end > limit) {  // last, partial tile: drop tokens >= limit
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (first + i < limit) ? x[i] : -INFINITY;
        const int n = min(max(limit - first, 0), 4);
        const uint32_t mx = (n >= 1 ? 0x0000FFFFu : 0u) | (n >= 2 ? 0xFFFF0000u : 0u);
        const uint32_t my = (n >= 3 ? 0x0000FFFFu : 0u) | (n >= 4 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int c = 0; c < DCH; ++c) {
          r.v[c].x &= mx;
          r.v[c].y &= my;
        }
      }
      if (r.bad) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __builtin_nanf("");
      }
      const float tmax = colmax4(max_nan(max_nan(x[0], x[1]), max_nan(x[2], x[3])));
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
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, r.v[c]),
                                                           pop, acc[c], 0, 0, 0);
    };

    // Software pipeline over the run's tiles, a ring of kRing register
    // tiles: while tile k is consumed, tiles k+1 .. k+kRing-1 are in flight.
    // Every load is issued unconditionally (past the last tile the ring
    // repeats the last tile, which the caches serve) and only the consumes
    // are guarded, so the wait before each tile covers exactly the loads
    // issued before it.  Block ids come from a table window; the window of
    // the next run of tiles is loaded when the current run starts.
    {
      constexpr int kWin = window_tiles<B>();
      static_assert(!kPair || (kRing == 2 && kWin % 2 == 0), "paired tiles assume a 2-tile ring");
      Tile<D> ring[kRing];
      uint2 carry[DCH];  // paired B = 32: a block's second tile's V, from its first tile
      int win = load_window(row, t_begin / B, nblk, lane);
      if (append) {
        // the row goes to LDS for the tile holding it, which also writes it
        // to its slot in the cache (only this wave reads that slot in this launch)
        stage_new_row<D>(nr, new_row_lds, lane);
      }
      // One tile's loads into a ring slot; kv: what of V the site fetches
      // (paired B = 32 only: fixed per site by the run's parity).
      auto load_at = [&](Tile<D>& r, const TileIds& id, int kd, auto kv) {
        if constexpr (kPair)
          load_tile_b32<D, decltype(kv)::value, kStream>(r, a, id, kvh, t0_of(kd), L, lane, k_off,
                                                         k_off_pair);
        else
          load_tile<D, B, kStream>(r, a, id, kvh, t0_of(kd), lane, k_off, v_off);
      };
      // par: the run starts at a block's second tile (paired B = 32; 0 otherwise)
      auto walk = [&](auto par) {
        constexpr int P = decltype(par)::value;
        for (int k0 = 0; k0 < ntile; k0 += kWin) {
          const int k1 = min(ntile, k0 + kWin);
          const int wb = t0_of(k0) / B;
          const int last = k1 - 1;
          TileIds id;
#pragma unroll
          for (int d = 0; d < kRing - 1; ++d) {
            const int kd = min(k0 + d, last);
            id = window_ids<B>(win, wb, t0_of(kd), nblk);
            load_at(ring[d], id, kd, std::integral_constant<int, P == 0 ? kVWide : kVHalf>{});
          }
          id = window_ids<B>(win, wb, t0_of(min(k0 + kRing - 1, last)), nblk);
          int nxt = win;  // issued after this window's first reads, so they do not wait for it
          if (k1 < ntile) nxt = load_window(row, t0_of(k1) / B, nblk, lane);
          // step d of the ring at tile k (k even): d is a compile-time index
          auto step = [&](int k, auto dd) {
            constexpr int d = decltype(dd)::value;
            const int kl = min(k + d + kRing - 1, last);
            // tile k + d + 1 is a block's first tile when P + d + 1 is even
            load_at(ring[(d + kRing - 1) % kRing], id, kl,
                    std::integral_constant<int, ((P + d + 1) & 1) == 0 ? kVWide : kVNone>{});
            id = window_ids<B>(win, wb, t0_of(min(k + d + kRing, last)), nblk);
            if (k + d < k1) {
              if constexpr (kPair) {
                if constexpr (((P + d) & 1) == 1) {  // a block's second tile
                  if (d > 0 || k > k0) {              // its first tile came just before
#pragma unroll
                    for (int c = 0; c < DCH; ++c) ring[d].v[c] = carry[c];
                  }
                } else {
#pragma unroll
                  for (int c = 0; c < DCH; ++c) carry[c] = ring[d].v2[c];
                }
              }
              if (append && k + d == tile_new - tin) {
                put_new_row<D>(ring[d], new_row_lds, rt_new, col, grp);
                if (unsigned(pb_new) < unsigned(a.num_blocks))
                  write_back(ring[d], pb_new, kvh, t0_of(k + d), rt_new, paired_new);
              }
              consume(ring[d], k + d);
              if (kParts && --part_left == 0 && k + d + 1 < ntile) {
                stage(part);
                ++part;
                part_left = tpp;
#pragma unroll
                for (int c = 0; c < DCH; ++c) acc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                m_run = -INFINITY;
                l_run = 0.f;
              }
            }
          };
          static_assert(kRing == 2, "the ring's steps are spelled out for two tiles");
          for (int k = k0; k < k1; k += kRing) {
            step(k, std::integral_constant<int, 0>{});
            step(k, std::integral_constant<int, 1>{});
          }
          win = nxt;
        }
      };
      if constexpr (kPair) {
        if ((t_begin / kTile) & 1)
          walk(std::integral_constant<int, 1>{});
        else
          walk(std::integral_constant<int, 0>{});
      } else {
        walk(std::integral_constant<int, 0>{});
      }
    }

    finish();
  };

  if constexpr (kGroups) {
    __shared__ int4 group_lds[kMaxGroups];
    const GroupTable gt{group_lds};  // filled by walk_unit_runs
    walk_unit_runs(a, gt, B, lane, blockIdx.x, [&](const UnitRun& r) {
      if (r.prefix) {
        run_prefix<D, B, kStream>(a, group_info(a, gt, r.seq), r.kvh, r.tin, r.ntile, r.wide,
                                  lane, k_off, v_off);
      } else {
        run(r.seq, r.kvh, r.shape.len, r.shape.tok0, r.tin, r.ntile, r.whole, r.slots, r.k0);
      }
    });
    if (staged > 0) drain();
    if (tb_used > 0) flush_write_backs();
  } else if constexpr (kSplit) {
    walk_slice_runs(a, B, lane, blockIdx.x,
                    [&](int s, int kvh, int L, int tin, int ntile, bool whole, PairSlots slots,
                        int k_first) { run(s, kvh, L, 0, tin, ntile, whole, slots, k_first); });
    if (staged > 0) drain();
    if (tb_used > 0) flush_write_backs();
  } else {
    // one worker per (sequence, KV head); consecutive workers are the KV
    // heads of one sequence (workgroup i runs on XCD i % 8)
    const int kvh = blockIdx.x % a.num_kv_heads;
    const int s = blockIdx.x / a.num_kv_heads;
    const int L = effective_len(a, s, B);
    if (L == 0) {
      uint16_t* o = out + (int64_t(s) * a.num_heads + int64_t(kvh) * G) * D;
      for (int i = lane; i < G * D; i += kThreads) o[i] = 0;
      if (a.lse && lane < G) a.lse[int64_t(s) * a.num_heads + int64_t(kvh) * G + lane] = -INFINITY;
      return;
    }
    run(s, kvh, L, 0, 0, (L + kTile - 1) / kTile, true, PairSlots{0, 0}, 0);
  }
}

template <int D, int B, bool kStream>
hipError_t launch_policy(const DecodeArgs& a, hipStream_t stream) {
  if (a.split && a.num_groups > 0)
    return launch(decode_bf16_mfma_kernel<D, B, true, kStream, true, true>,
                  dim3(unsigned(a.workers)), dim3(kThreads), 0, stream, a);
  if (a.split && a.max_partitions > 1)
    return launch(decode_bf16_mfma_kernel<D, B, true, kStream, true, false>,
                  dim3(unsigned(a.workers)), dim3(kThreads), 0, stream, a);
  if (a.split)
    return launch(decode_bf16_mfma_kernel<D, B, true, kStream, false, false>,
                  dim3(unsigned(a.workers)), dim3(kThreads), 0, stream, a);
  const int64_t grid = int64_t(a.num_seqs) * a.num_kv_heads;
  return launch(decode_bf16_mfma_kernel<D, B, false, kStream, false, false>, dim3(unsigned(grid)),
                dim3(kThreads), 0, stream, a);
}

template <int D, int B>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  return a.shared_blocks ? launch_policy<D, B, false>(a, stream)
                         : launch_policy<D, B, true>(a, stream);
}

// One worker count for every split variant: pa_decode_merge, which is not
// told the cache policy, rebuilds the same schedule from it.  It is taken
// from the variant with the most registers, so every variant fits that
// many workers on the device at once (all split variants use the same LDS).
template <int D, int B>
int workers_one(bool groups) {
  if (groups)  // the grouped kernels: their own occupancy, within the wide region's bound
    return std::min(kMaxGroupWorkers,
                    resident_workers(reinterpret_cast<const void*>(
                                         decode_bf16_mfma_kernel<D, B, true, true, true, true>),
                                     kThreads));
  return resident_workers(
      reinterpret_cast<const void*>(decode_bf16_mfma_kernel<D, B, true, true, true, false>),
      kThreads);
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

template <int D>
int workers_d(int block_size, bool groups) {
  switch (block_size) {
    case 8: return workers_one<D, 8>(groups);
    case 16: return workers_one<D, 16>(groups);
    case 32: return workers_one<D, 32>(groups);
    default: return 0;
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

int decode_workers_bf16_mfma(int head_dim, int block_size, bool groups) {
  switch (head_dim) {
    case 64: return workers_d<64>(block_size, groups);
    case 128: return workers_d<128>(block_size, groups);
    case 256: return workers_d<256>(block_size, groups);
    default: return 0;
  }
}

}  // namespace pa

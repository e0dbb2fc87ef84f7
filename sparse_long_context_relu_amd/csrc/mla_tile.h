// Sparse MLA tile layout and gather, shared by the forward passes
// (sparse_mla.hip) and the Stage-2 backward (sparse_bwd.hip).
//
// H = 128 heads, D = 576 (512 latent + 64 rope), Dv = 512.  A workgroup of 8
// waves gathers 32-row tiles of 1152-byte latent rows straight into LDS with
// the direct-to-LDS loads of gfx950; wave w owns heads 16w..16w+15.
#pragma once

#include "kernels.h"

namespace dsa {
namespace {

constexpr int kH = 128, kD = 576, kDv = 512;
constexpr int kWaves = kH / 16;               // 8 waves, 16 heads each
constexpr int kThreads = kWaves * 64;
constexpr int kR = 32;                        // latent rows per tile
// LDS tile layout: row r of the tile occupies kRowChunks 16-byte positions (72
// data chunks + 2 pad); data chunk c of row r sits at position c ^ swz(r).  With
// the 1184-byte row stride and this swizzle, the 16-byte logit-operand reads
// (16 rows, same chunk) and the transpose reads of the value product (4 rows x
// 32 bytes per 16 lanes) hit distinct LDS banks.
constexpr int kDataChunks = kD * 2 / 16;      // 72
constexpr int kRowChunks = kDataChunks + 2;   // row stride 1184 B
constexpr int kRowStride = kRowChunks * 16;
constexpr int kTileChunks = kR * kRowChunks;  // 2368
// A tile buffer is padded to 40 whole 64-lane loads, five per wave, so every
// load writes all of its lanes and every wave issues the same loads; the pad
// receives copies of a valid row.
constexpr int kWaveLoads = (kTileChunks + kThreads - 1) / kThreads;  // 5 direct loads per wave
constexpr int kTileLoads = kWaveLoads * kWaves;                      // 40
constexpr int kTileBufChunks = kTileLoads * 64;                      // 2560
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
constexpr int kKs = kD / 32;                  // 18 k-steps of the logits
constexpr int kDb = kDv / 16;                 // 32 value-dim blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplitRows = 2048;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// Running maxima are raised only when a tile's maximum exceeds them by more than
// this many binary orders of magnitude; in between, the softmax weights of a
// tile stay below 2^kLazy, exact in fp32 and in bf16 (the final result divides
// by the same running sum, so it does not depend on the base).
constexpr float kLazy = 8.f;

__device__ __forceinline__ int split_len(int k, int n_split) {
  int len = (k + n_split - 1) / n_split;
  return (len + kR - 1) / kR * kR;
}

// Block order.  Workgroups are dealt to the 8 XCDs round-robin by linear id,
// and each XCD has its own L2.
//   * Dense prefill lists: every query reads the same rows 0..t, so the
//     workgroups that run together on one XCD take the same split of
//     different queries (XCD x serves groups x, x+8, ..., split after split).
//     Their tiles then come from one 2048-row range of the cache, which that
//     L2 holds, instead of from every split's range at once.
//   * Otherwise the splits of one query are placed on the same XCD, so its
//     query rows are fetched once and then served by that XCD's L2.
__device__ __forceinline__ void mla_block(const MlaArgs &a, int groups, int &sp, int &r) {
  const int total = a.n_split * groups;
  int v = blockIdx.x;
  if (a.dense && a.sv.mode == DSA_PREFILL && (groups & 7) == 0) {
    const int per_xcd = groups >> 3, k = v >> 3;
    sp = k / per_xcd;
    r = (k - sp * per_xcd) * 8 + (v & 7);
    return;
  }
  if ((total & 7) == 0) v = (v & 7) * (total >> 3) + (v >> 3);
  r = v / a.n_split;
  sp = v - r * a.n_split;
}

constexpr int kBufs = 3;

// The direct-to-LDS gather of split rows [j0, j0+32) into the tile at LDS
// address `tile`.  Position p of the tile is (row p/74, slot p%74) and holds data
// chunk slot ^ swz(row) of that row; a wave's j-th load covers positions
// (8 j + wv) 64 + [0, 64).  The pad chunks and absent rows (slot -1) load a
// valid row (`fallback`), so every LDS byte the MFMAs read is finite; absent
// rows are masked in the softmax.  `slots` holds -1 past the split's last row,
// far enough for every lane's row.
struct TileLoads {
  const uint8_t *src[kWaveLoads];   // this lane's source of each of the wave's loads
};

// Per-lane coordinates of a wave's tile loads, the same for every tile: load
// j's tile row (5 bits) and its data chunk (7 bits, swizzled; 0 for a pad
// chunk), 12 bits a load: loads 0, 1 and the low byte of load 4 in the first
// word, loads 2, 3 and the high nibble of load 4 in the second.  Positions past
// the tile (rows 32..) only fill LDS that no one reads, so their row is kept
// modulo 32: they load some valid row.  Formed once per kernel; a tile then
// unpacks them with a few bit-field extracts instead of re-deriving row and
// chunk (two registers, where per-load values would not fit beside the MFMA
// operands).
static_assert(kWaveLoads == 5, "coordinate packing");
struct TileCoords {
  uint32_t w[2];
};
__device__ __forceinline__ TileCoords tile_coords(int wv, int lane) {
  uint32_t f[kWaveLoads];
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const int p = (j * kWaves + wv) * 64 + lane;
    const int row = p / kRowChunks, ch = p - row * kRowChunks;
    const int dc = ch < kDataChunks ? ch ^ swz(row) : 0;
    f[j] = (uint32_t)((row & 31) | (dc << 5));
  }
  TileCoords c;
  c.w[0] = f[0] | (f[1] << 12) | ((f[4] & 0xffu) << 24);
  c.w[1] = f[2] | (f[3] << 12) | ((f[4] >> 8) << 24);
  return c;
}
__device__ __forceinline__ uint32_t tile_coord(const TileCoords &c, int j) {
  if (j < 2) return (c.w[0] >> (12 * j)) & 0xfffu;
  if (j < 4) return (c.w[1] >> (12 * (j - 2))) & 0xfffu;
  return (c.w[0] >> 24) | ((c.w[1] >> 24) << 8);
}

// Sources of this wave's loads of the tile of split rows [j0, j0+32): slot reads
// first (independent LDS reads, one wait), then the addresses.  Rows past the
// tile (the pad) read the slot list's -1 tail and load the fallback row.
__device__ __forceinline__ TileLoads tile_loads(const uint8_t *kv, const int *slots, int j0, int fallback,
                                                const TileCoords &c0) {
  // unpacked per call (pinned so that the compiler does not hoist the
  // unpacked values out of the tile loop and keep them live across it)
  TileCoords c = c0;
  asm volatile("" : "+v"(c.w[0]), "+v"(c.w[1]));
  int sl[kWaveLoads], dc[kWaveLoads];
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const uint32_t f = tile_coord(c, j);
    sl[j] = slots[j0 + (int)(f & 31u)];
    dc[j] = (int)(f >> 5);
  }
  TileLoads t;
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const int s = sl[j] < 0 ? fallback : sl[j];
    t.src[j] = kv + (unsigned long long)(unsigned)s * (kD * 2) + dc[j] * 16;
  }
  return t;
}

// The wave's j-th load of a tile into the buffer at LDS address `tile`
// (kStream: streaming loads, for rows that no other workgroup reads again).
template <bool kStream = false>
__device__ __forceinline__ void tile_load(const TileLoads &t, int j, uint32_t tile, int wv) {
  if constexpr (kStream)
    lds_dma16_stream(t.src[j], tile + (j * kWaves + wv) * 1024);
  else
    lds_dma16(t.src[j], tile + (j * kWaves + wv) * 1024);
}

template <bool kStream = false>
__device__ __forceinline__ void issue_tile(uint32_t tile, const uint8_t *kv, const int *slots, int j0,
                                           int fallback, int wv, const TileCoords &c) {
  const TileLoads t = tile_loads(kv, slots, j0, fallback, c);
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) tile_load<kStream>(t, j, tile, wv);
}

// The same gather issued by half of the waves (h = wave index within the half,
// twice the loads each: load j covers positions (4 j + h) 64 + [0, 64)).  The
// passes without a value product alternate the halves from tile to tile: each
// tile's issue burst then stalls only four waves, while the other four go on
// with their logits.
constexpr int kHalfWaves = kWaves / 2;
constexpr int kHalfLoads = kTileLoads / kHalfWaves;   // 10
__device__ __forceinline__ void issue_tile_half(uint32_t tile, const uint8_t *kv, const int *slots, int j0,
                                                int fallback, int h, int lane) {
  asm volatile("" : "+v"(lane));
  // two batches of five: slot reads, then the loads
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    constexpr int kB = kHalfLoads / 2;
    int sl[kB], dc[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int p = ((b * kB + j) * kHalfWaves + h) * 64 + lane;
      const int row = p / kRowChunks, ch = p - row * kRowChunks;
      sl[j] = slots[j0 + row];
      dc[j] = ch < kDataChunks ? ch ^ swz(row) : 0;
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int src = sl[j] < 0 ? fallback : sl[j];
      lds_dma16(kv + (long long)src * (kD * 2) + dc[j] * 16, tile + ((b * kB + j) * kHalfWaves + h) * 1024);
    }
  }
}

// Sum over the 16 lanes of a row of the wave (the 16 heads of a lane group),
// in every lane of the row: two quad swaps, then the half-row and row mirrors.
__device__ __forceinline__ float sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

}  // namespace
}  // namespace dsa

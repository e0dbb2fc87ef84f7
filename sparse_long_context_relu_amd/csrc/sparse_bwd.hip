// Stage 2 of DSA training: the gradient of the sparse attention over each
// query's selected rows, and the indexer's KL loss restricted to the selection
// ("DeepSeek V3.2: How Far Can Open Models Go If You Actually Try?", section
// 3.3, Stage 2: the main attention switches to top-k, every parameter trains,
// and the indexer keeps learning from a loss on the selected subset S_t).
//
// For query t with selected rows c_j (j < k), logits z = sm_scale q c^T,
// weights P = exp(z - lse) (the forward's log-sum-exp) and output O:
//   Delta_h = sum_d dO[h,d] O[h,d]
//   dP = dO V^T,   dS = P (dP - Delta)                (per head, per row)
//   dq = sm_scale dS C                                 [H, D]
//   dc_j = sm_scale dS[:, j]^T Q + P[:, j]^T dO        [D] (key and value are one row)
// and the cache row of a token receives the sum of dc_j over every query that
// selected it.  Kernels, per chunk of up to 256 query rows:
//   bwd_delta     Delta from the forward output and dO
//   bwd_scores    gathers each query's rows into LDS (the forward's tiles); every
//                 tile operand read feeds the logit and the dP MFMA; writes
//                 P and sm_scale dS in bf16 (per tile for dq, per row for the row
//                 gradients) and the head-mean weights (the Stage-2 target)
//   bwd_dq        gathers the rows again: dq^T += C^T dS^T (LDS transpose reads)
//   bwd_contrib   the row gradients as a GEMM per query, [P | dS] rows against
//                 dO and Q slices staged in LDS: one bf16 row per (query, j)
//   bwd_jpos_*    which slot j of which query row selected each key
//   bwd_dkv       per key, its rows' gradients summed in fp32 in ascending query order,
//                 chunk after chunk: no atomics, so the result is deterministic.
#include "mla_tile.h"

namespace dsa {
namespace {

constexpr int kKv = kDv / 32;                 // 16 k-steps of dP over the value dims
constexpr int kDbAll = kD / 16;               // 36 dim blocks of the row and dq products
constexpr uint16_t kNoSlot = 0xFFFF;

// k-slot position of head h inside its group of 32 heads: the row-gradient
// product reads heads 4g..4g+3 and 16+4g..16+4g+3 of a group in lane group g,
// and they sit together so one 16-byte load fetches them.
__device__ __forceinline__ int head_slot(int h) {
  const int hh = h & 31;
  const int p = hh < 16 ? ((hh >> 2) << 3) + (hh & 3) : (((hh - 16) >> 2) << 3) + 4 + (hh & 3);
  return (h & ~31) + p;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) { return f32_to_bf16(x); }

// Slots of query t's k selected positions (prefill: sequence 0) into LDS, -1
// for absent entries and past the list; returns after a barrier with the
// largest present slot in *fallback (-1 when none).
__device__ void fill_slots(const MlaBwdArgs &a, int t, int n, int ntiles, int *slots, int *fallback) {
  if (threadIdx.x == 0) *fallback = -1;
  __syncthreads();
  const int32_t *irow = a.idx + (long long)t * a.k;
  const int nfill = ntiles * kR + 3 * kR;
  for (int j = threadIdx.x; j < nfill; j += kThreads) {
    int sl = -1;
    const int p = j < a.k ? irow[j] : -1;
    if (p >= 0 && p < n) {
      if (a.sv.block_table == nullptr) {
        sl = p;
      } else {
        const int blk = a.sv.block_table[p >> 6];
        if (blk >= 0 && blk < a.sv.num_blocks) sl = blk * 64 + (p & 63);
      }
    }
    slots[j] = sl;
    if (sl >= 0) atomicMax(fallback, sl);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- Delta

__global__ __launch_bounds__(256) void bwd_delta_kernel(MlaBwdArgs a) {
  const long long i = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= (long long)a.rows * kH) return;
  const int r = (int)(i / kH), h = (int)(i % kH);
  const long long base = ((long long)(a.q_begin + r) * kH + h) * kDv + lane_id() * 8;
  const uint4 o = ld16(reinterpret_cast<const uint16_t *>(a.out) + base);
  const uint4 d = ld16(reinterpret_cast<const uint16_t *>(a.dout) + base);
  const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, dw[4] = {d.x, d.y, d.z, d.w};
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    s = fmaf(__uint_as_float(ow[u] << 16), __uint_as_float(dw[u] << 16), s);
    s = fmaf(__uint_as_float(ow[u] & 0xFFFF0000u), __uint_as_float(dw[u] & 0xFFFF0000u), s);
  }
  s = wave_sum(s);
  if (lane_id() == 0) a.delta[i] = s;
}

// ---------------------------------------------------------------- P and dS

__global__ __launch_bounds__(kThreads) void bwd_scores_kernel(MlaBwdArgs a) {
  __shared__ uint4 tiles[kBufs][kTileBufChunks];
  __shared__ int slots[kMaxSplitRows + 4 * kR];
  __shared__ int fallback;
  __shared__ float psums[2][kWaves * kR];

  const int r = blockIdx.x;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int ntiles = (a.k + kR - 1) / kR;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int h = wv * 16 + col;

  // Q^T (dims 32 ks + 8 g + [0, 8), 18 k-steps) and dO^T (16 k-steps) of head h
  bf16x8 qb[kKs], ob[kKv];
  {
    const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q) + ((long long)t * kH + h) * (kD * 2);
    const uint8_t *orow = reinterpret_cast<const uint8_t *>(a.dout) + ((long long)t * kH + h) * (kDv * 2);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qb[ks] = as_bf16x8(ld16(qrow + ks * 64 + g * 16));
#pragma unroll
    for (int ks = 0; ks < kKv; ++ks) ob[ks] = as_bf16x8(ld16(orow + ks * 64 + g * 16));
  }
  const float lse2 = a.lse[(long long)t * kH + h] * kLog2e;
  const float dlt = a.delta[(long long)r * kH + h];
  const float scale2 = a.sm_scale * kLog2e;
  fill_slots(a, t, n, ntiles, slots, &fallback);
  const int fb = fallback;

  const uint32_t qk_off = col * kRowStride + (g ^ swz(col)) * 16;
  const uint32_t tile_lds = lds_addr(&tiles[0][0]);
  constexpr uint32_t kTileBytes = kTileBufChunks * 16;
  const uint8_t *kv = reinterpret_cast<const uint8_t *>(a.kv);
  // head sums of tile tt's weights (wave 0, after the barrier that follows the tile)
  auto write_probs = [&](int tt) {
    if (a.probs != nullptr && lane < kR) {
      const int j = tt * kR + lane;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += psums[tt & 1][w * kR + lane];
      if (j < a.k) a.probs[(long long)t * a.k + j] = v * (1.f / kH);
    }
  };

  // the bf16 outputs of tile tt (held in registers, stored at the start of the
  // next iteration: stores count in the vector-memory counter, and stored after
  // the next tile's loads they would make its in-order wait drain them too)
  const int hs = head_slot(h);
  auto store_tile = [&](int tt, const float (&pw)[8], const float (&sd)[8]) {
    uint4 pk;
    pk.x = pack_bf16x2(sd[0], sd[1]);
    pk.y = pack_bf16x2(sd[2], sd[3]);
    pk.z = pack_bf16x2(sd[4], sd[5]);
    pk.w = pack_bf16x2(sd[6], sd[7]);
    // sm_scale dS^T of the tile for the dq product: head h, rows in k-slot order
    st16(a.ds_t + (((long long)r * ntiles + tt) * kH + h) * kR + g * 8, pk);
    // P and sm_scale dS per row for the row-gradient product
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = tt * kR + 16 * rb + 4 * g + v;
        if (j < a.k) {
          uint16_t *row = a.pd + ((long long)r * a.k + j) * (2 * kH);
          row[hs] = bf16_bits(pw[rb * 4 + v]);
          row[kH + hs] = bf16_bits(sd[rb * 4 + v]);
        }
      }
  };

  if (fb >= 0) {
    const TileCoords tc = tile_coords(wv, lane);
    issue_tile(tile_lds, kv, slots, 0, fb, wv, tc);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);         // query, dO operands and tile 0
    if (ntiles > 1) issue_tile(tile_lds + kTileBytes, kv, slots, kR, fb, wv, tc);
    int cur = 0;
    float pw[8], sd[8];
    for (int tt = 0; tt < ntiles; ++tt) {
      if (tt + 1 >= ntiles)
        __builtin_amdgcn_s_waitcnt(kWaitVm0 & ~0x0F00);
      else
        __builtin_amdgcn_s_waitcnt(wait_vm(kWaveLoads) & ~0x0F00);
      lds_barrier();
      if (tt > 0) store_tile(tt - 1, pw, sd);
      if (tt + 2 < ntiles) issue_tile(tile_lds + (cur == 0 ? 2 : cur - 1) * kTileBytes, kv, slots, (tt + 2) * kR, fb,
                                      wv, tc);
      if (tt > 0 && wv == 0) write_probs(tt - 1);
      const uint32_t tile = tile_lds + cur * kTileBytes;
      const int row_slot = slots[tt * kR + (lane & (kR - 1))];
      f32x4 st[2] = {zero_vec<f32x4>(), zero_vec<f32x4>()};
      f32x4 dp[2] = {zero_vec<f32x4>(), zero_vec<f32x4>()};
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        u32x4 fr[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) fr[rb] = *(lds_u32x4 *)(uintptr_t)(tile + qk_off + rb * 16 * kRowStride + ks * 64);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          st[rb] = mfma16_bf16(__builtin_bit_cast(bf16x8, fr[rb]), qb[ks], st[rb]);
          if (ks < kKv) dp[rb] = mfma16_bf16(__builtin_bit_cast(bf16x8, fr[rb]), ob[ks], dp[rb]);
        }
      }
      // rows 16 rb + 4 g + v of the tile; head h
      const uint32_t rowmask = (uint32_t)__ballot(lane < kR && row_slot >= 0);
      const uint32_t mine = rowmask >> (4 * g);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool on = (mine >> (16 * rb + v)) & 1u;
          const float p = on ? __builtin_amdgcn_exp2f(st[rb][v] * scale2 - lse2) : 0.f;
          pw[rb * 4 + v] = p;
          sd[rb * 4 + v] = a.sm_scale * (p * (dp[rb][v] - dlt));
        }
      // the weights summed over this wave's 16 heads, per row
      if (a.probs != nullptr) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = sum16(pw[i]);
        float mine_e = e[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mine_e = col == i ? e[i] : mine_e;
        if (col < 8) psums[tt & 1][wv * kR + 16 * (col >> 2) + 4 * g + (col & 3)] = mine_e;
      }
      cur = cur == 2 ? 0 : cur + 1;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    lds_barrier();
    store_tile(ntiles - 1, pw, sd);
    if (wv == 0) write_probs(ntiles - 1);
  } else {
    // no selected row: P = dS = 0
    for (int i = threadIdx.x; i < ntiles * kH * kR / 8; i += kThreads)
      st16(a.ds_t + (long long)r * ntiles * kH * kR + i * 8, make_uint4(0, 0, 0, 0));
    for (int i = threadIdx.x; i < a.k * 2 * kH / 8; i += kThreads)
      st16(a.pd + (long long)r * a.k * 2 * kH + i * 8, make_uint4(0, 0, 0, 0));
    if (a.probs != nullptr)
      for (int j = threadIdx.x; j < a.k; j += kThreads) a.probs[(long long)t * a.k + j] = 0.f;
  }
}

// ---------------------------------------------------------------- dq

__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(MlaBwdArgs a) {
  __shared__ uint4 tiles[kBufs][kTileBufChunks];
  __shared__ uint4 dst[kBufs][kH * kR * 2 / 16];   // sm_scale dS^T of each buffered tile (8 KB)
  __shared__ int slots[kMaxSplitRows + 4 * kR];
  __shared__ int fallback;

  const int r = blockIdx.x;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int ntiles = (a.k + kR - 1) / kR;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int h = wv * 16 + col;
  fill_slots(a, t, n, ntiles, slots, &fallback);
  const int fb = fallback;

  f32x4 acc[kDbAll];
#pragma unroll
  for (int db = 0; db < kDbAll; ++db) acc[db] = zero_vec<f32x4>();
  if (fb >= 0) {
    const int vc = col & 3;
    const uint32_t pv_row = (4 * g + (col >> 2)) * kRowStride + (vc & 1) * 8;
    const uint32_t pv_even = pv_row + (((vc >> 1)) ^ g) * 16;
    const uint32_t pv_odd = pv_row + ((2 + (vc >> 1)) ^ g) * 16;
    const uint32_t tile_lds = lds_addr(&tiles[0][0]);
    const uint32_t ds_lds = lds_addr(&dst[0][0]);
    constexpr uint32_t kTileBytes = kTileBufChunks * 16;
    constexpr uint32_t kDsBytes = kH * kR * 2;
    const uint8_t *kv = reinterpret_cast<const uint8_t *>(a.kv);
    // wave wv's 1 KB of a tile's dS^T (heads 16 wv.., 32 rows each): lane l's 16 bytes
    const uint16_t *ds_src = a.ds_t + ((long long)r * ntiles * kH + wv * 16) * kR + lane * 8;
    const TileCoords tc = tile_coords(wv, lane);
    auto issue = [&](int bi, int tt) {
      issue_tile(tile_lds + bi * kTileBytes, kv, slots, tt * kR, fb, wv, tc);
      lds_dma16(ds_src + (long long)tt * kH * kR, ds_lds + bi * kDsBytes + wv * 1024);
    };
    constexpr int kLoads = kWaveLoads + 1;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (ntiles > 1) issue(1, 1);
    int cur = 0;
    for (int tt = 0; tt < ntiles; ++tt) {
      if (tt + 1 >= ntiles)
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      else
        __builtin_amdgcn_s_waitcnt(wait_vm(kLoads));
      lds_barrier();
      if (tt + 2 < ntiles) issue(cur == 0 ? 2 : cur - 1, tt + 2);
      const uint32_t tile = tile_lds + cur * kTileBytes;
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, *(lds_u32x4 *)(uintptr_t)(ds_lds + cur * kDsBytes + (wv * 16 + col) * (kR * 2) + g * 16));
#pragma unroll
      for (int db = 0; db < kDbAll; ++db) {
        const uint32_t v0 = tile + ((db & 1) ? pv_odd : pv_even) + (db >> 1) * 64;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)v0);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)(v0 + 16 * kRowStride));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = mfma16_bf16(av, pb, acc[db]);
      }
      // the dS^T read and the transpose reads three MFMAs ahead of their use
      constexpr int kAhead = 3;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead + 1, 1);
#pragma unroll
      for (int i = 0; i < kDbAll - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 1);
      cur = cur == 2 ? 0 : cur + 1;
    }
  }
  float *drow = a.dq + ((long long)t * kH + h) * kD;
#pragma unroll
  for (int db = 0; db < kDbAll; ++db)
    *reinterpret_cast<float4 *>(drow + db * 16 + 4 * g) = make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
}

// ---------------------------------------------------------------- row gradients

// One workgroup per (query row r, block of 128 selected slots); wave w owns slots
// 16 w.. of the block.  C^T[dims, slots] = dO^T[dims, heads] P^T[heads, slots]
// + Q^T[dims, heads] (sm_scale dS)^T[heads, slots], over four groups of 32
// heads whose dO and Q rows are staged in LDS in the tile layout.
constexpr int kContribRows = 128;

// The Q and dO rows of a head group (32 heads) go into LDS by direct-to-LDS
// loads in the tile layout (position p: row p/74, slot p%74, holding data
// chunk slot ^ swz(row); pad slots load the row's first chunk, never read):
// 37 loads of 64 lanes per array, five for waves 0..4 and four for 5..7.  The
// arrays come in as eight stages (Q, then dO, of each group) through three
// buffers, two stages ahead of the one being multiplied.  Each stage also
// brings the block's operand of its product into LDS (sm_scale dS of the
// group's heads for a Q stage, P for a dO stage: 64 bytes per slot, one load
// per wave), so that every load of the loop is one the explicit waits count.
constexpr int kStageLoads = (kTileChunks + 63) / 64;   // 37
constexpr int kStages = 2 * (kH / 32);
constexpr int kStageBufs = 3;
constexpr int kOpChunks = kContribRows * 64 / 16;      // 512: 128 slots x 32 heads x 2 bytes
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

__global__ __launch_bounds__(kThreads) void bwd_contrib_kernel(MlaBwdArgs a) {
  // the staged Q and dO arrays and the operands of their products; at the end
  // the row gradients on their way out
  __shared__ uint4 sbuf[kStageBufs][kTileChunks];
  __shared__ uint4 opbuf[kStageBufs][kOpChunks];
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, each XCD with
  // its own L2.  When the rows divide by 8, XCD x takes rows x, x+8, ..., every
  // slot block of a row in turn, so a row's Q and dO come into one L2 once and
  // serve all of its blocks (the grid's own order spreads a row's blocks over
  // every XCD, each fetching the row).
  int r = blockIdx.y, bx = blockIdx.x;
  if ((a.rows & 7) == 0) {
    const int v = blockIdx.x + gridDim.x * blockIdx.y, k = v >> 3;
    r = (k / (int)gridDim.x) * 8 + (v & 7);
    bx = k - (k / (int)gridDim.x) * (int)gridDim.x;
  }
  const int t = a.q_begin + r;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int jb = bx * kContribRows + wv * 16;
  const bool active = jb < a.k;                 // k is a multiple of 16

  const int vc = col & 3;
  const uint32_t pv_row = (4 * g + (col >> 2)) * kRowStride + (vc & 1) * 8;
  const uint32_t pv_even = pv_row + (((vc >> 1)) ^ g) * 16;
  const uint32_t pv_odd = pv_row + ((2 + (vc >> 1)) ^ g) * 16;
  const uint8_t *qsrc = reinterpret_cast<const uint8_t *>(a.q) + (long long)t * kH * (kD * 2);
  const uint8_t *osrc = reinterpret_cast<const uint8_t *>(a.dout) + (long long)t * kH * (kDv * 2);
  // this wave's operand load: slot (wv * 64 + lane) / 4 of the block, 16-byte
  // part lane % 4 of its 32 heads (slots past k read the last row, unused)
  int oslot = bx * kContribRows + ((wv * 64 + lane) >> 2);
  oslot = oslot < a.k ? oslot : a.k - 1;
  const uint16_t *osl = a.pd + ((long long)r * a.k + oslot) * (2 * kH) + (lane & 3) * 8;
  const int nloads = wv < kStageLoads - 4 * kWaves ? 5 : 4;    // wave-uniform
  // Stage st: Q (even st) or dO (odd st) of head group st / 2, and its
  // product's operand, into buffer st % 3.
  auto stage = [&](int st) {
    const int hg = st >> 1, bi = st % kStageBufs;
    const uint32_t base = lds_addr(&sbuf[bi][0]);
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      if (j < nloads) {
        const int p = (j * kWaves + wv) * 64 + lane;
        const int row = p / kRowChunks, ch = p - row * kRowChunks;
        const uint32_t m = __builtin_amdgcn_readfirstlane(base + (j * kWaves + wv) * 1024);
        if ((st & 1) == 0)
          lds_dma16(qsrc + (long long)(32 * hg + row) * (kD * 2) + (ch < kDataChunks ? ch ^ swz(row) : 0) * 16, m);
        else
          lds_dma16(osrc + (long long)(32 * hg + row) * (kDv * 2) + (ch < kDv / 8 ? ch ^ swz(row) : 0) * 16, m);
      }
    }
    lds_dma16(osl + ((st & 1) == 0 ? kH : 0) + 32 * hg,
              __builtin_amdgcn_readfirstlane(lds_addr(&opbuf[bi][0]) + wv * 1024));
  };

  f32x4 acc[kDbAll];
#pragma unroll
  for (int db = 0; db < kDbAll; ++db) acc[db] = zero_vec<f32x4>();
  // the products of one stage, transpose reads kAhead MFMAs ahead of their use
  constexpr int kAhead = 3;
  auto product = [&](uint32_t lds, const bf16x8 &op, auto nblk) {
    constexpr int kN = decltype(nblk)::value;
#pragma unroll
    for (int db = 0; db < kN; ++db) {
      const uint32_t off = ((db & 1) ? pv_odd : pv_even) + (db >> 1) * 64;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)(lds + off));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)(lds + off + 16 * kRowStride));
      acc[db] = mfma16_bf16(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)), op,
                            acc[db]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
    for (int i = 0; i < kN - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 1);
  };
  // Stages 0 and 1, then at stage st stage st+2.  Before stage st is used, the
  // stage issued after it (nloads + 1 loads) may still be in flight.
  stage(0);
  stage(1);
  const uint32_t op_off = ((wv * 16 + col) * 4 + g) * 16;   // this lane's operand: slot jb + col, heads 8 g..
  // stage st landed for this wave; the barrier covers every wave's and orders
  // the reads of stage st-1 before its buffer refills
  auto land = [&](int st) {
    if (st + 1 < kStages) {
      if (nloads == 5)
        __builtin_amdgcn_s_waitcnt(wait_vm(6));
      else
        __builtin_amdgcn_s_waitcnt(wait_vm(5));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    lds_barrier();
    if (st + 2 < kStages) stage(st + 2);
  };
  auto operand = [&](int st) {
    return __builtin_bit_cast(bf16x8, *(lds_u32x4 *)(uintptr_t)(lds_addr(&opbuf[st % kStageBufs][0]) + op_off));
  };
#pragma unroll 1
  for (int hg = 0; hg < kH / 32; ++hg) {
    const int sq = 2 * hg, so = 2 * hg + 1;
    land(sq);
    if (active) product(lds_addr(&sbuf[sq % kStageBufs][0]), operand(sq), std::integral_constant<int, kDbAll>());
    land(so);
    if (active) product(lds_addr(&sbuf[so % kStageBufs][0]), operand(so), std::integral_constant<int, kDv / 16>());
  }
  // bf16 rows (their sum per key stays fp32), staged through LDS: a wave's 16
  // rows are 18 KB in one piece of the row-gradient array, written with 16-byte
  // stores, 1 KB per instruction (where the accumulator layout would give 32
  // bytes of each of 16 rows per instruction); eight rows at a time.
  constexpr int kOutStride = kD * 2 + 16;      // LDS bytes per staged row (one pad chunk)
  static_assert(kWaves * 8 * kOutStride <= kStageBufs * kTileChunks * 16, "the staged rows fit the operand buffers");
  lds_barrier();                               // every wave is done with the last stage's operands
  if (!active) return;
  const uint32_t stg = lds_addr(&sbuf[0][0]) + wv * 8 * kOutStride;
  uint8_t *dst = reinterpret_cast<uint8_t *>(a.contrib + ((long long)r * a.k + jb) * kD);
  constexpr int kRowPieces = kD * 2 / 16;      // 72 16-byte pieces per row
  // The staged rows are written as 8-byte and read back as 16-byte vectors of
  // another type: the empty asm statements with a memory clobber keep the
  // compiler from reordering or merging those accesses (it would otherwise take
  // the two types as never aliasing).
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    asm volatile("" ::: "memory");
    if ((col >> 3) == half) {
#pragma unroll
      for (int db = 0; db < kDbAll; ++db) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[db][0], acc[db][1]);
        pk[1] = pack_bf16x2(acc[db][2], acc[db][3]);
        *(lds_u32x2 *)(uintptr_t)(stg + (col & 7) * kOutStride + (16 * db + 4 * g) * 2) = pk;
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int it = 0; it < 8 * kRowPieces / 64; ++it) {
      const int c = it * 64 + lane, row = c / kRowPieces, w = c - row * kRowPieces;
      const u32x4 v = *(lds_u32x4 *)(uintptr_t)(stg + row * kOutStride + w * 16);
      st16(dst + (half * 8 * kRowPieces + c) * 16, make_uint4(v[0], v[1], v[2], v[3]));
    }
  }
}

// ---------------------------------------------------------------- the reduction into the cache rows

__global__ __launch_bounds__(256) void bwd_jpos_fill_kernel(MlaBwdArgs a) {
  const long long words = (long long)a.nkeys * a.jstride / 8;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < words; i += (long long)gridDim.x * 256)
    st16(a.jpos + i * 8, make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu));
}

__global__ __launch_bounds__(256) void bwd_jpos_scatter_kernel(MlaBwdArgs a) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.k) return;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int s = a.idx[(long long)t * a.k + j];
  if (s >= 0 && s < n && s < a.nkeys) a.jpos[(long long)s * a.jstride + r] = (uint16_t)j;
}

// One wave per key position s of sequence 0: the gradients of the rows that
// selected it, in ascending query order, into its cache row.
__global__ __launch_bounds__(256) void bwd_dkv_kernel(MlaBwdArgs a) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= a.nkeys) return;
  const int lane = lane_id();
  long long slot = s;
  if (a.sv.block_table != nullptr) {
    const int blk = a.sv.block_table[s >> 6];
    slot = (blk >= 0 && blk < a.sv.num_blocks) ? (long long)blk * 64 + (s & 63) : -1;
  }
  if (slot < 0) return;
  // lane l sums dims 8 l .. 8 l + 7 and, for l < 8, dims 512 + 8 l .. + 7: one
  // 16-byte load per row (two for lanes 0..7)
  constexpr int kExt = (kD - 512) / 8;          // lanes with a second chunk (8)
  const bool ext = lane < kExt;
  float acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.f;
  const uint16_t *jrow = a.jpos + (long long)s * a.jstride;
  auto add8 = [&](const uint4 &v, int o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[o + 2 * i] += __uint_as_float(w[i] << 16);
      acc[o + 2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  };
  // Up to four rows' loads in flight at a time (streaming loads: each row is
  // read once); they are added in ascending query order.
  constexpr int kAhead = 4;
  for (int t0 = 0; t0 < a.rows; t0 += 64) {
    const int jv = t0 + lane < a.rows ? (int)jrow[t0 + lane] : (int)kNoSlot;
    unsigned long long m = __ballot(jv != kNoSlot);
    while (m) {
      int bs[kAhead];
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        if (m) {
          bs[u] = __ffsll((long long)m) - 1;
          m &= m - 1;
          cnt = u + 1;
        } else {
          bs[u] = bs[0];
        }
      }
      uint4 x[kAhead], y[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        const int j = __builtin_amdgcn_readlane(jv, bs[u]);
        const uint16_t *c = a.contrib + ((long long)(t0 + bs[u]) * a.k + j) * kD + 8 * lane;
        x[u] = ld16_stream(c);
        y[u] = ext ? ld16_stream(c + 512) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        if (u < cnt) {
          add8(x[u], 0);
          add8(y[u], 8);
        }
    }
  }
  float *drow = a.dkv + slot * kD;
  float4 *d0 = reinterpret_cast<float4 *>(drow + 8 * lane);
  float4 *d1 = reinterpret_cast<float4 *>(drow + 512 + 8 * lane);
  if (a.first) {
    d0[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    d0[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (ext) {
      d1[0] = make_float4(acc[8], acc[9], acc[10], acc[11]);
      d1[1] = make_float4(acc[12], acc[13], acc[14], acc[15]);
    }
  } else {
    const float4 o0 = d0[0], o1 = d0[1];
    d0[0] = make_float4(o0.x + acc[0], o0.y + acc[1], o0.z + acc[2], o0.w + acc[3]);
    d0[1] = make_float4(o1.x + acc[4], o1.y + acc[5], o1.z + acc[6], o1.w + acc[7]);
    if (ext) {
      const float4 p0 = d1[0], p1 = d1[1];
      d1[0] = make_float4(p0.x + acc[8], p0.y + acc[9], p0.z + acc[10], p0.w + acc[11]);
      d1[1] = make_float4(p1.x + acc[12], p1.y + acc[13], p1.z + acc[14], p1.w + acc[15]);
    }
  }
}

// ---------------------------------------------------------------- Stage-2 indexer KL

constexpr int kKlThreads = 256;
constexpr int kKlMaxWords = 262144 / 32;

__device__ float block_max(float v, float *red) {
  v = wave_max(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kKlThreads / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

__device__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kKlThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// One workgroup per query: softmax of the scores over the selected positions,
// the KL term against the target, and dL/dI written over the whole score row
// (softmax - p on the selection, 0 elsewhere).
__global__ __launch_bounds__(kKlThreads) void sparse_kl_kernel(SparseKlArgs a) {
  __shared__ uint32_t bits[kKlMaxWords];
  __shared__ float ival[kTopkMaxK];
  __shared__ float red[kKlThreads / 64];
  const int r = blockIdx.x;
  const int n = a.sv.candidates(r);
  float *srow = a.scores + (long long)r * a.ld;
  const int32_t *irow = a.idx + (long long)r * a.k;
  const float *prow = a.probs + (long long)r * a.k;
  const int words = (n + 31) >> 5;
  for (int i = threadIdx.x; i < words; i += kKlThreads) bits[i] = 0u;
  __syncthreads();
  float mx = neg_inf();
  for (int j = threadIdx.x; j < a.k; j += kKlThreads) {
    const int s = irow[j];
    float v = neg_inf();
    if (s >= 0 && s < n) {
      v = srow[s];
      atomicOr(&bits[s >> 5], 1u << (s & 31));
      mx = fmaxf(mx, v);
    }
    ival[j] = v;
  }
  mx = block_max(mx, red);
  float se = 0.f;
  for (int j = threadIdx.x; j < a.k; j += kKlThreads)
    if (ival[j] != neg_inf()) se += __expf(ival[j] - mx);
  se = block_sum(se, red);
  const float lse = mx + __logf(se);
  float kl = 0.f;
  for (int j = threadIdx.x; j < a.k; j += kKlThreads) {
    const float p = prow[j];
    if (ival[j] != neg_inf() && p > 0.f) kl += p * (__logf(p) - (ival[j] - lse));
  }
  kl = block_sum(kl, red);
  // 0 at every position outside the selection, then the gradient on it
  for (long long s = threadIdx.x; s < a.ld; s += kKlThreads)
    if (s >= n || !((bits[s >> 5] >> (s & 31)) & 1u)) srow[s] = 0.f;
  for (int j = threadIdx.x; j < a.k; j += kKlThreads)
    if (ival[j] != neg_inf()) srow[irow[j]] = __expf(ival[j] - lse) - prow[j];
  if (threadIdx.x == 0) a.loss[r] = mx == neg_inf() ? 0.f : kl;
}

}  // namespace

hipError_t launch_sparse_mla_bwd(const MlaBwdArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)(((long long)a.rows * kH + 3) / 4)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_scores_kernel, dim3(a.rows), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(a.rows), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL(bwd_contrib_kernel, dim3((a.k + kContribRows - 1) / kContribRows, a.rows), dim3(kThreads), 0, st,
                     a);
  const long long words = (long long)a.nkeys * a.jstride / 8;
  hipLaunchKernelGGL(bwd_jpos_fill_kernel, dim3((unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096)),
                     dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_jpos_scatter_kernel, dim3((a.k + 255) / 256, a.rows), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3((a.nkeys + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sparse_kl(const SparseKlArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(sparse_kl_kernel, dim3(a.rows), dim3(kKlThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

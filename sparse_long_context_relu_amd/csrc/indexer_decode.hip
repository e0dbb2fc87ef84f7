// Lightning indexer: I(t,s) = sum_j w(t,j) * ReLU(q(t,j) . k(s)) for every
// candidate s of query t ("DeepSeek V3.2: How Far Can Open Models Go If You
// Actually Try?", section 3.1, indexer equation; news.han.ihouse.idv.tw
// article 1495, DSA section: ReLU for throughput, FP8 execution).
//
// bf16 / e4m3fn (H_I = 64, d_I = 128): the q.k contraction runs on MFMA with
// the 64 heads of one query as the M dimension and 32 keys as N; the ReLU,
// the head weights and the head sum are applied to the accumulators in
// registers, so only one fp32 score per (query, key) leaves the kernel.
//   * decode tiling: one query per workgroup row of the grid, the candidate
//     keys split into chunks across workgroups; each wave streams 32-key
//     tiles straight from HBM into MFMA operand registers.
//   (this file; the prefill tiling and the fp32 path are in indexer.hip)
#include "indexer_common.h"

namespace dsa {
namespace {

constexpr int kDecodeChunk = 2048;  // keys per decode workgroup

// ------------------------------------------------------------------ decode tiling
//
// Each wave owns 32-key tiles (kRowBytes * 32 contiguous bytes: a tile never
// straddles a 64-token block).  It loads a tile with fully coalesced 16-byte
// loads -- one instruction covers whole rows -- into registers one tile ahead,
// stores it into a wave-private LDS buffer with the 16-byte chunks of row r
// XOR-swizzled by r, and reads the MFMA operands (lane: key l%32, chunks of
// k-group l/32) back from there without bank conflicts.

constexpr int kDecodeWaves = 4;

template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void indexer_decode_kernel(
    IndexerArgs a) {
  typedef IdxTraits<DT> Tr;
  constexpr int kChunks = Tr::kRowBytes / 16;       // 16-byte chunks per key row (16 bf16, 8 fp8)
  constexpr int kPer = 32 * kChunks / 64;           // chunks each lane loads per tile (8 or 4)
  __shared__ uint4 wtile[kDecodeWaves][32 * kChunks];
  __shared__ uint32_t lh[kTopkBins];

  const int r = blockIdx.y;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const int c0 = blockIdx.x * kDecodeChunk;
  float *srow = a.scores + (long long)r * a.ld;
  const long long cend = c0 + kDecodeChunk < a.ld ? c0 + kDecodeChunk : a.ld;
  if (a.fill_masked) {
    for (long long s = (c0 > n ? c0 : n) + threadIdx.x; s < cend; s += blockDim.x) srow[s] = neg_inf();
  }
  if (c0 >= n) return;
  const int c1 = c0 + kDecodeChunk < n ? c0 + kDecodeChunk : n;

  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const int g = lane >> 5, col = lane & 31;
  // Start-up, ordered so that the first tiles are in flight after one
  // block-table latency: the query operands and weights are loaded first (the
  // oldest loads), then the block-table entries of the chunk for the LDS copy
  // used from the third tile on, then the wave's first two tiles, whose slots
  // come straight from the table through the scalar cache.
  typename Tr::Op qa[2][Tr::kSteps];
  float wt[2][16];
  load_query<DT>(a, t, col, g, qa, wt);
  // Slot of the first key of each 64-token block of this chunk (-1: absent),
  // kept in LDS, so a tile's lookup in the loop is an LDS read that never waits
  // on the vector-memory counter (which also counts the score stores in flight).
  // Only the raw entry is loaded here; it is checked after the tile loads are
  // issued, so that no wait is placed before them.
  __shared__ long long blk0[kDecodeChunk / 64];
  const int my_s = c0 + (int)threadIdx.x * 64;
  const bool my_fill = threadIdx.x < kDecodeChunk / 64 && my_s < c1;
  int my_raw = 0;
  if (my_fill && a.sv.block_table != nullptr)
    my_raw = a.sv.block_table[(long long)b * a.sv.max_blocks + (my_s >> 6)];

  const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k_cache);
  uint4 *tile = wtile[wv];
  auto tile_slot = [&](int base) -> long long {
    const long long b0 = blk0[(base - c0) >> 6];
    return b0 >= 0 ? b0 + (base & 63) : -1;
  };
  // The same lookup for the wave's first two tiles, before the LDS copy exists:
  // both block-table entries are read at once, wave-uniformly, through the
  // scalar cache (a tile past the chunk reads the chunk's first entry and is
  // marked absent).
  auto first_slots = [&](int bA, int bB, long long &sA, long long &sB) {
    if (a.sv.block_table == nullptr) {
      sA = bA < c1 ? (long long)b * a.sv.max_seq_len + bA : -1;
      sB = bB < c1 ? (long long)b * a.sv.max_seq_len + bB : -1;
      return;
    }
    const __attribute__((address_space(4))) int32_t *bt =
        (const __attribute__((address_space(4))) int32_t *)(a.sv.block_table + (long long)b * a.sv.max_blocks);
    const int kA = bt[__builtin_amdgcn_readfirstlane((bA < c1 ? bA : c0) >> 6)];
    const int kB = bt[__builtin_amdgcn_readfirstlane((bB < c1 ? bB : c0) >> 6)];
    sA = (bA < c1 && kA >= 0 && kA < a.sv.num_blocks) ? (long long)kA * 64 + (bA & 63) : -1;
    sB = (bB < c1 && kB >= 0 && kB < a.sv.num_blocks) ? (long long)kB * 64 + (bB & 63) : -1;
  };
  // Coalesced fetch of the tile at key `base`: lane l takes chunk (i*64 + l) of
  // the tile for i < kPer, i.e. row (i*64 + l) / kChunks.  A tile lies inside
  // one 64-token block, so one wave-uniform lookup gives the slot of its first
  // row and the others follow.  Rows past c1 or in an absent block load zeros.
  // Every lane always loads (absent rows read the chunk's first row instead) and
  // `put` zeroes what is absent: no branches, and no register initialised
  // before a load that might be skipped.
  auto fetch = [&](int base, long long sl0, uint4 (&st)[kPer]) {
    const long long first = sl0 >= 0 ? sl0 : 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = i * 64 + lane;
      const int row = p / kChunks, ch = p % kChunks;
      const int rr = base + row < c1 ? row : 0;
      st[i] = ld16(kbase + (first + rr) * Tr::kRowBytes + ch * 16);
    }
  };
  auto put = [&](const uint4 (&st)[kPer], int base, long long sl0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = i * 64 + lane;
      const int row = p / kChunks, ch = p % kChunks;
      const bool ok = sl0 >= 0 && base + row < c1;
      tile[row * kChunks + (ch ^ (row & (kChunks - 1)))] = ok ? st[i] : make_uint4(0, 0, 0, 0);
    }
  };
  // Two tiles in flight per wave: stage A holds tile i+1 (loaded one tile ago),
  // stage B receives tile i+2 while tile i is multiplied from LDS.  The loop is
  // unrolled by two so the stages keep fixed registers.
  constexpr int kStep = kDecodeWaves * 32;
  uint4 sa[kPer], sb[kPer];
  int base = c0 + wv * 32;
  long long sl0, sla, slb = -1;
  first_slots(base, base + kStep, sl0, sla);
  fetch(base, sl0, sb);                            // tile 0, through stage B
  fetch(base + kStep, sla, sa);                    // tile 1
  // first radix digit of the top-k, counted per workgroup and added to the row's bins
  const bool hist = a.hist_mode == 1;
  if (hist)
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
  if (threadIdx.x < kDecodeChunk / 64) {
    long long v = -1;
    if (my_fill) {
      if (a.sv.block_table == nullptr)
        v = (long long)b * a.sv.max_seq_len + my_s;
      else if (my_raw >= 0 && my_raw < a.sv.num_blocks)
        v = (long long)my_raw * 64;
    }
    blk0[threadIdx.x] = v;
  }
  // LDS-only barrier: the tile loads stay in flight across it.
  lds_barrier();
  // The query, weight and table loads and tile 0 have landed once at most the
  // loads of tile 1 are outstanding; draining them here keeps every wait for
  // them out of the loop (where it would also wait for the prefetch).
  __builtin_amdgcn_s_waitcnt(wait_vm(kPer));
  put(sb, base, sl0);
  // Scores of the tile resident in LDS (valid in every lane for key col).
  auto consume = [&]() {
    typename Tr::Op kb[Tr::kSteps];
    const uint4 *trow = tile + col * kChunks;
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) {
      if constexpr (DT == DSA_BF16) {
        kb[ks] = __builtin_bit_cast(typename Tr::Op, trow[(g * 8 + ks) ^ (col & 15)]);
      } else {
        const int ch = g * 4 + ks * 2;
        const uint4 lo = trow[ch ^ (col & 7)], hi = trow[(ch + 1) ^ (col & 7)];
        typename Tr::Op o;
        o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
        o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
        kb[ks] = o;
      }
    }
    f32x16 c0a = zero_vec<f32x16>(), c1a = zero_vec<f32x16>();
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) {
      c0a = Tr::mma(qa[0][ks], kb[ks], c0a);
      c1a = Tr::mma(qa[1][ks], kb[ks], c1a);
    }
    return head_reduce(c0a, c1a, wt);
  };
  auto emit = [&](int tb, long long tsl, float sc) {
    const int s = tb + col;
    if (g == 0 && s < c1) {
      const float v = tsl >= 0 ? sc * key_scale<DT>(a, tsl + col) : neg_inf();
      srow[s] = v;
      if (hist) atomicAdd(&lh[score_key(v) >> 21], 1u);
    }
  };
  for (; base < c1; base += 2 * kStep) {
    const int b1 = base + kStep, b2 = base + 2 * kStep, b3 = base + 3 * kStep;
    // LDS: tile `base` (slot sl0); stage A: tile b1 (sla); tile b2 -> stage B.
    // The fetch is unconditional (past c1 it reads slot 0 and is discarded), so
    // the compiler's wait counts stay exact on every path.
    slb = b2 < c1 ? tile_slot(b2) : -1;
    fetch(b2, slb, sb);
    float sc = consume();
    put(sa, b1, sla);                              // the LDS reads above completed before the MFMAs
    emit(base, sl0, sc);
    if (b1 >= c1) break;
    // LDS: tile b1; stage B: tile b2 (slb); tile b3 -> stage A
    const long long s1 = sla;
    sla = b3 < c1 ? tile_slot(b3) : -1;
    fetch(b3, sla, sa);
    sc = consume();
    put(sb, b2, slb);                              // past c1 this stores zeros that are never read
    emit(b1, s1, sc);
    sl0 = slb;
  }
  if (hist) {
    __syncthreads();
    uint32_t *hrow = a.hist + (long long)r * a.hist_stride;
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x)
      if (lh[i]) atomicAdd(&hrow[i], lh[i]);
  }
}

}  // namespace

hipError_t launch_index_decode(const IndexerArgs &a, hipStream_t st) {
  const long long span = a.fill_masked ? a.ld : a.sv.max_ctx;
  dim3 grid((unsigned)((span + kDecodeChunk - 1) / kDecodeChunk), (unsigned)a.rows);
  if (a.dtype == DSA_BF16)
    hipLaunchKernelGGL(indexer_decode_kernel<DSA_BF16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(indexer_decode_kernel<DSA_FP8_E4M3FN>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

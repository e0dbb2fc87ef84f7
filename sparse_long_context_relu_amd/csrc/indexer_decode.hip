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
//     keys split into chunks across workgroups; each wave streams 8 KB key
//     tiles (32 bf16 or 64 e4m3fn keys) from HBM through registers and LDS
//     into MFMA operands.
//   (this file; the prefill tiling and the fp32 path are in indexer.hip)
#include "indexer_common.h"

namespace dsa {
namespace {

// Keys per decode workgroup: 2048, halved (down to 256) while the grid would
// have fewer than 1024 workgroups, so that short contexts still fill the chip.
constexpr int kDecodeChunk = 2048;
constexpr int kDecodeMinChunk = 256;
constexpr int kDecodeMinGrid = 1024;

// Length-balanced decode grid (at most kBalRows rows, no -inf fill).  With
// ragged contexts the fixed grid leaves a partial last round of workgroups on
// the chip (U[32K, 128K] contexts: ~1118 chunks of 2048 keys on 512 slots,
// 2.18 rounds).  Instead the batch is cut into about G = slots * round(K /
// (slots * 4096)) workgroups (at least `slots`), K the total candidate count:
// row r gets g_r = max(1, floor(n_r G / K)) of them (at most G + 2 rows in all,
// allowing one unit of fp64 rounding per row), each a 64-aligned chunk of
// ceil(n_r / g_r) keys, so the grid runs in whole rounds.  Every wave computes
// this schedule from the rows' candidate counts itself.  A chunk stays below
// kBlk0 * 64 keys: n_r / g_r < 2 K / G and K / G < 1.5 * 4096.  (Measured
// against a 2048-key target: the same on bf16 keys, e4m3fn 67.4 -> 65.0 us on
// 32 x U[32K, 128K]; a 1024-key target was slower on both.)
constexpr int kBalRows = 256;
constexpr int kBalTarget = 4096;
constexpr int kBlk0 = 256;                    // 64-token block entries a chunk may span

// keys < 2^40 and slots * kBalTarget < 2^31: the fp64 quotient floors exactly
__host__ __device__ inline long long bal_grid(long long keys, int slots) {
  const long long rounds = (long long)floor((double)(keys + (long long)slots * (kBalTarget / 2)) /
                                            (double)((long long)slots * kBalTarget));
  return (long long)slots * (rounds > 1 ? rounds : 1);
}

// ------------------------------------------------------------------ decode tiling
//
// Each wave owns 8 KB tiles: 32 bf16 keys or 64 e4m3fn keys, contiguous
// bytes that never straddle a 64-token block, so both types keep the same
// bytes in flight.  A wave loads a tile with fully coalesced 16-byte loads --
// one instruction covers whole rows -- into registers two tiles ahead, stores
// it into a wave-private LDS buffer with the 16-byte chunks of row r
// XOR-swizzled by r, and reads the MFMA operands (lane: key l%32 of a 32-key
// group, chunks of k-group l/32) back from there without bank conflicts.

constexpr int kDecodeWaves = 4;

template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void indexer_decode_kernel(
    IndexerArgs a) {
  typedef IdxTraits<DT> Tr;
  constexpr int kChunks = Tr::kRowBytes / 16;       // 16-byte chunks per key row (16 bf16, 8 fp8)
  constexpr int kTileKeys = 8192 / Tr::kRowBytes;   // keys per 8 KB tile (32 bf16, 64 fp8)
  constexpr int kGroups = kTileKeys / 32;           // 32-key MFMA groups per tile
  constexpr int kPer = kTileKeys * kChunks / 64;    // chunks each lane loads per tile (8)
  __shared__ uint4 wtile[kDecodeWaves][kTileKeys * kChunks];
  __shared__ uint32_t lh[kTopkBins];

  int r, chunk, c0, n;
  if (a.balanced) {
    // Schedule of the length-balanced grid, computed by every wave on its own
    // (no barrier, no LDS): lane l holds rows rpl*l .. rpl*l + rpl - 1, rpl =
    // ceil(rows / 64) <= 4.  The divisions run in fp64 (a 64-bit integer
    // division is a long instruction sequence here); every quotient they give
    // is a well-separated integer quotient (below 2^31, divisors below 2^31),
    // and the workgroup count of a row is fixed up in integers so that its
    // chunks tile [0, n_r) exactly.
    const int ln = lane_id();
    const int rpl = (a.rows + 63) >> 6;
    int nr[4];
    long long k = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = rpl * ln + j;
      nr[j] = j < rpl && row < a.rows ? a.sv.candidates(a.q_begin + row) : 0;
      k += nr[j];
    }
    for (int m = 32; m >= 1; m >>= 1) k += __shfl_xor(k, m, 64);
    if (k == 0) return;
    const long long G = bal_grid(k, a.slots);
    const double share = (double)G / (double)k;
    int cj[4], mj[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cj[j] = mj[j] = 0;
      if (j < rpl && nr[j] > 0) {
        const double gd = floor((double)nr[j] * share);
        const int g = gd > 1.0 ? (int)gd : 1;
        const int c = (int)ceil((double)nr[j] / (double)g);
        cj[j] = (c + 63) & ~63;
        int m = (int)ceil((double)nr[j] / (double)cj[j]);
        if ((long long)m * cj[j] < nr[j]) ++m;
        if (m > 1 && (long long)(m - 1) * cj[j] >= nr[j]) --m;
        mj[j] = m;
      }
      local += mj[j];
    }
    int x = local;                               // inclusive prefix of the counts over the lanes
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (ln >= d) x += y;
    }
    int first = x - local, hit = -1, hc = 0, hc0 = 0, hn = 0;
    const int id = (int)blockIdx.x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (mj[j] > 0 && id >= first && id < first + mj[j]) {
        hit = rpl * ln + j;
        hc = cj[j];
        hc0 = (id - first) * cj[j];
        hn = nr[j];
      }
      first += mj[j];
    }
    const unsigned long long owner = __ballot(hit >= 0);
    if (owner == 0) return;                      // past the last row's workgroups
    const int src = __builtin_amdgcn_readfirstlane(__ffsll((long long)owner) - 1);
    r = __builtin_amdgcn_readlane(hit, src);
    chunk = __builtin_amdgcn_readlane(hc, src);
    c0 = __builtin_amdgcn_readlane(hc0, src);
    n = __builtin_amdgcn_readlane(hn, src);
  } else {
    r = blockIdx.y;
    chunk = a.chunk;
    c0 = blockIdx.x * chunk;
    n = a.sv.candidates(a.q_begin + r);
  }
  const int t = a.q_begin + r;
  const int b = a.sv.seq_of(t);
  float *srow = a.scores + (long long)r * a.ld;
  const long long cend = c0 + chunk < a.ld ? c0 + chunk : a.ld;
  if (a.fill_masked) {
    for (long long s = (c0 > n ? c0 : n) + threadIdx.x; s < cend; s += blockDim.x) srow[s] = neg_inf();
  }
  if (c0 >= n) return;
  const int c1 = c0 + chunk < n ? c0 + chunk : n;

  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar loop control
  const int g = lane >> 5, col = lane & 31;
  const int ek = kGroups == 2 ? lane : col;         // key of the tile whose score this lane stores
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
  __shared__ long long blk0[kBlk0];
  const int my_s = c0 + (int)threadIdx.x * 64;
  const bool my_fill = threadIdx.x < chunk / 64 && my_s < c1;
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
  // Coalesced fetch of the tile at key `base` (streaming loads: each key is
  // read once per query): lane l takes chunk (i*64 + l) of
  // the tile for i < kPer, i.e. row (i*64 + l) / kChunks.  A tile lies inside
  // one 64-token block, so one wave-uniform lookup gives the slot of its first
  // row and the others follow.  Rows past c1 or in an absent block load zeros.
  // Every lane always loads (absent rows read the chunk's first row instead) and
  // `put` zeroes what is absent: no branches, and no register initialised
  // before a load that might be skipped.
  // For e4m3fn the scale of key ek is loaded with the tile, ahead of its rows,
  // so the wait for the rows covers it too.
  auto fetch = [&](int base, long long sl0, uint4 (&st)[kPer], float &scl) {
    const long long first = sl0 >= 0 ? sl0 : 0;
    if constexpr (DT != DSA_BF16) scl = __builtin_nontemporal_load(&a.k_scale[first + (base + ek < c1 ? ek : 0)]);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = i * 64 + lane;
      const int row = p / kChunks, ch = p % kChunks;
      const int rr = base + row < c1 ? row : 0;
      st[i] = ld16_stream(kbase + (first + rr) * Tr::kRowBytes + ch * 16);
    }
  };
  // Absent rows are zeroed with an opaque all-ones / zero mask: as a select the
  // compiler lowers this to branches with the load waits inside them, and the
  // merged wait state at the loop head then drains the other stage as well.
  auto put = [&](uint4 (&st)[kPer], int base, long long sl0, float &scl) {
    if constexpr (DT != DSA_BF16) asm volatile("" : "+v"(scl));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = i * 64 + lane;
      const int row = p / kChunks, ch = p % kChunks;
      uint32_t m = sl0 >= 0 && base + row < c1 ? ~0u : 0u;
      asm volatile("" : "+v"(m));
      const uint4 v = st[i];
      tile[row * kChunks + (ch ^ (row & (kChunks - 1)))] = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
    }
  };
  // Two tiles in flight per wave: stage A holds tile i+1 (loaded one tile ago),
  // stage B receives tile i+2 while tile i is multiplied from LDS.  The loop is
  // unrolled by two so the stages keep fixed registers.
  constexpr int kStep = kDecodeWaves * kTileKeys;
  uint4 sa[kPer], sb[kPer];
  float ka = 1.f, kb = 1.f;                        // key scales of stages A and B (e4m3fn)
  int base = c0 + wv * kTileKeys;
  long long sl0, sla, slb = -1;
  first_slots(base, base + kStep, sl0, sla);
  fetch(base, sl0, sb, kb);                        // tile 0, through stage B
  fetch(base + kStep, sla, sa, ka);                // tile 1
  // first radix digit of the top-k, counted per workgroup and added to the row's bins
  const bool hist = a.hist_mode == 1;
  if (hist)
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
  if (threadIdx.x < kBlk0) {
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
  __builtin_amdgcn_s_waitcnt(wait_vm(kPer + (DT != DSA_BF16)));
  put(sb, base, sl0, kb);
  float kt = kb;                                   // key scale of the tile in LDS
  // Half-wave head partials of 32-key group h of the tile resident in LDS.
  auto group = [&](int h) {
    typename Tr::Op kb[Tr::kSteps];
    const uint4 *trow = tile + (h * 32 + col) * kChunks;
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
    return head_partial(c0a, c1a, wt);
  };
  // Score of key ek of the tile resident in LDS.
  auto consume = [&]() {
    if constexpr (kGroups == 1) {
      const float p = group(0);
      return p + shfl_xor(p, 32);
    } else {
      return pair_head_total(group(0), group(1));
    }
  };
  auto emit = [&](int tb, long long tsl, float sc, float ksc) {
    const int s = tb + ek;
    if ((kGroups == 2 || g == 0) && s < c1) {
      const float v = tsl >= 0 ? (DT == DSA_BF16 ? sc : sc * ksc) : neg_inf();
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
    fetch(b2, slb, sb, kb);
    float sc = consume();
    put(sa, b1, sla, ka);                          // the LDS reads above completed before the MFMAs
    emit(base, sl0, sc, kt);
    kt = ka;
    // LDS: tile b1; stage B: tile b2 (slb); tile b3 -> stage A.  No exit in
    // between: past c1 tile b1 is all zeros and its scores are not stored (an
    // exit here would reach the loop head with stage B's loads outstanding on
    // that path, and the wait there would drain stage A every iteration).
    const long long s1 = sla;
    sla = b3 < c1 ? tile_slot(b3) : -1;
    fetch(b3, sla, sa, ka);
    sc = consume();
    put(sb, b2, slb, kb);                          // past c1 this stores zeros that are never read
    emit(b1, s1, sc, kt);
    kt = kb;
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
  IndexerArgs b = a;
  b.chunk = kDecodeChunk;
  b.balanced = 0;
  b.slots = 0;
  dim3 grid;
  // Two workgroups per CU run at once (two waves per SIMD, four-wave groups).
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      return hipErrorInvalidDevice;
    cus[dev] = c;
  }
  // The schedule costs each workgroup one dependent load of the rows' counts
  // before its first tile (about 2 us on a 16 x 8K batch, one round of 512
  // workgroups); it is taken where the fixed grid would need two rounds or more.
  const long long fixed_wgs = (long long)a.rows * ((span + kDecodeChunk - 1) / kDecodeChunk);
  if (!a.fill_masked && a.rows <= kBalRows && fixed_wgs >= 4LL * cus[dev]) {
    b.balanced = 1;
    b.slots = 2 * cus[dev];
    // the workgroups' own G never exceeds the first term (K <= rows * max_ctx, bal_grid is
    // monotone), and the rows' counts sum to at most G + 2 rows
    grid = dim3((unsigned)(bal_grid((long long)a.rows * span, b.slots) + 2 * a.rows), 1u);
  } else {
    while (b.chunk > kDecodeMinChunk && (long long)a.rows * ((span + b.chunk - 1) / b.chunk) < kDecodeMinGrid)
      b.chunk >>= 1;
    grid = dim3((unsigned)((span + b.chunk - 1) / b.chunk), (unsigned)a.rows);
  }
  if (a.dtype == DSA_BF16)
    hipLaunchKernelGGL(indexer_decode_kernel<DSA_BF16>, grid, dim3(256), 0, st, b);
  else
    hipLaunchKernelGGL(indexer_decode_kernel<DSA_FP8_E4M3FN>, grid, dim3(256), 0, st, b);
  return hipGetLastError();
}

}  // namespace dsa

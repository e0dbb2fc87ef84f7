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
//   * prefill tiling: 8 consecutive queries per workgroup (one per wave)
//     share 16 KB key tiles gathered straight into LDS, three deep.
// e4m3fn: scores = k_scale(s) * sum_j (w_j q_scale_j) ReLU(q8_j . k8_s),
// exact because ReLU(a x) = a ReLU(x) for a > 0.
//   (the decode tiling is in indexer_decode.hip)
#include <type_traits>

#include "indexer_common.h"

namespace dsa {
namespace {

// ------------------------------------------------------------------ prefill tiling

constexpr int kPrefillQ = 8;     // queries (waves) per workgroup


// Slot of the first key of the 64-token block holding key `s` of sequence 0,
// or -1 when the block is outside the pool.  `s` is wave-uniform; a paged
// lookup goes through the scalar cache (the block table is read-only here), so
// it never waits on the vector-memory counter that tracks the tile loads.
__device__ __forceinline__ long long block_slot(const SeqView &sv, int s) {
  if (sv.block_table == nullptr) return (long long)(s & ~63);
  const __attribute__((address_space(4))) int32_t *bt =
      (const __attribute__((address_space(4))) int32_t *)sv.block_table;
  const int blk = bt[__builtin_amdgcn_readfirstlane(s >> 6)];
  return (blk < 0 || blk >= sv.num_blocks) ? -1 : (long long)blk * 64;
}

// kHist: also count the row's scores into the top-k's first-digit histogram
// (the fused forward's hist_mode 2); kPaged: the cache is a block pool read
// through the block table (else one contiguous array).  Both are compile-time
// switches so that the group loop holds no branch and, for a contiguous cache,
// no block bookkeeping.
template <int DT, bool kHist, bool kPaged>
__global__ __launch_bounds__(kPrefillQ * 64) void indexer_prefill_kernel(IndexerArgs a) {
  typedef IdxTraits<DT> Tr;
  constexpr int kChunks = Tr::kRowBytes / 16;           // 16-byte chunks per key row (16 or 8)
  // keys per LDS tile: 64 for bf16, 128 for e4m3fn (the same 16 KB)
  constexpr int kPrefillKeys = DT == DSA_BF16 ? 64 : 128;
  constexpr int kBlocks = kPrefillKeys / 64;            // 64-token blocks per tile
  constexpr int kTileChunks = kPrefillKeys * kChunks;   // 1024 chunks per tile
  constexpr int kLoads = kTileChunks / (kPrefillQ * 64);   // tile loads per wave per tile (2)
  constexpr int kScaleKeys = kPrefillKeys / kPrefillQ;   // e4m3fn key scales each wave loads (16)
  constexpr bool kScaled = DT == DSA_FP8_E4M3FN;
  constexpr int kWaveLoads = kLoads + (kScaled ? 1 : 0);   // + the key scales (fp8)
  constexpr int kBufs = 3;                              // tiles tt+1, tt+2 stream in while tt is used
  constexpr uint32_t kTileBytes = kTileChunks * 16;
  __shared__ uint4 tile[kBufs][kTileChunks];
  // fp8 key scales: wave wv's load fills [wv][0, 64) of a buffer, its first
  // kScaleKeys entries being keys kScaleKeys wv + [0, kScaleKeys) of the tile
  __shared__ float kscale[kBufs][kScaled ? kPrefillQ * 64 : 1];

  const int grp = gridDim.x - 1 - blockIdx.x;           // longest rows first
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int r = grp * kPrefillQ + wv;
  const bool row_ok = r < a.rows;
  const int t = a.q_begin + (row_ok ? r : a.rows - 1);
  const int n = row_ok ? a.sv.candidates(t) : 0;
  int nmax = 0;
  for (int i = 0; i < kPrefillQ; ++i) {
    const int ri = grp * kPrefillQ + i;
    if (ri < a.rows) {
      const int ni = a.sv.candidates(a.q_begin + ri);
      nmax = ni > nmax ? ni : nmax;
    }
  }
  nmax = __builtin_amdgcn_readfirstlane(nmax);
  float *srow = a.scores + (long long)(row_ok ? r : 0) * a.ld;

  typename Tr::Op qa[2][Tr::kSteps];
  float wt[2][16];
  load_query<DT>(a, t, col, g, qa, wt);

  // first radix digit of the top-k: each wave owns its query row's bins
  __shared__ uint32_t wh[kPrefillQ][kHist ? kTopkBins : 1];
  if (kHist)
    for (int i = lane; i < kTopkBins; i += 64) wh[wv][i] = 0u;

  const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k_cache);
  // Tile gather: buffer loads straight into LDS.  Load j of wave wv fills tile
  // positions (kPrefillQ j + wv) 64 + [0, 64), i.e. the kChunks 16-byte chunks
  // of 64 / kChunks consecutive keys from key kf_j = (kPrefillQ j + wv) 64 / kChunks
  // of the tile, which lie in one 64-token block.  Position p holds data chunk
  // (p % kChunks) ^ swz(key) of key p / kChunks, so that the lanes of one MFMA
  // operand read touch distinct banks: swz = key mod 16 for bf16 (16 chunks a
  // row), (key / 2) mod 8 for e4m3fn (8 chunks a row; key mod 8 there leaves
  // about half the read cycles bank-conflicted, measured).  Each load's buffer
  // resource starts at the cache row of its first key and spans only the keys
  // below nmax of a block that is present; the hardware's range check returns
  // zeros (finite in both formats) for the rest, so the per-lane offsets are
  // constants and the loads need no per-tile vector work.
  constexpr int kLoadKeys = 64 / kChunks;                // keys per load instruction (8 or 4)
  // e4m3fn: the next group's key operands are read from LDS while the current
  // group is multiplied (two operand sets, 16 registers each); bf16 reads them
  // at the start of the group (its sets are twice the size)
  constexpr bool kPrefetchKb = DT != DSA_BF16;
  auto swz = [](int key) { return DT == DSA_BF16 ? (key & 15) : ((key >> 1) & 7); };
  uint32_t lane_off[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int p = (j * kPrefillQ + wv) * 64 + lane;
    const int key = p / kChunks, ch = (p % kChunks) ^ swz(key);
    lane_off[j] = (uint32_t)((lane / kChunks) * Tr::kRowBytes + ch * 16);
  }
  const uint32_t scale_off = lane < kScaleKeys ? (uint32_t)lane * 4u : kBufferDrop;
  const uint32_t tile_lds = lds_addr(&tile[0][0]);
  const uint32_t scale_lds = lds_addr(&kscale[0][0]);
  // Issues the tile at key `base` (< nmax) into buffer `bi`; returns its block
  // presence bits.
  // contiguous cache: one descriptor over the candidate rows of every query of
  // the workgroup (key s in row s), and the key offset goes into voffset
  const i32x4s dk_all = buffer_desc(kbase, kPaged ? 0 : nmax * Tr::kRowBytes);
  const i32x4s ds_all = buffer_desc(a.k_scale, kPaged || !kScaled ? 0 : nmax * 4);
  auto issue = [&](int base, int bi) -> uint32_t {
    if constexpr (!kPaged) {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int kf = (j * kPrefillQ + wv) * kLoadKeys;
        buffer_lds16(dk_all, tile_lds + bi * kTileBytes + (j * kPrefillQ + wv) * 1024,
                     lane_off[j] + (uint32_t)((base + kf) * Tr::kRowBytes));
      }
      if constexpr (kScaled)
        buffer_lds4(ds_all, scale_lds + (bi * kPrefillQ + wv) * 256,
                    scale_off + (uint32_t)((base + wv * kScaleKeys) * 4));
      return (1u << kBlocks) - 1;
    }
    long long sl0[kBlocks];
    uint32_t ok = 0;
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      sl0[j] = base + 64 * j < nmax ? block_slot(a.sv, base + 64 * j) : -1;
      ok |= (sl0[j] >= 0 ? 1u : 0u) << j;
    }
    // Resource from the cache row of tile key kf on: the keys below nmax of a
    // present block are in range (a range past the load's own keys changes
    // nothing), none otherwise.  Uniform scalar work: no clamp that would
    // select a vector instruction, and 32-bit slots.
    auto desc = [&](const void *arr, int row, int kf) {
      const int b0 = (int)(kBlocks == 1 ? sl0[0] : sl0[kf >> 6]);
      const int left = nmax - base - kf;
      const int bytes = b0 < 0 ? 0 : (left > 0 ? left : 0) * row;
      const int slot = b0 < 0 ? 0 : b0 + (kf & 63);
      return buffer_desc(reinterpret_cast<const uint8_t *>(arr) + (long long)slot * row, bytes);
    };
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int kf = (j * kPrefillQ + wv) * kLoadKeys;
      buffer_lds16(desc(kbase, Tr::kRowBytes, kf), tile_lds + bi * kTileBytes + (j * kPrefillQ + wv) * 1024,
                   lane_off[j]);
    }
    if constexpr (kScaled) {
      // keys kScaleKeys wv + [0, kScaleKeys); the other lanes are dropped by the
      // range check (and leave zeros in LDS that no one reads)
      buffer_lds4(desc(a.k_scale, 4, wv * kScaleKeys), scale_lds + (bi * kPrefillQ + wv) * 256, scale_off);
    }
    return ok;
  };

  // Key operands of 32-key group nb of the tile in buffer bi (rows nb*32 + col).
  typedef typename Tr::Op KOp[Tr::kSteps];
  auto read_kb = [&](int bi, int nb, KOp &kb) {
    const int key = nb * 32 + col;
    const uint4 *trow = &tile[bi][key * kChunks];
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) {
      if constexpr (DT == DSA_BF16) {
        const int ch = g * 8 + ks;
        kb[ks] = __builtin_bit_cast(typename Tr::Op, trow[ch ^ swz(key)]);
      } else {
        const int ch = g * 4 + ks * 2;
        const uint4 lo = trow[ch ^ swz(key)], hi = trow[(ch + 1) ^ swz(key)];
        typename Tr::Op o;
        o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
        o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
        kb[ks] = o;
      }
    }
  };
  // MFMAs of one group's key operands kb into (c0a, c1a), interleaved in program
  // order with the ReLU-weighted head sum of the previous group's accumulators
  // (p0a, p1a): each k-step's two MFMAs are followed by a slice of the
  // reduction, and scheduling barriers keep that order (MFMAs first), so the
  // VALU work runs while the matrix core is busy and never waits on a result
  // that has just been started.
  auto mma_reduce = [&](const KOp &kb, f32x16 &c0a, f32x16 &c1a, const f32x16 &p0a,
                        const f32x16 &p1a) -> float {
    c0a = zero_vec<f32x16>();
    c1a = zero_vec<f32x16>();
    constexpr int kPerStep = 16 / Tr::kSteps;     // reduction elements (per block) per k-step
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) {
      c0a = Tr::mma(qa[0][ks], kb[ks], c0a);
      c1a = Tr::mma(qa[1][ks], kb[ks], c1a);
      if constexpr (kPrefetchKb) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < kPerStep; ++e) {
        const int v = ks * kPerStep + e;
        r0 = fmaf(wt[0][v], __int_as_float(max(__float_as_int(p0a[v]), 0)), r0);
        r1 = fmaf(wt[1][v], __int_as_float(max(__float_as_int(p1a[v]), 0)), r1);
      }
      // pin this slice of the reduction here (the compiler would otherwise hoist
      // the whole reduction above the MFMAs it is meant to overlap)
      asm volatile("" : "+v"(r0), "+v"(r1));
      __builtin_amdgcn_sched_barrier(0);
    }
    return r0 + r1;   // this half-wave's heads; the other half's come in pair_total
  };
  // Scores of two consecutive groups: lanes 0..31 get the head sum of key
  // col of the even group (its two half-waves' partials added across the
  // halves), lanes 32..63 that of the odd group, with one lane swap.
  auto pair_total = [](float even_part, float odd_part) {
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(even_part), __float_as_uint(odd_part), false, false);
    return __uint_as_float(x[0]) + __uint_as_float(x[1]);
  };
  // Scores leave through a buffer store whose range is this row's first n
  // entries (none for a row past the last); the lanes of the upper half, and
  // keys at or past n, fall outside it and the hardware drops them.  The store
  // therefore needs no branch: a branch here would let the compiler move the
  // next group's MFMAs below it, behind the reduction they are meant to overlap.
  const __amdgpu_buffer_rsrc_t srsrc =
      __builtin_amdgcn_make_buffer_rsrc(srow, (short)0, row_ok ? n * 4 : 0, kBufferDword3);
  // 64 keys from `s0` (wave-uniform), lane l holding key s0 + l; `live` false
  // drops them.  The stored score is never -0 (the head sums start from +0,
  // and the e4m3fn key scale is applied as an fma with a +0 addend), so its
  // histogram bin, score_key(v) >> 21, is (u >> 21) ^ (sign ? 0x7ff : 0x400)
  // for its bits u.
  auto emit = [&](int s0, float v, bool gone, float kscl, bool live) {
    if (kScaled) v = fmaf(v, kscl, 0.f);
    if (kPaged) v = gone ? neg_inf() : v;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), srsrc,
                                          live ? (uint32_t)(s0 + lane) * 4u : kBufferDrop, 0, 0);
    if constexpr (kHist) {
      const uint32_t u = __float_as_uint(v);
      const uint32_t bin = (u >> 21) ^ (((uint32_t)((int)u >> 31) & 0x3ffu) | 0x400u);
      // every lane's bin is in range; only the stored lanes count
      const bool cnt = live && lane < n - s0 && row_ok;
      atomicAdd(&wh[wv][bin], cnt ? 1u : 0u);
    }
  };

  // Software pipeline over the 32-key groups of all tiles: while group i+1 is
  // multiplied, group i is reduced, and every second step the last two
  // groups' scores are written together.  Tile tt + kBufs - 1 goes into the
  // buffer of tile tt-1, which every wave has finished reading once the
  // barrier that opens tile tt is passed.  Each wave issues its share of that
  // tile after group K = wv mod kGroups rather than right after the barrier:
  // a vector-memory instruction holds its wave until the address unit takes
  // it, and eight waves queueing their loads at the same moment leave the
  // matrix cores idle meanwhile.  Past the last tile the loads repeat the last
  // tile (into a buffer no one reads), so every iteration issues the same
  // instructions and needs no branch.  Block presence bits travel with the
  // tile (kBufs x kBlocks bits); a pair of groups is one 64-token block, and
  // its fp8 key scales are read while its second group is multiplied (the
  // tile's buffer may be refilled once the next tile has begun).
  constexpr int kGroups = kPrefillKeys / 32;             // 32-key groups per tile (even)
  const int ntiles = (nmax + kPrefillKeys - 1) / kPrefillKeys;
  uint32_t okbits = 0;
  if (ntiles > 0) okbits |= issue(0, 0);
  // drain the query / weight loads (with tile 0) here, so that no wait for
  // them lands inside the loop, where it would also wait for the prefetches
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
  for (int j = 1; j < kBufs - 1; ++j)
    if (j < ntiles) okbits |= issue(j * kPrefillKeys, j) << (j * kBlocks);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = zero_vec<f32x16>();
  float part_even = 0.f;       // partial head sum of the pending even group
  float scl_pair = 1.f;        // key scale of this lane's key in the pending pair
  bool gone_pair = false;      // the pending pair's 64-token block is absent
  int bi = 0;
  auto tile_loop = [&](auto kc) {
    constexpr int K = decltype(kc)::value;               // group after which this wave issues
    // vector-memory operations issued after this wave's loads of a tile: the
    // pair stores of steps K+1.. of that iteration (even steps store), then
    // kBufs-2 whole iterations
    constexpr int kStoresAfter = (kGroups - 1) / 2 - K / 2;   // even steps in (K, kGroups)
    constexpr int kAfter = kStoresAfter + (kBufs - 2) * (kWaveLoads + kGroups / 2);
    static_assert(kStoresAfter >= 0 && kAfter < 64, "vmcnt field");
    for (int tt = 0; tt < ntiles; ++tt) {
      // tiles 1 .. kBufs-2 came from before the loop: wait for everything then
      if (tt >= kBufs - 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kAfter & 15) | ((kAfter >> 4) << 14));
      else if (tt > 0)
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      lds_barrier();
      const int nb2 = bi == 0 ? kBufs - 1 : bi - 1;      // (tt + kBufs - 1) % kBufs
      const bool fresh = tt + kBufs - 1 < ntiles;
      const int tn = fresh ? tt + kBufs - 1 : ntiles - 1;
      const uint32_t okt = okbits >> (bi * kBlocks);
      const int base = tt * kPrefillKeys;
      KOp kbs[kPrefetchKb ? 2 : 1];
      if constexpr (kPrefetchKb) read_kb(bi, 0, kbs[0]);
#pragma unroll
      for (int nb = 0; nb < kGroups; ++nb) {
        const int cur = nb & 1, prv = cur ^ 1;
        if constexpr (kPrefetchKb) {
          if (nb + 1 < kGroups) read_kb(bi, nb + 1, kbs[(nb + 1) & 1]);
        } else {
          read_kb(bi, nb, kbs[0]);
        }
        // multiplies group nb, reduces group nb-1 (the previous tile's last for nb = 0)
        const float part = mma_reduce(kbs[kPrefetchKb ? (nb & 1) : 0], acc[cur][0], acc[cur][1], acc[prv][0], acc[prv][1]);
        if (nb & 1) {
          // group nb-1 is even: hold it; read the scales and the presence of
          // the pair (nb-1, nb) while this tile is current
          part_even = part;
          if (kScaled) {
            const int k = (nb - 1) * 32 + lane;
            scl_pair = kscale[bi][(k / kScaleKeys) * 64 + k % kScaleKeys];
          }
          gone_pair = ((okt >> (nb >> 1)) & 1u) == 0;
        } else {
          // group nb-1 is odd: write the pair (nb-2, nb-1)
          emit(base + nb * 32 - 64, pair_total(part_even, part), gone_pair, scl_pair, tt > 0 || nb > 0);
        }
        if (nb == K) {
          const uint32_t ok = issue(tn * kPrefillKeys, nb2);
          okbits = fresh ? (okbits & ~(((1u << kBlocks) - 1) << (nb2 * kBlocks))) | (ok << (nb2 * kBlocks))
                         : okbits;
        }
      }
      bi = bi == kBufs - 1 ? 0 : bi + 1;
    }
    // the repeated loads of the last iterations land before the workgroup ends
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  };
  static_assert(kGroups == 2 || kGroups == 4, "issue groups");
  switch (wv & (kGroups - 1)) {
    case 0: tile_loop(std::integral_constant<int, 0>{}); break;
    case 1: tile_loop(std::integral_constant<int, 1>{}); break;
    case 2: tile_loop(std::integral_constant<int, (kGroups > 2 ? 2 : 0)>{}); break;
    default: tile_loop(std::integral_constant<int, (kGroups > 3 ? 3 : 0)>{}); break;
  }
  if (ntiles > 0) {
    // the last group (in acc[1], kGroups being even) is reduced alone and
    // written with the pending even group
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p0 = fmaf(wt[0][v], __int_as_float(max(__float_as_int(acc[1][0][v]), 0)), p0);
      p1 = fmaf(wt[1][v], __int_as_float(max(__float_as_int(acc[1][1][v]), 0)), p1);
    }
    emit(ntiles * kPrefillKeys - 64, pair_total(part_even, p0 + p1), gone_pair, scl_pair, true);
  }
  if (a.fill_masked && row_ok) {
    for (long long s = n + lane; s < a.ld; s += 64) srow[s] = neg_inf();
  }
  if (kHist && row_ok) {
    uint32_t *hrow = a.hist + (long long)r * a.hist_stride;
    for (int i = lane; i < kTopkBins; i += 64) hrow[i] = wh[wv][i];
  }
}

// ------------------------------------------------------------------ fp32, small shapes

__global__ __launch_bounds__(256) void indexer_f32_kernel(IndexerArgs a) {
  __shared__ float qs[4096];
  __shared__ float ws[64];
  const int r = blockIdx.y;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const int HD = a.H_I * a.d_I;
  const float *qrow = reinterpret_cast<const float *>(a.q_idx) + (long long)t * HD;
  for (int i = threadIdx.x; i < HD; i += blockDim.x) qs[i] = qrow[i];
  for (int i = threadIdx.x; i < a.H_I; i += blockDim.x) ws[i] = a.w[(long long)t * a.H_I + i];
  __syncthreads();
  const long long s = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  float *srow = a.scores + (long long)r * a.ld;
  if (s >= a.ld) return;
  if (s >= n) {
    if (a.fill_masked) srow[s] = neg_inf();
    return;
  }
  const long long sl = a.sv.slot(b, (int)s);
  if (sl < 0) {
    srow[s] = neg_inf();
    return;
  }
  const float *key = reinterpret_cast<const float *>(a.k_cache) + sl * a.d_I;
  float acc = 0.f;
  for (int j = 0; j < a.H_I; ++j) {
    float dot = 0.f;
    for (int d = 0; d < a.d_I; ++d) dot = fmaf(qs[j * a.d_I + d], key[d], dot);
    acc = fmaf(ws[j], fmaxf(dot, 0.f), acc);
  }
  srow[s] = acc;
}

}  // namespace

hipError_t launch_index_scores(const IndexerArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)((a.ld + 255) / 256), (unsigned)a.rows);
    hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const bool decode = a.sv.mode == DSA_DECODE;
  if (decode) return launch_index_decode(a, st);
  {
    dim3 grid((unsigned)((a.rows + kPrefillQ - 1) / kPrefillQ));
    const bool hist = a.hist_mode == 2, paged = a.sv.block_table != nullptr;
    const dim3 block(kPrefillQ * 64);
#define DSA_PREFILL_LAUNCH(D, H, P) hipLaunchKernelGGL((indexer_prefill_kernel<D, H, P>), grid, block, 0, st, a)
    if (a.dtype == DSA_BF16) {
      if (hist) { if (paged) DSA_PREFILL_LAUNCH(DSA_BF16, true, true); else DSA_PREFILL_LAUNCH(DSA_BF16, true, false); }
      else { if (paged) DSA_PREFILL_LAUNCH(DSA_BF16, false, true); else DSA_PREFILL_LAUNCH(DSA_BF16, false, false); }
    } else {
      if (hist) { if (paged) DSA_PREFILL_LAUNCH(DSA_FP8_E4M3FN, true, true); else DSA_PREFILL_LAUNCH(DSA_FP8_E4M3FN, true, false); }
      else { if (paged) DSA_PREFILL_LAUNCH(DSA_FP8_E4M3FN, false, true); else DSA_PREFILL_LAUNCH(DSA_FP8_E4M3FN, false, false); }
    }
#undef DSA_PREFILL_LAUNCH
  }
  return hipGetLastError();
}

}  // namespace dsa

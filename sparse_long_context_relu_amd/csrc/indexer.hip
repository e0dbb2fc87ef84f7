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

template <int DT>
__global__ __launch_bounds__(512) void indexer_prefill_kernel(IndexerArgs a) {
  typedef IdxTraits<DT> Tr;
  constexpr int kChunks = Tr::kRowBytes / 16;           // 16-byte chunks per key row (16 or 8)
  // keys per LDS tile: 64 for bf16, 128 for e4m3fn (the same 16 KB)
  constexpr int kPrefillKeys = DT == DSA_BF16 ? 64 : 128;
  constexpr int kBlocks = kPrefillKeys / 64;            // 64-token blocks per tile
  constexpr int kTileChunks = kPrefillKeys * kChunks;   // 1024 chunks per tile
  constexpr int kLoads = kTileChunks / 512;             // direct loads per wave per tile (2)
  constexpr bool kScaled = DT == DSA_FP8_E4M3FN;
  constexpr int kWaveLoads = kLoads + (kScaled ? 1 : 0);   // + the key scales (fp8)
  constexpr int kBufs = 3;                              // tiles tt+1, tt+2 stream in while tt is used
  constexpr uint32_t kTileBytes = kTileChunks * 16;
  __shared__ uint4 tile[kBufs][kTileChunks];
  __shared__ float kscale[kBufs][kScaled ? kPrefillKeys : 1];

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
  __shared__ uint32_t wh[kPrefillQ][kTopkBins];
  const bool hist = a.hist_mode == 2;
  if (hist)
    for (int i = lane; i < kTopkBins; i += 64) wh[wv][i] = 0u;

  const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k_cache);
  const uint32_t tile_lds = lds_addr(&tile[0][0]);
  const uint32_t scale_lds = lds_addr(&kscale[0][0]);
  // Direct-to-LDS gather of the tile at key `base` (< nmax) into buffer `bi`.
  // Position p of a tile holds data chunk (p % kChunks) ^ (key & (kChunks - 1))
  // of key p / kChunks, so the 16 lanes of one MFMA operand read touch distinct
  // bank groups; wave wv's j-th load fills positions (8 j + wv) 64 + [0, 64).
  // Keys at or past nmax load the last valid key, absent blocks slot 0: every
  // byte the MFMAs read is a finite cache entry, and neither is written out.
  // Returns the block presence bits of the tile.
  auto issue = [&](int base, int bi) -> uint32_t {
    long long sl0[kBlocks];
    uint32_t ok = 0;
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      sl0[j] = base + 64 * j < nmax ? block_slot(a.sv, base + 64 * j) : -1;
      ok |= (sl0[j] >= 0 ? 1u : 0u) << j;
    }
    const int last = nmax - 1 - base;                    // last valid key of the tile
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int p = (j * kPrefillQ + wv) * 64 + lane;
      const int key = p / kChunks, ch = (p % kChunks) ^ (key & (kChunks - 1));
      const int kk = key <= last ? key : last;
      const long long b0 = sl0[kk >> 6];
      const long long sl = b0 >= 0 ? b0 + (kk & 63) : 0;
      lds_dma16(kbase + sl * Tr::kRowBytes + ch * 16, tile_lds + bi * kTileBytes + (j * kPrefillQ + wv) * 1024);
    }
    if constexpr (kScaled) {
      // the 128 key scales, one per lane: wave wv's lanes 0..15 fetch keys 16 wv + lane
      if (lane < 16) {
        const int key = wv * 16 + lane;
        const int kk = key <= last ? key : last;
        const long long b0 = sl0[kk >> 6];
        const long long sl = b0 >= 0 ? b0 + (kk & 63) : 0;
        lds_dma4(a.k_scale + sl, scale_lds + bi * (kPrefillKeys * 4) + wv * 64);
      }
    }
    return ok;
  };

  // MFMAs of 32-key group nb of the tile in buffer bi (rows nb*32 + col) into
  // (c0a, c1a), interleaved in program order with the ReLU-weighted head sum of
  // the previous group's accumulators (p0a, p1a): each k-step's two MFMAs are
  // followed by a slice of the reduction, and scheduling barriers keep that
  // order, so the VALU work runs while the matrix core is busy.
  auto mma_reduce = [&](int bi, int nb, f32x16 &c0a, f32x16 &c1a, const f32x16 &p0a,
                        const f32x16 &p1a) -> float {
    const int key = nb * 32 + col;
    typename Tr::Op kb[Tr::kSteps];
    const uint4 *trow = &tile[bi][key * kChunks];
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) {
      if constexpr (DT == DSA_BF16) {
        const int ch = g * 8 + ks;
        kb[ks] = __builtin_bit_cast(typename Tr::Op, trow[ch ^ (key & 15)]);
      } else {
        const int ch = g * 4 + ks * 2;
        const uint4 lo = trow[ch ^ (key & 7)], hi = trow[(ch + 1) ^ (key & 7)];
        typename Tr::Op o;
        o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
        o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
        kb[ks] = o;
      }
    }
    c0a = zero_vec<f32x16>();
    c1a = zero_vec<f32x16>();
    constexpr int kPerStep = 16 / Tr::kSteps;     // reduction elements (per block) per k-step
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) {
      c0a = Tr::mma(qa[0][ks], kb[ks], c0a);
      c1a = Tr::mma(qa[1][ks], kb[ks], c1a);
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
    return sum_xor32(r0 + r1);
  };
  auto emit = [&](int s, float sc, bool gone, float kscl) {
    if (g == 0 && s < n && row_ok) {
      float v = neg_inf();
      if (!gone) {
        v = sc;
        if (kScaled) v *= kscl;
      }
      srow[s] = v;
      if (hist) atomicAdd(&wh[wv][score_key(v) >> 21], 1u);
    }
  };

  // Software pipeline over the 32-key groups of all tiles: while group i+1 is
  // multiplied, group i is reduced and written.  Tile tt+2 is issued right after
  // the barrier that opens tile tt, into the buffer of tile tt-1, which every
  // wave has finished reading by then.  Block presence bits travel with the
  // tile (3 buffers x kBlocks bits); fp8 key scales are read into registers one
  // group ahead of their use.
  constexpr int kGroups = kPrefillKeys / 32;             // 32-key groups per tile (even)
  const int ntiles = (nmax + kPrefillKeys - 1) / kPrefillKeys;
  uint32_t okbits = 0;
  if (ntiles > 0) okbits |= issue(0, 0);
  // drain the query / weight loads (with tile 0) here, so that no wait for
  // them lands inside the loop, where it would also wait for the prefetches
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (kBufs > 2 && ntiles > 1) okbits |= issue(kPrefillKeys, 1) << kBlocks;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = zero_vec<f32x16>();
  float scl[2] = {1.f, 1.f};
  bool gone_prev = false;
  int bi = 0;
  for (int tt = 0; tt < ntiles; ++tt) {
    // this wave's loads of tile tt have landed once at most the loads of tile
    // tt+1 are outstanding; the barrier then covers every wave's
    if (kBufs > 2 && tt + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(wait_vm(kWaveLoads));
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    lds_barrier();
    if (tt + kBufs - 1 < ntiles) {
      const int nb2 = bi == 0 ? kBufs - 1 : bi - 1;      // (tt + kBufs - 1) % kBufs
      okbits = (okbits & ~(((1u << kBlocks) - 1) << (nb2 * kBlocks))) |
               (issue((tt + kBufs - 1) * kPrefillKeys, nb2) << (nb2 * kBlocks));
    }
    const uint32_t okt = okbits >> (bi * kBlocks);
    const int base = tt * kPrefillKeys;
#pragma unroll
    for (int nb = 0; nb < kGroups; ++nb) {
      const int cur = nb & 1, prv = cur ^ 1;
      const float sc = mma_reduce(bi, nb, acc[cur][0], acc[cur][1], acc[prv][0], acc[prv][1]);
      if (kScaled) scl[cur] = kscale[bi][nb * 32 + col];
      if (tt > 0 || nb > 0) emit(base + nb * 32 - 32 + col, sc, gone_prev, scl[prv]);
      gone_prev = ((okt >> (nb >> 1)) & 1u) == 0;
    }
    bi = bi == kBufs - 1 ? 0 : bi + 1;
  }
  if (ntiles > 0) {
    // the last group (in acc[1], kGroups being even) is reduced alone
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p0 = fmaf(wt[0][v], __int_as_float(max(__float_as_int(acc[1][0][v]), 0)), p0);
      p1 = fmaf(wt[1][v], __int_as_float(max(__float_as_int(acc[1][1][v]), 0)), p1);
    }
    emit(ntiles * kPrefillKeys - 32 + col, sum_xor32(p0 + p1), gone_prev, scl[1]);
  }
  if (a.fill_masked && row_ok) {
    for (long long s = n + lane; s < a.ld; s += 64) srow[s] = neg_inf();
  }
  if (hist && row_ok) {
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
    if (a.dtype == DSA_BF16)
      hipLaunchKernelGGL(indexer_prefill_kernel<DSA_BF16>, grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL(indexer_prefill_kernel<DSA_FP8_E4M3FN>, grid, dim3(512), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dsa

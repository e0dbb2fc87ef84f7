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
//     share 64-key tiles staged through LDS.
// e4m3fn: scores = k_scale(s) * sum_j (w_j q_scale_j) ReLU(q8_j . k8_s),
// exact because ReLU(a x) = a ReLU(x) for a > 0.
//   (the decode tiling is in indexer_decode.hip)
#include "indexer_common.h"

namespace dsa {
namespace {

// ------------------------------------------------------------------ prefill tiling

constexpr int kPrefillQ = 8;     // queries (waves) per workgroup

template <int DT>
__global__ __launch_bounds__(512) void indexer_prefill_kernel(IndexerArgs a) {
  typedef IdxTraits<DT> Tr;
  constexpr int kChunks = Tr::kRowBytes / 16;           // 16-byte chunks per key row (16 or 8)
  // keys per LDS tile: 64 for bf16 (a larger tile spills registers), 128 for
  // e4m3fn (half the bytes per key, and twice the MFMA work per barrier)
  constexpr int kPrefillKeys = DT == DSA_BF16 ? 64 : 128;
  constexpr int kTileChunks = kPrefillKeys * kChunks;   // chunks per tile
  constexpr int kPerThread = kTileChunks / 512;         // 2 (bf16) or 1 (fp8)
  __shared__ uint4 tile[2][kTileChunks];

  const int grp = gridDim.x - 1 - blockIdx.x;           // longest rows first
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
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
  float *srow = a.scores + (long long)(row_ok ? r : 0) * a.ld;

  typename Tr::Op qa[2][Tr::kSteps];
  float wt[2][16];
  load_query<DT>(a, t, col, g, qa, wt);

  const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k_cache);
  // Stage the tile starting at key `base` into registers.
  uint4 stage[kPerThread];
  float stage_scale[kPerThread];
  // A tile covers whole 64-token blocks: one uniform lookup per block gives its
  // first slot, and whether the block is present at all (keys past nmax are
  // never written out, so their presence does not matter).
  constexpr int kBlocks = kPrefillKeys / 64;
  auto fetch = [&](int base, bool (&ok)[kBlocks]) {
    long long slb[kBlocks];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      slb[j] = base + 64 * j < nmax ? a.sv.slot(0, base + 64 * j) : -1;
      ok[j] = slb[j] >= 0;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = threadIdx.x + i * 512;
      const int key = c / kChunks, ch = c % kChunks;
      const long long sl0 = slb[key >> 6];
      const long long sl = (sl0 >= 0 && base + key < nmax) ? sl0 + (key & 63) : -1;
      stage[i] = sl >= 0 ? ld16(kbase + sl * Tr::kRowBytes + ch * 16) : make_uint4(0, 0, 0, 0);
      if (DT == DSA_FP8_E4M3FN) stage_scale[i] = (sl >= 0 && ch == 0) ? a.k_scale[sl] : 0.f;
    }
  };
  __shared__ float kscale[2][kPrefillKeys];
  // Swizzled store: chunk ch of key `key` goes to slot ch ^ (key & 15) of its row (bf16),
  // so the 16 lanes of one MFMA operand read touch 16 distinct bank groups.  The
  // fp8 key scales go beside the tile.
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = threadIdx.x + i * 512;
      const int key = c / kChunks, ch = c % kChunks;
      tile[buf][key * kChunks + (ch ^ (key & (kChunks - 1)))] = stage[i];
      if (DT == DSA_FP8_E4M3FN && ch == 0) kscale[buf][key] = stage_scale[i];
    }
  };
  // first radix digit of the top-k: each wave owns its query row's bins
  __shared__ uint32_t wh[kPrefillQ][kTopkBins];
  const bool hist = a.hist_mode == 2;
  if (hist)
    for (int i = lane; i < kTopkBins; i += 64) wh[wv][i] = 0u;

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
        if (DT == DSA_FP8_E4M3FN) v *= kscl;
      }
      srow[s] = v;
      if (hist) atomicAdd(&wh[wv][score_key(v) >> 21], 1u);
    }
  };

  // Software pipeline over 32-key groups: while group i+1 is multiplied, group
  // i is reduced and written.  The fp8 scales of a group are read into registers
  // before the barrier after which their buffer may be refilled; block presence
  // travels with the tile in wave-uniform flags.
  int buf = 0;
  bool okc[kBlocks], okn[kBlocks];          // the tile in LDS / the tile being fetched
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) okc[j] = okn[j] = true;
  if (nmax > 0) {
    fetch(0, okc);
    put(0);
  }
  __syncthreads();
  constexpr int kGroups = kPrefillKeys / 32;             // 32-key groups per tile (even)
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = zero_vec<f32x16>();
  float scl[2];
  (void)mma_reduce(0, 0, acc[0][0], acc[0][1], acc[1][0], acc[1][1]);
  scl[0] = DT == DSA_FP8_E4M3FN ? kscale[0][col] : 1.f;
  for (int base = 0; base < nmax; base += kPrefillKeys) {
    const bool more = base + kPrefillKeys < nmax;
    if (more) fetch(base + kPrefillKeys, okn);
    // group nb -> acc[nb & 1] while group nb - 1 is reduced and written
#pragma unroll
    for (int nb = 1; nb < kGroups; ++nb) {
      const int cur = nb & 1, prv = cur ^ 1;
      const float sc = mma_reduce(buf, nb, acc[cur][0], acc[cur][1], acc[prv][0], acc[prv][1]);
      scl[cur] = DT == DSA_FP8_E4M3FN ? kscale[buf][nb * 32 + col] : 1.f;
      emit(base + (nb - 1) * 32 + col, sc, !okc[(nb - 1) >> 1], scl[prv]);
    }
    if (more) put(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    // group 0 of the next tile -> acc[0] while the tile's last group (in acc[1])
    // is reduced (past the last tile this multiplies a stale buffer, unused)
    const float sc = mma_reduce(buf, 0, acc[0][0], acc[0][1], acc[1][0], acc[1][1]);
    const bool last_gone = !okc[kBlocks - 1];
    const float last_scl = scl[1];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) okc[j] = okn[j];
    scl[0] = DT == DSA_FP8_E4M3FN ? kscale[buf][col] : 1.f;
    emit(base + (kGroups - 1) * 32 + col, sc, last_gone, last_scl);
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

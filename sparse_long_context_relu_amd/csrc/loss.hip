// The lightning indexer's warm-up objective and its gradient ("DeepSeek V3.2:
// How Far Can Open Models Go If You Actually Try?", section 3.3, Stage 1: the
// main attention stays dense and frozen while the indexer is trained with a
// KL divergence towards its distribution; "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", Modeling, Objective Functions: the
// target is the dense attention aggregated over heads and L1-normalised).
//
//   L_I = sum_t KL(p_t || softmax(I_t)),   dL/dI(t, s) = softmax(I_t)_s - p_t(s)
//
// The head-aggregated target p comes from two passes of the attention kernel
// (sparse_mla.hip: the per-head log-sum-exp, then the weights summed over
// heads); this file holds the per-query KL rows.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kKlThreads = 256;
constexpr int kKlWaves = kKlThreads / 64;

// (max, sum of exp(x - max)) pairs, merged so that a -inf maximum carries no mass
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == neg_inf()) return;
  s = (m == neg_inf() ? 0.f : s * expf(m - M)) + (m2 == neg_inf() ? 0.f : s2 * expf(m2 - M));
  m = M;
}

// One workgroup per query row: log-sum-exp of the scores over the candidates,
// then the row's KL term and its gradient, written over the scores (0 past the
// last candidate).  Block reductions run in a fixed order (deterministic).
__global__ __launch_bounds__(kKlThreads) void indexer_kl_rows_kernel(KlArgs a) {
  __shared__ float red[2][kKlWaves];
  const int r = blockIdx.x;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  float *srow = a.scores + (long long)r * a.ld;
  const float *prow = a.probs + (long long)r * a.ld;
  const int lane = lane_id(), wv = threadIdx.x >> 6;

  float m = neg_inf(), sm = 0.f;
  for (int s = threadIdx.x; s < n; s += kKlThreads) lse_merge(m, sm, srow[s], 1.f);
  for (int o = 1; o < 64; o <<= 1) lse_merge(m, sm, shfl_xor(m, o), shfl_xor(sm, o));
  if (lane == 0) {
    red[0][wv] = m;
    red[1][wv] = sm;
  }
  __syncthreads();
  float M = neg_inf(), S = 0.f;
  for (int w = 0; w < kKlWaves; ++w) lse_merge(M, S, red[0][w], red[1][w]);
  const float lse = M == neg_inf() ? neg_inf() : M + logf(S);
  __syncthreads();

  float acc = 0.f;
  for (int s = threadIdx.x; s < n; s += kKlThreads) {
    const float p = prow[s];
    const float x = srow[s];
    // a score of -inf (absent key) has probability 0 under softmax(I)
    const float lq = x == neg_inf() ? neg_inf() : x - lse;
    if (p > 0.f) acc += p * (logf(p) - lq);
    srow[s] = (lq == neg_inf() ? 0.f : expf(lq)) - p;
  }
  for (long long s = (long long)n + threadIdx.x; s < a.ld; s += kKlThreads) srow[s] = 0.f;
  acc = wave_sum(acc);
  if (lane == 0) red[0][wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float l = 0.f;
    for (int w = 0; w < kKlWaves; ++w) l += red[0][w];
    a.loss[t] = l;
  }
}

// ------------------------------------------------------------------ backward
//
// With x(j, s) = q_j . k_s and g = dL/dI:
//   dw_j = sum_s g_s ReLU(x_js),  dq_j = sum_s G_js k_s,  dk_s = sum_j G_js q_j,
//   G_js = g_s w_j [x_js > 0].
// Both products have the shape of the attention kernel's: a first MFMA product
// of a streamed tile of rows against a column operand held in registers
// (S^T[rows, cols] = Tile . Op^T), an elementwise step that turns it into a
// bf16 operand P^T[rows, cols], and a second product accumulating
// Tile^T[dims, rows] . P^T into fp32 registers (dims x cols), the transposed
// tile read from LDS by ds_read_b64_tr_b16.  dq: rows = the query's keys,
// columns = its 64 heads (4 waves x 16).  dk: rows = the 64 head vectors of
// each query that sees the keys, columns = 128 keys (8 waves x 16).

constexpr int kBwdHeads = 64;                      // H_I
constexpr int kBwdDim = 128;                       // d_I
constexpr int kBwdRowBytes = kBwdDim * 2;          // bf16 rows
// LDS tile rows: a 288-byte stride (two pad chunks) and the two halves of
// each 32-byte pair of chunks swapped in rows 8..15 and 24..31 (chunk c of row
// r at position c ^ bwd_swz(r)).  With that, the 16-byte reads of the first
// product (16 rows, one chunk each) and the transpose reads of the second (4
// rows x 32 bytes per 16 lanes) both hit distinct LDS banks; the plain 272-byte
// stride left the transpose reads two-way conflicted.
constexpr int kBwdStride = kBwdRowBytes + 32;
constexpr int kBwdR = 32;                          // rows per tile
constexpr int kBwdTileBytes = kBwdR * kBwdStride;  // 9216
constexpr int kBwdKs = kBwdDim / 32;               // k-steps of the first product
constexpr int kBwdDb = kBwdDim / 16;               // 16-dim blocks of the second
constexpr int kBwdQParts = kBwdHeads * kBwdDim + kBwdHeads;   // floats of one dq split partial (dq, dw)
__device__ __forceinline__ int bwd_swz(int r) { return (r >> 3) & 1; }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// S^T: element v of st[rb] is row 16 rb + 4 g + v of the tile, column lane % 16.
__device__ __forceinline__ void tile_product(uint32_t tile, const bf16x8 (&op)[kBwdKs], f32x4 (&st)[2], int g,
                                             int col) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    st[rb] = zero_vec<f32x4>();
#pragma unroll
    for (int ks = 0; ks < kBwdKs; ++ks) {
      const u32x4 fr =
          *(lds_u32x4 *)(uintptr_t)(tile + (16 * rb + col) * kBwdStride + (4 * ks + (g ^ bwd_swz(col))) * 16);
      st[rb] = mfma16_bf16(__builtin_bit_cast(bf16x8, fr), op[ks], st[rb]);
    }
  }
}

// acc[db] (element v: dim 16 db + 4 g + v, column lane % 16) += Tile^T . P^T.
// k-slots 0..3 of this lane are tile rows 4 g + e, 4..7 rows 16 + 4 g + e, the
// rows it holds in P^T; lane 4 e + c of its group points the transpose read at
// row 4 g + e (16 + 4 g + e), dims 16 db + 4 c .. + 3.
__device__ __forceinline__ void tile_accumulate(uint32_t tile, const bf16x8 &pb, f32x4 (&acc)[kBwdDb], int g,
                                                int lane) {
  const int e = (lane & 15) >> 2, c = lane & 3;
  const uint32_t lo = tile + (4 * g + e) * kBwdStride + 16 * ((c >> 1) ^ bwd_swz(4 * g + e)) + 8 * (c & 1);
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db) {
    const v4s l4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)(lo + 32 * db));
    const v4s h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)(lo + 16 * kBwdStride + 32 * db));
    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7));
    acc[db] = mfma16_bf16(av, pb, acc[db]);
  }
}

__host__ __device__ constexpr int bwd_split_len(int span, int ns) { return ((span + ns - 1) / ns + 31) / 32 * 32; }

// dq, dw: one (query, split of its candidate keys) per workgroup, 4 waves, wave
// w owning heads 16 w .. 16 w + 15; rows with the most candidates first.  At
// most 128 registers per lane, so four workgroups share a CU (three at the
// 136 the compiler picks otherwise): 3-5 % faster.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void indexer_bwd_q_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kBwdTileBytes];
  const int ns = a.n_split;
  const int r = a.rows - 1 - (int)(blockIdx.x / ns);
  const int sp = blockIdx.x % ns;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const int len = bwd_split_len(a.span, ns);
  const int i0 = sp * len;
  const int i1 = i0 + len < n ? i0 + len : n;
  const int nk = i1 > i0 ? i1 - i0 : 0;
  if (nk == 0 && ns > 1) return;                 // the merge reads only splits that hold a key
  const int ntiles = (nk + kBwdR - 1) / kBwdR;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6, g = lane >> 4, col = lane & 15;
  const int h = wv * 16 + col;

  bf16x8 qb[kBwdKs];                             // this lane's head: dims 32 ks + 8 g + [0, 8)
  {
    const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q_idx) + ((long long)t * kBwdHeads + h) * kBwdRowBytes;
#pragma unroll
    for (int ks = 0; ks < kBwdKs; ++ks) qb[ks] = as_bf16x8(ld16(qrow + ks * 64 + g * 16));
  }
  const float wh = a.w[(long long)t * kBwdHeads + h];
  const float *grow = a.grad + (long long)r * a.ld + i0;
  const bool gvec = ((uintptr_t)grow & 15) == 0;
  const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k_cache);

  // Tile tt holds candidates i0 + tt*32 .. + 31 (inside one 64-token block).
  // Thread tid loads chunks tid and tid + 256 (row c / 16, chunk c % 16), and
  // the score gradients of the 8 rows it holds in S^T.
  uint4 pf[2];
  float gn[8];
  long long sn = -1;
  auto fetch = [&](int tt) {
    sn = a.sv.slot(b, i0 + tt * kBwdR);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u, row = c >> 4, ch = c & 15;
      const bool ok = sn >= 0 && tt * kBwdR + row < nk;
      pf[u] = ld16(kbase + (ok ? sn + row : 0) * kBwdRowBytes + ch * 16);
    }
    // rows 16 rb + 4 g + [0, 4): one 16-byte load each where the gradient row
    // is 16-byte aligned (kr is a multiple of 4), element loads otherwise
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int kr = tt * kBwdR + 16 * rb + 4 * g;
      if (gvec && kr + 3 < nk) {
        const float4 v4 = *reinterpret_cast<const float4 *>(grow + kr);
        gn[rb * 4 + 0] = v4.x; gn[rb * 4 + 1] = v4.y; gn[rb * 4 + 2] = v4.z; gn[rb * 4 + 3] = v4.w;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) gn[rb * 4 + v] = kr + v < nk ? grow[kr + v] : 0.f;
      }
    }
  };
  auto put = [&](int buf, int tt) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u, row = c >> 4, ch = c & 15;
      const bool ok = sn >= 0 && tt * kBwdR + row < nk;
      *reinterpret_cast<uint4 *>(&tiles[buf][row * kBwdStride + (ch ^ bwd_swz(row)) * 16]) =
          ok ? pf[u] : make_uint4(0, 0, 0, 0);
    }
  };

  f32x4 acc[kBwdDb];
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db) acc[db] = zero_vec<f32x4>();
  float dwa = 0.f;
  float gv[8];
  if (ntiles > 0) {
    fetch(0);
    put(0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = gn[i];
  }
  __syncthreads();
  for (int tt = 0; tt < ntiles; ++tt) {
    const int cur = tt & 1;
    float gc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) gc[i] = gv[i];
    if (tt + 1 < ntiles) fetch(tt + 1);
    const uint32_t tile = lds_addr(&tiles[cur][0]);
    f32x4 st[2];
    tile_product(tile, qb, st, g, col);
    bf16x8 pb;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float x = st[rb][v], gx = gc[rb * 4 + v];
        dwa = fmaf(gx, fmaxf(x, 0.f), dwa);
        pb[rb * 4 + v] = (__bf16)(x > 0.f ? gx * wh : 0.f);
      }
    tile_accumulate(tile, pb, acc, g, lane);
    if (tt + 1 < ntiles) {
      put(cur ^ 1, tt + 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) gv[i] = gn[i];
    }
    __syncthreads();
  }
  dwa += shfl_xor(dwa, 16);
  dwa += shfl_xor(dwa, 32);
  float *dqo, *dwo;
  if (ns == 1) {
    dqo = a.dq + ((long long)t * kBwdHeads + h) * kBwdDim;
    dwo = a.dw + (long long)t * kBwdHeads + h;
  } else {
    float *base = a.part + ((long long)r * ns + sp) * kBwdQParts;
    dqo = base + h * kBwdDim;
    dwo = base + kBwdHeads * kBwdDim + h;
  }
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db)
    *reinterpret_cast<float4 *>(dqo + 16 * db + 4 * g) = make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
  if (g == 0) *dwo = dwa;
}

// dq, dw over the selected keys only (Stage 2: the score gradient is zero
// outside each query's selection, so only those keys contribute): one query
// per workgroup, tiles of 32 consecutive entries of its selection list;
// otherwise the tile loop above.  The list's cache rows (through the block
// table) and score gradients are gathered into LDS first, so a tile's loads
// wait on no other global load.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void indexer_bwd_q_sel_kernel(
    BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kBwdTileBytes];
  __shared__ uint32_t srow[kTopkMaxK];             // cache row of each entry (0xFFFFFFFF: absent)
  __shared__ float sgrad[kTopkMaxK];               // its score gradient (0 when absent)
  const int r = blockIdx.x;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const int32_t *irow = a.sel + (long long)r * a.sel_k;
  const int ntiles = (a.sel_k + kBwdR - 1) / kBwdR;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6, g = lane >> 4, col = lane & 15;
  const int h = wv * 16 + col;
  const float *grow = a.grad + (long long)r * a.ld;
  for (int j = tid; j < ntiles * kBwdR; j += 256) {
    const int s = j < a.sel_k ? irow[j] : -1;
    const long long sl = (s >= 0 && s < n) ? a.sv.slot(b, s) : -1;
    srow[j] = sl >= 0 ? (uint32_t)sl : 0xFFFFFFFFu;
    sgrad[j] = sl >= 0 ? grow[s] : 0.f;
  }

  bf16x8 qb[kBwdKs];
  {
    const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q_idx) + ((long long)t * kBwdHeads + h) * kBwdRowBytes;
#pragma unroll
    for (int ks = 0; ks < kBwdKs; ++ks) qb[ks] = as_bf16x8(ld16(qrow + ks * 64 + g * 16));
  }
  const float wh = a.w[(long long)t * kBwdHeads + h];
  const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.k_cache);
  __syncthreads();

  // Tile tt holds selection entries tt*32 .. + 31.  Thread tid loads chunks tid
  // and tid + 256 (row c / 16, chunk c % 16), and the score gradients of the 8
  // rows it holds in S^T; an absent entry gives a zero row and gradient.
  uint4 pf[2];
  float gn[8];
  auto fetch = [&](int tt) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u, row = c >> 4, ch = c & 15;
      const uint32_t sl = srow[tt * kBwdR + row];
      pf[u] = sl != 0xFFFFFFFFu ? ld16(kbase + (unsigned long long)sl * kBwdRowBytes + ch * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) gn[rb * 4 + v] = sgrad[tt * kBwdR + 16 * rb + 4 * g + v];
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u, row = c >> 4, ch = c & 15;
      *reinterpret_cast<uint4 *>(&tiles[buf][row * kBwdStride + (ch ^ bwd_swz(row)) * 16]) = pf[u];
    }
  };

  f32x4 acc[kBwdDb];
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db) acc[db] = zero_vec<f32x4>();
  float dwa = 0.f;
  float gv[8];
  if (ntiles > 0) {
    fetch(0);
    put(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = gn[i];
  }
  __syncthreads();
  for (int tt = 0; tt < ntiles; ++tt) {
    const int cur = tt & 1;
    float gc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) gc[i] = gv[i];
    if (tt + 1 < ntiles) fetch(tt + 1);
    const uint32_t tile = lds_addr(&tiles[cur][0]);
    f32x4 st[2];
    tile_product(tile, qb, st, g, col);
    bf16x8 pb;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float x = st[rb][v], gx = gc[rb * 4 + v];
        dwa = fmaf(gx, fmaxf(x, 0.f), dwa);
        pb[rb * 4 + v] = (__bf16)(x > 0.f ? gx * wh : 0.f);
      }
    tile_accumulate(tile, pb, acc, g, lane);
    if (tt + 1 < ntiles) {
      put(cur ^ 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) gv[i] = gn[i];
    }
    __syncthreads();
  }
  dwa += shfl_xor(dwa, 16);
  dwa += shfl_xor(dwa, 32);
  float *dqo = a.dq + ((long long)t * kBwdHeads + h) * kBwdDim;
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db)
    *reinterpret_cast<float4 *>(dqo + 16 * db + 4 * g) = make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
  if (g == 0) a.dw[(long long)t * kBwdHeads + h] = dwa;
}

// dq, dw of several key splits: summed in split order over the splits that
// hold a key.
__global__ __launch_bounds__(256) void indexer_bwd_q_merge_kernel(BwdArgs a) {
  const int r = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= kBwdQParts) return;
  const int t = a.q_begin + r;
  const int ns = a.n_split;
  const int len = bwd_split_len(a.span, ns);
  const int n = a.sv.candidates(t);
  int nm = n <= 0 ? 0 : (n + len - 1) / len;
  nm = nm < ns ? nm : ns;
  const float *p = a.part + (long long)r * ns * kBwdQParts + i;
  float v = 0.f;
  for (int sp = 0; sp < nm; ++sp) v += p[(long long)sp * kBwdQParts];
  if (i < kBwdHeads * kBwdDim)
    a.dq[(long long)t * kBwdHeads * kBwdDim + i] = v;
  else
    a.dw[(long long)t * kBwdHeads + (i - kBwdHeads * kBwdDim)] = v;
}

// dk: one (block of 128 key positions, set of queries) per workgroup, 8 waves,
// wave w owning keys 16 w .. 16 w + 15 of the block.  Prefill: query split y
// (q_per_split queries of sequence 0), partials merged by the next kernel.
// Decode: y = the sequence, whose only query is query y; written directly.
__global__ __launch_bounds__(512) void indexer_bwd_k_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kBwdTileBytes];
  __shared__ int act[512];                       // active queries (that see a key of the block)
  __shared__ int actpos[512];
  __shared__ int nact;
  const bool decode = a.sv.mode == DSA_DECODE;
  const int kb = blockIdx.x, y = blockIdx.y;
  const int kb0 = kb * kBwdKeysPerBlock;
  const int b = decode ? y : 0;
  const int q_lo = decode ? y : y * a.q_per_split;
  const int q_hi = decode ? y + 1 : (q_lo + a.q_per_split < a.rows ? q_lo + a.q_per_split : a.rows);
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6, g = lane >> 4, col = lane & 15;

  const int kp = kb0 + wv * 16 + col;            // this lane's key position
  bf16x8 kq[kBwdKs];
  {
    const long long sl = kp < a.sv.max_ctx ? a.sv.slot(b, kp) : -1;
    const uint8_t *krow = reinterpret_cast<const uint8_t *>(a.k_cache) + (sl >= 0 ? sl : 0) * kBwdRowBytes;
#pragma unroll
    for (int ks = 0; ks < kBwdKs; ++ks) {
      const uint4 v = ld16(krow + ks * 64 + g * 16);
      kq[ks] = as_bf16x8(sl >= 0 ? v : make_uint4(0, 0, 0, 0));
    }
  }

  // tile i: rows = heads 32 (i & 1) .. + 31 of active query act[i >> 1]; thread
  // tid loads chunk tid (row tid / 16, chunk tid % 16), and the 8 head weights
  // of the rows it holds in S^T plus (for the query) its key's score gradient
  uint4 pf;
  float wn[8], gkn = 0.f;
  auto fetch = [&](int i) {
    const int q = act[i >> 1], half = i & 1;
    const int t = a.q_begin + q;
    pf = ld16(reinterpret_cast<const uint8_t *>(a.q_idx) +
              ((long long)t * kBwdHeads + 32 * half + (tid >> 4)) * kBwdRowBytes + (tid & 15) * 16);
    const float *wr = a.w + (long long)t * kBwdHeads + 32 * half + 4 * g;
    const float4 w0 = *reinterpret_cast<const float4 *>(wr), w1 = *reinterpret_cast<const float4 *>(wr + 16);
    wn[0] = w0.x; wn[1] = w0.y; wn[2] = w0.z; wn[3] = w0.w;
    wn[4] = w1.x; wn[5] = w1.y; wn[6] = w1.z; wn[7] = w1.w;
    gkn = kp <= actpos[i >> 1] ? a.grad[(long long)q * a.ld + kp] : 0.f;
  };
  auto put = [&](int buf) {
    *reinterpret_cast<uint4 *>(&tiles[buf][(tid >> 4) * kBwdStride + ((tid & 15) ^ bwd_swz(tid >> 4)) * 16]) = pf;
  };

  f32x4 acc[kBwdDb];
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db) acc[db] = zero_vec<f32x4>();
  float wc[8], gkc = 0.f;
  int last_pos = -1;                             // decode: the query's position
  // rounds of up to 512 queries of the set: the ones whose last candidate
  // reaches the block, compacted in order, then their tiles
  for (int base = q_lo; base < q_hi; base += 512) {
  {
    const int q = base + tid;
    const int pos = q < q_hi ? a.sv.candidates(a.q_begin + q) - 1 : -1;
    const bool on = pos >= kb0;
    const uint64_t m = __ballot(on);
    const int before = __popcll(m & ((1ull << lane) - 1));
    __shared__ int wbase[8];
    if (lane == 0) wbase[wv] = __popcll(m);
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wv; ++w) off += wbase[w];
    if (on) {
      act[off + before] = q;
      actpos[off + before] = pos;
    }
    if (tid == 511) nact = off + before + (on ? 1 : 0);
  }
  __syncthreads();
  const int na = nact;
  if (na > 0) last_pos = actpos[na - 1];
  const int ntiles = 2 * na;
  if (ntiles > 0) {
    fetch(0);
    put(0);
  }
  __syncthreads();
  for (int i = 0; i < ntiles; ++i) {
    const int cur = i & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) wc[j] = wn[j];
    gkc = gkn;
    if (i + 1 < ntiles) fetch(i + 1);
    const uint32_t tile = lds_addr(&tiles[cur][0]);
    f32x4 st[2];
    tile_product(tile, kq, st, g, col);
    bf16x8 pb;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float x = st[rb][v];
        pb[rb * 4 + v] = (__bf16)(x > 0.f ? gkc * wc[rb * 4 + v] : 0.f);
      }
    tile_accumulate(tile, pb, acc, g, lane);
    if (i + 1 < ntiles) put(cur ^ 1);
    __syncthreads();
  }
  }
  // acc[db]: dims 16 db + 4 g + v of key column col
  const int kl = wv * 16 + col;
  float *out;
  if (decode) {
    if (last_pos < 0 || kp > last_pos) return;   // keys past the query's position are not seen
    const long long sl = a.sv.slot(b, kp);
    if (sl < 0) return;
    out = a.dk + sl * kBwdDim;
  } else {
    out = a.part + ((long long)y * gridDim.x + kb) * (kBwdKeysPerBlock * kBwdDim) + kl * kBwdDim;
  }
#pragma unroll
  for (int db = 0; db < kBwdDb; ++db)
    *reinterpret_cast<float4 *>(out + 16 * db + 4 * g) = make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
}

// Prefill dk: the query splits' partials of each key, summed in split order,
// written to the key's cache slot (positions 0 .. max_ctx - 1 of sequence 0).
__global__ __launch_bounds__(256) void indexer_bwd_k_merge_kernel(BwdArgs a, int nkb) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int kp = (int)(i / kBwdDim), d = (int)(i % kBwdDim);
  if (kp >= a.sv.max_ctx) return;
  const long long sl = a.sv.slot(0, kp);
  if (sl < 0) return;
  const int kb = kp / kBwdKeysPerBlock, kl = kp % kBwdKeysPerBlock;
  const float *p = a.part + (long long)kb * (kBwdKeysPerBlock * kBwdDim) + kl * kBwdDim + d;
  float v = 0.f;
  for (int qs = 0; qs < a.n_split; ++qs) v += p[(long long)qs * nkb * (kBwdKeysPerBlock * kBwdDim)];
  a.dk[sl * kBwdDim + d] = v;
}

}  // namespace

int bwd_q_splits(int rows, int span) {
  if (rows >= 256) return 1;
  int s = (span + 2047) / 2048;
  return s < 1 ? 1 : (s > 128 ? 128 : s);
}

hipError_t launch_indexer_bwd_q(const BwdArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_bwd_q_kernel, dim3((unsigned)(a.rows * a.n_split)), dim3(256), 0, st, a);
  if (a.n_split > 1)
    hipLaunchKernelGGL(indexer_bwd_q_merge_kernel, dim3((kBwdQParts + 255) / 256, (unsigned)a.rows), dim3(256), 0, st,
                       a);
  return hipGetLastError();
}

hipError_t launch_indexer_bwd_q_sel(const BwdArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_bwd_q_sel_kernel, dim3((unsigned)a.rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_indexer_bwd_k(const BwdArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const int nkb = (a.sv.max_ctx + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock;
  const bool decode = a.sv.mode == DSA_DECODE;
  const int ny = decode ? a.rows : a.n_split;
  hipLaunchKernelGGL(indexer_bwd_k_kernel, dim3((unsigned)nkb, (unsigned)ny), dim3(512), 0, st, a);
  if (!decode) {
    const long long total = (long long)nkb * kBwdKeysPerBlock * kBwdDim;
    hipLaunchKernelGGL(indexer_bwd_k_merge_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a, nkb);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_kl(const KlArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_kl_rows_kernel, dim3(a.rows), dim3(kKlThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

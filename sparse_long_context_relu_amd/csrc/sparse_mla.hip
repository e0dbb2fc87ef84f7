// Sparse MLA in MQA mode over the selected latent rows ("DeepSeek V3.2: How
// Far Can Open Models Go If You Actually Try?", section 3.1, selection-then-
// attention equation and the MQA-mode paragraph: one shared latent row per
// token, every head reads the same fetched rows; "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", Novel Architectural Elements).
//
// bf16 path (H = 128, D = 576, Dv = 512): a workgroup of 8 waves owns one
// query (and one split of its selected rows).  Each 32-row tile is gathered
// from HBM once, straight into LDS by the direct-to-LDS loads of gfx950 (no
// staging registers), double-buffered so the next tile streams in while the
// current one is multiplied; every head of the query is served from that one
// fetch.  Wave w owns heads 16w..16w+15 (two waves per SIMD, so the MFMA
// accumulators of one stay in architectural registers):
//   S^T[rows, heads] = C_tile[rows, 576] . Q^T          (16x16x32 bf16 MFMA)
//   online softmax in fp32 (base-2 exponent, running max and sum per head)
//   O^T[dims, heads] += V^T[dims, rows] . P^T[rows, heads]
// V^T operands come from the row-major tile through the LDS transpose read
// (ds_read_b64_tr_b16), so the tile is stored once.  With several splits per
// query the unnormalised partials (acc, max, sum) are merged by a second
// kernel in a fixed order.
#include "mla_tile.h"

namespace dsa {
namespace {

// What a pass over the rows computes.
constexpr int kModeAttn = 0;    // softmax attention: output rows and lse
constexpr int kModeLse = 1;     // the logits' log-sum-exp per head only
constexpr int kModeProbs = 2;   // softmax weights given the lse, summed over the heads

// Logits, then per mode: online softmax and value product (attention), online
// softmax only (lse), or the normalised weights summed over this wave's heads
// (probs; 32 rows into prow + q kWaves kR, given each head's lse in base 2).
// The lse and probs passes serve kQ queries of one sequence from each tile:
// every operand read feeds kQ MFMAs, and query q sees the tile's first
// nrow[q] - j0 rows.
//
// The operand reads are issued ahead of the MFMAs that consume them (fixed
// instruction groups below), so several LDS reads are in flight while the
// matrix core works.
template <int kMode, int kQ>
__device__ __forceinline__ void consume_tile(uint32_t tile, const int *slots, int j0, const bf16x8 (&qb)[kQ][kKs],
                                             f32x4 (&acc)[kDb], float (&m_run)[kQ], float (&l_run)[kQ],
                                             float scale2, uint32_t qk_off, uint32_t pv_even, uint32_t pv_odd, int g,
                                             const float (&lse2)[kQ], const int (&nrow)[kQ], float *prow) {
  static_assert(kMode != kModeAttn || kQ == 1, "attention serves one query per workgroup");
  // ---- S^T for 32 rows x this wave's 16 heads.  The 36 operand reads go in
  // batches of kBatch, each batch issued before the MFMAs of the previous one
  // (scheduling barriers keep the compiler from sinking the reads to their uses).
  constexpr int kBatch = 3;
  constexpr int kSteps = 2 * kKs / kBatch;
  // Row presence of the tile, read before the logits so that its LDS latency
  // is covered by them (row lane%32's slot; -1: absent).
  const int lane = lane_id();
  const int row_slot = slots[j0 + (lane & (kR - 1))];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 st[kQ][2];
#pragma unroll
  for (int q = 0; q < kQ; ++q) st[q][0] = st[q][1] = zero_vec<f32x4>();
  u32x4 fr[2][kBatch];
  auto read = [&](int i, int buf) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int q = i * kBatch + u, ks = q >> 1, rb = q & 1;
      fr[buf][u] = *(lds_u32x4 *)(uintptr_t)(tile + qk_off + rb * 16 * kRowStride + ks * 64);
    }
  };
  read(0, 0);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    if (i + 1 < kSteps) read(i + 1, (i + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = i * kBatch + u, ks = k >> 1, rb = k & 1;
#pragma unroll
      for (int q = 0; q < kQ; ++q)
        st[q][rb] = mfma16_bf16(__builtin_bit_cast(bf16x8, fr[i & 1][u]), qb[q][ks], st[q][rb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int q = 0; q < kQ; ++q) {
  // ---- online softmax (base 2), one head per lane column.
  // Row validity of the tile as a wave-uniform mask (bit j: row j present).
  const uint32_t rowmask =
      (uint32_t)__ballot(lane < kR && row_slot >= 0 && (kQ == 1 || j0 + (lane & (kR - 1)) < nrow[q]));
  const uint32_t mine = rowmask >> (4 * g);     // bit v: row 4g+v; bit 16+v: row 16+4g+v
  if constexpr (kMode == kModeProbs) {
    // weight of each present row for this lane's head, summed over the 16 heads
    float e[8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        e[rb * 4 + v] =
            sum16(((mine >> (16 * rb + v)) & 1u) ? __builtin_amdgcn_exp2f(st[q][rb][v] * scale2 - lse2[q]) : 0.f);
    // lane with column c < 8 keeps row 16 (c / 4) + 4 g + c % 4
    const int c = lane & 15;
    float mine_e = e[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mine_e = c == i ? e[i] : mine_e;
    if (c < 8) prow[q * kWaves * kR + 16 * (c >> 2) + 4 * g + (c & 3)] = mine_e;
    continue;
  }
  float mx = neg_inf();
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      st[q][rb][v] = ((mine >> (16 * rb + v)) & 1u) ? st[q][rb][v] * scale2 : neg_inf();
      mx = fmaxf(mx, st[q][rb][v]);
    }
  mx = max_over_rows(mx);
  if (__any(mx > m_run[q] + kLazy)) {
    // raise the base of every head whose maximum moved (a head with no row yet
    // present keeps -inf and a zero accumulator)
    const float m_new = fmaxf(m_run[q], mx);
    const float alpha = m_run[q] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(m_run[q] - m_new);
    l_run[q] *= alpha;
    if constexpr (kMode == kModeAttn) {
#pragma unroll
      for (int db = 0; db < kDb; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[db][v] *= alpha;
    }
    m_run[q] = m_new;
  }
  // exponent base 0 while the head has seen nothing: -inf - 0 stays -inf (weight 0)
  const float base = m_run[q] == neg_inf() ? 0.f : m_run[q];
  bf16x8 pb;
  float psum = 0.f;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float pv = __builtin_amdgcn_exp2f(st[q][rb][v] - base);
      psum += pv;
      pb[rb * 4 + v] = (__bf16)pv;
    }
  l_run[q] += psum;
  if constexpr (kMode == kModeLse) continue;
  // ---- O^T += V^T . P^T.  k-slots 0..3 = tile rows 4g+e, 4..7 = rows 16+4g+e (e = 0..3),
  // matching the rows this lane holds in P^T.  Lane 4e+c of group g points the
  // transpose read at row 4g+e (resp. 16+4g+e), dims d0+4c..d0+4c+3, and receives
  // V[row_e][d0 + (lane%16)] for e = 0..3.  The swizzle permutes chunks within
  // aligned groups of four, so even and odd value blocks have their own lane offsets.
  // The per-lane bases are formed once per tile (pinned as vector values) so
  // that each block's part of the address lands in the reads' offset field
  // instead of costing an add per read.
  uint32_t pvb[2] = {tile + pv_even, tile + pv_odd};
  asm volatile("" : "+v"(pvb[0]), "+v"(pvb[1]));
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
    const uint32_t v0 = pvb[db & 1] + (db >> 1) * 64;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)v0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)(v0 + 16 * kRowStride));
    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    acc[db] = mfma16_bf16(av, pb, acc[db]);
  }
  constexpr int kAheadV = 3;     // 64 transpose reads, 32 MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAheadV, 1);
#pragma unroll
  for (int i = 0; i < kDb - kAheadV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAheadV, 1);
  }
}

// One workgroup per (group of kQ query rows, split of their lists); kQ > 1
// only for the lse and probs passes of a prefill (dense lists of sequence 0,
// one tile serving every query of the group).  kStream: the rows are gathered
// with streaming loads (decode: no other query of the launch reads them).
template <int kMode, int kQ, bool kStream = false>
__global__ __launch_bounds__(kThreads) void mla_bf16_kernel(MlaArgs a) {
  __shared__ uint4 tiles[kBufs][kTileBufChunks];
  __shared__ int slots[kMaxSplitRows + 4 * kR];
  __shared__ int fallback;
  // probs: each wave's head sums of the last two tiles' rows, per query
  __shared__ float psums[kMode == kModeProbs ? 2 : 1][kMode == kModeProbs ? kQ * kWaves * kR : 1];

  int sp, rg;
  mla_block(a, (a.rows + kQ - 1) / kQ, sp, rg);
  const int r = rg * kQ;                      // first row of the group
  const int t = a.q_begin + r;
  const int b = a.sv.seq_of(t);
  // rows of the group past the launch's last row see nothing and write nothing
  int nq[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) nq[q] = r + q < a.rows ? a.sv.candidates(t + q) : 0;
  int n = nq[0];
#pragma unroll
  for (int q = 1; q < kQ; ++q) n = nq[q] > n ? nq[q] : n;
  const int32_t *irow = a.dense ? nullptr : a.idx + (long long)r * a.k;
  const int len = split_len(a.k, a.n_split);
  const int i0 = sp * len;
  int i1 = i0 + len < a.k ? i0 + len : a.k;
  if (a.dense && i1 > n) i1 = n;              // dense lists end at the last candidate
  const int rows = i1 > i0 ? i1 - i0 : 0;
  int nrow[kQ];                               // list entries (from the split's start) each query sees
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int e = (i1 < nq[q] ? i1 : nq[q]) - i0;
    nrow[q] = e > 0 ? e : 0;
  }
  if constexpr (kMode == kModeProbs) {
    // positions of this split past each query's last candidate (and, for the
    // last split, up to the row's end) hold 0
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (r + q >= a.rows) break;
      float *prow = a.probs + (long long)(r + q) * a.ld;
      const long long z0 = i0 + nrow[q], z1 = sp + 1 == a.n_split ? a.ld : (i0 + len < a.ld ? i0 + len : a.ld);
      for (long long s = z0 + threadIdx.x; s < z1; s += kThreads) prow[s] = 0.f;
    }
  }
  // A dense split past the last candidate has nothing to merge; the combine
  // reads only the splits that hold a position.
  if (a.dense && rows == 0 && (a.n_split > 1 || kMode == kModeProbs)) return;
  const int ntiles = (rows + kR - 1) / kR;

  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;

  if (threadIdx.x == 0) fallback = -1;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  lds_barrier();
  // Slots of this split's rows (-1: absent, and past the last row), so the
  // gather depends on LDS only.  All of a thread's positions are loaded first.
  // With a block table, the sequence's entries up to its last candidate are
  // loaded at the same time (they do not depend on the positions) into the
  // tile buffers, idle until the first gather, and looked up there: one global
  // round trip in all.  A table too long for that room is read per position
  // after the positions have landed: two dependent round trips.
  constexpr int kFill = (kMaxSplitRows + 4 * kR + kThreads - 1) / kThreads;
  // block-table entries the tile buffers hold (less one pass of the copy below)
  constexpr int kTableCap = kBufs * kTileBufChunks * 4 - 4 * kThreads;
  const int nfill = ntiles * kR + 3 * kR;
  int pos[kFill];
#pragma unroll
  for (int u = 0; u < kFill; ++u) {
    const int j = threadIdx.x + u * kThreads;
    pos[u] = j < rows ? (a.dense ? i0 + j : irow[i0 + j]) : -1;
  }
  const int nblk = (n + 63) >> 6;
  int sl[kFill];
  if (a.sv.block_table == nullptr) {
#pragma unroll
    for (int u = 0; u < kFill; ++u)
      sl[u] = (pos[u] >= 0 && pos[u] < n) ? (int)((long long)b * a.sv.max_seq_len + pos[u]) : -1;
  } else if (nblk <= kTableCap) {
    const int32_t *bt = a.sv.block_table + (long long)b * a.sv.max_blocks;
    int32_t *tbl = reinterpret_cast<int32_t *>(&tiles[0][0]);
    // Every lane loads (entries past the last needed one read that one) and
    // stores; entries past nblk are never looked up.  No branches.
    // The first pass (contexts up to 128K) is straight-line code, so that its
    // loads are not held back by a wait at a loop head.
    const int last = nblk > 0 ? nblk - 1 : 0;
    auto copy_pass = [&](int e0) {
      int te[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + (int)threadIdx.x + u * kThreads;
        te[u] = bt[e < last ? e : last];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) tbl[e0 + threadIdx.x + u * kThreads] = te[u];
    };
    copy_pass(0);
    for (int e0 = 4 * kThreads; e0 < nblk; e0 += 4 * kThreads) copy_pass(e0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const bool ok = pos[u] >= 0 && pos[u] < n;
      const int blk = tbl[ok ? (pos[u] >> 6) : 0];
      sl[u] = (ok && blk >= 0 && blk < a.sv.num_blocks) ? blk * 64 + (pos[u] & 63) : -1;
    }
  } else {
    // every lane loads (an invalid position reads the sequence's first entry),
    // so the loads are issued back to back
    const int32_t *bt = a.sv.block_table + (long long)b * a.sv.max_blocks;
    int blk[kFill];
#pragma unroll
    for (int u = 0; u < kFill; ++u) blk[u] = bt[(pos[u] >= 0 && pos[u] < n) ? (pos[u] >> 6) : 0];
#pragma unroll
    for (int u = 0; u < kFill; ++u)
      sl[u] = (pos[u] >= 0 && pos[u] < n && blk[u] >= 0 && blk[u] < a.sv.num_blocks) ? blk[u] * 64 + (pos[u] & 63)
                                                                                     : -1;
  }
  // Q^T operands for this wave's heads: lane holds head 16 wv + col,
  // dims 32 ks + 8 g + [0, 8).  Issued only now: vector-memory waits are in
  // order, so query loads issued before the index and page-table loads would
  // be drained by the waits for those.  From here they stream in with the
  // first tile; the barriers up to it wait for LDS work only.
  bf16x8 qb[kQ][kKs];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int tq = r + q < a.rows ? t + q : t;
    const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q) + ((long long)tq * kH + wv * 16 + col) * (kD * 2);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qb[q][ks] = as_bf16x8(ld16(qrow + ks * 64 + g * 16));
  }
#pragma unroll
  for (int u = 0; u < kFill; ++u) {
    const int j = threadIdx.x + u * kThreads;
    if (j < nfill) {
      slots[j] = sl[u];
      if (sl[u] >= 0) atomicMax(&fallback, sl[u]);
    }
  }

  f32x4 acc[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db) acc[db] = zero_vec<f32x4>();
  float m_run[kQ], l_run[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    m_run[q] = neg_inf();
    l_run[q] = 0.f;
  }
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t *kv = reinterpret_cast<const uint8_t *>(a.kv);
  // per-lane LDS byte offsets: the logit operand (row col, data chunk 4 ks + g)
  // and the transpose reads (row 4 g + col/4, dims 4 (col%4).. of each 16-dim block)
  const uint32_t qk_off = col * kRowStride + (g ^ swz(col)) * 16;
  const int vc = col & 3;
  const uint32_t pv_row = (4 * g + (col >> 2)) * kRowStride + (vc & 1) * 8;
  const uint32_t pv_even = pv_row + (((vc >> 1)) ^ g) * 16;
  const uint32_t pv_odd = pv_row + ((2 + (vc >> 1)) ^ g) * 16;
  const uint32_t tile_lds = lds_addr(&tiles[0][0]);
  constexpr uint32_t kTileBytes = kTileBufChunks * 16;
  // probs: this lane's head's log-sum-exp in base 2, per query
  float lse2[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    lse2[q] = kMode == kModeProbs && r + q < a.rows ? a.lse[(long long)(t + q) * kH + wv * 16 + col] * kLog2e : 0.f;
  // probs: the normalised weights of tile tt's rows, summed over every head in a
  // fixed order (wave 0, after the barrier that follows the tile)
  auto write_probs = [&](int tt) {
    if (lane < kR) {
      const int j = tt * kR + lane;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += psums[tt & 1][(q * kWaves + w) * kR + lane];
        if (j < nrow[q]) a.probs[(long long)(r + q) * a.ld + i0 + j] = v * (1.f / kH);
      }
    }
  };
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  lds_barrier();
  const int fb = fallback;

  if (fb >= 0) {
    // Three tile buffers: tiles tt+1 and tt+2 stream in while tile tt is used.
    // tile tt's gather: every wave (attention), or half (tt even: waves 0-3, odd: 4-7)
    constexpr bool kHalf = kMode != kModeAttn;
    const int half = wv / kHalfWaves, hw = wv % kHalfWaves;
    const TileCoords tc = tile_coords(wv, lane);
    auto issue = [&](uint32_t buf, int tt) {
      if constexpr (kHalf) {
        if ((tt & 1) == half) issue_tile_half(buf, kv, slots, tt * kR, fb, hw, lane);
      } else {
        issue_tile<kStream>(buf, kv, slots, tt * kR, fb, wv, tc);
      }
    };
    issue(tile_lds, 0);
    // Drain the query operand loads (with tile 0) here, so that no wait for them
    // is placed inside the loop, where it would also wait for the prefetches.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (ntiles > 1) issue(tile_lds + kTileBytes, 1);
    int cur = 0;
    for (int tt = 0; tt < ntiles; ++tt) {
      // This wave's loads of tile tt have landed once at most the loads of tile
      // tt+1 are outstanding; the barrier then covers every wave's, and also
      // orders every wave's reads of tile tt-1 before its buffer is refilled.
      // (probs: the head sums of tile tt-1 written to LDS are complete as well)
      constexpr int kLgkm = kMode == kModeProbs ? 0x0F00 : 0;
      // (halves: a wave's only outstanding loads are of its own half's tile, tt or tt+1)
      if (kHalf ? (tt & 1) == half : tt + 1 >= ntiles)
        __builtin_amdgcn_s_waitcnt(kWaitVm0 & ~kLgkm);
      else
        __builtin_amdgcn_s_waitcnt((kHalf ? kWaitNone : wait_vm(kWaveLoads)) & ~kLgkm);
      lds_barrier();
      if (tt + 2 < ntiles) {
        const int nb = cur == 0 ? 2 : cur - 1;     // (tt + 2) % 3
        issue(tile_lds + nb * kTileBytes, tt + 2);
      }
      if (kMode == kModeProbs && tt > 0 && wv == 0) write_probs(tt - 1);
      consume_tile<kMode, kQ>(tile_lds + cur * kTileBytes, slots, tt * kR, qb, acc, m_run, l_run, scale2, qk_off,
                              pv_even, pv_odd, g, lse2, nrow,
                              &psums[kMode == kModeProbs ? (tt & 1) : 0][kMode == kModeProbs ? wv * kR : 0]);
      cur = cur == 2 ? 0 : cur + 1;
    }
  }
  if constexpr (kMode == kModeProbs) {
    if (fb >= 0 && ntiles > 0) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      lds_barrier();
      if (wv == 0) write_probs(ntiles - 1);
    } else {
#pragma unroll
      for (int q = 0; q < kQ; ++q)                // none present: every weight is 0
        for (int j = threadIdx.x; j < nrow[q]; j += kThreads) a.probs[(long long)(r + q) * a.ld + i0 + j] = 0.f;
    }
    return;
  }

  const int h = wv * 16 + col;
  if constexpr (kMode == kModeLse) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const float lq = sum_over_rows(l_run[q]);
      if (g == 0 && r + q < a.rows) {
        if (a.n_split == 1) {
          if (a.lse != nullptr)
            a.lse[(long long)(t + q) * kH + h] = lq > 0.f ? (m_run[q] + __log2f(lq)) * kLn2 : neg_inf();
        } else {
          reinterpret_cast<float2 *>(a.part)[((long long)(r + q) * a.n_split + sp) * kH + h] =
              make_float2(m_run[q], lq);
        }
      }
    }
    return;
  }
  const float l_tot = sum_over_rows(l_run[0]);
  // One split: the output row.  Several: this split's normalised output in
  // bf16 (a weighted mean of value rows, so within their range) and its
  // (max, sum), merged by the combine kernel.
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const long long orow_i = a.n_split == 1 ? (long long)t * kH + h : ((long long)r * a.n_split + sp) * kH + h;
  uint16_t *orow = reinterpret_cast<uint16_t *>(a.n_split == 1 ? a.out : a.part) + orow_i * kDv;
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
    const int d = db * 16 + 4 * g;
    uint2 pk;
    pk.x = pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv);
    pk.y = pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv);
    *reinterpret_cast<uint2 *>(orow + d) = pk;
  }
  if (g == 0) {
    if (a.n_split == 1) {
      if (a.lse != nullptr) a.lse[orow_i] = l_tot > 0.f ? (m_run[0] + __log2f(l_tot)) * kLn2 : neg_inf();
    } else {
      float2 *ml = reinterpret_cast<float2 *>(reinterpret_cast<uint16_t *>(a.part) +
                                              (long long)a.rows * a.n_split * kH * kDv);
      ml[orow_i] = make_float2(m_run[0], l_tot);
    }
  }
}

// Merge the split partials of one (query, head): one wave per head, each lane
// owning 8 consecutive value dims.  Lanes s and s + 64 read the running maximum
// and sum of splits s and s + 64 (up to 128 splits); split s weighs
// exp2(max_s - M) sum_s, normalised over the splits.  The loads of up to eight
// splits are issued together, and the weighted sum runs in split order.  A
// dense list merges only the splits that hold a position.
// The combine's (query, head group) of workgroup blockIdx.x, placed on the XCD
// whose workgroups wrote that query's split partials (mla_block), so that the
// partials are read from that XCD's L2.
__device__ __forceinline__ void combine_block(const MlaArgs &a, int &r, int &hg) {
  constexpr int kGroups = kH / 4;
  const int v = blockIdx.x;
  if ((a.rows & 7) == 0) {
    const int x = v & 7, k = v >> 3;
    hg = k % kGroups;
    if (a.dense && a.sv.mode == DSA_PREFILL)
      r = (k / kGroups) * 8 + x;                  // XCD x: queries x, x+8, ...
    else
      r = x * (a.rows >> 3) + k / kGroups;        // XCD x: a contiguous eighth of the queries
    return;
  }
  r = v / kGroups;
  hg = v - r * kGroups;
}

__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a) {
  const int lane = lane_id();
  int r, hg;
  combine_block(a, r, hg);
  const int h = hg * 4 + (threadIdx.x >> 6);
  const int t = a.q_begin + r;
  const int ns = a.n_split;
  int nm = ns;
  if (a.dense) {
    const int len = split_len(a.k, ns);
    const int n = a.sv.candidates(t);
    nm = n <= 0 ? 0 : (n + len - 1) / len;
    if (nm > ns) nm = ns;
  }
  const uint16_t *po = reinterpret_cast<const uint16_t *>(a.part) + ((long long)r * ns * kH + h) * kDv + lane * 8;
  const float2 *ml = reinterpret_cast<const float2 *>(reinterpret_cast<const uint16_t *>(a.part) +
                                                      (long long)a.rows * ns * kH * kDv) +
                     (long long)r * ns * kH + h;
  // The first eight splits' partials are loaded together with the (max, sum)
  // pairs, ahead of them, so that one memory latency covers both; split
  // indices past the last are clamped to it, and those loads are not used.
  uint4 v[8];
  const int slast = nm > 0 ? nm - 1 : 0;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    v[u] = *reinterpret_cast<const uint4 *>(po + (long long)(u < slast ? u : slast) * kH * kDv);
  float ms0 = neg_inf(), ls0 = 0.f, ms1 = neg_inf(), ls1 = 0.f;
  if (lane < nm) {
    const float2 v = ml[(long long)lane * kH];
    ms0 = v.x;
    ls0 = v.y;
  }
  if (lane + 64 < nm) {
    const float2 v = ml[(long long)(lane + 64) * kH];
    ms1 = v.x;
    ls1 = v.y;
  }
  const float M = wave_max(fmaxf(ms0, ms1));
  const float w0 = ms0 == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(ms0 - M) * ls0;
  const float w1 = ms1 == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(ms1 - M) * ls1;
  const float L = wave_sum(w0 + w1);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // splits s0..s0+7 (those below nm) added in split order
  auto accumulate = [&](int s0) {
    const float w = s0 < 64 ? w0 : w1;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < nm) {
        const float wu =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (s0 + u) & 63));
        const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = fmaf(wu, __builtin_bit_cast(float, x[i] << 16), o[2 * i]);
          o[2 * i + 1] = fmaf(wu, __builtin_bit_cast(float, x[i] & 0xFFFF0000u), o[2 * i + 1]);
        }
      }
  };
  accumulate(0);
  for (int s0 = 8; s0 < nm; s0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int su = s0 + u < nm ? s0 + u : nm - 1;
      v[u] = *reinterpret_cast<const uint4 *>(po + (long long)su * kH * kDv);
    }
    accumulate(s0);
  }
  uint16_t *orow = reinterpret_cast<uint16_t *>(a.out) + ((long long)t * kH + h) * kDv + lane * 8;
  uint4 pk;
  pk.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  pk.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  pk.z = pack_bf16x2(o[4] * inv, o[5] * inv);
  pk.w = pack_bf16x2(o[6] * inv, o[7] * inv);
  *reinterpret_cast<uint4 *>(orow) = pk;
  if (lane == 0 && a.lse != nullptr) a.lse[(long long)t * kH + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : neg_inf();
}

// lse pass with several splits: one thread per (query, head) merges the
// splits' (max, sum) pairs in split order.
__global__ __launch_bounds__(256) void mla_lse_combine_kernel(MlaArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)a.rows * kH) return;
  const int r = (int)(i / kH), h = (int)(i % kH);
  const int t = a.q_begin + r;
  const int ns = a.n_split;
  int nm = ns;
  if (a.dense) {
    const int len = split_len(a.k, ns);
    const int n = a.sv.candidates(t);
    nm = n <= 0 ? 0 : (n + len - 1) / len;
    if (nm > ns) nm = ns;
  }
  const float2 *ml = reinterpret_cast<const float2 *>(a.part) + (long long)r * ns * kH + h;
  float M = neg_inf();
  for (int s = 0; s < nm; ++s) M = fmaxf(M, ml[(long long)s * kH].x);
  float L = 0.f;
  for (int s = 0; s < nm; ++s) {
    const float2 v = ml[(long long)s * kH];
    if (v.x != neg_inf()) L += __builtin_amdgcn_exp2f(v.x - M) * v.y;
  }
  a.lse[(long long)t * kH + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : neg_inf();
}

// fp32, small shapes (H <= 16, D <= 128, k <= 1024): one workgroup per query,
// logits in LDS, exact two-pass softmax.
__global__ __launch_bounds__(256) void mla_f32_kernel(MlaArgs a) {
  extern __shared__ __attribute__((aligned(8))) float sm[];
  const int H = a.H, D = a.D, Dv = a.Dv, K = a.k;
  long long *slots = reinterpret_cast<long long *>(sm);   // [K]
  float *qs = sm + 2 * K;         // [H, D]
  float *z = qs + H * D;          // [H, K]
  float *stat = z + H * K;        // [H, 2]
  const int r = blockIdx.x;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const float *q = reinterpret_cast<const float *>(a.q) + (long long)t * H * D;
  const float *kv = reinterpret_cast<const float *>(a.kv);
  const int32_t *irow = a.dense ? nullptr : a.idx + (long long)r * K;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) qs[i] = q[i];
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    const int s = a.dense ? j : irow[j];
    slots[j] = (s >= 0 && s < n) ? a.sv.slot(b, s) : -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < H * K; i += blockDim.x) {
    const int hh = i / K, j = i - hh * K;
    float zz = neg_inf();
    if (slots[j] >= 0) {
      const float *row = kv + slots[j] * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[hh * D + d], row[d], dot);
      zz = dot * a.sm_scale;
    }
    z[i] = zz;
  }
  __syncthreads();
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  for (int hh = wv; hh < H; hh += blockDim.x / 64) {
    float mx = neg_inf();
    for (int j = lane; j < K; j += 64) mx = fmaxf(mx, z[hh * K + j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < K; j += 64) {
      const float zz = z[hh * K + j];
      const float p = zz == neg_inf() ? 0.f : expf(zz - mx);
      z[hh * K + j] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      stat[2 * hh] = mx;
      stat[2 * hh + 1] = sum;
    }
  }
  __syncthreads();
  float *out = reinterpret_cast<float *>(a.out) + (long long)t * H * Dv;
  for (int i = threadIdx.x; i < H * Dv; i += blockDim.x) {
    const int hh = i / Dv, d = i - hh * Dv;
    float o = 0.f;
    for (int j = 0; j < K; ++j)
      if (slots[j] >= 0) o = fmaf(z[hh * K + j], kv[slots[j] * D + d], o);
    const float l = stat[2 * hh + 1];
    out[i] = l > 0.f ? o / l : 0.f;
  }
  if (a.lse != nullptr)
    for (int hh = threadIdx.x; hh < H; hh += blockDim.x) {
      const float l = stat[2 * hh + 1];
      a.lse[(long long)t * H + hh] = l > 0.f ? stat[2 * hh] + logf(l) : neg_inf();
    }
}

}  // namespace

int mla_splits(int rows, int k) {
  int s = (256 + rows - 1) / rows;
  int cap = (k + 2 * kR - 1) / (2 * kR);
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

// A dense list of `span` entries: splits of at most kMaxSplitRows entries (the
// slot list of a workgroup), and at least as many as fill the chip.
int mla_dense_splits(int rows, int span) {
  int s = (span + kMaxSplitRows - 1) / kMaxSplitRows;
  const int fill = mla_splits(rows, span);
  if (s < fill) s = fill;
  return s > kMlaMaxSplits ? kMlaMaxSplits : s;
}

size_t mla_f32_lds(int H, int D, int k) {
  return (size_t)(2 * k + H * D + H * k + 2 * H) * sizeof(float);
}

hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.dtype == DSA_F32) {
    const size_t lds = mla_f32_lds(a.H, a.D, a.k);
    if (lds > 65536) {
      const hipError_t e =
          hipFuncSetAttribute((const void *)mla_f32_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(mla_f32_kernel, dim3(a.rows), dim3(256), lds, st, a);
    return hipGetLastError();
  }
  const dim3 grid(a.n_split * a.rows);
  // the lse and probs passes of a prefill serve two queries from each tile
  const bool pair = a.dense && a.sv.mode == DSA_PREFILL && a.rows > 1;
  const dim3 grid2(a.n_split * ((a.rows + 1) / 2));
  if (a.mode == kModeLse) {
    if (pair)
      hipLaunchKernelGGL((mla_bf16_kernel<kModeLse, 2>), grid2, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((mla_bf16_kernel<kModeLse, 1>), grid, dim3(kThreads), 0, st, a);
    if (a.n_split > 1)
      hipLaunchKernelGGL(mla_lse_combine_kernel, dim3((unsigned)(((long long)a.rows * kH + 255) / 256)), dim3(256), 0,
                         st, a);
  } else if (a.mode == kModeProbs) {
    if (pair)
      hipLaunchKernelGGL((mla_bf16_kernel<kModeProbs, 2>), grid2, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((mla_bf16_kernel<kModeProbs, 1>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (a.sv.mode == DSA_DECODE)
      hipLaunchKernelGGL((mla_bf16_kernel<kModeAttn, 1, true>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((mla_bf16_kernel<kModeAttn, 1>), grid, dim3(kThreads), 0, st, a);
    if (a.n_split > 1) hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(kH / 4) * (unsigned)a.rows), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dsa

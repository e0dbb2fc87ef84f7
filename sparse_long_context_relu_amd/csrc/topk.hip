// Fine-grained top-k token selection: for every query, the first
// m = min(k, n) candidates in the order (score descending, position
// ascending) ("DeepSeek V3.2: How Far Can Open Models Go If You Actually
// Try?", section 3.1, selection equation; "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", System Modules, top-k operation).
//
// Exact integer radix select on order-preserving 32-bit keys, no float
// arithmetic:
//   hist1   11-bit histogram of key[31:21] over the row -> top digit d1.
//           Built by the indexer's epilogue inside the fused path, or by
//           topk_hist1_kernel for scores handed in from outside.
//   collect one pass over the row: keys with key[31:21] > d1 are selected
//           outright (fewer than m of them); keys with key[31:21] == d1 are
//           the candidates.
//   select  radix passes over the candidates (key[20:10], then key[9:0])
//           give the exact threshold T; keys above T are selected and keys
//           equal to T are taken lowest position first.  The selection is
//           written in ascending position order through LDS bitmaps: the
//           output is deterministic and needs no sort.
// Few long rows (decode): collect splits every row over workgroups; each
// writes its selected positions and candidates to its own region (no global
// atomics) and adds the candidates' second-digit histogram to the row's; one
// workgroup per row then selects.  Many rows (prefill): one workgroup per row
// does collect and select, candidates in LDS.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kNT = 256;
constexpr int kRowNT = 512;
constexpr int kLdsCap = 2048;    // candidates held in LDS by the one-workgroup-per-row path (4 workgroups per CU at 64K)
constexpr int kTieCap = 4096;    // second-digit ties held in LDS by the sliced select

struct RowWs {
  uint32_t *hist1, *hist2, *info, *counts, *sel, *cand;
};

__device__ __forceinline__ RowWs row_ws(const TopkArgs &a, int r) {
  uint32_t *base = a.ws + (long long)r * a.row_words;
  RowWs w;
  w.hist1 = base;
  w.hist2 = base + kTopkHist2;
  w.info = base + kTopkInfo;
  w.counts = base + kTopkCounts;
  w.sel = base + kTopkRegions;
  w.cand = w.sel + (long long)a.slices * a.sel_seg;
  return w;
}

// Exclusive prefix over the threads of a block (NT a multiple of 64); `tmp`
// holds NT/64 ints of LDS.  Returns the exclusive prefix, sets `total`.
template <int NT>
__device__ int block_exclusive_scan(int v, int *tmp, int &total) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int x = tmp[i];
    before += i < wv ? x : 0;
    total += x;
  }
  __syncthreads();
  return before + inc - v;
}

// Given a histogram (nbins, in LDS) and 1 <= need <= total, find the digit d
// with count(bins > d) < need <= count(bins >= d).  Writes d and
// count(bins > d) to out[0..1] (LDS) and returns after a barrier.
template <int NT>
__device__ void find_digit(const uint32_t *hist, int nbins, int need, int *out, int *tmp) {
  const int per = nbins / NT;
  // thread i owns bins [nbins - (i+1) per, nbins - i per): descending order
  const int hi = nbins - threadIdx.x * per;
  int local = 0;
  for (int j = 1; j <= per; ++j) local += (int)hist[hi - j];
  int total;
  const int above = block_exclusive_scan<NT>(local, tmp, total);
  if (above < need && above + local >= need) {
    int acc = above;
    for (int j = 1; j <= per; ++j) {
      const int c = (int)hist[hi - j];
      if (acc + c >= need) {
        out[0] = hi - j;
        out[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Ascending-position compaction of the selection: the bits of selmap, plus the
// first `quota` bits of eqmap (ties at the threshold, lowest position first),
// written to out[0, m); out[m, k) = -1.  Thread i owns words [i*wpt, (i+1)*wpt).
// `quota` is block-uniform.
template <int NT>
__device__ void compact_selection(uint32_t *selmap, const uint32_t *eqmap, int W, int quota, int m, int k,
                                  int32_t *out, int *tmp) {
  const int wpt = (W + NT - 1) / NT;
  const int w0 = threadIdx.x * wpt;
  const int w1 = w0 + wpt < W ? w0 + wpt : W;
  int tot;
  int cnt = 0;
  if (quota > 0) {
    int eq_local = 0;
    for (int i = w0; i < w1; ++i) eq_local += __popc(eqmap[i]);
    int eq_before = block_exclusive_scan<NT>(eq_local, tmp, tot);
    for (int i = w0; i < w1; ++i) {
      uint32_t e = eqmap[i];
      uint32_t take = 0u;
      while (e && eq_before < quota) {
        const uint32_t low = e & (0u - e);
        take |= low;
        e ^= low;
        ++eq_before;
      }
      const uint32_t bits = selmap[i] | take;
      selmap[i] = bits;
      cnt += __popc(bits);
    }
  } else {
    for (int i = w0; i < w1; ++i) cnt += __popc(selmap[i]);
  }
  int pos = block_exclusive_scan<NT>(cnt, tmp, tot);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = selmap[i];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < m) out[pos] = i * 32 + b;
      ++pos;
    }
  }
  for (int i = m + threadIdx.x; i < k; i += NT) out[i] = -1;
}

// Load one round of row[s], s in [base, base + NT*16) clipped to [.., s1),
// into x: thread t holds elements base + (i*NT + t)*4 + c.  Sixteen scores per
// thread are in flight together (16-byte loads when the row is aligned).
// Buffer loads over [row, row + s1): elements past s1 read as zero (their
// keys are masked by the caller), so no load needs a branch; a branch per
// element group made the compiler wait for each group's loads in turn.
template <int NT>
__device__ __forceinline__ void load_round(const float *row, int base, int s1, bool vec, float (&x)[4][4]) {
  const __amdgpu_buffer_rsrc_t d =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), (short)0, s1 * 4, kBufferDword3);
  if (vec) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = base + (i * NT + (int)threadIdx.x) * 4;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(d, e * 4, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[i][c] = __uint_as_float(v[c]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        x[i][c] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(d, (base + (i * NT + (int)threadIdx.x) * 4 + c) * 4, 0, 0));
  }
}

// Visit row[s], s in [s0, s1) (s0 a multiple of 4), in rounds that every lane
// of the block takes part in: f(s, key, valid).
template <int NT, typename F>
__device__ __forceinline__ void scan_row(const float *row, int s0, int s1, F &&f) {
  const bool vec = ((uintptr_t)(row + s0) & 15) == 0;
  for (int base = s0; base < s1; base += NT * 16) {
    float x[4][4];
    load_round<NT>(row, base, s1, vec, x);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int sidx = base + (i * NT + (int)threadIdx.x) * 4 + c;
        f(sidx, score_key(x[i][c]), sidx < s1);
      }
  }
}

// Slice b of a row of n candidates: [b per, min(n, (b+1) per)), per a multiple of 64.
__device__ __forceinline__ void slice_range(const TopkArgs &a, int n, int b, int &s0, int &s1) {
  const int per = ((n + a.slices - 1) / a.slices + 63) & ~63;
  s0 = b * per;
  s1 = s0 + per < n ? s0 + per : n;
  if (s1 < s0) s1 = s0;
}

__global__ __launch_bounds__(kNT) void topk_zero_kernel(TopkArgs a) {
  // rows start 16-byte aligned (row_words and the workspace base are multiples of 4 words)
  static_assert(kTopkHdrWords % 4 == 0, "16-byte stores");
  uint4 *base = reinterpret_cast<uint4 *>(a.ws + (long long)blockIdx.x * a.row_words);
  for (int i = threadIdx.x; i < kTopkHdrWords / 4; i += kNT) base[i] = make_uint4(0u, 0u, 0u, 0u);
}

// hist1 for scores handed in from outside (the fused path builds it in the indexer).
__global__ __launch_bounds__(kNT) void topk_hist1_kernel(TopkArgs a) {
  const int r = blockIdx.y;
  const int n = a.sv.candidates(a.q_begin + r);
  if (n <= a.k) return;
  __shared__ uint32_t h[kTopkBins];
  for (int i = threadIdx.x; i < kTopkBins; i += kNT) h[i] = 0u;
  __syncthreads();
  int s0, s1;
  slice_range(a, n, blockIdx.x, s0, s1);
  const float *row = a.scores + (long long)r * a.ld;
  scan_row<kNT>(row, s0, s1, [&](int, uint32_t key, bool valid) {
    if (valid) atomicAdd(&h[key >> 21], 1u);
  });
  __syncthreads();
  RowWs w = row_ws(a, r);
  for (int i = threadIdx.x; i < kTopkBins; i += kNT)
    if (h[i]) atomicAdd(&w.hist1[i], h[i]);
}

// Sliced collect: keys above the top digit go to this slice's selected
// region, keys in it to its candidate region, and the candidates' second
// digits to the row's second histogram.  The first round of scores is in
// flight while the top digit is searched.
__global__ __launch_bounds__(kNT) void topk_collect_kernel(TopkArgs a) {
  const int r = blockIdx.y, b = blockIdx.x;
  const int n = a.sv.candidates(a.q_begin + r);
  if (n <= a.k) return;
  __shared__ uint32_t h[kTopkBins];   // hist1 for the digit search, then this slice's hist2
  __shared__ int res[2];
  __shared__ int tmp[kNT / 64];
  __shared__ uint32_t wcnt[2][kNT / 64];
  RowWs w = row_ws(a, r);
  int s0, s1;
  slice_range(a, n, b, s0, s1);
  const float *row = a.scores + (long long)r * a.ld;
  const bool vec = ((uintptr_t)(row + s0) & 15) == 0;
  float x[4][4];
  load_round<kNT>(row, s0, s1, vec, x);
  {
    // all of this thread's bins in flight at once
    uint32_t hv[kTopkBins / kNT];
#pragma unroll
    for (int j = 0; j < kTopkBins / kNT; ++j) hv[j] = w.hist1[threadIdx.x + j * kNT];
#pragma unroll
    for (int j = 0; j < kTopkBins / kNT; ++j) h[threadIdx.x + j * kNT] = hv[j];
  }
  __syncthreads();
  find_digit<kNT>(h, kTopkBins, a.k, res, tmp);
  const uint32_t d1 = (uint32_t)res[0];
  if (b == 0 && threadIdx.x == 0) {
    w.info[0] = d1;
    w.info[1] = (uint32_t)res[1];
  }
  for (int i = threadIdx.x; i < kTopkBins; i += kNT) h[i] = 0u;
  __syncthreads();

  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t *sel = w.sel + (long long)b * a.sel_seg;
  uint32_t *cand = w.cand + 2ll * b * a.slice_len;
  uint32_t ns_run = 0u, nc_run = 0u;   // block-uniform running counts
  for (int base = s0; base < s1; base += kNT * 16) {
    if (base != s0) load_round<kNT>(row, base, s1, vec, x);
    uint32_t key[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = base + (i * kNT + (int)threadIdx.x) * 4 + c;
        key[i][c] = e < s1 ? score_key(x[i][c]) : 0u;   // key 0: digit 0, below every valid key
      }
    uint32_t ns = 0u, nc = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t dig = key[i][c] >> 21;
        ns += (uint32_t)__popcll(__ballot(dig > d1));
        nc += (uint32_t)__popcll(__ballot(dig == d1));
      }
    if (lane == 0) {
      wcnt[0][wv] = ns;
      wcnt[1][wv] = nc;
    }
    __syncthreads();
    uint32_t os = ns_run, oc = nc_run;
#pragma unroll
    for (int j = 0; j < kNT / 64; ++j) {
      const uint32_t a0 = wcnt[0][j], a1 = wcnt[1][j];
      if (j < wv) {
        os += a0;
        oc += a1;
      }
      ns_run += a0;
      nc_run += a1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = key[i][c];
        const uint32_t dig = kk >> 21;
        const bool is_sel = dig > d1;
        const bool is_cand = dig == d1;
        const unsigned long long ms = __ballot(is_sel);
        const unsigned long long mc = __ballot(is_cand);
        const int sidx = base + (i * kNT + (int)threadIdx.x) * 4 + c;
        if (is_sel) {
          const uint32_t pos = os + __popcll(ms & below);
          if (pos < (uint32_t)a.sel_seg) sel[pos] = (uint32_t)sidx;
        }
        if (is_cand) {
          const uint32_t pos = oc + __popcll(mc & below);
          cand[2 * pos] = kk & 0x1fffffu;
          cand[2 * pos + 1] = (uint32_t)sidx;
          atomicAdd(&h[(kk & 0x1fffffu) >> 10], 1u);
        }
        os += (uint32_t)__popcll(ms);
        oc += (uint32_t)__popcll(mc);
      }
    __syncthreads();   // wcnt is rewritten by the next round; h is complete after the last
  }
  // The row's second histogram gets this slice's nonzero bins.  Buffer atomics
  // with a constant lane offset and the bin block in the scalar offset: no
  // address register is rewritten between them, so they issue back to back
  // (a rewritten address register makes the compiler wait for the previous
  // atomic to complete).
  static_assert(kTopkBins % kNT == 0, "bins per thread");
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(w.hist2, (short)0, kTopkBins * 4, kBufferDword3);
  uint32_t hv[kTopkBins / kNT];
#pragma unroll
  for (int j = 0; j < kTopkBins / kNT; ++j) hv[j] = h[threadIdx.x + j * kNT];
#pragma unroll
  for (int j = 0; j < kTopkBins / kNT; ++j)
    if (hv[j]) __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32((int)hv[j], hr, (int)threadIdx.x * 4, j * kNT * 4, 0);
  // last: a store's address registers rewritten after it would make the
  // compiler wait for the store
  if (threadIdx.x == 0) {
    w.counts[b] = ns_run;
    w.counts[kTopkMaxSlices + b] = nc_run;
  }
}

// Sliced select, one workgroup per row: the second digit from the collected
// histogram, one pass over the slices' lists (selected positions and
// candidates above the second digit go to the bitmap, ties of the second digit
// to an LDS list), the third digit over those ties, then the compaction.
// Thread t serves slice t % slices, entries t / slices, t / slices + tps, ...
__global__ __launch_bounds__(kRowNT) void topk_select_sliced_kernel(TopkArgs a) {
  extern __shared__ uint32_t smem[];
  const int r = blockIdx.x;
  const int n = a.sv.candidates(a.q_begin + r);
  int32_t *out = a.idx + (long long)r * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kRowNT) out[i] = i < n ? i : -1;
    return;
  }
  const int m = a.k;
  const int Wmax = (a.sv.max_ctx + 31) >> 5;
  const int W = (n + 31) >> 5;
  uint32_t *selmap = smem;
  uint32_t *eqmap = smem + Wmax;
  uint32_t *h = smem + 2 * Wmax;                 // kTopkBins words
  uint32_t *ties = h + kTopkBins;                // 2 * kTieCap words: (low key bits, position)
  __shared__ int res[6];
  __shared__ int tmp[kRowNT / 64];
  __shared__ uint32_t cnt_s[kTopkMaxSlices], cnt_c[kTopkMaxSlices];
  __shared__ uint32_t nties;

  RowWs w = row_ws(a, r);
  const int sb = threadIdx.x % a.slices;         // this thread's slice
  const int tps = kRowNT / a.slices;             // threads per slice
  const int t0 = threadIdx.x / a.slices;
  const bool active = t0 < tps;
  const uint32_t *ssel = w.sel + (long long)sb * a.sel_seg;
  const uint32_t *scand = w.cand + 2ll * sb * a.slice_len;
  // This thread's first list entries are loaded before the slice counts and
  // the second digit are known (the loads depend on neither; entries past a
  // slice's count are read but not used), so the list reads overlap the
  // histogram read instead of following it.
  constexpr int kSelPT = 4, kCandPT = 16;
  uint32_t s_pre[kSelPT];
  uint2 c_pre[kCandPT];
  // (indices clamped into the slice's regions, so the loads need no branch and
  // go out back to back; the use below masks them by the counts)
#pragma unroll
  for (int u = 0; u < kSelPT; ++u) {
    const int i = t0 + u * tps;
    s_pre[u] = ssel[i < a.sel_seg ? i : a.sel_seg - 1];
  }
#pragma unroll
  for (int u = 0; u < kCandPT; ++u) {
    const int i = t0 + u * tps;
    c_pre[u] = *reinterpret_cast<const uint2 *>(scand + 2 * (i < a.slice_len ? i : a.slice_len - 1));
  }
  {
    uint32_t hv[kTopkBins / kRowNT];
#pragma unroll
    for (int j = 0; j < kTopkBins / kRowNT; ++j) hv[j] = w.hist2[threadIdx.x + j * kRowNT];
#pragma unroll
    for (int j = 0; j < kTopkBins / kRowNT; ++j) h[threadIdx.x + j * kRowNT] = hv[j];
  }
  for (int i = threadIdx.x; i < W; i += kRowNT) {
    selmap[i] = 0u;
    eqmap[i] = 0u;
  }
  if (threadIdx.x < a.slices) {
    cnt_s[threadIdx.x] = w.counts[threadIdx.x];
    cnt_c[threadIdx.x] = w.counts[kTopkMaxSlices + threadIdx.x];
  }
  if (threadIdx.x == 0) {
    res[0] = (int)w.info[0];
    res[1] = (int)w.info[1];
    nties = 0u;
  }
  __syncthreads();
  const int need = m - res[1];                   // still to take among the candidates (>= 1)
  find_digit<kRowNT>(h, kTopkBins, need, res + 2, tmp);
  const uint32_t d2 = (uint32_t)res[2];
  const int need3 = need - res[3];

  const int nsel = active ? (int)min(cnt_s[sb], (uint32_t)a.sel_seg) : 0;
  const int ncand = active ? (int)cnt_c[sb] : 0;
  // selected outright
#pragma unroll
  for (int u = 0; u < kSelPT; ++u)
    if (t0 + u * tps < nsel && s_pre[u] < (uint32_t)n) atomicOr(&selmap[s_pre[u] >> 5], 1u << (s_pre[u] & 31));
  for (int i = t0 + kSelPT * tps; i < nsel; i += tps) {
    const uint32_t sv = ssel[i];
    if (sv < (uint32_t)n) atomicOr(&selmap[sv >> 5], 1u << (sv & 31));
  }
  // candidates: above the second digit -> selected; equal -> the tie list
  auto candidate = [&](uint2 e) {
    const uint32_t lo = e.x & 0x1fffffu, sv = e.y;
    if (sv >= (uint32_t)n) return;
    const uint32_t dig = lo >> 10;
    if (dig > d2) {
      atomicOr(&selmap[sv >> 5], 1u << (sv & 31));
    } else if (dig == d2) {
      const uint32_t p = atomicAdd(&nties, 1u);
      if (p < (uint32_t)kTieCap) {
        ties[2 * p] = lo;
        ties[2 * p + 1] = sv;
      }
    }
  };
#pragma unroll
  for (int u = 0; u < kCandPT; ++u)
    if (t0 + u * tps < ncand) candidate(c_pre[u]);
  for (int i0 = t0 + kCandPT * tps; i0 < ncand; i0 += 4 * tps) {
    uint2 e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      e[u] = i0 + u * tps < ncand ? *reinterpret_cast<const uint2 *>(scand + 2 * (i0 + u * tps))
                                  : make_uint2(0u, 0xffffffffu);
#pragma unroll
    for (int u = 0; u < 4; ++u) candidate(e[u]);
  }
  __syncthreads();
  const int nt = (int)nties;
  int quota = 0;
  if (nt <= 64) {
    // Few ties (the usual case): wave 0 ranks them exactly in the order (low key
    // bits descending, position ascending) and takes the first need3.
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      const uint32_t lo = i < nt ? ties[2 * i] : 0u, s = i < nt ? ties[2 * i + 1] : 0xffffffffu;
      int rank = 0;
      for (int j = 0; j < nt; ++j) {
        const uint32_t lj = (uint32_t)__builtin_amdgcn_readlane((int)lo, j);
        const uint32_t sj = (uint32_t)__builtin_amdgcn_readlane((int)s, j);
        rank += (lj > lo || (lj == lo && sj < s)) ? 1 : 0;
      }
      if (i < nt && rank < need3) atomicOr(&selmap[s >> 5], 1u << (s & 31));
    }
  } else {
    // Visit every tie of the second digit: from the LDS list, or from the slices'
    // candidate lists again when it overflowed.
    auto for_each_tie = [&](auto &&f) {
      if (nt <= kTieCap) {
        for (int i = threadIdx.x; i < nt; i += kRowNT) f(ties[2 * i], ties[2 * i + 1]);
      } else {
        for (int i = t0; i < ncand; i += tps) {
          const uint2 e = *reinterpret_cast<const uint2 *>(scand + 2 * i);
          const uint32_t lo = e.x & 0x1fffffu;
          if (e.y < (uint32_t)n && (lo >> 10) == d2) f(lo, e.y);
        }
      }
    };
    // ---- third digit key[9:0]
    for (int i = threadIdx.x; i < 1024; i += kRowNT) h[i] = 0u;
    __syncthreads();
    for_each_tie([&](uint32_t lo, uint32_t) { atomicAdd(&h[lo & 1023u], 1u); });
    __syncthreads();
    find_digit<kRowNT>(h, 1024, need3, res + 4, tmp);
    const uint32_t T = (d2 << 10) | (uint32_t)res[4];
    quota = need3 - res[5];
    for_each_tie([&](uint32_t lo, uint32_t s) {
      if (lo > T) atomicOr(&selmap[s >> 5], 1u << (s & 31));
      else if (lo == T) atomicOr(&eqmap[s >> 5], 1u << (s & 31));
    });
  }
  __syncthreads();
  compact_selection<kRowNT>(selmap, eqmap, W, quota, m, a.k, out, tmp);
}

// One workgroup per row (many rows): one pass over the row selects the keys
// above the top digit straight into the bitmap, counts the second-digit
// histogram of the candidates (keys in the top digit) and keeps the candidates
// in LDS while they fit.  The second digit then comes from that histogram.  The
// third-digit histogram runs over the candidates in LDS or, when they did not
// fit, over a second pass of the row that also keeps the ties of the second
// digit in LDS (a third pass only when those do not fit either); then the
// exact threshold and the compaction.
__global__ __launch_bounds__(kRowNT) void topk_select_rows_kernel(TopkArgs a) {
  extern __shared__ uint32_t smem[];
  const int r = blockIdx.x;
  const int n = a.sv.candidates(a.q_begin + r);
  int32_t *out = a.idx + (long long)r * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kRowNT) out[i] = i < n ? i : -1;
    return;
  }
  const int m = a.k;
  const int Wmax = (a.sv.max_ctx + 31) >> 5;
  const int W = (n + 31) >> 5;
  uint32_t *selmap = smem;
  uint32_t *eqmap = smem + Wmax;
  uint32_t *h = smem + 2 * Wmax;                 // kTopkBins words
  uint32_t *lcand = h + kTopkBins;               // 2 * kLdsCap words: (low 21 key bits, position)
  __shared__ int res[6];
  __shared__ int tmp[kRowNT / 64];
  __shared__ uint32_t lcount;

  RowWs w = row_ws(a, r);
  {
    uint32_t hv[kTopkBins / kRowNT];
#pragma unroll
    for (int j = 0; j < kTopkBins / kRowNT; ++j) hv[j] = w.hist1[threadIdx.x + j * kRowNT];
#pragma unroll
    for (int j = 0; j < kTopkBins / kRowNT; ++j) h[threadIdx.x + j * kRowNT] = hv[j];
  }
  for (int i = threadIdx.x; i < W; i += kRowNT) {
    selmap[i] = 0u;
    eqmap[i] = 0u;
  }
  if (threadIdx.x == 0) lcount = 0u;
  const float *row = a.scores + (long long)r * a.ld;
  const int lane = lane_id();
  __syncthreads();
  find_digit<kRowNT>(h, kTopkBins, m, res, tmp);
  const uint32_t d1 = (uint32_t)res[0];
  const int need = m - res[1];                   // still to take among the candidates (>= 1)
  for (int i = threadIdx.x; i < kTopkBins; i += kRowNT) h[i] = 0u;
  __syncthreads();

  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // Appends (low key bits, position) of the lanes with `take` to the LDS list.
  auto append = [&](bool take, uint32_t lo, int s) {
    const unsigned long long mc = __ballot(take);
    if (mc == 0ull) return;
    uint32_t bc = 0u;
    if (lane == 0) bc = atomicAdd(&lcount, (uint32_t)__popcll(mc));
    bc = __shfl(bc, 0, kWave);
    if (take) {
      const uint32_t pos = bc + __popcll(mc & below);
      if (pos < (uint32_t)kLdsCap) {
        lcand[2 * pos] = lo;
        lcand[2 * pos + 1] = (uint32_t)s;
      }
    }
  };
  // ---- pass 1: selected keys, second-digit histogram and list of the candidates
  scan_row<kRowNT>(row, 0, n, [&](int s, uint32_t key, bool valid) {
    const uint32_t dig = key >> 21;
    if (valid && dig > d1) atomicOr(&selmap[s >> 5], 1u << (s & 31));
    const bool is_cand = valid && dig == d1;
    if (is_cand) atomicAdd(&h[(key >> 10) & (kTopkBins - 1)], 1u);
    append(is_cand, key & 0x1fffffu, s);
  });
  __syncthreads();
  const bool fit = lcount <= (uint32_t)kLdsCap;   // every candidate is in the list
  // ---- second digit key[20:10]
  find_digit<kRowNT>(h, kTopkBins, need, res + 2, tmp);
  const uint32_t d2 = (uint32_t)res[2];
  const int need3 = need - res[3];
  // ---- third-digit histogram key[9:0] over the ties of the second digit;
  // candidates above the second digit are selected
  for (int i = threadIdx.x; i < 1024; i += kRowNT) h[i] = 0u;
  if (!fit && threadIdx.x == 0) lcount = 0u;      // the list now collects the ties
  __syncthreads();
  if (fit) {
    const int nc = (int)lcount;
    for (int i = threadIdx.x; i < nc; i += kRowNT) {
      const uint32_t lo = lcand[2 * i], sv = lcand[2 * i + 1];
      const uint32_t dig = lo >> 10;
      if (dig > d2) atomicOr(&selmap[sv >> 5], 1u << (sv & 31));
      else if (dig == d2) atomicAdd(&h[lo & 1023u], 1u);
    }
  } else {
    scan_row<kRowNT>(row, 0, n, [&](int s, uint32_t key, bool valid) {
      const bool cand = valid && (key >> 21) == d1;
      const uint32_t lo = key & 0x1fffffu, dig = lo >> 10;
      if (cand && dig > d2) atomicOr(&selmap[s >> 5], 1u << (s & 31));
      const bool tie = cand && dig == d2;
      if (tie) atomicAdd(&h[lo & 1023u], 1u);
      append(tie, lo, s);
    });
  }
  __syncthreads();
  // ties of the second digit: the candidate list filtered by it, the tie list,
  // or a pass over the row when the tie list overflowed too
  const int nlist = (int)lcount;
  const bool tie_fit = fit || nlist <= kLdsCap;
  find_digit<kRowNT>(h, 1024, need3, res + 4, tmp);
  const uint32_t T = (d2 << 10) | (uint32_t)res[4];
  const int quota = need3 - res[5];
  auto mark = [&](uint32_t lo, uint32_t sv) {
    if ((lo >> 10) != d2) return;
    if (lo > T) atomicOr(&selmap[sv >> 5], 1u << (sv & 31));
    else if (lo == T) atomicOr(&eqmap[sv >> 5], 1u << (sv & 31));
  };
  if (tie_fit) {
    for (int i = threadIdx.x; i < nlist; i += kRowNT) mark(lcand[2 * i], lcand[2 * i + 1]);
  } else {
    for (int s = threadIdx.x; s < n; s += kRowNT) {
      const uint32_t key = score_key(row[s]);
      if ((key >> 21) == d1) mark(key & 0x1fffffu, (uint32_t)s);
    }
  }
  __syncthreads();
  compact_selection<kRowNT>(selmap, eqmap, W, quota, m, a.k, out, tmp);
}

// The selection when no query has more than k candidates: every candidate, in
// ascending position order, then -1.
__global__ __launch_bounds__(256) void topk_all_kernel(TopkArgs a) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.k) return;
  const int n = a.sv.candidates(a.q_begin + r);
  a.idx[(long long)r * a.k + j] = j < n ? j : -1;
}

hipError_t set_lds(const void *kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace

bool topk_sliced(int rows) { return rows < 256; }

TopkLayout topk_layout(int rows, int max_ctx) {
  TopkLayout L;
  if (!topk_sliced(rows)) {
    L.slices = 1;
    L.slice_len = 0;
    L.sel_seg = 0;
    L.row_words = kTopkHdrWords;
    return L;
  }
  int s = (2048 + rows - 1) / rows;
  const int cap = (max_ctx + 4095) / 4096;
  if (s > cap) s = cap;
  if (s > kTopkMaxSlices) s = kTopkMaxSlices;
  L.slices = s < 1 ? 1 : s;
  L.slice_len = ((max_ctx + L.slices - 1) / L.slices + 63) & ~63;
  L.sel_seg = L.slice_len < kTopkMaxK ? L.slice_len : kTopkMaxK;
  L.row_words = kTopkRegions + (long long)L.slices * (L.sel_seg + 2ll * L.slice_len);
  return L;
}

hipError_t launch_topk_zero(const TopkArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3(a.rows), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const int Wmax = (a.sv.max_ctx + 31) / 32;
  if (topk_sliced(a.rows)) {
    hipLaunchKernelGGL(topk_collect_kernel, dim3(a.slices, a.rows), dim3(kNT), 0, st, a);
    const size_t lds = (size_t)(2 * Wmax + kTopkBins + 2 * kTieCap) * sizeof(uint32_t);
    if (hipError_t e = set_lds((const void *)topk_select_sliced_kernel, lds)) return e;
    hipLaunchKernelGGL(topk_select_sliced_kernel, dim3(a.rows), dim3(kRowNT), lds, st, a);
  } else {
    const size_t lds = (size_t)(2 * Wmax + kTopkBins + 2 * kLdsCap) * sizeof(uint32_t);
    if (hipError_t e = set_lds((const void *)topk_select_rows_kernel, lds)) return e;
    hipLaunchKernelGGL(topk_select_rows_kernel, dim3(a.rows), dim3(kRowNT), lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_topk_all(const TopkArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_all_kernel, dim3((a.k + 255) / 256, a.rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3(a.rows), dim3(kNT), 0, st, a);
  hipLaunchKernelGGL(topk_hist1_kernel, dim3(a.slices, a.rows), dim3(kNT), 0, st, a);
  return launch_topk_select(a, st);
}

}  // namespace dsa

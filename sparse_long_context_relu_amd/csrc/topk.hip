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
//   select  two radix passes over the candidates (key[20:10], then key[9:0])
//           give the exact threshold T; keys above T are selected and keys
//           equal to T are taken lowest position first.  The selection is
//           written in ascending position order through LDS bitmaps: the
//           output is deterministic and needs no sort.
// Few long rows (decode): collect splits every row over workgroups that
// append to global lists; one workgroup per row then selects.  Many rows
// (prefill): one workgroup per row does collect and select, candidates in LDS.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kNT = 256;
constexpr int kRowNT = 512;
constexpr int kLdsCap = 8192;   // candidates held in LDS by the one-workgroup-per-row path

struct RowWs {
  uint32_t *hist1, *counters, *sel, *cand;
};

__device__ __forceinline__ RowWs row_ws(uint32_t *ws, long long row_words, int r) {
  uint32_t *base = ws + (long long)r * row_words;
  RowWs w;
  w.hist1 = base;
  w.counters = base + kTopkBins;  // [0] selected, [1] candidates
  w.sel = base + kTopkHdrWords;
  w.cand = base + kTopkHdrWords + kTopkMaxK;
  return w;
}

// Exclusive prefix over the threads of a block (NT a multiple of 64); `tmp`
// holds NT/64 + 1 ints of LDS.  Returns the exclusive prefix, sets `total`.
template <int NT>
__device__ int block_exclusive_scan(int v, int *tmp, int &total) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < NT / 64; ++i) {
      const int x = tmp[i];
      tmp[i] = acc;
      acc += x;
    }
    tmp[NT / 64] = acc;
  }
  __syncthreads();
  const int res = tmp[wv] + inc - v;
  total = tmp[NT / 64];
  __syncthreads();
  return res;
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

// Visit row[s], s in [s0, s1) (s0 a multiple of 4), in rounds that every lane
// of the block takes part in: f(s, key, valid).  Each thread loads 16 scores
// (four 16-byte loads when the row is 16-byte aligned) before using any, so a
// round has NT*16 scores in flight.
template <int NT, typename F>
__device__ __forceinline__ void scan_row(const float *row, int s0, int s1, F &&f) {
  const bool vec = ((uintptr_t)(row + s0) & 15) == 0;
  for (int base = s0; base < s1; base += NT * 16) {
    float x[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = base + (i * NT + (int)threadIdx.x) * 4;
      if (vec && e + 3 < s1) {
        const float4 v = *reinterpret_cast<const float4 *>(row + e);
        x[i][0] = v.x; x[i][1] = v.y; x[i][2] = v.z; x[i][3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[i][c] = e + c < s1 ? row[e + c] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int sidx = base + (i * NT + (int)threadIdx.x) * 4 + c;
        f(sidx, score_key(x[i][c]), sidx < s1);
      }
  }
}

__device__ __forceinline__ void slice_range(const TopkArgs &a, int n, int &s0, int &s1) {
  const int per = ((n + a.slices - 1) / a.slices + 63) & ~63;
  s0 = blockIdx.x * per;
  s1 = s0 + per < n ? s0 + per : n;
}

__global__ __launch_bounds__(kNT) void topk_zero_kernel(TopkArgs a) {
  uint32_t *base = a.ws + (long long)blockIdx.x * a.row_words;
  for (int i = threadIdx.x; i < kTopkHdrWords; i += kNT) base[i] = 0u;
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
  slice_range(a, n, s0, s1);
  const float *row = a.scores + (long long)r * a.ld;
  scan_row<kNT>(row, s0, s1, [&](int, uint32_t key, bool valid) {
    if (valid) atomicAdd(&h[key >> 21], 1u);
  });
  __syncthreads();
  RowWs w = row_ws(a.ws, a.row_words, r);
  for (int i = threadIdx.x; i < kTopkBins; i += kNT)
    if (h[i]) atomicAdd(&w.hist1[i], h[i]);
}

// Sliced collect: keys above the top digit go to the row's selected list,
// keys in it to the row's candidate list (count kept past the capacity).  Per
// round of kNT*16 scores the workgroup counts both kinds with wave ballots,
// reserves its space with one atomic per list, then writes.
__global__ __launch_bounds__(kNT) void topk_collect_kernel(TopkArgs a) {
  const int r = blockIdx.y;
  const int n = a.sv.candidates(a.q_begin + r);
  if (n <= a.k) return;
  __shared__ uint32_t h[kTopkBins];
  __shared__ int res[2];
  __shared__ int tmp[kNT / 64 + 1];
  __shared__ uint32_t wcnt[2][kNT / 64];
  __shared__ uint32_t gbase[2];
  RowWs w = row_ws(a.ws, a.row_words, r);
  for (int i = threadIdx.x; i < kTopkBins; i += kNT) h[i] = w.hist1[i];
  __syncthreads();
  find_digit<kNT>(h, kTopkBins, a.k, res, tmp);
  const uint32_t d1 = (uint32_t)res[0];
  int s0, s1;
  slice_range(a, n, s0, s1);
  const float *row = a.scores + (long long)r * a.ld;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool vec = ((uintptr_t)(row + s0) & 15) == 0;
  for (int base = s0; base < s1; base += kNT * 16) {
    uint32_t key[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = base + (i * kNT + (int)threadIdx.x) * 4;
      float x[4];
      if (vec && e + 3 < s1) {
        const float4 v = *reinterpret_cast<const float4 *>(row + e);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = e + c < s1 ? row[e + c] : 0.f;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) key[i][c] = e + c < s1 ? score_key(x[c]) : 0u;   // key 0: never d1 > 0
    }
    // counts of this round, per wave
    uint32_t ns = 0u, nc = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t dig = key[i][c] >> 21;
        ns += (uint32_t)__popcll(__ballot(dig > d1 && key[i][c] != 0u));
        nc += (uint32_t)__popcll(__ballot(dig == d1 && key[i][c] != 0u));
      }
    if (lane == 0) {
      wcnt[0][wv] = ns;
      wcnt[1][wv] = nc;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      uint32_t tot = 0u;
      for (int j = 0; j < kNT / 64; ++j) tot += wcnt[threadIdx.x][j];
      gbase[threadIdx.x] = tot ? atomicAdd(&w.counters[threadIdx.x], tot) : 0u;
    }
    __syncthreads();
    uint32_t os = gbase[0], oc = gbase[1];
    for (int j = 0; j < wv; ++j) {
      os += wcnt[0][j];
      oc += wcnt[1][j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = key[i][c];
        const uint32_t dig = kk >> 21;
        const bool is_sel = dig > d1 && kk != 0u;
        const bool is_cand = dig == d1 && kk != 0u;
        const unsigned long long ms = __ballot(is_sel);
        const unsigned long long mc = __ballot(is_cand);
        const int sidx = base + (i * kNT + (int)threadIdx.x) * 4 + c;
        if (is_sel) {
          const uint32_t pos = os + __popcll(ms & below);
          if (pos < (uint32_t)kTopkMaxK) w.sel[pos] = (uint32_t)sidx;
        }
        if (is_cand) {
          const uint32_t pos = oc + __popcll(mc & below);
          if (pos < (uint32_t)kTopkCap) {
            w.cand[2 * pos] = kk & 0x1fffffu;
            w.cand[2 * pos + 1] = (uint32_t)sidx;
          }
        }
        os += (uint32_t)__popcll(ms);
        oc += (uint32_t)__popcll(mc);
      }
    __syncthreads();
  }
}

// One workgroup per row: exact threshold among the candidates, then the
// ascending bitmap compaction.  GLOBAL_LISTS: the selected and candidate lists
// come from topk_collect_kernel; otherwise this workgroup collects them itself
// (selected keys straight into the bitmap, candidates into LDS).
template <bool GLOBAL_LISTS>
__global__ __launch_bounds__(kRowNT) void topk_select_kernel(TopkArgs a) {
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
  uint32_t *lcand = h + kTopkBins;               // 2 * kLdsCap words: the candidates
  __shared__ int res[6];
  __shared__ int tmp[kRowNT / 64 + 1];
  __shared__ uint32_t lcount;

  RowWs w = row_ws(a.ws, a.row_words, r);
  for (int i = threadIdx.x; i < kTopkBins; i += kRowNT) h[i] = w.hist1[i];
  for (int i = threadIdx.x; i < W; i += kRowNT) {
    selmap[i] = 0u;
    eqmap[i] = 0u;
  }
  if (threadIdx.x == 0) lcount = 0u;
  const float *row = a.scores + (long long)r * a.ld;
  const int lane = lane_id();
  const uint32_t *cand = lcand;
  int ncand = 0;
  if (GLOBAL_LISTS) {
    // the lists do not depend on the digits: fetch them before the digit search
    ncand = (int)w.counters[1];
    if (ncand <= kLdsCap) {                      // stage the list in LDS for the three passes
      const uint4 *src = reinterpret_cast<const uint4 *>(w.cand);
      uint4 *dst = reinterpret_cast<uint4 *>(lcand);
      for (int i = threadIdx.x; i < (ncand + 1) / 2; i += kRowNT) dst[i] = src[i];
    } else {
      cand = w.cand;
      ncand = ncand <= kTopkCap ? ncand : -1;    // -1: list overflowed, rescan the row
    }
  }
  __syncthreads();
  if (GLOBAL_LISTS) {
    const int nsel = (int)min(w.counters[0], (uint32_t)m);
    for (int i = threadIdx.x; i < nsel; i += kRowNT) {
      const uint32_t s = w.sel[i];
      if (s < (uint32_t)n) atomicOr(&selmap[s >> 5], 1u << (s & 31));
    }
  }
  find_digit<kRowNT>(h, kTopkBins, m, res, tmp);
  const uint32_t d1 = (uint32_t)res[0];
  const int need = m - res[1];                   // still to take among the candidates (>= 1)

  // ---- per-row path: selected keys straight into the bitmap, candidates into LDS
  if (!GLOBAL_LISTS) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    scan_row<kRowNT>(row, 0, n, [&](int s, uint32_t key, bool valid) {
      const uint32_t dig = key >> 21;
      if (valid && dig > d1) atomicOr(&selmap[s >> 5], 1u << (s & 31));
      const bool is_cand = valid && dig == d1;
      const unsigned long long mc = __ballot(is_cand);
      if (mc == 0ull) return;
      uint32_t bc = 0u;
      if (lane == 0) bc = atomicAdd(&lcount, (uint32_t)__popcll(mc));
      bc = __shfl(bc, 0, kWave);
      if (is_cand) {
        const uint32_t pos = bc + __popcll(mc & below);
        if (pos < (uint32_t)kLdsCap) {
          lcand[2 * pos] = key & 0x1fffffu;
          lcand[2 * pos + 1] = (uint32_t)s;
        }
      }
    });
    __syncthreads();
    ncand = (int)lcount;
    ncand = ncand <= kLdsCap ? ncand : -1;
  }
  // Visit every candidate (low 21 key bits, position): from the list, or by
  // rescanning the row when the list overflowed.
  auto for_each_cand = [&](auto &&f) {
    if (ncand >= 0) {
      for (int i = threadIdx.x; i < ncand; i += kRowNT) {
        const uint32_t s = cand[2 * i + 1];
        if (s < (uint32_t)n) f(cand[2 * i] & 0x1fffffu, s);
      }
    } else {
      for (int s = threadIdx.x; s < n; s += kRowNT) {
        const uint32_t key = score_key(row[s]);
        if ((key >> 21) == d1) f(key & 0x1fffffu, (uint32_t)s);
      }
    }
  };

  // ---- second digit key[20:10]
  __syncthreads();
  for (int i = threadIdx.x; i < kTopkBins; i += kRowNT) h[i] = 0u;
  __syncthreads();
  for_each_cand([&](uint32_t lo, uint32_t) { atomicAdd(&h[lo >> 10], 1u); });
  __syncthreads();
  find_digit<kRowNT>(h, kTopkBins, need, res + 2, tmp);
  const uint32_t d2 = (uint32_t)res[2];
  const int need3 = need - res[3];
  // ---- third digit key[9:0]
  for (int i = threadIdx.x; i < 1024; i += kRowNT) h[i] = 0u;
  __syncthreads();
  for_each_cand([&](uint32_t lo, uint32_t) {
    if ((lo >> 10) == d2) atomicAdd(&h[lo & 1023u], 1u);
  });
  __syncthreads();
  find_digit<kRowNT>(h, 1024, need3, res + 4, tmp);
  const uint32_t T = (d2 << 10) | (uint32_t)res[4];
  const int quota = need3 - res[5];
  for_each_cand([&](uint32_t lo, uint32_t s) {
    if (lo > T) atomicOr(&selmap[s >> 5], 1u << (s & 31));
    else if (lo == T) atomicOr(&eqmap[s >> 5], 1u << (s & 31));
  });
  __syncthreads();

  // ---- ascending-position compaction: thread i owns words [i*wpt, (i+1)*wpt)
  const int wpt = (W + kRowNT - 1) / kRowNT;
  const int w0 = threadIdx.x * wpt;
  const int w1 = w0 + wpt < W ? w0 + wpt : W;
  int eq_local = 0;
  for (int i = w0; i < w1; ++i) eq_local += __popc(eqmap[i]);
  int tot;
  int eq_before = block_exclusive_scan<kRowNT>(eq_local, tmp, tot);
  int cnt = 0;
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
  int pos = block_exclusive_scan<kRowNT>(cnt, tmp, tot);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = selmap[i];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < m) out[pos] = i * 32 + b;
      ++pos;
    }
  }
  for (int i = m + threadIdx.x; i < a.k; i += kRowNT) out[i] = -1;
}

}  // namespace

int topk_slices(int rows, int max_ctx) {
  int s = (2048 + rows - 1) / rows;
  const int cap = (max_ctx + 4095) / 4096;
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

bool topk_sliced(int rows) { return rows < 256; }

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
    const size_t lds = (size_t)(2 * Wmax + kTopkBins + 2 * kLdsCap) * sizeof(uint32_t);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute((const void *)topk_select_kernel<true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(a.rows), dim3(kRowNT), lds, st, a);
  } else {
    const size_t lds = (size_t)(2 * Wmax + kTopkBins + 2 * kLdsCap) * sizeof(uint32_t);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute((const void *)topk_select_kernel<false>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3(a.rows), dim3(kRowNT), lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3(a.rows), dim3(kNT), 0, st, a);
  hipLaunchKernelGGL(topk_hist1_kernel, dim3(a.slices, a.rows), dim3(kNT), 0, st, a);
  return launch_topk_select(a, st);
}

}  // namespace dsa

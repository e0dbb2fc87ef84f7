// Fine-grained top-k token selection: for every query, the first
// m = min(k, n) candidates in the order (score descending, position
// ascending) ("DeepSeek V3.2: How Far Can Open Models Go If You Actually
// Try?", section 3.1, selection equation; "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", System Modules, top-k operation).
//
// Exact integer radix select on order-preserving 32-bit keys, no float
// arithmetic:
//   hist1   11-bit histogram of key[31:21] over the row            -> digit d1
//   hist2   11-bit histogram of key[20:10] among keys with d1      -> digit d2
//   collect keys with key[31:10] above the 22-bit prefix P = (d1,d2) are
//           selected outright; keys equal to P are kept as candidates
//   final   10-bit histogram of key[9:0] over the candidates        -> exact
//           threshold T; keys equal to T are taken lowest position first;
//           the selection is written in ascending position order through an
//           LDS bitmap (deterministic output, no sort).
// The first three stages split every row over `slices` workgroups (decode has
// few, long rows); the final stage takes one workgroup per row.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kNT = 256;

struct RowWs {
  uint32_t *hist1, *hist2, *counters, *sel, *cand;
};

__device__ __forceinline__ RowWs row_ws(uint32_t *ws, int r) {
  uint32_t *base = ws + (long long)r * kTopkRowWords;
  RowWs w;
  w.hist1 = base;
  w.hist2 = base + kTopkBins;
  w.counters = base + 2 * kTopkBins;  // [0] selected, [1] candidates
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

// Given a histogram (nbins, in LDS) and need >= 1 <= total, find the digit d
// with count(bins > d) < need <= count(bins >= d).  Writes d and count(bins > d)
// to out[0..1] (LDS) and returns after a barrier.
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

__device__ __forceinline__ void slice_range(const TopkArgs &a, int n, int &s0, int &s1) {
  const int per = (n + a.slices - 1) / a.slices;
  s0 = blockIdx.x * per;
  s1 = s0 + per < n ? s0 + per : n;
}

__global__ __launch_bounds__(kNT) void topk_zero_kernel(TopkArgs a) {
  uint32_t *base = a.ws + (long long)blockIdx.x * kTopkRowWords;
  for (int i = threadIdx.x; i < kTopkHdrWords; i += kNT) base[i] = 0u;
}

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
  for (int s = s0 + threadIdx.x; s < s1; s += kNT) atomicAdd(&h[score_key(row[s]) >> 21], 1u);
  __syncthreads();
  RowWs w = row_ws(a.ws, r);
  for (int i = threadIdx.x; i < kTopkBins; i += kNT)
    if (h[i]) atomicAdd(&w.hist1[i], h[i]);
}

// Digits of the first two passes, recomputed from the global histograms.
__device__ void load_digits(const RowWs &w, int m, bool second, uint32_t *h, int *res, int *tmp) {
  for (int i = threadIdx.x; i < kTopkBins; i += kNT) h[i] = w.hist1[i];
  __syncthreads();
  find_digit<kNT>(h, kTopkBins, m, res, tmp);
  if (!second) return;
  const int need2 = m - res[1];
  for (int i = threadIdx.x; i < kTopkBins; i += kNT) h[i] = w.hist2[i];
  __syncthreads();
  find_digit<kNT>(h, kTopkBins, need2, res + 2, tmp);
}

__global__ __launch_bounds__(kNT) void topk_hist2_kernel(TopkArgs a) {
  const int r = blockIdx.y;
  const int n = a.sv.candidates(a.q_begin + r);
  if (n <= a.k) return;
  __shared__ uint32_t h[kTopkBins];
  __shared__ int res[4];
  __shared__ int tmp[kNT / 64 + 1];
  RowWs w = row_ws(a.ws, r);
  load_digits(w, a.k, false, h, res, tmp);
  const uint32_t d1 = (uint32_t)res[0];
  for (int i = threadIdx.x; i < kTopkBins; i += kNT) h[i] = 0u;
  __syncthreads();
  int s0, s1;
  slice_range(a, n, s0, s1);
  const float *row = a.scores + (long long)r * a.ld;
  for (int s = s0 + threadIdx.x; s < s1; s += kNT) {
    const uint32_t key = score_key(row[s]);
    if ((key >> 21) == d1) atomicAdd(&h[(key >> 10) & 2047u], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kTopkBins; i += kNT)
    if (h[i]) atomicAdd(&w.hist2[i], h[i]);
}

__global__ __launch_bounds__(kNT) void topk_collect_kernel(TopkArgs a) {
  const int r = blockIdx.y;
  const int n = a.sv.candidates(a.q_begin + r);
  if (n <= a.k) return;
  __shared__ uint32_t h[kTopkBins];
  __shared__ int res[4];
  __shared__ int tmp[kNT / 64 + 1];
  RowWs w = row_ws(a.ws, r);
  load_digits(w, a.k, true, h, res, tmp);
  const uint32_t P = ((uint32_t)res[0] << 11) | (uint32_t)res[2];
  int s0, s1;
  slice_range(a, n, s0, s1);
  const float *row = a.scores + (long long)r * a.ld;
  const int lane = lane_id();
  for (int base = s0 + (threadIdx.x & ~63); base < s1; base += kNT) {
    const int s = base + lane;
    uint32_t key = 0u;
    if (s < s1) key = score_key(row[s]);
    const uint32_t pre = key >> 10;
    const bool is_sel = s < s1 && pre > P;
    const bool is_cand = s < s1 && pre == P;
    const unsigned long long ms = __ballot(is_sel);
    const unsigned long long mc = __ballot(is_cand);
    uint32_t bs = 0u, bc = 0u;
    if (lane == 0) {
      if (ms) bs = atomicAdd(&w.counters[0], (uint32_t)__popcll(ms));
      if (mc) bc = atomicAdd(&w.counters[1], (uint32_t)__popcll(mc));
    }
    bs = __shfl(bs, 0, kWave);
    bc = __shfl(bc, 0, kWave);
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (is_sel) {
      const uint32_t pos = bs + __popcll(ms & below);
      if (pos < (uint32_t)kTopkMaxK) w.sel[pos] = (uint32_t)s;
    }
    if (is_cand) {
      const uint32_t pos = bc + __popcll(mc & below);
      if (pos < (uint32_t)kTopkCap) {
        w.cand[2 * pos] = key & 1023u;
        w.cand[2 * pos + 1] = (uint32_t)s;
      }
    }
  }
}

constexpr int kFinNT = 1024;

__global__ __launch_bounds__(kFinNT) void topk_final_kernel(TopkArgs a) {
  extern __shared__ uint32_t smem[];
  const int r = blockIdx.x;
  const int n = a.sv.candidates(a.q_begin + r);
  int32_t *out = a.idx + (long long)r * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kFinNT) out[i] = i < n ? i : -1;
    return;
  }
  const int m = a.k;
  const int W = (n + 31) >> 5;
  uint32_t *selmap = smem;
  uint32_t *eqmap = smem + W;
  uint32_t *h = smem + 2 * W;        // 2048 words (hist1/hist2 copies, then hist3)
  __shared__ int res[8];
  __shared__ int tmp[kFinNT / 64 + 1];

  RowWs w = row_ws(a.ws, r);
  // digits d1, d2 (block of 1024 threads: 2 bins each)
  for (int i = threadIdx.x; i < kTopkBins; i += kFinNT) h[i] = w.hist1[i];
  __syncthreads();
  find_digit<kFinNT>(h, kTopkBins, m, res, tmp);
  const int above1 = res[1];
  for (int i = threadIdx.x; i < kTopkBins; i += kFinNT) h[i] = w.hist2[i];
  __syncthreads();
  find_digit<kFinNT>(h, kTopkBins, m - above1, res + 2, tmp);
  const uint32_t P = ((uint32_t)res[0] << 11) | (uint32_t)res[2];
  const int need3 = m - above1 - res[3];

  for (int i = threadIdx.x; i < 2 * W; i += kFinNT) smem[i] = 0u;
  for (int i = threadIdx.x; i < 1024; i += kFinNT) h[i] = 0u;
  __syncthreads();
  const int nsel = (int)min(w.counters[0], (uint32_t)m);
  for (int i = threadIdx.x; i < nsel; i += kFinNT) {
    const uint32_t s = w.sel[i];
    if (s < (uint32_t)n) atomicOr(&selmap[s >> 5], 1u << (s & 31));
  }
  const int ncand = (int)w.counters[1];
  const float *row = a.scores + (long long)r * a.ld;
  const bool listed = ncand <= kTopkCap;
  // hist3 over the low 10 bits of the candidates
  if (listed) {
    for (int i = threadIdx.x; i < ncand; i += kFinNT) atomicAdd(&h[w.cand[2 * i] & 1023u], 1u);
  } else {
    for (int s = threadIdx.x; s < n; s += kFinNT) {
      const uint32_t key = score_key(row[s]);
      if ((key >> 10) == P) atomicAdd(&h[key & 1023u], 1u);
    }
  }
  __syncthreads();
  find_digit<kFinNT>(h, 1024, need3, res + 4, tmp);
  const uint32_t d3 = (uint32_t)res[4];
  const int quota = need3 - res[5];
  if (listed) {
    for (int i = threadIdx.x; i < ncand; i += kFinNT) {
      const uint32_t lo = w.cand[2 * i], s = w.cand[2 * i + 1];
      if (s >= (uint32_t)n) continue;
      if (lo > d3) atomicOr(&selmap[s >> 5], 1u << (s & 31));
      else if (lo == d3) atomicOr(&eqmap[s >> 5], 1u << (s & 31));
    }
  } else {
    for (int s = threadIdx.x; s < n; s += kFinNT) {
      const uint32_t key = score_key(row[s]);
      if ((key >> 10) == P) {
        const uint32_t lo = key & 1023u;
        if (lo > d3) atomicOr(&selmap[s >> 5], 1u << (s & 31));
        else if (lo == d3) atomicOr(&eqmap[s >> 5], 1u << (s & 31));
      }
    }
  }
  __syncthreads();
  // Ascending-position compaction: thread i owns words [i*wpt, (i+1)*wpt).
  const int wpt = (W + kFinNT - 1) / kFinNT;
  const int w0 = threadIdx.x * wpt;
  const int w1 = w0 + wpt < W ? w0 + wpt : W;
  int eq_local = 0;
  for (int i = w0; i < w1; ++i) eq_local += __popc(eqmap[i]);
  int tot;
  int eq_before = block_exclusive_scan<kFinNT>(eq_local, tmp, tot);
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
  int pos = block_exclusive_scan<kFinNT>(cnt, tmp, tot);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = selmap[i];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < m) out[pos] = i * 32 + b;
      ++pos;
    }
  }
  for (int i = m + threadIdx.x; i < a.k; i += kFinNT) out[i] = -1;
}

}  // namespace

int topk_slices(int rows, int max_ctx) {
  int s = (2048 + rows - 1) / rows;
  const int cap = (max_ctx + 2047) / 2048;
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_zero_kernel, dim3(a.rows), dim3(kNT), 0, st, a);
  dim3 grid(a.slices, a.rows);
  hipLaunchKernelGGL(topk_hist1_kernel, grid, dim3(kNT), 0, st, a);
  hipLaunchKernelGGL(topk_hist2_kernel, grid, dim3(kNT), 0, st, a);
  hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kNT), 0, st, a);
  const int W = (a.sv.max_ctx + 31) / 32;
  const size_t lds = (size_t)(2 * W + kTopkBins) * sizeof(uint32_t);
  if (lds > 65536)
    hipFuncSetAttribute((const void *)topk_final_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(topk_final_kernel, dim3(a.rows), dim3(kFinNT), lds, st, a);
  return hipGetLastError();
}

}  // namespace dsa

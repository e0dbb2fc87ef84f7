// Internal launch interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

// Rows [q_begin, q_begin + rows) of the query set are processed by one launch;
// row r of every row-indexed output buffer belongs to query q_begin + r.

struct IndexerArgs {
  SeqView sv;
  int H_I, d_I, dtype;
  const void *q_idx;
  const float *q_scale;
  const float *w;
  const void *k_cache;
  const float *k_scale;
  float *scores;
  long long ld;
  int q_begin, rows;
  int fill_masked;  // write -inf to scores[r, s] for n_t <= s < ld
  // Optional 2048-bin histogram of score_key >> 21 per row (the top-k's first
  // radix digit): hist_mode 1 adds into zeroed rows with atomics (decode:
  // rows split over workgroups), 2 stores each row whole (prefill: one wave
  // per row).  Row r's bins start at hist + r * hist_stride.
  uint32_t *hist;
  long long hist_stride;
  int hist_mode;
};

struct TopkArgs {
  SeqView sv;
  int k;
  const float *scores;
  long long ld;
  int q_begin, rows;
  int32_t *idx;  // [rows, k]
  uint32_t *ws;  // [rows, row_words]
  long long row_words;
  int slices;
};

struct MlaArgs {
  SeqView sv;
  int H, D, Dv, k, dtype;
  float sm_scale;
  const void *q;
  const void *kv;
  const int32_t *idx;  // [rows, k]
  void *out;
  float *lse;
  int q_begin, rows;
  int n_split;
  float *part;  // [rows, n_split, H, Dv + 4] when n_split > 1 (acc[Dv], max, sum, pad)
};

// top-k workspace, per row, in 32-bit words: the first-digit histogram and two
// counters (zeroed per call), then -- for the sliced path only -- the list of
// selected positions and the candidate list (low 21 key bits, position).
constexpr int kTopkBins = 2048;        // 11-bit radix digits
constexpr int kTopkCap = 16384;        // candidates listed per row by the sliced path
constexpr int kTopkHdrWords = kTopkBins + 64;
constexpr int kTopkMaxK = 2048;
constexpr long long kTopkSlicedRowWords = kTopkHdrWords + kTopkMaxK + 2 * kTopkCap;

int topk_slices(int rows, int max_ctx);
bool topk_sliced(int rows);
inline long long topk_row_words(int rows) { return topk_sliced(rows) ? kTopkSlicedRowWords : kTopkHdrWords; }
int mla_splits(int rows, int k);
size_t mla_f32_lds(int H, int D, int k);

hipError_t launch_index_scores(const IndexerArgs &a, hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);         // zero + hist1 + select
hipError_t launch_topk_zero(const TopkArgs &a, hipStream_t s);    // zero the per-row headers
hipError_t launch_topk_select(const TopkArgs &a, hipStream_t s);  // collect + select (hist1 ready)
hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t s);

}  // namespace dsa

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
};

struct TopkArgs {
  SeqView sv;
  int k;
  const float *scores;
  long long ld;
  int q_begin, rows;
  int32_t *idx;  // [rows, k]
  uint32_t *ws;  // [rows, kTopkRowWords]
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

// top-k workspace, per row, in 32-bit words
constexpr int kTopkBins = 2048;        // 11-bit radix digits
constexpr int kTopkCap = 4096;         // candidates kept after the 22-bit prefix
constexpr int kTopkHdrWords = 2 * kTopkBins + 64;  // two histograms + counters (zeroed per call)
constexpr int kTopkMaxK = 2048;
constexpr long long kTopkRowWords = kTopkHdrWords + kTopkMaxK + 2 * kTopkCap;

int topk_slices(int rows, int max_ctx);
int mla_splits(int rows, int k);
size_t mla_f32_lds(int H, int D, int k);

hipError_t launch_index_scores(const IndexerArgs &a, hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t s);

}  // namespace dsa

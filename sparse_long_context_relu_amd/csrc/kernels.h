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
  int chunk;        // decode tiling: candidate keys per workgroup (set by its launcher)
  // decode tiling, set by its launcher: 1 when each workgroup derives its row
  // and key range from the candidate counts of all rows (a grid of G_max
  // workgroups, `slots` of which run at once); 0 for the fixed row x chunk grid
  int balanced;
  int slots;
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
  int slices;     // workgroups per row in the sliced path
  int slice_len;  // the longest slice (a multiple of 64): size of a slice's candidate region
  int sel_seg;    // size of a slice's selected-position region
};

struct MlaArgs {
  SeqView sv;
  int H, D, Dv, k, dtype;
  float sm_scale;
  const void *q;
  const void *kv;
  const int32_t *idx;  // [rows, k]; unused when dense
  // dense: entry j of query t's list is position j itself (present while
  // j < n_t), for j < k; idx is not read.  k then only sets how the lists are
  // split.  A split with no position writes no partial.
  int dense;
  // 0: attention (out, lse); 1: lse only (bf16, dense lists; split partials are
  // fp32 (max, sum) pairs [rows, n_split, H, 2] in part); 2: the softmax
  // weights given lse (input), summed over heads and divided by H, written to
  // probs[r * ld + position] (bf16, dense lists; 0 past the last candidate)
  int mode;
  float *probs;
  long long ld;
  void *out;
  float *lse;
  int q_begin, rows;
  int n_split;
  // when n_split > 1: the normalised split outputs, bf16 [rows, n_split, H, Dv],
  // followed by their (running max in log2 units, sum) pairs, fp32 [rows, n_split, H, 2]
  void *part;
};

// top-k workspace, per row, in 32-bit words.  Header (zeroed before every
// call): the histogram of the first radix digit (key[31:21]), the histogram of
// the second digit (key[20:10]) of the candidates, and a few words of row
// results.  The sliced path (few long rows) adds the per-slice counts of
// selected positions and candidates, then per slice a region of selected
// positions and a region of candidates (low 21 key bits, position).
constexpr int kTopkBins = 2048;        // 11-bit radix digits
constexpr int kTopkMaxK = 2048;
constexpr int kTopkMaxSlices = 64;
constexpr int kTopkHist2 = kTopkBins;                 // word offset of the second histogram
constexpr int kTopkInfo = 2 * kTopkBins;              // d1, count above d1
constexpr int kTopkHdrWords = 2 * kTopkBins + 64;
constexpr int kTopkCounts = kTopkHdrWords;            // [2][kTopkMaxSlices]: selected, candidates
constexpr int kTopkRegions = kTopkCounts + 2 * kTopkMaxSlices;

// Per-row e4m3fn quantisation: src [rows, len] (bf16 / fp32) -> dst [rows, len]
// codes and scale[rows * scale_repeat] (each row's scale repeated).
struct QuantArgs {
  long long rows;
  int len, src_dtype, scale_repeat;
  const void *src;
  uint8_t *dst;
  float *scale;
};

// Append of one new index key per query token into the e4m3fn key cache.
struct AppendArgs {
  SeqView sv;
  int len, src_dtype;
  const void *src;   // [T, len]
  uint8_t *cache;    // key cache rows of len codes
  float *scale;      // key scales, one per cache row
};

// Per-query KL rows of the indexer's warm-up objective.
struct KlArgs {
  SeqView sv;
  int q_begin, rows;
  float *scores;        // [rows, ld]: I in, dL/dI out (0 past the last candidate)
  const float *probs;   // [rows, ld]: the target distribution
  long long ld;
  float *loss;          // [T]: indexed by query
};

// Gradient of the indexer scores into q_I, w and k_I (bf16 indexer operands).
struct BwdArgs {
  SeqView sv;
  int q_begin, rows;        // query rows of this launch (grad row r = query q_begin + r)
  const void *q_idx;        // [T, 64, 128] bf16
  const float *w;           // [T, 64]
  const void *k_cache;      // key cache, bf16 rows of 128
  const float *grad;        // [rows, ld]: dL/dI
  long long ld;
  float *dq;                // [T, 64, 128]
  float *dw;                // [T, 64]
  float *dk;                // key cache layout, fp32 rows of 128
  int span;                 // dq: list length the splits cut (max_ctx)
  int n_split;              // dq: key splits per query; dk: query splits
  int q_per_split;          // dk: queries per split (prefill)
  float *part;              // split partials
  const int32_t *sel;       // dq over a selection: [rows, sel_k] positions (ascending; -1 or out of range: none)
  int sel_k;
};

// Stage-2 gradient of the sparse attention (bf16, H = 128, D = 576, Dv = 512),
// one chunk of query rows [q_begin, q_begin + rows) of a prefill per call of
// the launcher.  Buffers marked ws are the caller's workspace.
struct MlaBwdArgs {
  SeqView sv;
  int k;                    // selection length (a multiple of 16)
  float sm_scale;
  const void *q;            // [T, H, D]
  const void *kv;           // latent cache
  const int32_t *idx;       // [T, k] selected positions (entries < 0 or > q_pos: absent)
  const void *out;          // [T, H, Dv] forward output
  const float *lse;         // [T, H] forward log-sum-exp (natural log)
  const void *dout;         // [T, H, Dv] dL/dout
  float *dq;                // [T, H, D]
  float *dkv;               // latent cache layout, fp32 rows of D
  float *probs;             // [T, k] head-mean weights over the selection, or null
  int q_begin, rows;
  float *delta;             // ws [rows, H]: sum_d dout * out
  uint16_t *ds_t;           // ws [rows, k / 32, H, 32] bf16: sm_scale dS per tile, rows in k-slot order
  uint16_t *pd;             // ws [rows, k, 2, H] bf16: P and sm_scale dS per row, heads in k-slot order
  uint16_t *contrib;        // ws [rows, k, D] bf16: each selected row's gradient from its query
  uint16_t *jpos;           // ws [nkeys, jstride]: slot j of query row r that selected key s, or 0xFFFF
  int jstride;              // rows rounded up to 8
  int nkeys;                // keys reduced (positions 0..nkeys-1 of sequence 0)
  int first;                // 1: dkv rows are written; 0: added to
};

// Stage-2 indexer KL over each query's selection.
struct SparseKlArgs {
  SeqView sv;
  int rows, k;
  float *scores;            // [rows, ld]: I in, dL/dI out (0 outside the selection)
  long long ld;
  const int32_t *idx;       // [rows, k]
  const float *probs;       // [rows, k] target over the selection
  float *loss;              // [rows]
};

struct TopkLayout {
  int slices, slice_len, sel_seg;
  long long row_words;
};
TopkLayout topk_layout(int rows, int max_ctx);
bool topk_sliced(int rows);
int mla_splits(int rows, int k);
int mla_dense_splits(int rows, int span);   // splits of a dense list of `span` entries
constexpr int kMlaMaxSplits = 128;
size_t mla_f32_lds(int H, int D, int k);

hipError_t launch_index_scores(const IndexerArgs &a, hipStream_t s);
hipError_t launch_index_decode(const IndexerArgs &a, hipStream_t s);   // decode tiling of the above
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);         // zero + hist1 + select
hipError_t launch_topk_zero(const TopkArgs &a, hipStream_t s);    // zero the per-row headers
hipError_t launch_topk_select(const TopkArgs &a, hipStream_t s);  // collect + select (hist1 ready)
hipError_t launch_topk_all(const TopkArgs &a, hipStream_t s);     // every candidate (all n_t <= k)
hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t s);     // also the dense lists
hipError_t launch_indexer_kl(const KlArgs &a, hipStream_t s);
hipError_t launch_indexer_bwd_q(const BwdArgs &a, hipStream_t s);   // dq, dw (+ split merge)
hipError_t launch_indexer_bwd_k(const BwdArgs &a, hipStream_t s);   // dk (+ split merge)
hipError_t launch_indexer_bwd_q_sel(const BwdArgs &a, hipStream_t s);   // dq, dw over the selected keys only
constexpr int kBwdKeysPerBlock = 128;                                // keys per dk workgroup
int bwd_q_splits(int rows, int span);                                // dq key splits per query
hipError_t launch_sparse_mla_bwd(const MlaBwdArgs &a, hipStream_t s);   // one query chunk
hipError_t launch_sparse_kl(const SparseKlArgs &a, hipStream_t s);
hipError_t launch_fp8_quantize(const QuantArgs &a, hipStream_t s);
hipError_t launch_fp8_append(const AppendArgs &a, hipStream_t s);

// Read-rate measurement with the decode indexer's access shape (ceiling.hip):
// one workgroup per kReadCeilingChunk bytes, one XOR word per wave into sink.
constexpr long long kReadCeilingChunk = 512 * 1024;
hipError_t launch_read_ceiling(const void *src, long long bytes, bool paged, bool cached, uint32_t *sink,
                               hipStream_t s);

}  // namespace dsa

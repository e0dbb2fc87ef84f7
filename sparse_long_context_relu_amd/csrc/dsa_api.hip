// C ABI of the DSA forward path: host-side argument checks, workspace carving
// and kernel orchestration on the caller's stream.  See include/dsa.h for the
// contract of every entry point.
#include <mutex>
#include <stdint.h>

#include "kernels.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

using namespace dsa;

// Scratch memory of dsa_forward_noalloc: one array per GPU, held from the
// library's load until the process ends.  In host code `scratch` names a host
// stand-in, not device memory; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t kNoallocScratchBytes = 128ull << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxCtx = 262144;
constexpr long long kScoreBudget = 256ll << 20;  // bytes of score rows per prefill chunk
constexpr long long kMinChunkRows = 8192;        // query rows per prefill chunk, at least
constexpr int kQuantMaxLen = 65536;              // values per quantised row
constexpr int kQuantMaxRepeat = 1024;            // copies of each row's scale
constexpr long long kQuantMaxRows = 2147483647;  // one workgroup (or a quarter) per row
constexpr int kAppendMaxDim = 2048;              // index key width for the append
constexpr long long kDenseWsBudget = 1ll << 30;  // bytes of split partials per dense query chunk
constexpr int kDenseF32MaxCtx = 1024;            // fp32 dense lists live in one workgroup's LDS

long long align256(long long x) { return (x + 255) & ~255ll; }

int check_seqs(const dsa_seqs *s) {
  if (s == nullptr) return DSA_ERR_INVALID_ARG;
  if (s->mode != DSA_PREFILL && s->mode != DSA_DECODE) return DSA_ERR_INVALID_ARG;
  if (s->num_seqs < 1 || s->num_q < 0 || s->reserved != 0) return DSA_ERR_INVALID_ARG;
  if (s->max_ctx < 1) return DSA_ERR_INVALID_ARG;
  if (s->max_ctx > kMaxCtx) return DSA_ERR_UNSUPPORTED;
  if (s->num_q > 0 && s->q_pos == nullptr) return DSA_ERR_INVALID_ARG;
  if (s->mode == DSA_DECODE && s->num_q > s->num_seqs) return DSA_ERR_INVALID_ARG;
  if (s->block_table != nullptr) {
    if (s->block_size != 64) return DSA_ERR_UNSUPPORTED;
    if (s->num_blocks < 1 || s->max_blocks < (s->max_ctx + 63) / 64) return DSA_ERR_INVALID_ARG;
  } else {
    if (s->max_seq_len < s->max_ctx) return DSA_ERR_INVALID_ARG;
  }
  return DSA_OK;
}

int check_index_dims(const dsa_dims *d) {
  if (d == nullptr || d->index_heads < 1 || d->index_dim < 1) return DSA_ERR_INVALID_ARG;
  switch (d->index_dtype) {
    case DSA_F32:
      if (d->index_heads > 64 || d->index_dim > 128 || d->index_heads * d->index_dim > 4096)
        return DSA_ERR_UNSUPPORTED;
      return DSA_OK;
    case DSA_BF16:
    case DSA_FP8_E4M3FN:
      return (d->index_heads == 64 && d->index_dim == 128) ? DSA_OK : DSA_ERR_UNSUPPORTED;
    default:
      return DSA_ERR_INVALID_ARG;
  }
}

int check_k(int k) {
  if (k < 1) return DSA_ERR_INVALID_ARG;
  return k <= kTopkMaxK ? DSA_OK : DSA_ERR_UNSUPPORTED;
}

int check_mla_dims(const dsa_dims *d) {
  if (d == nullptr || d->heads < 1 || d->qk_dim < 1 || d->v_dim < 1 || d->v_dim > d->qk_dim)
    return DSA_ERR_INVALID_ARG;
  if (int e = check_k(d->topk)) return e;
  switch (d->mla_dtype) {
    case DSA_BF16:
      return (d->heads == 128 && d->qk_dim == 576 && d->v_dim == 512) ? DSA_OK : DSA_ERR_UNSUPPORTED;
    case DSA_F32:
      if (d->heads > 16 || d->qk_dim > 128 || d->topk > 1024)
        return DSA_ERR_UNSUPPORTED;
      return DSA_OK;
    case DSA_FP8_E4M3FN:
      return DSA_ERR_UNSUPPORTED;
    default:
      return DSA_ERR_INVALID_ARG;
  }
}

int check_dense_dims(const dsa_seqs *s, const dsa_dims *d) {
  if (d == nullptr || d->heads < 1 || d->qk_dim < 1 || d->v_dim < 1 || d->v_dim > d->qk_dim)
    return DSA_ERR_INVALID_ARG;
  switch (d->mla_dtype) {
    case DSA_BF16:
      return (d->heads == 128 && d->qk_dim == 576 && d->v_dim == 512) ? DSA_OK : DSA_ERR_UNSUPPORTED;
    case DSA_F32:
      if (d->heads > 16 || d->qk_dim > 128 || s->max_ctx > kDenseF32MaxCtx) return DSA_ERR_UNSUPPORTED;
      return DSA_OK;
    case DSA_FP8_E4M3FN:
      return DSA_ERR_UNSUPPORTED;
    default:
      return DSA_ERR_INVALID_ARG;
  }
}

SeqView view(const dsa_seqs *s) {
  SeqView v;
  v.mode = s->mode;
  v.num_seqs = s->num_seqs;
  v.num_q = s->num_q;
  v.max_ctx = s->max_ctx;
  v.q_pos = s->q_pos;
  v.block_table = s->block_table;
  v.max_blocks = s->max_blocks;
  v.num_blocks = s->num_blocks;
  v.block_size = s->block_size;
  v.max_seq_len = s->max_seq_len;
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

long long score_ld(const dsa_seqs *s) { return ((long long)s->max_ctx + 63) & ~63ll; }

int mla_split_count(const dsa_dims *d, int rows) {
  return d->mla_dtype == DSA_BF16 ? mla_splits(rows, d->topk) : 1;
}

long long mla_ws_bytes(const dsa_dims *d, int rows) {
  const int ns = mla_split_count(d, rows);
  if (ns <= 1) return 0;
  return (long long)rows * ns * d->heads * ((long long)d->v_dim * 2 + 2 * (long long)sizeof(float));
}

long long topk_ws_bytes(int rows, int max_ctx) {
  return (long long)rows * topk_layout(rows, max_ctx).row_words * (long long)sizeof(uint32_t);
}

// Query rows per prefill chunk: as many as kScoreBudget bytes of score rows
// hold, but never fewer than kMinChunkRows (the prefill indexer runs 8 rows per
// workgroup; each chunk's launches end in a ragged tail, so chunks span the 256
// CUs several times over; at long contexts that takes more score memory than
// the budget: 2 GiB of rows at 64K).
int forward_chunk_rows(const dsa_seqs *s) {
  if (s->mode == DSA_DECODE || s->num_q == 0) return s->num_q;
  long long rows = kScoreBudget / (score_ld(s) * 4);
  rows = rows / 8 * 8;
  if (rows < kMinChunkRows) rows = kMinChunkRows;
  return rows < s->num_q ? (int)rows : s->num_q;
}

struct ForwardLayout {
  int chunk;
  long long ld, off_scores, off_idx, off_topk, off_mla, total;
};

// Every chunk of a call starts its regions at the same offsets, and a region's
// size depends on the chunk's row count: a short last chunk takes the sliced
// top-k layout (longer rows) and splits its attention rows (partials that a
// full chunk does not have).  Each region is therefore sized for the larger of
// the full chunk and the tail chunk.
ForwardLayout forward_layout(const dsa_seqs *s, const dsa_dims *d) {
  ForwardLayout L;
  L.chunk = forward_chunk_rows(s);
  L.ld = score_ld(s);
  const int tail = L.chunk > 0 ? s->num_q % L.chunk : 0;
  long long topk_b = topk_ws_bytes(L.chunk, s->max_ctx);
  long long mla_b = mla_ws_bytes(d, L.chunk);
  if (tail > 0) {
    const long long tt = topk_ws_bytes(tail, s->max_ctx), tm = mla_ws_bytes(d, tail);
    topk_b = tt > topk_b ? tt : topk_b;
    mla_b = tm > mla_b ? tm : mla_b;
  }
  L.off_scores = 0;
  L.off_idx = align256(L.ld * L.chunk * 4);
  L.off_topk = L.off_idx + align256((long long)L.chunk * d->topk * 4);
  L.off_mla = L.off_topk + align256(topk_b);
  L.total = L.off_mla + align256(mla_b);
  return L;
}

// Dense MLA: every query's list is its max_ctx candidate positions, cut into
// n_split pieces of at most 2048; queries run in chunks whose split partials
// fit kDenseWsBudget (one chunk when they all fit, and always for decode
// batches of up to 64 queries at 128K).
struct DenseLayout {
  int chunk, n_split;
  long long total;
};

DenseLayout dense_layout(const dsa_seqs *s, const dsa_dims *d) {
  DenseLayout L;
  const int T = s->num_q;
  L.chunk = T;
  L.n_split = d->mla_dtype == DSA_BF16 ? mla_dense_splits(T, s->max_ctx) : 1;
  L.total = 0;
  if (L.n_split > 1) {
    const long long per_row = (long long)L.n_split * d->heads * ((long long)d->v_dim * 2 + 8);
    if ((long long)T * per_row > kDenseWsBudget) {
      const long long c = kDenseWsBudget / per_row;
      L.chunk = c < 1 ? 1 : (int)c;
    }
    L.total = (long long)L.chunk * per_row;
  }
  return L;
}

// Warm-up target: per-head log-sum-exp of every query (kept in the workspace
// unless the caller asks for it), then the head-aggregated weights.  The lse
// pass's split partials are fp32 (max, sum) pairs; queries run in chunks
// whose partials fit kDenseWsBudget.
struct ProbsLayout {
  int chunk, n_split;
  long long off_part, total;
};

ProbsLayout probs_layout(const dsa_seqs *s, const dsa_dims *d) {
  ProbsLayout L;
  const int T = s->num_q;
  L.n_split = mla_dense_splits(T, s->max_ctx);
  const long long per_row = L.n_split > 1 ? (long long)L.n_split * d->heads * 8 : 0;
  L.chunk = T;
  if (per_row > 0 && (long long)T * per_row > kDenseWsBudget) {
    const long long c = kDenseWsBudget / per_row;
    L.chunk = c < 1 ? 1 : (int)c;
  }
  L.off_part = align256((long long)T * d->heads * 4);
  L.total = L.off_part + align256((long long)L.chunk * per_row);
  return L;
}

int check_probs_dims(const dsa_seqs *s, const dsa_dims *d) {
  if (int e = check_dense_dims(s, d)) return e;
  return d->mla_dtype == DSA_BF16 ? DSA_OK : DSA_ERR_UNSUPPORTED;
}

// Indexer backward: dq key-split partials (few queries only) and dk query-split
// partials (prefill), the latter bounded by kDenseWsBudget.
struct BwdLayout {
  int q_splits, k_qsplits, q_per_split;
  long long off_k, total;
};

constexpr long long kBwdQPartBytes = (64ll * 128 + 64) * 4;

BwdLayout bwd_layout(const dsa_seqs *s) {
  BwdLayout L;
  const int T = s->num_q;
  L.q_splits = bwd_q_splits(T, s->max_ctx);
  const long long qpart = L.q_splits > 1 ? (long long)T * L.q_splits * kBwdQPartBytes : 0;
  L.off_k = align256(qpart);
  L.k_qsplits = 1;
  L.q_per_split = T;
  long long kpart = 0;
  if (s->mode == DSA_PREFILL) {
    const long long nkb = (s->max_ctx + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock;
    const long long per_split = nkb * kBwdKeysPerBlock * 128 * 4;
    long long want = (T + 511) / 512;                     // 512 queries per split
    long long cap = kDenseWsBudget / per_split;
    if (cap < 1) cap = 1;
    L.k_qsplits = (int)(want < cap ? want : cap);
    L.q_per_split = (T + L.k_qsplits - 1) / L.k_qsplits;
    kpart = (long long)L.k_qsplits * per_split;
  }
  L.total = L.off_k + align256(kpart);
  return L;
}

int check_bwd_dims(const dsa_dims *d) {
  if (d == nullptr) return DSA_ERR_INVALID_ARG;
  if (d->index_dtype != DSA_BF16 || d->index_heads != 64 || d->index_dim != 128) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

struct KlLossLayout {
  long long ld, off_probs, off_ws, total;
};

KlLossLayout kl_loss_layout(const dsa_seqs *s, const dsa_dims *d) {
  KlLossLayout L;
  L.ld = score_ld(s);
  const long long rowbytes = align256((long long)s->num_q * L.ld * 4);
  L.off_probs = rowbytes;
  L.off_ws = 2 * rowbytes;
  const long long a = probs_layout(s, d).total, b = bwd_layout(s).total;
  L.total = L.off_ws + (a > b ? a : b);
  return L;
}

// Device address of `scratch` on the current device, looked up on the first
// call per device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

// Stage-2 attention backward: per chunk of up to kSBwdChunk query rows, the
// bf16 weights and score gradients, the bf16 row gradients and the key map.
constexpr int kSBwdChunk = 256;

struct SBwdLayout {
  int chunk, jstride;
  long long off_dst, off_pd, off_contrib, off_jpos, total;
};

SBwdLayout sbwd_layout(const dsa_seqs *s, const dsa_dims *d) {
  SBwdLayout L;
  const int T = s->num_q;
  L.chunk = T < kSBwdChunk ? T : kSBwdChunk;
  L.jstride = (L.chunk + 7) / 8 * 8;
  const long long c = L.chunk, k = d->topk, ntk = (k + 31) / 32;
  L.off_dst = align256(c * d->heads * 4);
  L.off_pd = L.off_dst + align256(c * ntk * d->heads * 32 * 2);
  L.off_contrib = L.off_pd + align256(c * k * 2 * d->heads * 2);
  L.off_jpos = L.off_contrib + align256(c * k * d->qk_dim * 2);
  L.total = L.off_jpos + align256((long long)s->max_ctx * L.jstride * 2);
  return L;
}

int check_sbwd(const dsa_seqs *s, const dsa_dims *d) {
  if (int e = check_mla_dims(d)) return e;
  if (d->mla_dtype != DSA_BF16 || s->mode != DSA_PREFILL || d->topk % 16 != 0) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

int check_ws(size_t need, const void *ws, size_t ws_bytes) {
  if (need == 0) return DSA_OK;
  // the kernels address workspace regions with 16-byte accesses; every region
  // offset is a multiple of 256 bytes, so the base must be too
  if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return DSA_ERR_WORKSPACE;
  return DSA_OK;
}

IndexerArgs indexer_args(const dsa_seqs *s, const dsa_dims *d, const void *q_idx, const float *q_scale,
                         const float *w, const void *k_cache, const float *k_scale, float *scores,
                         long long ld, int q_begin, int rows, int fill) {
  IndexerArgs a;
  a.sv = view(s);
  a.H_I = d->index_heads;
  a.d_I = d->index_dim;
  a.dtype = d->index_dtype;
  a.q_idx = q_idx;
  a.q_scale = q_scale;
  a.w = w;
  a.k_cache = k_cache;
  a.k_scale = k_scale;
  a.scores = scores;
  a.ld = ld;
  a.q_begin = q_begin;
  a.rows = rows;
  a.fill_masked = fill;
  a.hist = nullptr;
  a.hist_stride = 0;
  a.hist_mode = 0;
  return a;
}

TopkArgs topk_args(const dsa_seqs *s, int k, const float *scores, long long ld, int32_t *idx, void *ws,
                   int q_begin, int rows) {
  TopkArgs a;
  a.sv = view(s);
  a.k = k;
  a.scores = scores;
  a.ld = ld;
  a.q_begin = q_begin;
  a.rows = rows;
  a.idx = idx;
  a.ws = reinterpret_cast<uint32_t *>(ws);
  const TopkLayout L = topk_layout(rows, s->max_ctx);
  a.row_words = L.row_words;
  a.slices = L.slices;
  a.slice_len = L.slice_len;
  a.sel_seg = L.sel_seg;
  return a;
}

MlaArgs mla_args(const dsa_seqs *s, const dsa_dims *d, float sm_scale, const void *q, const void *kv,
                 const int32_t *idx, void *out, float *lse, void *ws, int q_begin, int rows) {
  MlaArgs a;
  a.sv = view(s);
  a.H = d->heads;
  a.D = d->qk_dim;
  a.Dv = d->v_dim;
  a.k = d->topk;
  a.dtype = d->mla_dtype;
  a.sm_scale = sm_scale;
  a.q = q;
  a.kv = kv;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.q_begin = q_begin;
  a.rows = rows;
  a.n_split = mla_split_count(d, rows);
  a.part = ws;
  a.dense = 0;
  a.mode = 0;
  a.probs = nullptr;
  a.ld = 0;
  return a;
}

int check_index_ptrs(const dsa_dims *d, const void *q_idx, const float *q_scale, const float *w,
                     const void *k_cache, const float *k_scale) {
  if (q_idx == nullptr || w == nullptr || k_cache == nullptr) return DSA_ERR_INVALID_ARG;
  if (d->index_dtype == DSA_FP8_E4M3FN && (q_scale == nullptr || k_scale == nullptr)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

}  // namespace

DSA_EXPORT size_t dsa_workspace_size(int op, const dsa_seqs *seqs, const dsa_dims *dims) {
  if (check_seqs(seqs) != DSA_OK || dims == nullptr || seqs->num_q == 0) return 0;
  switch (op) {
    case DSA_OP_INDEX_SCORES:
      return 0;
    case DSA_OP_TOPK:
      if (check_k(dims->topk) != DSA_OK) return 0;
      return (size_t)topk_ws_bytes(seqs->num_q, seqs->max_ctx);
    case DSA_OP_SPARSE_MLA:
      if (check_mla_dims(dims) != DSA_OK) return 0;
      return (size_t)mla_ws_bytes(dims, seqs->num_q);
    case DSA_OP_FORWARD:
      if (check_index_dims(dims) != DSA_OK || check_mla_dims(dims) != DSA_OK) return 0;
      return (size_t)forward_layout(seqs, dims).total;
    case DSA_OP_DENSE_MLA:
      if (check_dense_dims(seqs, dims) != DSA_OK) return 0;
      return (size_t)dense_layout(seqs, dims).total;
    case DSA_OP_ATTENTION_PROBS:
      if (check_probs_dims(seqs, dims) != DSA_OK) return 0;
      return (size_t)probs_layout(seqs, dims).total;
    case DSA_OP_INDEXER_BACKWARD:
      if (check_bwd_dims(dims) != DSA_OK) return 0;
      return (size_t)bwd_layout(seqs).total;
    case DSA_OP_INDEXER_KL_LOSS:
      if (check_bwd_dims(dims) != DSA_OK || check_probs_dims(seqs, dims) != DSA_OK) return 0;
      return (size_t)kl_loss_layout(seqs, dims).total;
    case DSA_OP_SPARSE_MLA_BACKWARD:
      if (check_sbwd(seqs, dims) != DSA_OK) return 0;
      return (size_t)sbwd_layout(seqs, dims).total;
    default:
      return 0;
  }
}

DSA_EXPORT int64_t dsa_forward_chunk_rows(const dsa_seqs *seqs, const dsa_dims *dims) {
  if (check_seqs(seqs) != DSA_OK || check_index_dims(dims) != DSA_OK || check_mla_dims(dims) != DSA_OK) return 0;
  return forward_chunk_rows(seqs);
}

DSA_EXPORT int dsa_index_scores(const dsa_seqs *seqs, const dsa_dims *dims, const void *q_idx,
                                const float *q_scale, const float *w, const void *k_cache,
                                const float *k_scale, float *scores, int64_t ld_scores,
                                hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_index_dims(dims)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (int e = check_index_ptrs(dims, q_idx, q_scale, w, k_cache, k_scale)) return e;
  if (scores == nullptr || ld_scores < seqs->max_ctx) return DSA_ERR_INVALID_ARG;
  IndexerArgs a = indexer_args(seqs, dims, q_idx, q_scale, w, k_cache, k_scale, scores, ld_scores, 0,
                               seqs->num_q, 1);
  return hip_status(launch_index_scores(a, stream));
}

DSA_EXPORT int dsa_topk(const dsa_seqs *seqs, int32_t k, const float *scores, int64_t ld_scores,
                        int32_t *topk_idx, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_k(k)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (scores == nullptr || topk_idx == nullptr || ld_scores < seqs->max_ctx) return DSA_ERR_INVALID_ARG;
  if (int e = check_ws((size_t)topk_ws_bytes(seqs->num_q, seqs->max_ctx), ws, ws_bytes)) return e;
  TopkArgs a = topk_args(seqs, k, scores, ld_scores, topk_idx, ws, 0, seqs->num_q);
  return hip_status(launch_topk(a, stream));
}

DSA_EXPORT int dsa_sparse_mla(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                              const void *kv_cache, const int32_t *topk_idx, void *out, float *lse,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_mla_dims(dims)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (q == nullptr || kv_cache == nullptr || topk_idx == nullptr || out == nullptr) return DSA_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return DSA_ERR_INVALID_ARG;
  if (int e = check_ws((size_t)mla_ws_bytes(dims, seqs->num_q), ws, ws_bytes)) return e;
  MlaArgs a = mla_args(seqs, dims, sm_scale, q, kv_cache, topk_idx, out, lse, ws, 0, seqs->num_q);
  return hip_status(launch_sparse_mla(a, stream));
}

namespace {

int check_forward(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_forward_args *args) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_index_dims(dims)) return e;
  if (int e = check_mla_dims(dims)) return e;
  if (args == nullptr || args->reserved != 0) return DSA_ERR_INVALID_ARG;
  if (seqs->num_q == 0) return DSA_OK;
  if (int e = check_index_ptrs(dims, args->q_idx, args->q_scale, args->w, args->k_cache, args->k_scale))
    return e;
  if (args->q == nullptr || args->kv_cache == nullptr || args->out == nullptr) return DSA_ERR_INVALID_ARG;
  if (!(args->sm_scale == args->sm_scale)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

}  // namespace

DSA_EXPORT int dsa_forward(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_forward_args *args,
                           void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_forward(seqs, dims, args)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  const ForwardLayout L = forward_layout(seqs, dims);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;

  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  float *scores = reinterpret_cast<float *>(base + L.off_scores);
  int32_t *idx_ws = reinterpret_cast<int32_t *>(base + L.off_idx);
  void *topk_ws = base + L.off_topk;
  void *mla_ws = base + L.off_mla;
  hipEvent_t const *ev = reinterpret_cast<hipEvent_t const *>(args->stage_events);

  // Short prompts: when no query has more than k candidates the selection is
  // every candidate whatever the scores, so the indexer and the top-k are
  // skipped and the attention walks the candidate positions directly (the
  // same lists, split the same way, so the same bytes out).
  const bool all_selected = seqs->max_ctx <= dims->topk;
  const int T = seqs->num_q;
  for (int c0 = 0; c0 < T; c0 += L.chunk) {
    const int rows = c0 + L.chunk < T ? L.chunk : T - c0;
    const bool timed = ev != nullptr && c0 == 0;
    int32_t *idx = args->topk_idx != nullptr ? args->topk_idx + (long long)c0 * dims->topk : idx_ws;
    TopkArgs ta = topk_args(seqs, dims->topk, scores, L.ld, idx, topk_ws, c0, rows);
    if (all_selected) {
      if (timed && hipEventRecord(ev[0], stream) != hipSuccess) return DSA_ERR_HIP;
      if (timed && hipEventRecord(ev[1], stream) != hipSuccess) return DSA_ERR_HIP;
      if (args->topk_idx != nullptr && launch_topk_all(ta, stream) != hipSuccess) return DSA_ERR_HIP;
      if (timed && hipEventRecord(ev[2], stream) != hipSuccess) return DSA_ERR_HIP;
      MlaArgs ma = mla_args(seqs, dims, args->sm_scale, args->q, args->kv_cache, nullptr, args->out, args->lse,
                            mla_ws, c0, rows);
      ma.dense = 1;
      if (launch_sparse_mla(ma, stream) != hipSuccess) return DSA_ERR_HIP;
      if (timed && hipEventRecord(ev[3], stream) != hipSuccess) return DSA_ERR_HIP;
      continue;
    }
    IndexerArgs ia = indexer_args(seqs, dims, args->q_idx, args->q_scale, args->w, args->k_cache,
                                  args->k_scale, scores, L.ld, c0, rows, 0);
    // The MFMA indexers count the top-k's first radix digit as they write the
    // scores: decode adds per-workgroup counts into rows zeroed first; prefill
    // stores whole rows (the sliced select still needs its counters zeroed).
    const bool fused = dims->index_dtype != DSA_F32;
    if (fused) {
      ia.hist = ta.ws;
      ia.hist_stride = ta.row_words;
      ia.hist_mode = seqs->mode == DSA_DECODE ? 1 : 2;
      if ((ia.hist_mode == 1 || topk_sliced(rows)) && launch_topk_zero(ta, stream) != hipSuccess)
        return DSA_ERR_HIP;
    }
    if (timed && hipEventRecord(ev[0], stream) != hipSuccess) return DSA_ERR_HIP;
    if (launch_index_scores(ia, stream) != hipSuccess) return DSA_ERR_HIP;
    if (timed && hipEventRecord(ev[1], stream) != hipSuccess) return DSA_ERR_HIP;
    if ((fused ? launch_topk_select(ta, stream) : launch_topk(ta, stream)) != hipSuccess) return DSA_ERR_HIP;
    if (timed && hipEventRecord(ev[2], stream) != hipSuccess) return DSA_ERR_HIP;
    MlaArgs ma = mla_args(seqs, dims, args->sm_scale, args->q, args->kv_cache, idx, args->out, args->lse,
                          mla_ws, c0, rows);
    if (launch_sparse_mla(ma, stream) != hipSuccess) return DSA_ERR_HIP;
    if (timed && hipEventRecord(ev[3], stream) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

DSA_EXPORT int dsa_forward_noalloc(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_forward_args *args,
                                   hipStream_t stream) {
  if (int e = check_forward(seqs, dims, args)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if ((size_t)forward_layout(seqs, dims).total > kNoallocScratchBytes) return DSA_ERR_SCRATCH_LIMIT;
  void *ptr = nullptr;
  if (int e = scratch_on_current_device(&ptr)) return e;
  return dsa_forward(seqs, dims, args, ptr, kNoallocScratchBytes, stream);
}

DSA_EXPORT int dsa_dense_mla(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                             const void *kv_cache, void *out, float *lse, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_dense_dims(seqs, dims)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (q == nullptr || kv_cache == nullptr || out == nullptr) return DSA_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return DSA_ERR_INVALID_ARG;
  const DenseLayout L = dense_layout(seqs, dims);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;
  const int T = seqs->num_q;
  for (int c0 = 0; c0 < T; c0 += L.chunk) {
    const int rows = c0 + L.chunk < T ? L.chunk : T - c0;
    MlaArgs a = mla_args(seqs, dims, sm_scale, q, kv_cache, nullptr, out, lse, ws, c0, rows);
    a.dense = 1;
    a.k = seqs->max_ctx;
    a.n_split = L.n_split;
    if (launch_sparse_mla(a, stream) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

DSA_EXPORT int dsa_attention_probs(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                                   const void *kv_cache, float *probs, int64_t ld_probs, float *lse,
                                   int32_t lse_given, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_probs_dims(seqs, dims)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (q == nullptr || kv_cache == nullptr || probs == nullptr || ld_probs < seqs->max_ctx) return DSA_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return DSA_ERR_INVALID_ARG;
  if (lse_given != 0 && (lse_given != 1 || lse == nullptr)) return DSA_ERR_INVALID_ARG;
  const ProbsLayout L = probs_layout(seqs, dims);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  float *lse_buf = lse != nullptr ? lse : reinterpret_cast<float *>(base);
  void *part = base + L.off_part;
  const int T = seqs->num_q;
  for (int c0 = 0; c0 < T; c0 += L.chunk) {
    const int rows = c0 + L.chunk < T ? L.chunk : T - c0;
    MlaArgs a = mla_args(seqs, dims, sm_scale, q, kv_cache, nullptr, nullptr, lse_buf, part, c0, rows);
    a.dense = 1;
    a.k = seqs->max_ctx;
    a.n_split = L.n_split;
    if (!lse_given) {
      a.mode = 1;
      if (launch_sparse_mla(a, stream) != hipSuccess) return DSA_ERR_HIP;
    }
    a.mode = 2;
    a.probs = probs + (long long)c0 * ld_probs;
    a.ld = ld_probs;
    if (launch_sparse_mla(a, stream) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

DSA_EXPORT int dsa_indexer_kl(const dsa_seqs *seqs, float *scores, const float *probs, int64_t ld, float *loss,
                              hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (scores == nullptr || probs == nullptr || loss == nullptr || ld < seqs->max_ctx) return DSA_ERR_INVALID_ARG;
  KlArgs a;
  a.sv = view(seqs);
  a.q_begin = 0;
  a.rows = seqs->num_q;
  a.scores = scores;
  a.probs = probs;
  a.ld = ld;
  a.loss = loss;
  return hip_status(launch_indexer_kl(a, stream));
}

DSA_EXPORT int dsa_indexer_backward(const dsa_seqs *seqs, const dsa_dims *dims, const void *q_idx, const float *w,
                                    const void *k_cache, const float *grad_scores, int64_t ld, float *dq_idx,
                                    float *dw, float *dk, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_bwd_dims(dims)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (q_idx == nullptr || w == nullptr || k_cache == nullptr || grad_scores == nullptr || ld < seqs->max_ctx)
    return DSA_ERR_INVALID_ARG;
  if (dq_idx == nullptr || dw == nullptr || dk == nullptr) return DSA_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(seqs);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;
  BwdArgs a;
  a.sv = view(seqs);
  a.q_begin = 0;
  a.rows = seqs->num_q;
  a.q_idx = q_idx;
  a.w = w;
  a.k_cache = k_cache;
  a.grad = grad_scores;
  a.ld = ld;
  a.dq = dq_idx;
  a.dw = dw;
  a.dk = dk;
  a.span = seqs->max_ctx;
  a.n_split = L.q_splits;
  a.q_per_split = L.q_per_split;
  a.part = reinterpret_cast<float *>(ws);
  a.sel = nullptr;
  a.sel_k = 0;
  if (launch_indexer_bwd_q(a, stream) != hipSuccess) return DSA_ERR_HIP;
  a.n_split = L.k_qsplits;
  a.part = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + L.off_k);
  return hip_status(launch_indexer_bwd_k(a, stream));
}

DSA_EXPORT int dsa_indexer_backward_selected(const dsa_seqs *seqs, const dsa_dims *dims, const void *q_idx,
                                             const float *w, const void *k_cache, const float *grad_scores,
                                             int64_t ld, const int32_t *topk_idx, int32_t k, float *dq_idx,
                                             float *dw, float *dk, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_bwd_dims(dims)) return e;
  if (int e = check_k(k)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (q_idx == nullptr || w == nullptr || k_cache == nullptr || grad_scores == nullptr || topk_idx == nullptr ||
      ld < seqs->max_ctx)
    return DSA_ERR_INVALID_ARG;
  if (dq_idx == nullptr || dw == nullptr || dk == nullptr) return DSA_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(seqs);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;
  BwdArgs a;
  a.sv = view(seqs);
  a.q_begin = 0;
  a.rows = seqs->num_q;
  a.q_idx = q_idx;
  a.w = w;
  a.k_cache = k_cache;
  a.grad = grad_scores;
  a.ld = ld;
  a.dq = dq_idx;
  a.dw = dw;
  a.dk = dk;
  a.span = seqs->max_ctx;
  a.sel = topk_idx;
  a.sel_k = k;
  a.n_split = 1;
  a.q_per_split = L.q_per_split;
  a.part = nullptr;
  if (launch_indexer_bwd_q_sel(a, stream) != hipSuccess) return DSA_ERR_HIP;
  a.n_split = L.k_qsplits;
  a.part = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + L.off_k);
  return hip_status(launch_indexer_bwd_k(a, stream));
}

DSA_EXPORT int dsa_indexer_kl_loss(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_kl_args *args, void *ws,
                                   size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_bwd_dims(dims)) return e;
  if (int e = check_probs_dims(seqs, dims)) return e;
  if (args == nullptr || args->reserved != 0) return DSA_ERR_INVALID_ARG;
  if (seqs->num_q == 0) return DSA_OK;
  if (args->q_idx == nullptr || args->w == nullptr || args->k_cache == nullptr || args->q == nullptr ||
      args->kv_cache == nullptr || args->loss == nullptr)
    return DSA_ERR_INVALID_ARG;
  const bool bwd = args->dq_idx != nullptr;
  if (bwd && (args->dw == nullptr || args->dk == nullptr)) return DSA_ERR_INVALID_ARG;
  if (!(args->sm_scale == args->sm_scale)) return DSA_ERR_INVALID_ARG;
  const KlLossLayout L = kl_loss_layout(seqs, dims);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  float *scores = reinterpret_cast<float *>(base);
  float *probs = reinterpret_cast<float *>(base + L.off_probs);
  void *sub = base + L.off_ws;
  const size_t sub_bytes = ws_bytes - (size_t)L.off_ws;
  hipEvent_t const *ev = reinterpret_cast<hipEvent_t const *>(args->stage_events);
  auto mark = [&](int i) { return ev == nullptr || hipEventRecord(ev[i], stream) == hipSuccess; };
  if (!mark(0)) return DSA_ERR_HIP;
  if (int e = dsa_attention_probs(seqs, dims, args->sm_scale, args->q, args->kv_cache, probs, L.ld,
                                  const_cast<float *>(args->lse), args->lse != nullptr ? 1 : 0, sub, sub_bytes,
                                  stream))
    return e;
  if (!mark(1)) return DSA_ERR_HIP;
  if (int e = dsa_index_scores(seqs, dims, args->q_idx, nullptr, args->w, args->k_cache, nullptr, scores, L.ld,
                               stream))
    return e;
  if (!mark(2)) return DSA_ERR_HIP;
  if (int e = dsa_indexer_kl(seqs, scores, probs, L.ld, args->loss, stream)) return e;
  if (!mark(3)) return DSA_ERR_HIP;
  if (bwd) {
    if (int e = dsa_indexer_backward(seqs, dims, args->q_idx, args->w, args->k_cache, scores, L.ld, args->dq_idx,
                                     args->dw, args->dk, sub, sub_bytes, stream))
      return e;
  }
  if (!mark(4)) return DSA_ERR_HIP;
  return DSA_OK;
}

DSA_EXPORT int dsa_sparse_mla_backward(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                                       const void *kv_cache, const int32_t *topk_idx, const void *out,
                                       const float *lse, const void *dout, float *dq, float *dkv, float *probs,
                                       void *ws, size_t ws_bytes, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_sbwd(seqs, dims)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (q == nullptr || kv_cache == nullptr || topk_idx == nullptr || out == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dkv == nullptr)
    return DSA_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return DSA_ERR_INVALID_ARG;
  const SBwdLayout L = sbwd_layout(seqs, dims);
  if (int e = check_ws((size_t)L.total, ws, ws_bytes)) return e;
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  MlaBwdArgs a;
  a.sv = view(seqs);
  a.k = dims->topk;
  a.sm_scale = sm_scale;
  a.q = q;
  a.kv = kv_cache;
  a.idx = topk_idx;
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dkv = dkv;
  a.probs = probs;
  a.delta = reinterpret_cast<float *>(base);
  a.ds_t = reinterpret_cast<uint16_t *>(base + L.off_dst);
  a.pd = reinterpret_cast<uint16_t *>(base + L.off_pd);
  a.contrib = reinterpret_cast<uint16_t *>(base + L.off_contrib);
  a.jpos = reinterpret_cast<uint16_t *>(base + L.off_jpos);
  a.jstride = L.jstride;
  a.nkeys = seqs->max_ctx;
  const int T = seqs->num_q;
  for (int c0 = 0; c0 < T; c0 += L.chunk) {
    a.q_begin = c0;
    a.rows = c0 + L.chunk < T ? L.chunk : T - c0;
    a.first = c0 == 0 ? 1 : 0;
    if (launch_sparse_mla_bwd(a, stream) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

DSA_EXPORT int dsa_sparse_indexer_kl(const dsa_seqs *seqs, float *scores, int64_t ld, const int32_t *topk_idx,
                                     int32_t k, const float *probs, float *loss, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (int e = check_k(k)) return e;
  if (seqs->num_q == 0) return DSA_OK;
  if (scores == nullptr || topk_idx == nullptr || probs == nullptr || loss == nullptr || ld < seqs->max_ctx)
    return DSA_ERR_INVALID_ARG;
  SparseKlArgs a;
  a.sv = view(seqs);
  a.rows = seqs->num_q;
  a.k = k;
  a.scores = scores;
  a.ld = ld;
  a.idx = topk_idx;
  a.probs = probs;
  a.loss = loss;
  return hip_status(launch_sparse_kl(a, stream));
}

DSA_EXPORT int dsa_quantize_fp8(int64_t rows, int32_t len, int32_t src_dtype, const void *src, void *dst,
                                float *scale, int32_t scale_repeat, hipStream_t stream) {
  if (rows < 0 || len < 1 || scale_repeat < 1) return DSA_ERR_INVALID_ARG;
  if (src_dtype != DSA_BF16 && src_dtype != DSA_F32) return DSA_ERR_INVALID_ARG;
  if (len % 4 != 0 || len > kQuantMaxLen || scale_repeat > kQuantMaxRepeat) return DSA_ERR_UNSUPPORTED;
  if (rows == 0) return DSA_OK;
  if (rows > kQuantMaxRows) return DSA_ERR_UNSUPPORTED;
  if (src == nullptr || dst == nullptr || scale == nullptr) return DSA_ERR_INVALID_ARG;
  QuantArgs a;
  a.rows = rows;
  a.len = len;
  a.src_dtype = src_dtype;
  a.scale_repeat = scale_repeat;
  a.src = src;
  a.dst = reinterpret_cast<uint8_t *>(dst);
  a.scale = scale;
  return hip_status(launch_fp8_quantize(a, stream));
}

DSA_EXPORT int dsa_append_index_keys(const dsa_seqs *seqs, int32_t index_dim, int32_t src_dtype,
                                     const void *k_new, void *k_cache, float *k_scale, hipStream_t stream) {
  if (int e = check_seqs(seqs)) return e;
  if (index_dim < 1) return DSA_ERR_INVALID_ARG;
  if (src_dtype != DSA_BF16 && src_dtype != DSA_F32) return DSA_ERR_INVALID_ARG;
  if (index_dim % 4 != 0 || index_dim > kAppendMaxDim) return DSA_ERR_UNSUPPORTED;
  if (seqs->num_q == 0) return DSA_OK;
  if (k_new == nullptr || k_cache == nullptr || k_scale == nullptr) return DSA_ERR_INVALID_ARG;
  AppendArgs a;
  a.sv = view(seqs);
  a.len = index_dim;
  a.src_dtype = src_dtype;
  a.src = k_new;
  a.cache = reinterpret_cast<uint8_t *>(k_cache);
  a.scale = k_scale;
  return hip_status(launch_fp8_append(a, stream));
}

DSA_EXPORT int dsa_read_ceiling(const void *src, int64_t bytes, int32_t flags, uint32_t *sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      (flags & ~(DSA_READ_PAGED | DSA_READ_CACHED)) != 0)
    return DSA_ERR_INVALID_ARG;
  if (bytes % kReadCeilingChunk != 0 || bytes / kReadCeilingChunk > INT32_MAX) return DSA_ERR_UNSUPPORTED;
  const int64_t nblk = bytes / 16384;
  const bool paged = (flags & DSA_READ_PAGED) != 0;
  if (paged && (nblk & (nblk - 1)) != 0) return DSA_ERR_UNSUPPORTED;
  return hip_status(launch_read_ceiling(src, bytes, paged, (flags & DSA_READ_CACHED) != 0, sink, stream));
}

DSA_EXPORT const char *dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape or type not supported";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: kernel launch failed";
    case DSA_ERR_SCRATCH_LIMIT:
      return "DSA_ERR_SCRATCH_LIMIT: the problem needs more than the 128 MiB static scratch of dsa_forward_noalloc";
    default: return "unknown dsa_status";
  }
}

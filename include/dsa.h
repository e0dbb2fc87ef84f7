/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) forward path for
 * AMD Instinct MI355X (gfx950).
 *
 * The path has three steps.  Sources, cited below by tag:
 *   [ZS] "DeepSeek V3.2: How Far Can Open Models Go If You Actually Try?"
 *        (zeroshot.it.com), section 3.1 (indexer equation, selection-then-
 *        attention equation, MQA mode) and section 3.4 (short prompts).
 *   [LD] "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models"
 *        (papers.lunadong.com summary), Pipeline Flow, System Modules, Key
 *        Hyperparameters (selected_tokens_k = 2048, 128K context).
 *   [BT] baseten.co "DeepSeek-V3.2", section (1) DSA + MLA.
 *   [NH] news.han.ihouse.idv.tw article 1495, section "Introducing DSA
 *        Efficient Sparse Attention Mechanism" (ReLU, FP8, k = 2048).
 *
 *   1. lightning indexer  I(t,s) = sum_j w(t,j) * ReLU(q(t,j) . k(s))  over
 *      every candidate s of query t                     [ZS 3.1; LD; NH]
 *   2. fine-grained top-k: the k best candidates of each query
 *                                                       [ZS 3.1; LD; BT]
 *   3. MLA in MQA mode over the selected rows of the shared latent cache:
 *      every head attends over the same fetched rows    [ZS 3.1; LD]
 *
 * Conventions (every entry point):
 *   - Pointers are DEVICE pointers unless marked "host".  Structs passed by
 *     pointer are host memory, read during the call only.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     null stream).  The library never synchronises, never allocates device
 *     memory and keeps no state between calls; callers own every buffer,
 *     including the workspace sized by dsa_workspace_size() (its base
 *     256-byte aligned, as every hipMalloc and torch allocation is).  The one
 *     exception is dsa_forward_noalloc, whose scratch is a static device
 *     array of the library (see there).
 *   - Arguments are checked on the host before any launch; a failed check
 *     returns a negative dsa_status and launches nothing.  A launch failure
 *     returns DSA_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Device-side metadata is bounds-checked in the kernels and never makes
 *     them read outside the caches: a query position is clamped to
 *     [-1, max_ctx-1] (a negative position means no candidates); a block
 *     table entry outside [0, num_blocks) makes the tokens of that block
 *     absent (score -inf, never attended); a selected index that is negative
 *     or above the query's position is skipped.
 *   - Candidates: query t at position p = q_pos[t] sees the positions
 *     s = 0..p of its sequence, p included (n_t = p + 1).  Reading of the
 *     pages' "preceding tokens"; with k >= n_t the path is dense causal MLA.
 *   - Results are deterministic: the same inputs give the same bytes.
 *
 * Layouts (row-major, last index fastest; all arrays dense):
 *   indexer queries  q_idx    [T, H_I, d_I]   index_dtype
 *   indexer q scales q_scale  [T, H_I] fp32   (e4m3fn only, > 0)
 *   head weights     w        [T, H_I] fp32   (any sign)
 *   indexer keys     k_cache  contiguous [B, max_seq_len, d_I] or paged
 *                             [num_blocks, block_size, d_I]     index_dtype
 *   key scales       k_scale  [B, max_seq_len] / [num_blocks, block_size]
 *                             fp32 (e4m3fn only, > 0)
 *   MLA queries      q        [T, H, D]   mla_dtype (already absorbed into
 *                             the latent space; D = latent Dv + rope)
 *   latent cache     kv_cache contiguous [B, max_seq_len, D] or paged
 *                             [num_blocks, block_size, D]       mla_dtype
 *   scores           [T, ld_scores] fp32
 *   selected         topk_idx [T, k] int32
 *   output           out      [T, H, Dv]  mla_dtype;  lse [T, H] fp32
 *
 * Supported shapes (others return DSA_ERR_UNSUPPORTED):
 *   indexer  bf16 / e4m3fn: H_I = 64, d_I = 128;
 *            fp32: H_I <= 64, d_I <= 128, H_I * d_I <= 4096
 *   MLA      bf16: H = 128, D = 576, Dv = 512;
 *            fp32: H <= 16, D <= 128, Dv <= D, k <= 1024
 *   1 <= k <= 2048; max_ctx <= 262144; paged block_size = 64.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_dtype {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3FN = 2 /* OCP FP8 E4M3 (max 448, no infinities); indexer only */
} dsa_dtype;

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shape */
  DSA_ERR_UNSUPPORTED = -2, /* valid but outside the supported shapes/types */
  DSA_ERR_WORKSPACE = -3,   /* workspace missing, smaller than required, or not 256-byte aligned */
  DSA_ERR_HIP = -4,         /* a kernel launch failed */
  DSA_ERR_SCRATCH_LIMIT = -5 /* dsa_forward_noalloc: the problem needs more than its static scratch */
} dsa_status;

typedef enum dsa_mode {
  DSA_PREFILL = 0, /* all T queries belong to sequence 0 of the caches */
  DSA_DECODE = 1   /* query t belongs to sequence t (T <= B) */
} dsa_mode;

typedef enum dsa_op {
  DSA_OP_INDEX_SCORES = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_MLA = 2,
  DSA_OP_FORWARD = 3,
  DSA_OP_DENSE_MLA = 4,
  DSA_OP_ATTENTION_PROBS = 5,
  DSA_OP_INDEXER_BACKWARD = 6,
  DSA_OP_INDEXER_KL_LOSS = 7,
  DSA_OP_SPARSE_MLA_BACKWARD = 8
} dsa_op;

/* Where each query sits and which cache rows it may read (host struct). */
typedef struct dsa_seqs {
  int32_t mode;              /* dsa_mode */
  int32_t num_seqs;          /* B: sequences in the caches (prefill: >= 1, only sequence 0 is read) */
  int32_t num_q;             /* T >= 0 */
  int32_t max_ctx;           /* host bound: max over t of q_pos[t] + 1 (1..262144); sizes grids */
  const int32_t *q_pos;      /* [T] device: position of query t in its sequence */
  const int32_t *block_table;/* [B, max_blocks] device, or NULL for contiguous caches */
  int32_t max_blocks;        /* columns of block_table (>= ceil(max_ctx / block_size)) */
  int32_t num_blocks;        /* blocks in each paged pool */
  int32_t block_size;        /* tokens per block: 64 (paged only) */
  int32_t reserved;          /* must be 0 */
  int64_t max_seq_len;       /* contiguous caches: token slots per sequence (>= max_ctx) */
} dsa_seqs;

/* Problem dimensions and element types (host struct). */
typedef struct dsa_dims {
  int32_t index_heads; /* H_I */
  int32_t index_dim;   /* d_I */
  int32_t topk;        /* k */
  int32_t heads;       /* H */
  int32_t qk_dim;      /* D (score dim: latent + rope) */
  int32_t v_dim;       /* Dv (value dim: latent) */
  int32_t index_dtype; /* dsa_dtype of q_idx / k_cache */
  int32_t mla_dtype;   /* dsa_dtype of q / kv_cache / out (F32 or BF16) */
} dsa_dims;

/* Inputs and outputs of dsa_forward (host struct of device pointers). */
typedef struct dsa_forward_args {
  const void *q_idx;     /* [T, H_I, d_I] */
  const float *q_scale;  /* [T, H_I] (e4m3fn only, else NULL) */
  const float *w;        /* [T, H_I] */
  const void *k_cache;   /* indexer key cache */
  const float *k_scale;  /* key scales (e4m3fn only, else NULL) */
  const void *q;         /* [T, H, D] */
  const void *kv_cache;  /* latent cache */
  float sm_scale;        /* softmax scale applied to q . c (e.g. 1/sqrt(D)) */
  int32_t reserved;      /* must be 0 */
  int32_t *topk_idx;     /* optional [T, k] output of the selection, or NULL */
  void *out;             /* [T, H, Dv] */
  float *lse;            /* optional [T, H], or NULL */
  /* optional host array of 4 hipEvent_t recorded on `stream` at the start and
   * after the indexer, top-k and attention stages of the first query chunk
   * (decode always runs as one chunk); NULL records nothing */
  void *const *stage_events;
} dsa_forward_args;

/* Inputs and outputs of dsa_indexer_kl_loss (host struct of device pointers). */
typedef struct dsa_kl_args {
  const void *q_idx;     /* [T, H_I, d_I] bf16: the indexer (trained) */
  const float *w;        /* [T, H_I] */
  const void *k_cache;   /* indexer key cache, bf16 */
  const void *q;         /* [T, H, D] bf16: the main attention (frozen) */
  const void *kv_cache;  /* latent cache, bf16 */
  float sm_scale;        /* softmax scale of the main attention */
  int32_t reserved;      /* must be 0 */
  const float *lse;      /* [T, H]: the main attention's per-head lse (e.g. from
                            dsa_dense_mla), or NULL to compute it */
  float *loss;           /* [T]: KL term of each query (L_I is their sum) */
  float *dq_idx;         /* [T, H_I, d_I] fp32, or NULL: no backward */
  float *dw;             /* [T, H_I] fp32 (NULL with dq_idx) */
  float *dk;             /* key cache layout, fp32 (NULL with dq_idx) */
  /* optional host array of 5 hipEvent_t recorded on `stream` at the start and
   * after the target distribution, the scores, the KL rows and the backward;
   * NULL records nothing */
  void *const *stage_events;
} dsa_kl_args;

/* Bytes of workspace the given entry point needs for these shapes (0 when
 * none).  op is a dsa_op.  Returns 0 as well for invalid arguments; the
 * entry point itself then reports the error. */
size_t dsa_workspace_size(int op, const dsa_seqs *seqs, const dsa_dims *dims);

/* Step 1, the lightning indexer [ZS 3.1 indexer equation; LD System Modules;
 * NH: ReLU chosen for throughput, FP8].
 * scores[t, s] = sum_j w[t,j] * ReLU(q_idx[t,j,:] . k(s)) for s = 0..q_pos[t];
 * with e4m3fn operands q = q8 * q_scale[t,j] and k = k8 * k_scale(s), which
 * the kernel folds out of the ReLU (scales must be positive).  Entries
 * q_pos[t] < s < ld_scores are set to -inf.  Products are accumulated in
 * fp32 (bf16 / e4m3fn / fp32 operands); the head sum is fp32.
 * ld_scores >= max_ctx.  No workspace. */
int dsa_index_scores(const dsa_seqs *seqs, const dsa_dims *dims, const void *q_idx,
                     const float *q_scale, const float *w, const void *k_cache,
                     const float *k_scale, float *scores, int64_t ld_scores,
                     hipStream_t stream);

/* Step 2, fine-grained top-k [ZS 3.1 selection equation; LD "Top-k
 * operation"; LD Key Hyperparameters k = 2048].
 * For each query the first m = min(k, q_pos[t]+1) positions in the order
 * (score descending, position ascending) -- ties go to the lower position,
 * -0.0 equals +0.0 -- written in ASCENDING position order to topk_idx[t, 0..m)
 * and -1 to topk_idx[t, m..k).  Reads scores[t, 0..q_pos[t]] only; scores
 * must not be NaN.  Exact: integer radix select on order-preserving keys.
 * Workspace: dsa_workspace_size(DSA_OP_TOPK, ...). */
int dsa_topk(const dsa_seqs *seqs, int32_t k, const float *scores, int64_t ld_scores,
             int32_t *topk_idx, void *ws, size_t ws_bytes, hipStream_t stream);

/* Step 3, sparse MLA in MQA mode [ZS 3.1 selection equation and MQA-mode
 * paragraph: one shared latent row per token, every head reads the same
 * fetched rows; LD Novel Architectural Elements].
 * For query t and head h over the valid entries s of topk_idx[t, :]:
 *   z_s = sm_scale * (q[t,h,:] . c(s)[0:D]),  p = softmax(z),
 *   out[t,h,:] = sum_s p_s * c(s)[0:Dv],  lse[t,h] = max z + ln sum exp(z - max z).
 * bf16 operands, fp32 logits / softmax / accumulation, bf16 round-to-nearest-
 * even output (fp32 throughout for DSA_F32).  An empty selection gives
 * out = 0 and lse = -inf.  lse may be NULL.
 * Workspace: dsa_workspace_size(DSA_OP_SPARSE_MLA, ...). */
int dsa_sparse_mla(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                   const void *kv_cache, const int32_t *topk_idx, void *out, float *lse,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* Steps 1-3 fused into one call for prefill or decode [LD Pipeline Flow:
 * indexer, then token selection, then sparse attention].  Results equal
 * dsa_index_scores -> dsa_topk -> dsa_sparse_mla on the same inputs.
 * Prefill runs in query chunks so the score rows of a chunk stay on chip.
 * Short prompts [ZS 3.4: DSA then behaves as dense attention]: when
 * max_ctx <= k every query keeps all of its candidates whatever their
 * scores, so the indexer and top-k are not run; the attention walks the
 * candidate positions and the output bytes are the same.  topk_idx, if
 * given, then receives 0..n_t-1 followed by -1.
 * Workspace: dsa_workspace_size(DSA_OP_FORWARD, ...). */
int dsa_forward(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_forward_args *args,
                void *ws, size_t ws_bytes, hipStream_t stream);

/* dsa_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation, kernels and results as dsa_forward, with the workspace
 * taken from a static device array of the library: 128 MiB on each GPU,
 * reserved when the library's code object is loaded on that GPU and held
 * until the process ends.  The array of the current device (hipGetDevice) is
 * used, so `stream` must belong to it.  The call allocates nothing (no
 * hipMalloc, no library allocation).  A problem whose
 * dsa_workspace_size(DSA_OP_FORWARD, ...) exceeds 128 MiB is rejected on the
 * host with DSA_ERR_SCRATCH_LIMIT and launches nothing; 128 MiB holds, e.g.,
 * a decode of 32 sequences at 128K context, or a prefill of 2048 tokens.
 * Every call on one GPU shares that GPU's array (the kernels clear what must
 * start at zero on every call), so calls that overlap on one GPU -- on
 * different streams, or from different host threads -- race; order them. */
int dsa_forward_noalloc(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_forward_args *args,
                        hipStream_t stream);

/* Query rows per chunk that dsa_forward processes at a time for these shapes
 * (all num_q rows for decode), so a caller can time or split work the way the
 * call runs it.  0 for invalid arguments.  Host only; launches nothing. */
int64_t dsa_forward_chunk_rows(const dsa_seqs *seqs, const dsa_dims *dims);

/* Dense MLA, the attention DSA is measured against [ZS 3.4: at a 128K context
 * DSA decodes about twice as cheaply as dense MLA; LD: the dense warm-up
 * stage keeps dense attention]: step 3 over EVERY candidate s = 0..q_pos[t]
 * of each query, with no indexer and no selection.  Logits, softmax, output,
 * lse and precision as dsa_sparse_mla; dims->topk and the indexer fields are
 * not read.  bf16: each query's candidates are cut into up to 128 splits of
 * at most 2048 rows, merged in split order; queries run in chunks whose split
 * partials fit 1 GiB of workspace (so a decode batch is one chunk).
 * Supported: bf16 H = 128, D = 576, Dv = 512 (max_ctx <= 262144); fp32
 * H <= 16, D <= 128, max_ctx <= 1024.
 * Workspace: dsa_workspace_size(DSA_OP_DENSE_MLA, ...). */
int dsa_dense_mla(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                  const void *kv_cache, void *out, float *lse, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* The indexer's warm-up target [ZS 3.3, Stage 1: the main attention stays
 * dense and the indexer learns its distribution; LD Modeling, Objective
 * Functions: the dense attention aggregated over heads, L1-normalised].
 * For every query t and candidate s = 0..q_pos[t]:
 *   probs[t, s] = (1/H) sum_h softmax_s(sm_scale * q[t,h,:] . c(s))
 * (each head's weights sum to 1, so dividing the head sum by H is its L1
 * normalisation); probs[t, s] = 0 for q_pos[t] < s < ld_probs.  lse [T, H]
 * holds each head's log-sum-exp: with lse_given = 0 it is computed first (a
 * pass of the attention kernel over every candidate) and stored there unless
 * lse is NULL; with lse_given = 1 the caller's values are used, e.g. the lse
 * that dsa_dense_mla returns for the frozen dense attention.  The weights take
 * one more pass; bf16 operands, fp32 arithmetic and output.  ld_probs >=
 * max_ctx.  Supported: bf16 H = 128, D = 576, Dv = 512.
 * Workspace: dsa_workspace_size(DSA_OP_ATTENTION_PROBS, ...). */
int dsa_attention_probs(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                        const void *kv_cache, float *probs, int64_t ld_probs, float *lse, int32_t lse_given,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* One KL term of the warm-up objective per query [ZS 3.3:
 * L_I = sum_t KL(p_t || softmax(I_t))], and its gradient with respect to the
 * scores.  scores [T, ld] holds I (e.g. from dsa_index_scores) on entry and
 * dL/dI = softmax(I_t) - p_t on return (0 for s > q_pos[t]); probs [T, ld]
 * holds p (e.g. from dsa_attention_probs).  loss[t] = sum_s p (log p - log
 * softmax(I)_s) over the candidates with p > 0 (L_I is the sum over t).  A
 * score of -inf (absent key) has softmax weight 0.  fp32; deterministic.  No
 * workspace. */
int dsa_indexer_kl(const dsa_seqs *seqs, float *scores, const float *probs, int64_t ld, float *loss,
                   hipStream_t stream);

/* Gradient of step 1 for the warm-up objective [ZS 3.3; the indexer is the
 * only part trained in Stage 1]: given dL/dI in grad_scores [T, ld] (e.g.
 * from dsa_indexer_kl), with x_js = q_idx[t,j,:] . k(s) over the candidates
 * s = 0..q_pos[t]:
 *   dw[t, j]        = sum_s g(t,s) ReLU(x_js)
 *   dq_idx[t, j, :] = sum_s g(t,s) w[t,j] [x_js > 0] k(s)
 *   dk(s)           = sum_t sum_j g(t,s) w[t,j] [x_js > 0] q_idx[t,j,:]
 * (ReLU'(0) = 0).  dq_idx [T, H_I, d_I] and dw [T, H_I] fp32; dk fp32 in the
 * key cache's layout (contiguous [B, max_seq_len, d_I] or paged
 * [num_blocks, block_size, d_I]): the rows of positions 0..max_ctx-1 of
 * sequence 0 (prefill) or 0..q_pos[t] of sequence t (decode) are written,
 * 0 where no query sees the key; other rows are left as they are.  The
 * products run on bf16 MFMA (the masked, weighted score gradient rounded to
 * bf16 as an operand) with fp32 accumulation; split partials are summed in a
 * fixed order (deterministic).  Supported: bf16 indexer, H_I = 64, d_I = 128.
 * Workspace: dsa_workspace_size(DSA_OP_INDEXER_BACKWARD, ...). */
int dsa_indexer_backward(const dsa_seqs *seqs, const dsa_dims *dims, const void *q_idx, const float *w,
                         const void *k_cache, const float *grad_scores, int64_t ld, float *dq_idx,
                         float *dw, float *dk, void *ws, size_t ws_bytes, hipStream_t stream);

/* dsa_indexer_backward for a score gradient that is zero outside each query's
 * selection [ZS 3.3 Stage 2: the indexer's loss is restricted to the selected
 * set S_t, e.g. grad_scores from dsa_sparse_indexer_kl]: dq_idx and dw are
 * summed over the entries s of topk_idx[t, 0..k) only (ascending positions as
 * dsa_topk writes them; an entry outside [0, q_pos[t]] adds nothing), where
 * dsa_indexer_backward visits every candidate; dk as dsa_indexer_backward.
 * Equal to dsa_indexer_backward on such a gradient up to the fp32 order of the
 * sums.  Same types, layouts and workspace (DSA_OP_INDEXER_BACKWARD); k as
 * dsa_topk. */
int dsa_indexer_backward_selected(const dsa_seqs *seqs, const dsa_dims *dims, const void *q_idx, const float *w,
                                  const void *k_cache, const float *grad_scores, int64_t ld,
                                  const int32_t *topk_idx, int32_t k, float *dq_idx, float *dw, float *dk, void *ws,
                                  size_t ws_bytes, hipStream_t stream);

/* The indexer's warm-up objective in one call [ZS 3.3 Stage 1; LD Objective
 * Functions]: dsa_attention_probs (target p, from args->lse when given),
 * dsa_index_scores (I),
 * dsa_indexer_kl (loss and dL/dI) and, when dq_idx is not NULL,
 * dsa_indexer_backward, with the same contracts and results.  Scores and
 * target are kept in the workspace ([T, ld] fp32 each, ld = max_ctx rounded
 * up to 64).  Supported: bf16 indexer (H_I = 64, d_I = 128) and bf16 MLA
 * (H = 128, D = 576, Dv = 512).
 * Workspace: dsa_workspace_size(DSA_OP_INDEXER_KL_LOSS, ...). */
int dsa_indexer_kl_loss(const dsa_seqs *seqs, const dsa_dims *dims, const dsa_kl_args *args, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/* Stage 2 of training, the main attention's gradient [ZS 3.3, Stage 2: the
 * main attention switches to top-k sparse and every parameter trains]: the
 * backward of dsa_sparse_mla over each query's selection.  Given the forward's
 * out [T, H, Dv] and lse [T, H] (natural log) and dout = dL/dout [T, H, Dv],
 * with P = exp(sm_scale q . c(s) - lse) over the selected rows c(s):
 *   dS[h, s] = P (dout[h] . c(s)[0:Dv] - sum_d dout[h,d] out[h,d])
 *   dq[t, h, :] = sm_scale sum_s dS[h, s] c(s)                       [T, H, D] fp32
 *   the cache row of token s gets sm_scale sum_h dS[h, s] q[t, h, :] plus
 *   sum_h P[h, s] dout[t, h, :] (its first Dv entries), summed over every
 *   query that selected s                           dkv: latent cache layout, fp32
 * The rows of positions 0..max_ctx-1 of sequence 0 are written (0 where no
 * query selected the token); other rows are left as they are.  The selection
 * has no gradient.  probs, if not NULL, receives the Stage-2 target of the
 * indexer, the attention weights over the selection averaged over the heads
 * ([T, k] fp32, 0 at absent entries).  Entries of topk_idx outside
 * 0..q_pos[t] are absent; a query must not select a position twice.
 * bf16 operands (P and sm_scale dS rounded to bf16 as MFMA operands), fp32
 * accumulation; each query's contribution to a cache row is rounded to bf16
 * once before the token sums, which run in fp32 in ascending query order, so
 * the result is deterministic.  Supported: prefill (training runs over whole sequences),
 * bf16 H = 128, D = 576, Dv = 512, k a multiple of 16.
 * Workspace: dsa_workspace_size(DSA_OP_SPARSE_MLA_BACKWARD, ...). */
int dsa_sparse_mla_backward(const dsa_seqs *seqs, const dsa_dims *dims, float sm_scale, const void *q,
                            const void *kv_cache, const int32_t *topk_idx, const void *out, const float *lse,
                            const void *dout, float *dq, float *dkv, float *probs, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* Stage 2 of training, the indexer's loss on the selected subset [ZS 3.3,
 * Stage 2: the indexer keeps learning from a loss on S_t].  Per query,
 *   loss[t] = KL(p_t || softmax over S_t of I(t, .))
 * with p_t = probs[t, :] (e.g. from dsa_sparse_mla_backward) over the entries
 * of topk_idx[t, :] that lie in 0..q_pos[t].  scores [T, ld] holds I on entry
 * and dL/dI on return: softmax_S(I) - p at the selected positions, 0 at every
 * other position < ld (feed it to dsa_indexer_backward).  fp32;
 * deterministic.  No workspace. */
int dsa_sparse_indexer_kl(const dsa_seqs *seqs, float *scores, int64_t ld, const int32_t *topk_idx, int32_t k,
                          const float *probs, float *loss, hipStream_t stream);

/* Upstream of step 1: per-row fp8 quantisation for an indexer that "runs in
 * FP8" [ZS 3.1; BT (1)].  The pages fix neither scale nor rounding; the
 * reading taken: for each row r of src [rows, len] (DSA_BF16 or DSA_F32),
 *   scale[r]   = max_i |src[r,i]| / 448   (1 when the row is all zeros),
 *   dst[r, i]  = e4m3fn code of clamp(src[r,i] / scale[r], -448, 448),
 *                rounded to nearest, ties to even,
 * both fp32 IEEE operations.  scale[r] is stored scale_repeat times, at
 * scale[r * scale_repeat + j], j < scale_repeat: quantising indexer queries
 * with one scale per token gives len = H_I * d_I, scale_repeat = H_I (the
 * q_scale [T, H_I] layout); keys take len = d_I, scale_repeat = 1.
 * dst [rows, len] bytes, scale [rows * scale_repeat] fp32, both owned by the
 * caller.  src must be finite.  Supported: len % 4 == 0, len <= 65536,
 * scale_repeat <= 1024.  No workspace. */
int dsa_quantize_fp8(int64_t rows, int32_t len, int32_t src_dtype, const void *src, void *dst,
                     float *scale, int32_t scale_repeat, hipStream_t stream);

/* Append the new index key of every query token to an e4m3fn key cache
 * [ZS 3.1 "runs in FP8"; the decode step upstream of the indexer].  Token t
 * belongs to sequence t (decode) or 0 (prefill) at position q_pos[t]; its key
 * k_new[t, 0..index_dim) (DSA_BF16 or DSA_F32, layout [T, index_dim]) is
 * quantised as by dsa_quantize_fp8 (one scale per key) and written with its
 * scale to that position's slot of k_cache / k_scale (the layouts of
 * dsa_index_scores; through the block table when paged).  A token whose
 * position is negative, past the contiguous slots or the table's columns, or
 * in a block outside the pool is skipped.  Tokens must name distinct slots.
 * Supported: index_dim % 4 == 0, index_dim <= 2048.  No workspace. */
int dsa_append_index_keys(const dsa_seqs *seqs, int32_t index_dim, int32_t src_dtype, const void *k_new,
                          void *k_cache, float *k_scale, hipStream_t stream);

/* Measurement aid, not a step of the method: streams `bytes` of device memory
 * at `src` with the decode indexer's read shape and no arithmetic, so that its
 * duration gives the HBM read rate that shape can reach.  One 256-thread
 * workgroup per 512 KB (524288 B) chunk; its four waves read the chunk's 8 KB
 * tiles w, w+4, ... with two tiles in flight and 16-byte streaming
 * (nontemporal) loads, as the indexer does.  `flags`: DSA_READ_PAGED reads the
 * buffer as 16 KB (64-key) blocks scattered over it: block b comes from
 * physical block (b * 0x9E3779B1) mod (bytes / 16384), which must then be a
 * power of two; DSA_READ_CACHED uses loads with the default cache policy
 * instead of streaming ones.  Each wave writes the XOR of every 32-bit word it
 * read to sink[chunk * 4 + wave] (bytes / 131072 entries, owned by the
 * caller), so the reads are observable.  src must be 16-byte aligned; bytes a
 * positive multiple of 524288.  Errors: DSA_ERR_INVALID_ARG (null pointers,
 * misaligned src, bytes <= 0, unknown flags), DSA_ERR_UNSUPPORTED (other
 * sizes).  No workspace. */
enum { DSA_READ_PAGED = 1, DSA_READ_CACHED = 2 };
int dsa_read_ceiling(const void *src, int64_t bytes, int32_t flags, uint32_t *sink, hipStream_t stream);

/* Static string naming a dsa_status value. */
const char *dsa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */

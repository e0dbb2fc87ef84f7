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

}  // namespace

hipError_t launch_indexer_kl(const KlArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_kl_rows_kernel, dim3(a.rows), dim3(kKlThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

// Lightning indexer: pieces shared by the decode and prefill tilings
// ("DeepSeek V3.2: How Far Can Open Models Go If You Actually Try?",
// section 3.1, indexer equation).
#pragma once
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kHeads = 64;
constexpr int kDim = 128;

// ------------------------------------------------------------------ helpers

template <int DT>
struct IdxTraits;

// bf16: 8 k-steps of 16; lane group g holds d = 64 g + 8 ks + [0, 8).
template <>
struct IdxTraits<DSA_BF16> {
  static constexpr int kSteps = 8;
  static constexpr int kRowBytes = kDim * 2;
  typedef bf16x8 Op;
  __device__ static Op load(const uint8_t *row, int g, int ks) {
    return as_bf16x8(ld16(row + g * 128 + ks * 16));
  }
  __device__ static f32x16 mma(Op a, Op b, f32x16 c) { return mfma32_bf16(a, b, c); }
};

// e4m3fn: 2 k-steps of 64; lane group g holds d = 64 g + 32 ks + [0, 32).
template <>
struct IdxTraits<DSA_FP8_E4M3FN> {
  static constexpr int kSteps = 2;
  static constexpr int kRowBytes = kDim;
  typedef i32x8 Op;
  __device__ static Op load(const uint8_t *row, int g, int ks) {
    const uint8_t *p = row + g * 64 + ks * 32;
    uint4 lo = ld16(p), hi = ld16(p + 16);
    Op o;
    o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
    o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
    return o;
  }
  __device__ static f32x16 mma(Op a, Op b, f32x16 c) { return mfma32_fp8(a, b, c); }
};

// Weight of accumulator element v of head block hb for lane group g.
__device__ __forceinline__ int acc_head(int hb, int v, int g) { return hb * 32 + 8 * (v >> 2) + 4 * g + (v & 3); }

template <int DT>
__device__ __forceinline__ void load_query(const IndexerArgs &a, int t, int col, int g,
                                           typename IdxTraits<DT>::Op (&qa)[2][IdxTraits<DT>::kSteps],
                                           float (&wt)[2][16]) {
  typedef IdxTraits<DT> Tr;
  const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q_idx) + (long long)t * kHeads * Tr::kRowBytes;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int ks = 0; ks < Tr::kSteps; ++ks) qa[hb][ks] = Tr::load(qrow + (hb * 32 + col) * Tr::kRowBytes, g, ks);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int h = acc_head(hb, v, g);
      float wv = a.w[(long long)t * kHeads + h];
      if (DT == DSA_FP8_E4M3FN) wv *= a.q_scale[(long long)t * kHeads + h];
      wt[hb][v] = wv;
    }
}

// ReLU-weighted sum, for the key in column l%32, of the heads whose
// accumulator rows this half-wave holds (the other half-wave holds the rest).
__device__ __forceinline__ float head_partial(const f32x16 &c0, const f32x16 &c1, const float (&wt)[2][16]) {
  // ReLU as an integer max on the float's bits: non-negative floats are
  // non-negative integers, negative floats (and -0.0) negative ones.
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    p0 = fmaf(wt[0][v], __int_as_float(max(__float_as_int(c0[v]), 0)), p0);
    p1 = fmaf(wt[1][v], __int_as_float(max(__float_as_int(c1[v]), 0)), p1);
  }
  return p0 + p1;
}

// The full head sum of the two 32-head accumulator blocks for the key in
// column l%32; the result is valid in every lane.
__device__ __forceinline__ float head_reduce(const f32x16 &c0, const f32x16 &c1, const float (&wt)[2][16]) {
  const float p = head_partial(c0, c1, wt);
  return p + shfl_xor(p, 32);
}

// Full head sums of two 32-key groups from their half-wave partials: lanes
// 0..31 get key l of group 0, lanes 32..63 key l-32 of group 1 (one lane swap
// exchanges the halves the other lanes need).
__device__ __forceinline__ float pair_head_total(float part0, float part1) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1), false, false);
  return __uint_as_float(x[0]) + __uint_as_float(x[1]);
}

}  // namespace
}  // namespace dsa

// fp8 quantisation upstream of the indexer, which runs in FP8 ("DeepSeek V3.2:
// How Far Can Open Models Go If You Actually Try?", section 3.1; baseten.co
// "DeepSeek-V3.2", section (1)): per-row OCP e4m3fn codes with an fp32 scale,
// and the append of each new token's index key into the (paged) key cache.
//
// Per row: scale = amax|x| / 448 (1 for an all-zero row), code = RNE(clamp(x /
// scale, -448, 448)), both fp32 IEEE operations; the rounding to e4m3fn is the
// gfx950 converter (round to nearest, ties to even).  The rows are read twice
// (the maximum, then the codes); the second pass hits the cache.
#include "kernels.h"

namespace dsa {
namespace {

constexpr float kE4M3Max = 448.f;

// Four consecutive source values as fp32 (exact for bf16).
__device__ __forceinline__ void load4(const void *src, int dtype, long long e, float (&v)[4]) {
  if (dtype == DSA_BF16) {
    const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(src) + e);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(src) + e);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

// Codes of four values at one scale, packed little-endian into a word.
__device__ __forceinline__ uint32_t encode4(const float (&v)[4], float scale) {
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(v[i] / scale, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  return (uint32_t)w;
}

// Quantise one row of `len` values (len % 4 == 0) with G threads (G = 64: one
// wave; G = 256: four waves, `red` holds their partial maxima).  Returns the
// row's scale in every thread of the group.
template <int G>
__device__ __forceinline__ float quantize_row(const void *src, int dtype, long long e0, int len, uint8_t *dst,
                                              float *red) {
  const int tid = threadIdx.x % G;
  float amax = 0.f;
  for (int i = tid * 4; i < len; i += G * 4) {
    float v[4];
    load4(src, dtype, e0 + i, v);
#pragma unroll
    for (int c = 0; c < 4; ++c) amax = fmaxf(amax, fabsf(v[c]));
  }
  amax = wave_max(amax);
  if (G > 64) {
    const int wv = tid >> 6;
    if ((tid & 63) == 0) red[wv] = amax;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G / 64; ++j) amax = fmaxf(amax, red[j]);
  }
  const float scale = amax > 0.f ? amax / kE4M3Max : 1.f;
  for (int i = tid * 4; i < len; i += G * 4) {
    float v[4];
    load4(src, dtype, e0 + i, v);
    *reinterpret_cast<uint32_t *>(dst + i) = encode4(v, scale);
  }
  return scale;
}

// Rows of len <= 2048: one wave per row, four rows per workgroup.
__global__ __launch_bounds__(256) void fp8_quantize_wave_kernel(QuantArgs a) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  const float scale = quantize_row<64>(a.src, a.src_dtype, r * a.len, a.len, a.dst + r * a.len, nullptr);
  for (int j = lane_id(); j < a.scale_repeat; j += 64) a.scale[r * a.scale_repeat + j] = scale;
}

// Longer rows: one workgroup per row.
__global__ __launch_bounds__(256) void fp8_quantize_block_kernel(QuantArgs a) {
  __shared__ float red[4];
  const long long r = blockIdx.x;
  const float scale = quantize_row<256>(a.src, a.src_dtype, r * a.len, a.len, a.dst + r * a.len, red);
  for (int j = threadIdx.x; j < a.scale_repeat; j += 256) a.scale[r * a.scale_repeat + j] = scale;
}

// One wave per new token: quantise its key and store it at its position's slot.
__global__ __launch_bounds__(256) void fp8_append_kernel(AppendArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.sv.num_q) return;
  const int b = a.sv.seq_of(t);
  const int pos = a.sv.q_pos[t];
  if (pos < 0) return;
  long long slot;
  if (a.sv.block_table == nullptr) {
    if (pos >= a.sv.max_seq_len) return;
    slot = (long long)b * a.sv.max_seq_len + pos;
  } else {
    if ((pos >> 6) >= a.sv.max_blocks) return;
    slot = a.sv.slot(b, pos);
    if (slot < 0) return;
  }
  const float scale = quantize_row<64>(a.src, a.src_dtype, (long long)t * a.len, a.len,
                                       a.cache + slot * a.len, nullptr);
  if (lane_id() == 0) a.scale[slot] = scale;
}

}  // namespace

hipError_t launch_fp8_quantize(const QuantArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.len <= 2048)
    hipLaunchKernelGGL(fp8_quantize_wave_kernel, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(fp8_quantize_block_kernel, dim3((unsigned)a.rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fp8_append(const AppendArgs &a, hipStream_t st) {
  if (a.sv.num_q <= 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_append_kernel, dim3((unsigned)((a.sv.num_q + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

// Sparse MLA in MQA mode over the selected latent rows ("DeepSeek V3.2: How
// Far Can Open Models Go If You Actually Try?", section 3.1, selection-then-
// attention equation and the MQA-mode paragraph: one shared latent row per
// token, every head reads the same fetched rows; "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", Novel Architectural Elements).
//
// bf16 path (H = 128, D = 576, Dv = 512): a workgroup of 8 waves owns one
// query (and one split of its selected rows).  Each 32-row tile is gathered
// from HBM once into LDS, in two layouts: row-major for the logits and
// transposed (value dim major) for the value product, so every head of the
// query is served from the single fetch.  Wave w owns heads 16w..16w+15:
//   S^T[rows, heads] = C_tile[rows, 576] . Q^T          (16x16x32 bf16 MFMA)
//   online softmax in fp32 (base-2 exponent, running max and sum per head)
//   O^T[dims, heads] += V^T[dims, rows] . P^T[rows, heads]
// With several splits per query the unnormalised partials (acc, max, sum)
// are merged by a second kernel in a fixed order.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kH = 128, kD = 576, kDv = 512;
constexpr int kR = 32;              // latent rows per tile
constexpr int kRowStride = 1168;    // bytes per row in the row-major tile (1152 + 16 pad)
constexpr int kVtStride = 80;       // bytes per value dim in the transposed tile (64 + 16 pad)
constexpr int kChunks = kD * 2 / 16;   // 72 16-byte chunks per row
constexpr int kVChunks = kDv * 2 / 16; // 64 of them hold value dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int split_len(int k, int n_split) {
  int len = (k + n_split - 1) / n_split;
  return (len + kR - 1) / kR * kR;
}

__global__ __launch_bounds__(512) void mla_bf16_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t rm[kR * kRowStride];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kDv * kVtStride];
  __shared__ int rowok[kR];

  const int sp = blockIdx.x;
  const int r = blockIdx.y;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const int32_t *irow = a.idx + (long long)r * a.k;
  const int len = split_len(a.k, a.n_split);
  const int i0 = sp * len;
  const int i1 = i0 + len < a.k ? i0 + len : a.k;

  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int h = wv * 16 + col;

  // Q^T operand for this wave's 16 heads: lane holds head h, dims 32 ks + 8 g + [0, 8).
  const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q) + ((long long)t * kH + h) * (kD * 2);
  bf16x8 qb[kD / 32];
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks) qb[ks] = as_bf16x8(ld16(qrow + ks * 64 + g * 16));

  f32x4 acc[kDv / 16];
#pragma unroll
  for (int db = 0; db < kDv / 16; ++db) acc[db] = zero_vec<f32x4>();
  float m_run = neg_inf();
  float l_run = 0.f;
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t *kv = reinterpret_cast<const uint8_t *>(a.kv);

  for (int i = i0; i < i1; i += kR) {
    // ---- gather the tile: 32 rows x 72 chunks over 512 threads
    for (int c = threadIdx.x; c < kR * kChunks; c += 512) {
      const int row = c / kChunks, ch = c - row * kChunks;
      const int ii = i + row;
      const int s = ii < i1 ? irow[ii] : -1;
      const long long sl = (s >= 0 && s < n) ? a.sv.slot(b, s) : -1;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (sl >= 0) v = ld16(kv + sl * (kD * 2) + ch * 16);
      *reinterpret_cast<uint4 *>(rm + row * kRowStride + ch * 16) = v;
      if (ch < kVChunks) {
        const uint16_t e[8] = {(uint16_t)(v.x & 0xffff), (uint16_t)(v.x >> 16), (uint16_t)(v.y & 0xffff),
                               (uint16_t)(v.y >> 16),    (uint16_t)(v.z & 0xffff), (uint16_t)(v.z >> 16),
                               (uint16_t)(v.w & 0xffff), (uint16_t)(v.w >> 16)};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint16_t *>(vt + (ch * 8 + j) * kVtStride + row * 2) = e[j];
      }
      if (ch == 0) rowok[row] = sl >= 0;
    }
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int j = 0; j < kR; ++j) any |= rowok[j] != 0;
    if (any) {
      // ---- logits S^T for 32 rows x this wave's 16 heads
      f32x4 st[2] = {zero_vec<f32x4>(), zero_vec<f32x4>()};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const uint8_t *arow = rm + (rb * 16 + col) * kRowStride + g * 16;
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks)
          st[rb] = mfma16_bf16(as_bf16x8(*reinterpret_cast<const uint4 *>(arow + ks * 64)), qb[ks], st[rb]);
      }
      // ---- online softmax (base 2), per head = per lane column
      float z[2][4];
      float mx = neg_inf();
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = rb * 16 + 4 * g + v;
          z[rb][v] = rowok[row] ? st[rb][v] * scale2 : neg_inf();
          mx = fmaxf(mx, z[rb][v]);
        }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == neg_inf() ? 0.f : exp2f(m_run - m_new);
      float p[2][4];
      float psum = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[rb][v] = z[rb][v] == neg_inf() ? 0.f : exp2f(z[rb][v] - m_new);
          psum += p[rb][v];
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[db][v] *= alpha;
      }
      bf16x8 pb;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pb[v] = (__bf16)p[0][v];
        pb[4 + v] = (__bf16)p[1][v];
      }
      // ---- O^T += V^T . P^T: k-slots 0..3 = tile rows 4g.., 4..7 = rows 16 + 4g..
#pragma unroll
      for (int db = 0; db < kDv / 16; ++db) {
        const uint8_t *vrow = vt + (db * 16 + col) * kVtStride;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + g * 8);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 32 + g * 8);
        const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        acc[db] = mfma16_bf16(as_bf16x8(av), pb, acc[db]);
      }
    }
    __syncthreads();
  }

  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  if (a.n_split == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t *orow = reinterpret_cast<uint16_t *>(a.out) + ((long long)t * kH + h) * kDv;
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
      const int d = db * 16 + 4 * g;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc[db][0] * inv) | ((uint32_t)f32_to_bf16(acc[db][1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc[db][2] * inv) | ((uint32_t)f32_to_bf16(acc[db][3] * inv) << 16);
      *reinterpret_cast<uint2 *>(orow + d) = pk;
    }
    if (a.lse != nullptr && g == 0)
      a.lse[(long long)t * kH + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : neg_inf();
  } else {
    float *prow = a.part + (((long long)r * a.n_split + sp) * kH + h) * (kDv + 4);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
      const int d = db * 16 + 4 * g;
      *reinterpret_cast<float4 *>(prow + d) = make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
    }
    if (g == 0) {
      prow[kDv] = m_run;
      prow[kDv + 1] = l_tot;
    }
  }
}

// Merge the split partials of one (query, head) in split order.
template <bool BF16>
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaArgs a) {
  const int h = blockIdx.x, r = blockIdx.y;
  const int t = a.q_begin + r;
  const int H = a.H, Dv = a.Dv;
  const long long stride = (long long)H * (Dv + 4);
  const float *base = a.part + ((long long)r * a.n_split * H + h) * (Dv + 4);
  float M = neg_inf();
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, base[s * stride + Dv]);
  float L = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float ms = base[s * stride + Dv];
    if (ms != neg_inf()) L += exp2f(ms - M) * base[s * stride + Dv + 1];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = threadIdx.x * 4; d < Dv; d += 128 * 4) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < a.n_split; ++s) {
      const float ms = base[s * stride + Dv];
      if (ms == neg_inf()) continue;
      const float wgt = exp2f(ms - M);
      const float4 v = *reinterpret_cast<const float4 *>(base + s * stride + d);
      o.x = fmaf(wgt, v.x, o.x);
      o.y = fmaf(wgt, v.y, o.y);
      o.z = fmaf(wgt, v.z, o.z);
      o.w = fmaf(wgt, v.w, o.w);
    }
    const long long ob = ((long long)t * H + h) * Dv + d;
    if (BF16) {
      uint16_t *out = reinterpret_cast<uint16_t *>(a.out);
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(o.x * inv) | ((uint32_t)f32_to_bf16(o.y * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(o.z * inv) | ((uint32_t)f32_to_bf16(o.w * inv) << 16);
      *reinterpret_cast<uint2 *>(out + ob) = pk;
    } else {
      float *out = reinterpret_cast<float *>(a.out);
      *reinterpret_cast<float4 *>(out + ob) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    }
  }
  if (threadIdx.x == 0 && a.lse != nullptr)
    a.lse[(long long)t * H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : neg_inf();
}

// fp32, small shapes (H <= 16, D <= 128, k <= 1024): one workgroup per query,
// logits in LDS, exact two-pass softmax.
__global__ __launch_bounds__(256) void mla_f32_kernel(MlaArgs a) {
  extern __shared__ __attribute__((aligned(8))) float sm[];
  const int H = a.H, D = a.D, Dv = a.Dv, K = a.k;
  long long *slots = reinterpret_cast<long long *>(sm);   // [K]
  float *qs = sm + 2 * K;         // [H, D]
  float *z = qs + H * D;          // [H, K]
  float *stat = z + H * K;        // [H, 2]
  const int r = blockIdx.x;
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const float *q = reinterpret_cast<const float *>(a.q) + (long long)t * H * D;
  const float *kv = reinterpret_cast<const float *>(a.kv);
  const int32_t *irow = a.idx + (long long)r * K;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) qs[i] = q[i];
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    const int s = irow[j];
    slots[j] = (s >= 0 && s < n) ? a.sv.slot(b, s) : -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < H * K; i += blockDim.x) {
    const int hh = i / K, j = i - hh * K;
    float zz = neg_inf();
    if (slots[j] >= 0) {
      const float *row = kv + slots[j] * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[hh * D + d], row[d], dot);
      zz = dot * a.sm_scale;
    }
    z[i] = zz;
  }
  __syncthreads();
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  for (int hh = wv; hh < H; hh += blockDim.x / 64) {
    float mx = neg_inf();
    for (int j = lane; j < K; j += 64) mx = fmaxf(mx, z[hh * K + j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < K; j += 64) {
      const float zz = z[hh * K + j];
      const float p = zz == neg_inf() ? 0.f : expf(zz - mx);
      z[hh * K + j] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      stat[2 * hh] = mx;
      stat[2 * hh + 1] = sum;
    }
  }
  __syncthreads();
  float *out = reinterpret_cast<float *>(a.out) + (long long)t * H * Dv;
  for (int i = threadIdx.x; i < H * Dv; i += blockDim.x) {
    const int hh = i / Dv, d = i - hh * Dv;
    float o = 0.f;
    for (int j = 0; j < K; ++j)
      if (slots[j] >= 0) o = fmaf(z[hh * K + j], kv[slots[j] * D + d], o);
    const float l = stat[2 * hh + 1];
    out[i] = l > 0.f ? o / l : 0.f;
  }
  if (a.lse != nullptr)
    for (int hh = threadIdx.x; hh < H; hh += blockDim.x) {
      const float l = stat[2 * hh + 1];
      a.lse[(long long)t * H + hh] = l > 0.f ? stat[2 * hh] + logf(l) : neg_inf();
    }
}

}  // namespace

int mla_splits(int rows, int k) {
  int s = (256 + rows - 1) / rows;
  int cap = (k + 2 * kR - 1) / (2 * kR);
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

size_t mla_f32_lds(int H, int D, int k) {
  return (size_t)(2 * k + H * D + H * k + 2 * H) * sizeof(float);
}

hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.dtype == DSA_F32) {
    const size_t lds = mla_f32_lds(a.H, a.D, a.k);
    if (lds > 65536) hipFuncSetAttribute((const void *)mla_f32_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(mla_f32_kernel, dim3(a.rows), dim3(256), lds, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(mla_bf16_kernel, dim3(a.n_split, a.rows), dim3(512), 0, st, a);
  if (a.n_split > 1) hipLaunchKernelGGL(mla_combine_kernel<true>, dim3(a.H, a.rows), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

// Sparse MLA in MQA mode over the selected latent rows ("DeepSeek V3.2: How
// Far Can Open Models Go If You Actually Try?", section 3.1, selection-then-
// attention equation and the MQA-mode paragraph: one shared latent row per
// token, every head reads the same fetched rows; "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", Novel Architectural Elements).
//
// bf16 path (H = 128, D = 576, Dv = 512): a workgroup of 8 waves owns one
// query (and one split of its selected rows).  Each 32-row tile is gathered
// from HBM once, straight into LDS by the direct-to-LDS loads of gfx950 (no
// staging registers), double-buffered so the next tile streams in while the
// current one is multiplied; every head of the query is served from that one
// fetch.  Wave w owns heads 16w..16w+15 (two waves per SIMD, so the MFMA
// accumulators of one stay in architectural registers):
//   S^T[rows, heads] = C_tile[rows, 576] . Q^T          (16x16x32 bf16 MFMA)
//   online softmax in fp32 (base-2 exponent, running max and sum per head)
//   O^T[dims, heads] += V^T[dims, rows] . P^T[rows, heads]
// V^T operands come from the row-major tile through the LDS transpose read
// (ds_read_b64_tr_b16), so the tile is stored once.  With several splits per
// query the unnormalised partials (acc, max, sum) are merged by a second
// kernel in a fixed order.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kH = 128, kD = 576, kDv = 512;
constexpr int kHB = 1;                        // 16-head blocks per wave
constexpr int kWaves = kH / (16 * kHB);       // 8 waves, one head block each
constexpr int kThreads = kWaves * 64;
constexpr int kR = 32;                        // latent rows per tile
constexpr int kRowChunks = kD * 2 / 16 + 1;   // 72 data chunks + 1 pad: row stride 1168 B
constexpr int kRowStride = kRowChunks * 16;
constexpr int kTileChunks = kR * kRowChunks;  // 2336
constexpr int kWaveLoads = (kTileChunks + kThreads - 1) / kThreads;  // 10 direct loads per wave
constexpr int kKs = kD / 32;                  // 18 k-steps of the logits
constexpr int kDb = kDv / 16;                 // 32 value-dim blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplitRows = 2048;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int split_len(int k, int n_split) {
  int len = (k + n_split - 1) / n_split;
  return (len + kR - 1) / kR * kR;
}

// Block order: the splits of one query are placed on the same XCD (workgroups
// are dealt to the 8 XCDs round-robin by linear id), so its query rows are
// fetched from HBM once and then served by that XCD's L2.
__device__ __forceinline__ void mla_block(const MlaArgs &a, int &sp, int &r) {
  const int total = a.n_split * a.rows;
  int v = blockIdx.x;
  if ((total & 7) == 0) v = (v & 7) * (total >> 3) + (v >> 3);
  r = v / a.n_split;
  sp = v - r * a.n_split;
}

// One 16-byte direct-to-LDS load: lane l's 16 bytes land at lds_dst + 16 l.
// It returns nothing in registers.  It is written out here because the
// compiler's wait insertion cannot tell the two tile buffers apart and would
// otherwise stall the consumer of one buffer on the loads still streaming into
// the other; the kernel waits for these loads itself (s_waitcnt vmcnt(0) and a
// barrier) before any wave reads the buffer they fill.
__device__ __forceinline__ void lds_dma16(const void *gsrc, const uint4 *lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gsrc)
               : "memory", "m0");
}

// Issue the direct-to-LDS gather of tile rows [j0, j0+32) of the split into
// `tile`: lane l of a load writes LDS bytes base + 16 l.  Chunk position p
// holds (row p/73, chunk p%73); the pad chunk and absent rows load a valid row
// (`fallback`) so every LDS byte the MFMAs read is finite; absent rows are
// masked in the softmax.
__device__ __forceinline__ void issue_tile(uint4 *tile, const uint8_t *kv, const int *slots, int j0, int jend,
                                           int fallback, int wv, int lane) {
  // Keep the per-lane chunk coordinates from being hoisted out of the tile loop
  // (they are cheap to recompute; holding them would cost registers).
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const int base = (j * kWaves + wv) * 64;
    const int p = base + lane;
    if (base < kTileChunks) {
      const int row = p / kRowChunks;
      const int ch = p - row * kRowChunks;
      int sl = (j0 + row < jend) ? slots[j0 + row] : -1;
      if (sl < 0) sl = fallback;
      const uint8_t *src = kv + (long long)sl * (kD * 2) + (ch < kRowChunks - 1 ? ch : 0) * 16;
      if (p < kTileChunks) lds_dma16(src, tile + base);
    }
  }
}

// Logits, online softmax and value product for one resident tile.
__device__ __forceinline__ void consume_tile(const uint8_t *tile, const int *slots, int j0, int jend,
                                             const bf16x8 (&qb)[kHB][kKs], f32x4 (&acc)[kHB][kDb],
                                             float (&m_run)[kHB], float (&l_run)[kHB], float scale2, int col,
                                             int g) {
  // ---- S^T for 32 rows x this wave's heads
  f32x4 st[2][kHB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) st[rb][hb] = zero_vec<f32x4>();
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4 *>(tile + (rb * 16 + col) * kRowStride + g * 16 + ks * 64));
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) st[rb][hb] = mfma16_bf16(a, qb[hb][ks], st[rb][hb]);
    }
  // ---- online softmax (base 2), one head per lane column and head block.
  // Row validity of the tile as a wave-uniform 32-bit mask (bit j: row j present).
  const int lane = lane_id();
  const uint32_t rowmask = (uint32_t)__ballot(lane < kR && j0 + lane < jend && slots[j0 + (lane & (kR - 1))] >= 0);
  bool ok[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) ok[rb][v] = (rowmask >> (rb * 16 + 4 * g + v)) & 1u;
  bf16x8 pb[kHB];
  bool rescale = false;
  float alpha[kHB];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    float mx = neg_inf();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        st[rb][hb][v] = ok[rb][v] ? st[rb][hb][v] * scale2 : neg_inf();
        mx = fmaxf(mx, st[rb][hb][v]);
      }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run[hb], mx);
    alpha[hb] = m_run[hb] == neg_inf() ? 0.f : exp2f(m_run[hb] - m_new);
    float psum = 0.f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float pv = st[rb][hb][v] == neg_inf() ? 0.f : exp2f(st[rb][hb][v] - m_new);
        psum += pv;
        pb[hb][rb * 4 + v] = (__bf16)pv;
      }
    l_run[hb] = l_run[hb] * alpha[hb] + psum;
    m_run[hb] = m_new;
    rescale |= alpha[hb] != 1.f;
  }
  if (__any(rescale)) {
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
      for (int db = 0; db < kDb; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[hb][db][v] *= alpha[hb];
  }
  // ---- O^T += V^T . P^T.  k-slots 0..3 = tile rows 4g+e, 4..7 = rows 16+4g+e (e = 0..3),
  // matching the rows this lane holds in P^T.  Lane 4e+c of group g points the
  // transpose read at row 4g+e (resp. 16+4g+e), dims d0+4c..d0+4c+3, and receives
  // V[row_e][d0 + (lane%16)] for e = 0..3.
  const int e = col >> 2, c = col & 3;
  const uint8_t *v0 = tile + (4 * g + e) * kRowStride + c * 8;
  const uint8_t *v1 = v0 + 16 * kRowStride;
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(v0 + db * 32));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(v1 + db * 32));
    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) acc[hb][db] = mfma16_bf16(av, pb[hb], acc[hb][db]);
  }
}

__global__ __launch_bounds__(kThreads) void mla_bf16_kernel(MlaArgs a) {
  __shared__ uint4 tile0[kTileChunks];
  __shared__ uint4 tile1[kTileChunks];
  __shared__ int slots[kMaxSplitRows];
  __shared__ int fallback;

  int sp, r;
  mla_block(a, sp, r);
  const int t = a.q_begin + r;
  const int n = a.sv.candidates(t);
  const int b = a.sv.seq_of(t);
  const int32_t *irow = a.idx + (long long)r * a.k;
  const int len = split_len(a.k, a.n_split);
  const int i0 = sp * len;
  const int i1 = i0 + len < a.k ? i0 + len : a.k;
  const int rows = i1 > i0 ? i1 - i0 : 0;

  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;

  if (threadIdx.x == 0) fallback = -1;
  __syncthreads();
  // Slots of this split's rows (-1: absent), so the gather depends on LDS only.
  for (int j = threadIdx.x; j < rows; j += kThreads) {
    const int s = irow[i0 + j];
    const int sl = (s >= 0 && s < n) ? (int)a.sv.slot(b, s) : -1;
    slots[j] = sl;
    if (sl >= 0) atomicMax(&fallback, sl);
  }

  // Q^T operands for this wave's heads: lane holds head 16 (kHB wv + hb) + col,
  // dims 32 ks + 8 g + [0, 8).
  bf16x8 qb[kHB][kKs];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    const uint8_t *qrow =
        reinterpret_cast<const uint8_t *>(a.q) + ((long long)t * kH + (wv * kHB + hb) * 16 + col) * (kD * 2);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qb[hb][ks] = as_bf16x8(ld16(qrow + ks * 64 + g * 16));
  }

  f32x4 acc[kHB][kDb];
  float m_run[kHB], l_run[kHB];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
#pragma unroll
    for (int db = 0; db < kDb; ++db) acc[hb][db] = zero_vec<f32x4>();
    m_run[hb] = neg_inf();
    l_run[hb] = 0.f;
  }
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t *kv = reinterpret_cast<const uint8_t *>(a.kv);
  __syncthreads();
  const int fb = fallback;

  if (fb >= 0) {
    const int ntiles = (rows + kR - 1) / kR;
    issue_tile(tile0, kv, slots, 0, rows, fb, wv, lane);
    for (int tt = 0; tt < ntiles; ++tt) {
      // tile tt (in flight) lands; every wave is done with the other buffer
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      uint4 *cur = (tt & 1) ? tile1 : tile0;
      uint4 *nxt = (tt & 1) ? tile0 : tile1;
      if (tt + 1 < ntiles) issue_tile(nxt, kv, slots, (tt + 1) * kR, rows, fb, wv, lane);
      consume_tile(reinterpret_cast<const uint8_t *>(cur), slots, tt * kR, rows, qb, acc, m_run, l_run, scale2,
                   col, g);
    }
  }

#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    const int h = (wv * kHB + hb) * 16 + col;
    float l_tot = l_run[hb] + shfl_xor(l_run[hb], 16);
    l_tot += shfl_xor(l_tot, 32);
    if (a.n_split == 1) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t *orow = reinterpret_cast<uint16_t *>(a.out) + ((long long)t * kH + h) * kDv;
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int d = db * 16 + 4 * g;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(acc[hb][db][0] * inv) | ((uint32_t)f32_to_bf16(acc[hb][db][1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc[hb][db][2] * inv) | ((uint32_t)f32_to_bf16(acc[hb][db][3] * inv) << 16);
        *reinterpret_cast<uint2 *>(orow + d) = pk;
      }
      if (a.lse != nullptr && g == 0)
        a.lse[(long long)t * kH + h] = l_tot > 0.f ? (m_run[hb] + __log2f(l_tot)) * kLn2 : neg_inf();
    } else {
      float *prow = a.part + (((long long)r * a.n_split + sp) * kH + h) * (kDv + 4);
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int d = db * 16 + 4 * g;
        *reinterpret_cast<float4 *>(prow + d) =
            make_float4(acc[hb][db][0], acc[hb][db][1], acc[hb][db][2], acc[hb][db][3]);
      }
      if (g == 0) {
        prow[kDv] = m_run[hb];
        prow[kDv + 1] = l_tot;
      }
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
  hipLaunchKernelGGL(mla_bf16_kernel, dim3(a.n_split * a.rows), dim3(kThreads), 0, st, a);
  if (a.n_split > 1) hipLaunchKernelGGL(mla_combine_kernel<true>, dim3(a.H, a.rows), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

// Device-side building blocks shared by the DSA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- direct-to-LDS tiles

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One 16-byte direct-to-LDS load: lane l's 16 bytes land at LDS address
// m0 + 16 l (m0 wave-uniform); inactive lanes write nothing.  It returns
// nothing in registers.  It is written out here because the compiler's wait
// insertion cannot tell tile buffers apart and would otherwise stall the
// consumer of one buffer on the loads still streaming into another; a kernel
// using it waits for these loads itself (s_waitcnt vmcnt and a barrier) before
// any wave reads the buffer they fill.  Vector-memory loads complete in issue
// order, so vmcnt(n) means "all but this wave's n most recent loads landed"
// (stores issued in between can only make such a wait stricter).
__device__ __forceinline__ void lds_dma16(const void *gsrc, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gsrc)
               : "memory", "m0");
}

// The same load with the streaming (nontemporal) cache policy, for rows that
// are read once.
__device__ __forceinline__ void lds_dma16_stream(const void *gsrc, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(m0), "v"(gsrc)
               : "memory", "m0");
}

// The 4-byte form: lane l's 4 bytes land at LDS address m0 + 4 l.
__device__ __forceinline__ void lds_dma4(const void *gsrc, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(m0), "v"(gsrc)
               : "memory", "m0");
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm0 = 0x0F70;      // vector-memory count <= 0, the others free
__host__ __device__ constexpr int wait_vm(int n) { return 0x0F70 | n; }   // vmcnt <= n (n < 16)
constexpr int kWaitLgkm0 = 0xC07F;    // LDS / scalar counts <= 0, vector memory left in flight
constexpr int kWaitNone = 0xCF7F;     // every count at its maximum: no wait

// Buffer resources (raw, stride 0): the fourth descriptor word of the gfx9
// family (32-bit data format; the format does not affect untyped accesses),
// and an offset past any range used here, whose accesses the hardware's
// range check drops (stores) or returns as zero (loads).
constexpr int kBufferDword3 = 0x00020000;
constexpr uint32_t kBufferDrop = 0x80000000u;

// Raw buffer descriptor (stride 0) over `bytes` bytes from `base`; the values
// are wave-uniform and end up in scalar registers.
typedef int i32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4s buffer_desc(const void *base, int bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4s d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  d[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu));
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = kBufferDword3;
  return d;
}

// Buffer loads straight into LDS: lane i's 16 (or 4) bytes at voffset land at
// LDS address m0 + 16 i (4 i); lanes outside the descriptor's range write
// zeros.  Written as asm so that the compiler does not wait for them before
// every later LDS access (it cannot tell which LDS bytes they write): the
// caller waits on the vector-memory count itself, as for lds_dma16.
__device__ __forceinline__ void buffer_lds16(i32x4s d, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(d)
               : "memory", "m0");
}
__device__ __forceinline__ void buffer_lds4(i32x4s d, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(d)
               : "memory", "m0");
}

// Workgroup barrier without a memory fence: the fence of __syncthreads would
// also wait for the tile loads still streaming into the other buffers.  LDS
// reads are complete once their values are used, and the direct-to-LDS writes
// are covered by each wave's own s_waitcnt before it arrives here.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even, by the gfx950 converter
// (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 -> two bf16 in one 32-bit word (lo in bits 15:0), one converter op.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

// OCP e4m3fn byte -> fp32 via the gfx950 converter.
__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(int(byte), 0);
}

// Order-preserving unsigned key of an fp32 score: a > b  <=>  key(a) > key(b);
// -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xff800000u); }

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// v + v[lane ^ 32] in every lane, through the gfx950 half-wave swap (a VALU
// op; no LDS round trip).  Lanes below 32 add v[l] + v[l + 32], the others
// v[l - 32] + v[l]: the same sums as an exchange with lane ^ 32.
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// through the gfx950 row swaps (VALU ops; no LDS round trip).  The 16-lane swap
// exchanges odd rows of one operand with even rows of the other, so with both
// operands = v the pair holds (v[l], v[l ^ 16]) in every lane; the 32-lane swap
// then does the same across the halves.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return sum_xor32(__uint_as_float(a[0]) + __uint_as_float(a[1]));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (l >= d) v += o;
  }
  return v;
}

// ---------------------------------------------------------------- MFMA
//
// 32x32x16 bf16:  A lane l holds row l%32, 8 k-values of k-group l/32;
//                 B lane l holds column l%32, the same 8 k-values;
//                 C element v (0..15) of lane l: row 8*(v/4) + 4*(l/32) + v%4, column l%32.
// 16x16x32 bf16:  A lane l: row l%16, 8 k-values of k-group l/16; B likewise by column;
//                 C element v (0..3) of lane l: row 4*(l/16) + v, column l%16.
// 32x32x64 fp8:   A lane l: row l%32, 32 k-values of k-group l/32 (e4m3, byte-packed); B likewise.
// Because A and B map (lane, slot) to k identically, any fixed permutation of
// the reduction index applied to both operands leaves the product unchanged;
// the kernels use that to make each lane read contiguous bytes.

__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// e4m3 x e4m3 with unit block scales (E8M0 127 == 2^0).
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <typename V>
__device__ __forceinline__ V zero_vec() {
  V v;
#pragma unroll
  for (int i = 0; i < int(sizeof(V) / sizeof(v[0])); ++i) v[i] = 0;
  return v;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// 16-byte streaming load (the nontemporal cache policy: data read once).  On
// this part a stream of such loads reaches a higher HBM read rate than the same
// loads with the default policy (about 6.8 against 6.0 TB/s for the decode
// indexer's 8 KB tiles).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- geometry

struct SeqView {
  int mode;
  int num_seqs;
  int num_q;
  int max_ctx;
  const int32_t *q_pos;
  const int32_t *block_table;
  int max_blocks;
  int num_blocks;
  int block_size;
  long long max_seq_len;

  // Candidates of query t: positions 0..n-1, n = q_pos + 1 clamped to [0, max_ctx].
  __device__ __forceinline__ int candidates(int t) const {
    int p = q_pos[t];
    p = p < -1 ? -1 : p;
    p = p > max_ctx - 1 ? max_ctx - 1 : p;
    return p + 1;
  }
  __device__ __forceinline__ int seq_of(int t) const { return mode == DSA_DECODE ? t : 0; }

  // Slot (row index into a [slots, width] cache) of logical position s of
  // sequence b, or -1 when the position is absent (block outside the pool).
  __device__ __forceinline__ long long slot(int b, int s) const {
    if (block_table == nullptr) return (long long)b * max_seq_len + s;
    const int blk = block_table[(long long)b * max_blocks + (s >> 6)];
    if (blk < 0 || blk >= num_blocks) return -1;
    return (long long)blk * 64 + (s & 63);
  }
};

}  // namespace dsa

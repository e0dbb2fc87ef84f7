// Measurement aid, not a step of the method: the HBM read rate that the decode
// indexer's access shape can reach with no arithmetic at all.
//
// Each 256-thread workgroup streams one 512 KB chunk (2048 bf16 index keys of
// 256 B), its four waves taking the chunk's 8 KB tiles w, w + 4, ... with two
// tiles in flight in registers, 16-byte loads, eight per lane and tile -- the
// decode indexer's tiling (indexer_decode.hip).  With `paged`, the chunk's
// 16 KB blocks (64 keys) are scattered over the buffer as a paged key cache
// is: block b of the buffer's sequence of blocks is read from physical block
// (b * 0x9E3779B1) mod nblk, a bijection since nblk is a power of two and the
// multiplier odd.  The loads are streaming (nontemporal) loads as in the
// indexer; with `cached` they use the default cache policy instead, which
// shows what the streaming policy gains.  Every word read is folded into an
// XOR that the wave writes out, so no load is dead.
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kTileBytes = 8192;
constexpr int kTilesPerChunk = kReadCeilingChunk / kTileBytes;   // 64
constexpr int kWaveTiles = kTilesPerChunk / 4;                   // 16 per wave
constexpr int kLoads = kTileBytes / (64 * 16);                   // 8 per lane and tile

template <bool kPaged, bool kStream>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void read_ceiling_kernel(
    const uint8_t *src, long long nblk, uint32_t *sink) {
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto fetch = [&](int t, uint4 (&st)[kLoads]) {
    const long long g = (long long)blockIdx.x * kTilesPerChunk + t * 4 + wv;   // tile of the buffer
    const long long phys = kPaged ? ((((g >> 1) * 0x9E3779B1LL) & (nblk - 1)) << 1) | (g & 1) : g;
    const uint8_t *p = src + phys * kTileBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) st[i] = kStream ? ld16_stream(p + i * 1024) : ld16(p + i * 1024);
  };
  uint32_t acc = 0;
  auto fold = [&](const uint4 (&st)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) acc ^= st[i].x ^ st[i].y ^ st[i].z ^ st[i].w;
  };
  uint4 sa[kLoads], sb[kLoads];
  fetch(0, sb);
  fetch(1, sa);
  // fully unrolled, so the tiles past the last are skipped at compile time
#pragma unroll
  for (int t = 0; t < kWaveTiles; t += 2) {
    fold(sb);
    if (t + 2 < kWaveTiles) fetch(t + 2, sb);
    fold(sa);
    if (t + 3 < kWaveTiles) fetch(t + 3, sa);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  if (lane == 0) sink[(long long)blockIdx.x * 4 + wv] = acc;
}

}  // namespace

hipError_t launch_read_ceiling(const void *src, long long bytes, bool paged, bool cached, uint32_t *sink,
                               hipStream_t st) {
  const long long chunks = bytes / kReadCeilingChunk;
  const long long nblk = bytes / (2 * kTileBytes);
  const uint8_t *s = reinterpret_cast<const uint8_t *>(src);
  const dim3 grid((unsigned)chunks);
  if (paged && cached)
    hipLaunchKernelGGL((read_ceiling_kernel<true, false>), grid, dim3(256), 0, st, s, nblk, sink);
  else if (paged)
    hipLaunchKernelGGL((read_ceiling_kernel<true, true>), grid, dim3(256), 0, st, s, nblk, sink);
  else if (cached)
    hipLaunchKernelGGL((read_ceiling_kernel<false, false>), grid, dim3(256), 0, st, s, nblk, sink);
  else
    hipLaunchKernelGGL((read_ceiling_kernel<false, true>), grid, dim3(256), 0, st, s, nblk, sink);
  return hipGetLastError();
}

}  // namespace dsa

// stream.hip -- a plain streaming read of device memory with the same
// 16-byte non-temporal loads the decode kernels use: the read rate this GPU
// reaches on its own, a reference for the decode kernels' bandwidth. Not part
// of the attention path. Every 32-bit word is XOR-folded into one value so
// the loads cannot be dropped and the result can be checked.
#include "decode_common.h"

namespace parallax {
namespace {

using dec::load16;
using dec::u32x4;

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;      // 16-byte loads in flight per lane
constexpr int kStreamBlocks = 512;    // two streams per CU: fewer, longer streams read faster

// Workgroup b reads one contiguous share of the buffer, in tiles of
// kStreamThreads * kStreamUnroll 16-byte words (32 KiB), each lane keeping
// kStreamUnroll loads in flight: the access pattern of a decode workgroup
// streaming its rows.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* src,
                                                                     int64_t n16,
                                                                     unsigned* sink) {
  constexpr int TILE = kStreamThreads * kStreamUnroll;
  const int64_t ntiles = (n16 + TILE - 1) / TILE;
  const int64_t per = (ntiles + gridDim.x - 1) / gridDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * per;
  const int64_t t1 = t0 + per < ntiles ? t0 + per : ntiles;
  const int tid = threadIdx.x;
  unsigned x = 0;
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t base = t * TILE + tid;
    u32x4 w[kStreamUnroll];
    if ((t + 1) * TILE <= n16) {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) w[u] = load16(src + base + u * kStreamThreads);
    } else {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int64_t i = base + u * kStreamThreads;
        const u32x4 z = {0u, 0u, 0u, 0u};
        w[u] = i < n16 ? load16(src + i) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= (w[u][0] ^ w[u][1]) ^ (w[u][2] ^ w[u][3]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (unsigned)__shfl_xor((int)x, o);
  if ((tid & 63) == 0) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t tiles = (n16 + kStreamThreads * kStreamUnroll - 1) /
                        (kStreamThreads * kStreamUnroll);
  const int64_t blocks = tiles < kStreamBlocks ? tiles : kStreamBlocks;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0,
                     stream, reinterpret_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace parallax

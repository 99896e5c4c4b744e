// pack.hip -- transposed tile images for the matrix-core kernels.
//
// A matrix-core contraction over keys (or queries) reads its left operand
// as 16 rows (head-dimension entries) by 32 contraction indices per lane
// group; the kernels keep that operand in LDS transposed, [D][T] for a tile
// of T consecutive rows of a [B, N, H, D] tensor. This kernel writes each
// tile once, in exactly the LDS order the consumer loads, so the consumer
// stages it with plain 16-byte LDS-DMA copies:
//   element (d, n) of a 64-row tile (n = row within the tile) sits in the
//   128-byte LDS row d, 16-byte unit u = 4 * (n / 32) + (n % 16) / 4 stored
//   at slot u ^ ((d >> 1) & 7), element 4 * ((n % 32) / 16) + n % 4.
// Inside each 32-row group this puts the eight rows one lane feeds to a
// contraction (rows 4g..4g+3 and 16+4g..16+4g+3 for lane group g, the rows
// that lane holds in the accumulator layout of the producing contraction)
// in one unit; the slot swizzle gives the 16 lanes of a fragment load 16
// distinct bank groups. Rows past N are zero (tiles that
// start past a packed sequence's end are not written). Optionally
// bf16 is converted to fp16 on the way (exact for |x| in [2^-14, 65504]).
#include "internal.h"
#include "mfma_common.h"

namespace parallax {
namespace {

using namespace mfma;

template <int D, int T, bool F16>
__global__ __launch_bounds__(256) void pack_t_kernel(PackParams p) {
  static_assert(T == 64, "tile rows");
  constexpr int TILE = T * D;
  constexpr int CPR = D / 8;
  __shared__ __attribute__((aligned(16))) unsigned short img[TILE];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  int N = p.N;
  int64_t boff = (int64_t)b * p.sb;
  if (p.cu_seqlens != nullptr) {   // packed: rows [cu[b], cu[b+1])
    const int a = p.cu_seqlens[b];
    N = min(max(p.cu_seqlens[b + 1] - a, 0), p.N);
    boff = (int64_t)a * p.sn;
  }
  if (t * T >= N) return;           // no consumer reads this tile
  const char* base = reinterpret_cast<const char*>(p.src) + (boff + h * p.sh) * 2;
  const int64_t span = (int64_t)(N - 1) * p.sn * 2 + D * 2;
  const int64_t off0 = (int64_t)t * T * p.sn * 2;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + off0, span - off0);
#pragma unroll
  for (int c = tid; c < T * CPR; c += 256) {
    const int n = c / CPR, dc = c % CPR;
    const u32x4 w = buf_load16(rs, n * (int)p.sn * 2 + dc * 16);
    const int unit = 4 * (n >> 5) + ((n >> 2) & 3);
    const int el = 4 * ((n >> 4) & 1) + (n & 3);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned hv = F16 ? bf16x2_to_f16x2(w[q]) : w[q];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int d = 8 * dc + 2 * q + hf;
        img[d * 64 + ((unit ^ ((d >> 1) & 7)) << 3) + el] =
            (unsigned short)(hf ? (hv >> 16) : (hv & 0xffffu));
      }
    }
  }
  __syncthreads();
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<unsigned short*>(p.dst) +
                                         ((int64_t)(b * p.H + h) * p.tiles + t) * TILE);
  const u32x4* src = reinterpret_cast<const u32x4*>(img);
#pragma unroll
  for (int c = tid; c < TILE / 8; c += 256) dst[c] = src[c];
}

template <int D, int T>
hipError_t launch(const PackParams& p, bool to_f16, hipStream_t stream) {
  const dim3 grid(p.tiles, p.H, p.B);
  if (to_f16)
    hipLaunchKernelGGL((pack_t_kernel<D, T, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((pack_t_kernel<D, T, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_t(const PackParams& p, int D, int T, bool to_f16,
                         hipStream_t stream) {
  if (T != 64) return hipErrorInvalidValue;
  return D == 128 ? launch<128, 64>(p, to_f16, stream) : launch<64, 64>(p, to_f16, stream);
}

}  // namespace parallax

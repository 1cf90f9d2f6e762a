// Measurement support: the read bandwidth of the two K/V lane layouts.
//
// The decode's cost is reading the paged KV cache ([P2] background: K/V are
// read page by page out of the paged cache), so how HBM serves its 16-byte
// loads decides the kernel's ceiling. This kernel reads blocks of 16 rows of
// row_bytes bytes (one 16-token block of a cache page, K or V) with the
// partition pass's two lane layouts and the non-temporal policy, and nothing
// else: load i of lane l reads bytes 1024 i + 16 l of the block (linear), or
// bytes [64 i + 16 j, +16) of row c for lane (c = l % 16, j = l / 16) (rows).
// Wave w of the grid reads blocks blocks[w * per + k], k < per, two blocks at
// a time, where per = num_blocks / waves in the grid rounded down to even;
// it folds the loaded words into one value per lane, written to sink, so the
// loads are not removed. Block indices are clamped to the buffer's blocks, so
// every access stays inside it whatever the list holds.
#include "pa_common.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int ROWB, bool LIN>
__global__ __launch_bounds__(1024) void read_probe_kernel(const uint8_t* buf, int32_t nbuf,
                                                          const int32_t* blocks, int32_t per,
                                                          float* sink) {
  constexpr int LPB = ROWB / 64;  // 16-byte loads per lane per block
  constexpr int BLK = 16 * ROWB;
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  u32x4 acc = {0, 0, 0, 0};
  for (int32_t k = 0; k < per; k += 2) {
    u32x4 v[2][LPB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t b = min(max(__builtin_amdgcn_readfirstlane(blocks[wave * per + k + h]), 0), nbuf - 1);
      const auto r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(buf + static_cast<int64_t>(b) * BLK), static_cast<short>(0), BLK,
          0x00020000);
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        const uint32_t off = LIN ? 1024u * i + 16u * lane
                                 : static_cast<uint32_t>((lane & 15) * ROWB + 16 * (lane >> 4) + 64 * i);
        v[h][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < LPB; ++i) acc ^= v[h][i];
  }
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] =
      static_cast<float>(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

template <int ROWB>
void launch_t(bool lin, int grid, int waves, const uint8_t* buf, int32_t nbuf, const int32_t* blocks,
              int32_t per, float* sink, hipStream_t s) {
  if (lin)
    hipLaunchKernelGGL((read_probe_kernel<ROWB, true>), dim3(grid), dim3(64 * waves), 0, s, buf, nbuf,
                       blocks, per, sink);
  else
    hipLaunchKernelGGL((read_probe_kernel<ROWB, false>), dim3(grid), dim3(64 * waves), 0, s, buf, nbuf,
                       blocks, per, sink);
}

}  // namespace

hipError_t launch_read_probe(const uint8_t* buf, int32_t nbuf, const int32_t* blocks, int32_t num_blocks,
                             int row_bytes, bool linear, int grid, int waves, float* sink, hipStream_t s) {
  const int32_t per = num_blocks / (grid * waves) / 2 * 2;
  switch (row_bytes) {
    case 128: launch_t<128>(linear, grid, waves, buf, nbuf, blocks, per, sink, s); break;
    case 256: launch_t<256>(linear, grid, waves, buf, nbuf, blocks, per, sink, s); break;
    default: launch_t<512>(linear, grid, waves, buf, nbuf, blocks, per, sink, s); break;
  }
  return hipGetLastError();
}

}  // namespace pa

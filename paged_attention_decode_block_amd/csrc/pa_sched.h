// Device helpers of the work-list rule: the item ranges of workgroups (lo,
// owner), the segment index of an item inside its (sequence, kv head) pair,
// exact integer division through a double reciprocal, and a block-wide
// prefix sum.
#pragma once

#include "pa_common.h"

namespace pa {

// Exclusive prefix sums of two values per thread over a workgroup of WAVES
// waves: wave scans with lane shuffles, then the wave totals through LDS.
template <int WAVES>
__device__ __forceinline__ int2 block_exclusive_scan2(int2 v, int2* wsum, int2* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int2 x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int yx = __shfl_up(x.x, off), yy = __shfl_up(x.y, off);
    if (lane >= off) {
      x.x += yx;
      x.y += yy;
    }
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int2 before = make_int2(0, 0), tot = make_int2(0, 0);
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const int2 s = wsum[w];
    tot.x += s.x;
    tot.y += s.y;
    if (w < wave) {
      before.x += s.x;
      before.y += s.y;
    }
  }
  *total = tot;
  __syncthreads();
  return make_int2(before.x + x.x - v.x, before.y + x.y - v.y);
}

// floor(a / b) for 0 <= a < 2^53 and 0 < b < 2^31 when the quotient is below
// 2^31: the double product a * (1/b) is within 2^-21 of a / b, so its
// truncation is off by at most one, which one exact remainder test fixes.
struct Div {
  int64_t b;
  double inv;
  __device__ explicit Div(int64_t d) : b(d), inv(1.0 / static_cast<double>(d)) {}
  __device__ __forceinline__ int32_t operator()(int64_t a) const {
    int32_t q = static_cast<int32_t>(static_cast<double>(a) * inv);
    const int64_t r = a - static_cast<int64_t>(q) * b;
    q += (r >= b) ? 1 : 0;
    q -= (r < 0) ? 1 : 0;
    return q;
  }
};

struct Sched {
  int64_t N, G;
  Div byG, byN;
  __device__ Sched(int64_t n, int64_t g) : N(n), G(g), byG(g), byN(n > 0 ? n : 1) {}
  // first item of workgroup w: floor(w N / G)
  __device__ __forceinline__ int32_t wg_lo(int64_t w) const { return byG(w * N); }
  // workgroup owning item x: floor(((x + 1) G - 1) / N)
  __device__ __forceinline__ int32_t owner(int64_t x) const { return byN((x + 1) * G - 1); }
  __device__ __forceinline__ int32_t seg_index(int32_t x, int32_t A) const {
    return N >= G ? owner(x) - owner(A) : x - A;
  }
};

__device__ __forceinline__ int32_t items_of(const Div& byP, int32_t ctx, int32_t P) {
  return byP(static_cast<int64_t>(ctx) + P - 1);
}

}  // namespace pa

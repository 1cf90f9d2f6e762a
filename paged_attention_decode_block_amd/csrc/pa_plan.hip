// Persistent work-list builder (one workgroup).
//
// The metadata scheduler of "[Kernel][Perf] Optimize paged-attention metadata
// decode" (ROCm/FlyDSL PR #910, "Pull request overview" and the code excerpt:
// a persistent grid of CU count x multiplier) is described there only by what
// it produces. The list format here is this library's (see include/pa.h,
// pa_plan): items in (sequence, kv head, partition) order, contiguous item
// ranges per workgroup, segments = same-pair runs inside a range, partial
// slots only for pairs split over several workgroups.
//
// Method: prefix sums (items per sequence, segments per pair, both owned by
// thread chunks) and a closed form per item; each thread writes a contiguous
// run of items. With N items over G workgroups, workgroup w starts at
// lo(w) = floor(w N / G) and item x belongs to owner(x) = floor(((x+1) G - 1) / N),
// the largest w with lo(w) <= x. When N >= G every range is non-empty, so
// the segment index of item x inside its pair (first item A) is
// owner(x) - owner(A); when N < G every non-empty range holds one item and the
// index is x - A. Item x starts a segment when x == A or x == lo(owner(x)).
#include "pa_common.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kLdsSeqs = 4096;   // sequences whose item bases are kept in LDS
constexpr int kLdsPairs = 4096;  // pairs whose segment counts / bases are kept in LDS

// Exclusive prefix sum of one value per thread over the workgroup: a wave
// scan with lane shuffles, then the 16 wave totals through LDS.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* wsum, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int32_t s = wsum[w];
    tot += s;
    before += w < wave ? s : 0;
  }
  *total = tot;
  __syncthreads();
  return before + x - v;
}

// floor(a / b) for 0 <= a < 2^53, 0 < b < 2^31: a double quotient, then an
// exact integer correction (the quotient can be off by one near integers).
// Avoids the long emulated 64-bit integer division.
struct Div {
  int64_t b;
  double inv;
  __device__ explicit Div(int64_t d) : b(d), inv(1.0 / static_cast<double>(d)) {}
  __device__ __forceinline__ int64_t operator()(int64_t a) const {
    int64_t q = static_cast<int64_t>(static_cast<double>(a) * inv);
    int64_t r = a - q * b;
    while (r < 0) { --q; r += b; }
    while (r >= b) { ++q; r -= b; }
    return q;
  }
};

struct Sched {
  int64_t N, G;
  Div byG, byN;
  __device__ Sched(int64_t n, int64_t g) : N(n), G(g), byG(g), byN(n > 0 ? n : 1) {}
  // first item of workgroup w: floor(w N / G)
  __device__ __forceinline__ int32_t wg_lo(int64_t w) const { return static_cast<int32_t>(byG(w * N)); }
  // workgroup owning item x: floor(((x + 1) G - 1) / N)
  __device__ __forceinline__ int32_t owner(int64_t x) const {
    return static_cast<int32_t>(byN((x + 1) * G - 1));
  }
  __device__ __forceinline__ int32_t seg_index(int32_t x, int32_t A) const {
    return N >= G ? owner(x) - owner(A) : x - A;
  }
};

__device__ __forceinline__ int32_t items_of(int32_t ctx, int32_t P) { return (max(ctx, 0) + P - 1) / P; }

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int32_t wsum[kPlanWaves];
  __shared__ int32_t bad;
  __shared__ int32_t l_base[kLdsSeqs + 1];
  __shared__ int32_t l_nseg[kLdsPairs], l_sbase[kLdsPairs], l_pbase[kLdsPairs];
  const int tid = threadIdx.x;
  const int32_t B = a.batch, H = a.num_kv_heads, P = a.partition, G = a.grid;
  const int32_t pairs = B * H;
  // per-sequence / per-pair tables: LDS when they fit, else the workspace
  int32_t* base_t = B < kLdsSeqs ? l_base : a.batch_base;
  int32_t* nseg_t = pairs <= kLdsPairs ? l_nseg : a.nseg;
  int32_t* sbase_t = pairs <= kLdsPairs ? l_sbase : a.seg_base;
  int32_t* pbase_t = pairs <= kLdsPairs ? l_pbase : a.pseg_base;
  if (tid == 0) bad = 0;
  __syncthreads();

  // 1. thread t owns sequences [b_lo, b_hi): validate, count items, and
  //    find the first item of each by a prefix sum
  const int32_t per_b = (B + kPlanThreads - 1) / kPlanThreads;
  const int32_t b_lo = min(B, tid * per_b), b_hi = min(B, b_lo + per_b);
  int32_t sum = 0;
  for (int32_t b = b_lo; b < b_hi; ++b) {
    const int32_t c = a.context_lens[b];
    if (c < max(1, a.q_len) || c > a.capacity) atomicOr(&bad, 1);
    sum += H * items_of(c, P);
  }
  int32_t N = 0;
  const int32_t first = block_exclusive_scan(sum, wsum, &N);
  const Sched sc(N, G);
  if (bad) {
    for (int i = tid; i <= G; i += kPlanThreads) { a.wg_begin[i] = 0; a.wg_seg_begin[i] = 0; }
    for (int i = tid; i < pairs; i += kPlanThreads) a.nseg[i] = 0;
    for (int i = tid; i <= pairs; i += kPlanThreads) { a.seg_base[i] = 0; a.pseg_base[i] = 0; }
    for (int i = tid; i <= B; i += kPlanThreads) a.batch_base[i] = 0;
    if (tid == 0) {
      a.status[ST_BITS] = PA_DEV_BAD_CONTEXT;
      a.status[ST_ITEMS] = 0;
      a.status[ST_SEGS] = 0;
    }
    return;
  }

  // 2. the same thread's pairs: segment counts, then slot bases (split pairs
  //    only) and segment bases by two more prefix sums
  int32_t split = 0, all = 0;
  {
    int32_t A = first;
    for (int32_t b = b_lo; b < b_hi; ++b) {
      const int32_t n = items_of(a.context_lens[b], P);
      for (int32_t g = 0; g < H; ++g, A += n) {
        const int32_t ns = sc.seg_index(A + n - 1, A) + 1;
        split += ns > 1 ? ns : 0;
        all += ns;
      }
    }
  }
  int32_t slots = 0, S = 0;
  int32_t run_split = block_exclusive_scan(split, wsum, &slots);
  int32_t run_all = block_exclusive_scan(all, wsum, &S);
  {
    int32_t A = first;
    for (int32_t b = b_lo; b < b_hi; ++b) {
      const int32_t n = items_of(a.context_lens[b], P);
      base_t[b] = A;
      a.batch_base[b] = A;
      for (int32_t g = 0; g < H; ++g, A += n) {
        const int32_t p = b * H + g;
        const int32_t ns = sc.seg_index(A + n - 1, A) + 1;
        nseg_t[p] = ns;
        sbase_t[p] = run_split;
        pbase_t[p] = run_all;
        a.nseg[p] = ns;
        a.seg_base[p] = run_split;
        a.pseg_base[p] = run_all;
        run_split += ns > 1 ? ns : 0;
        run_all += ns;
      }
    }
  }
  if (tid == 0) {
    base_t[B] = N;
    a.batch_base[B] = N;
    a.seg_base[pairs] = slots;
    a.pseg_base[pairs] = S;
  }
  __syncthreads();

  // 3. thread t writes items [x0, x1): each item, the segment it opens, and
  //    the segment-range start of every workgroup whose range starts there.
  //    The owning workgroup w (and its range [lo_w, hi_w)) advances with x.
  const int32_t per_x = (N + kPlanThreads - 1) / kPlanThreads;
  const int32_t x0 = min(N, tid * per_x), x1 = min(N, x0 + per_x);
  if (x0 < x1) {
    int lo = 0, hi = B;  // largest b with base_t[b] <= x0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (base_t[mid] <= x0) lo = mid; else hi = mid;
    }
    int32_t b = lo;
    int32_t ctx = a.context_lens[b];
    int32_t n = items_of(ctx, P);
    int32_t g = (x0 - base_t[b]) / n;
    int32_t k = x0 - base_t[b] - g * n;
    int32_t p = b * H + g;
    int32_t A = base_t[b] + g * n;
    int32_t ns = nseg_t[p], sb = sbase_t[p], pb = pbase_t[p];
    int32_t w = sc.owner(x0);
    int32_t lo_w = sc.wg_lo(w), hi_w = sc.wg_lo(w + 1);
    int32_t w_A = sc.owner(A);
    for (int32_t x = x0; x < x1; ++x) {
      while (x >= hi_w) {  // skips empty ranges too
        ++w;
        lo_w = hi_w;
        hi_w = sc.wg_lo(w + 1);
      }
      if (x == A) w_A = w;
      const int32_t j = N >= G ? w - w_A : x - A;
      Span it;
      it.pair = p;
      it.tok_begin = k * P;
      it.tok_end = min((k + 1) * P, ctx);
      it.slot = ns > 1 ? sb + j : -1;
      a.items[x] = it;
      if (x == A || x == lo_w) {
        const int32_t last = min(A + n, hi_w) - 1;
        Span sg = it;
        sg.tok_end = min((last - A + 1) * P, ctx);
        a.segs[pb + j] = sg;
      }
      if (x == lo_w) {
        // workgroups ceil(x G / N) .. w all start their (possibly empty) range at x
        for (int32_t w2 = w; w2 >= 0 && (w2 == w || sc.wg_lo(w2) == x); --w2)
          a.wg_seg_begin[w2] = pb + j;
      }
      if (++k == n) {  // next pair: next kv head, or the next sequence
        k = 0;
        A += n;
        if (++g == H) {
          g = 0;
          if (++b < B) {
            ctx = a.context_lens[b];
            n = items_of(ctx, P);
          }
        }
        p = b * H + g;
        if (x + 1 < x1) {
          ns = nseg_t[p];
          sb = sbase_t[p];
          pb = pbase_t[p];
        }
      }
    }
  }

  // 4. item ranges
  for (int32_t w = tid; w <= G; w += kPlanThreads) a.wg_begin[w] = sc.wg_lo(w);
  if (tid == 0) {
    a.wg_seg_begin[G] = S;
    a.status[ST_BITS] = 0;
    a.status[ST_ITEMS] = N;
    a.status[ST_SEGS] = S;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa

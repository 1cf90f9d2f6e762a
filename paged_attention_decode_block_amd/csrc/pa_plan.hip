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
// Method: two prefix sums (items per sequence, segments per pair) and a closed
// form per item. With N items over G workgroups, workgroup w starts at
// lo(w) = floor(w N / G) and item x belongs to owner(x) = floor(((x+1) G - 1) / N),
// the largest w with lo(w) <= x. When N >= G every range is non-empty, so
// the segment index of item x inside its pair (first item A) is
// owner(x) - owner(A); when N < G every non-empty range holds one item and the
// index is x - A. Item x starts a segment when x == A or x == lo(owner(x)).
#include "pa_common.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

// In-place exclusive prefix sum of data[0, n) in global memory; returns the
// total. Thread t owns a contiguous chunk; chunk sums are scanned in LDS.
__device__ int32_t block_exclusive_scan(int32_t* data, int32_t n, int32_t* lds) {
  const int tid = threadIdx.x;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, tid * per);
  const int hi = min(n, lo + per);
  int32_t sum = 0;
  for (int x = lo; x < hi; ++x) sum += data[x];
  lds[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int32_t v = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += v;
    __syncthreads();
  }
  int32_t run = lds[tid] - sum;
  const int32_t total = lds[kPlanThreads - 1];
  for (int x = lo; x < hi; ++x) {
    const int32_t v = data[x];
    data[x] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

__device__ __forceinline__ int32_t wg_lo(int64_t w, int64_t N, int64_t G) {
  return static_cast<int32_t>(w * N / G);
}

__device__ __forceinline__ int32_t owner(int64_t x, int64_t N, int64_t G) {
  return static_cast<int32_t>(((x + 1) * G - 1) / N);
}

__device__ __forceinline__ int32_t seg_index(int32_t x, int32_t A, int64_t N, int64_t G) {
  return N >= G ? owner(x, N, G) - owner(A, N, G) : x - A;
}

// Largest b in [0, B) with batch_base[b] <= x (batch_base has B + 1 entries).
__device__ __forceinline__ int32_t find_seq(const int32_t* batch_base, int32_t B, int32_t x) {
  int lo = 0, hi = B;  // invariant: batch_base[lo] <= x < batch_base[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (batch_base[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

struct ItemPos {
  int32_t pair, A, n, k, ctx;
};

__device__ __forceinline__ ItemPos locate(const PlanArgs& a, int32_t x) {
  const int32_t b = find_seq(a.batch_base, a.batch, x);
  const int32_t base = a.batch_base[b];
  const int32_t n = (a.batch_base[b + 1] - base) / a.num_kv_heads;
  const int32_t r = x - base;
  const int32_t g = r / n;
  ItemPos ip;
  ip.pair = b * a.num_kv_heads + g;
  ip.A = base + g * n;
  ip.n = n;
  ip.k = r - g * n;
  ip.ctx = a.context_lens[b];
  return ip;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int32_t lds[kPlanThreads];
  __shared__ int32_t bad;
  const int tid = threadIdx.x;
  const int32_t B = a.batch, H = a.num_kv_heads, P = a.partition, G = a.grid;
  const int32_t pairs = B * H;
  if (tid == 0) bad = 0;
  __syncthreads();

  // 1. validate context lengths; items per sequence = H * ceil(ctx / P)
  for (int b = tid; b < B; b += kPlanThreads) {
    const int32_t c = a.context_lens[b];
    if (c < max(1, a.q_len) || c > a.capacity) atomicOr(&bad, 1);
    a.batch_base[b] = H * ((max(c, 0) + P - 1) / P);
  }
  __syncthreads();
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
  const int32_t N = block_exclusive_scan(a.batch_base, B, lds);
  if (tid == 0) a.batch_base[B] = N;
  __syncthreads();

  // 2. segments per pair, then slot bases (split pairs) and segment bases (all)
  for (int p = tid; p < pairs; p += kPlanThreads) {
    const int32_t b = p / H, g = p - b * H;
    const int32_t n = (a.batch_base[b + 1] - a.batch_base[b]) / H;
    const int32_t A = a.batch_base[b] + g * n;
    const int32_t ns = seg_index(A + n - 1, A, N, G) + 1;
    a.nseg[p] = ns;
    a.seg_base[p] = ns > 1 ? ns : 0;
    a.pseg_base[p] = ns;
  }
  __syncthreads();
  const int32_t slots = block_exclusive_scan(a.seg_base, pairs, lds);
  const int32_t S = block_exclusive_scan(a.pseg_base, pairs, lds);
  if (tid == 0) {
    a.seg_base[pairs] = slots;
    a.pseg_base[pairs] = S;
  }
  __syncthreads();

  // 3. items, and the segment each segment-starting item opens
  for (int32_t x = tid; x < N; x += kPlanThreads) {
    const ItemPos ip = locate(a, x);
    const int32_t j = seg_index(x, ip.A, N, G);
    const int32_t ns = a.nseg[ip.pair];
    Span it;
    it.pair = ip.pair;
    it.tok_begin = ip.k * P;
    it.tok_end = min((ip.k + 1) * P, ip.ctx);
    it.slot = ns > 1 ? a.seg_base[ip.pair] + j : -1;
    a.items[x] = it;
    const int32_t w = owner(x, N, G);
    if (x == ip.A || x == wg_lo(w, N, G)) {
      const int32_t last = min(ip.A + ip.n, wg_lo(w + 1, N, G)) - 1;
      Span sg = it;
      sg.tok_end = min((last - ip.A + 1) * P, ip.ctx);
      a.segs[a.pseg_base[ip.pair] + j] = sg;
    }
  }

  // 4. per-workgroup item and segment ranges
  for (int32_t w = tid; w <= G; w += kPlanThreads) {
    const int32_t lo = wg_lo(w, N, G);
    a.wg_begin[w] = lo;
    int32_t sb = S;
    if (lo < N) {
      const ItemPos ip = locate(a, lo);
      sb = a.pseg_base[ip.pair] + seg_index(lo, ip.A, N, G);
    }
    a.wg_seg_begin[w] = sb;
  }
  if (tid == 0) {
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

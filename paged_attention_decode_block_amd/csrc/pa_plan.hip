// Persistent work-list builder.
//
// The metadata scheduler of "[Kernel][Perf] Optimize paged-attention metadata
// decode" (ROCm/FlyDSL PR #910, "Pull request overview" and the code excerpt:
// a persistent grid of CU count x multiplier) is described there only by what
// it produces. The list format here is this library's (see include/pa.h,
// pa_plan): items in (sequence, kv head, partition) order, contiguous item
// ranges per workgroup, segments = same-pair runs inside a range, partial
// slots only for pairs split over several workgroups.
//
// Method: prefix sums (items per sequence, then split slots and segments per
// pair) and a closed form per item. With N items over G workgroups,
// workgroup w starts at lo(w) = floor(w N / G) and item x belongs to
// owner(x) = floor(((x+1) G - 1) / N), the largest w with lo(w) <= x. When
// N >= G every range is non-empty, so the segment index of item x inside its
// pair (first item A) is owner(x) - owner(A); when N < G every non-empty range
// holds one item and the index is x - A. Item x starts a segment when x == A
// or x == lo(owner(x)); a workgroup's first segment is the one that holds item
// lo(w), so empty ranges need no special case.
//
// Latency is the whole cost of this kernel, so: the per-sequence and per-pair
// tables live in LDS whenever they fit (typed LDS accesses, which never wait
// on outstanding global stores), every global store sits after the loads of
// its phase, and divisions go through a double reciprocal with one exact
// correction instead of the emulated 64-bit integer division. When the tables
// fit in LDS, several workgroups run: each recomputes the (small) tables in
// its own LDS and writes only its slice of the items, ranges and tables, so
// the item writes are spread over several CUs with no inter-workgroup
// synchronisation. Otherwise one workgroup keeps the tables in the workspace.
#include "pa_plan.h"
#include "pa_sched.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 512;
constexpr int kPlanWaves = kPlanThreads / 64;
// LDS tables: context and first item per sequence; segment count, first split
// slot and first segment per pair. Two capacities: 4096 sequences and 4096
// pairs with every table, and as many as the 160 KiB of a gfx950 workgroup
// hold (less a little for the scan's wave sums) with only the first items and
// bases: context lengths are then reread from the input (cached after their
// first pass) and segment counts recomputed by their closed form where
// needed. The recomputation (a few double-precision reciprocals) costs the
// small batches about 0.4 us, so they keep every table.
constexpr int kLdsBytes = 160 * 1024;
constexpr int kLdsSeqsSmall = 4096, kLdsPairsSmall = 4096;
constexpr int kLdsSeqsBig = 8192;
constexpr int kLdsPairsBig = ((kLdsBytes - 256) / 4 - (kLdsSeqsBig + 1)) / 2 / 16 * 16;  // 16336
constexpr int kPlanMaxBlocks = 256;

// Per-sequence and per-pair tables: LDS arrays when they fit, else the
// workspace arrays of the same meaning. Context lengths are in LDS only with
// kCtx; otherwise they are reread from the input.
template <bool kCtx>
struct Tables {
  int32_t* ctx;    // [B]      context length (kCtx only)
  int32_t* base;   // [B + 1]  first item of each sequence
  int32_t* nseg;   // [pairs]  (absent from the largest LDS tables)
  int32_t* sbase;  // [pairs]  first split slot
  int32_t* pbase;  // [pairs]  first segment
  const int32_t* in_ctx;
  int32_t off;     // ctx_offset, subtracted from the input lengths
  __device__ __forceinline__ int32_t context(int32_t b) const {
    if constexpr (kCtx) return ctx[b];
    return in_ctx[b] - off;
  }
};

// 3. Items [X0, X1) of the list; thread tid writes the run [x0, x1) of them:
//    each item and the segment it opens. The owning workgroup w (and its
//    range [lo_w, hi_w)) advances with x. Shared by the plan kernel (tables in
//    LDS or the workspace) and the items kernel (tables in the workspace).
template <bool kCtx, bool kNseg>
__device__ __forceinline__ void write_items(const PlanArgs& a, const Tables<kCtx>& t, const Sched& sc,
                                            const Div& byP, int32_t N, int32_t X0, int32_t X1,
                                            int tid) {
  const int32_t B = a.batch, H = a.num_kv_heads, P = a.partition, G = a.grid;
  auto items_of = [&](int32_t ctx) { return byP(static_cast<int64_t>(ctx) + P - 1); };
  auto nseg_at = [&](int32_t p, int32_t A, int32_t n) {
    if constexpr (kNseg) return t.nseg[p];
    return sc.seg_index(A + n - 1, A) + 1;
  };
  const int32_t per_x = (X1 - X0 + kPlanThreads - 1) / kPlanThreads;
  const int32_t x0 = min(X1, X0 + tid * per_x), x1 = min(X1, x0 + per_x);
  if (x0 < x1) {
    int lo = 0, hi = B;  // largest b with base[b] <= x0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (t.base[mid] <= x0) lo = mid; else hi = mid;
    }
    int32_t b = lo;
    int32_t ctx = t.context(b);
    int32_t n = items_of(ctx);
    const int32_t bb = t.base[b];
    int32_t g = Div(n)(x0 - bb);
    int32_t k = x0 - bb - g * n;
    int32_t p = b * H + g;
    int32_t A = bb + g * n;
    int32_t ns = nseg_at(p, A, n), sb = t.sbase[p], pb = t.pbase[p];
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
      if (x == A || x == lo_w) {
        const int32_t last = min(A + n, hi_w) - 1;
        Span sg = it;
        sg.tok_end = min((last - A + 1) * P, ctx);
        a.segs[pb + j] = sg;
        // the decode's record: everything a segment needs in one 32-byte load
        int4* si = reinterpret_cast<int4*>(a.seg_info + 8 * static_cast<int64_t>(pb + j));
        si[0] = make_int4(b, g, sg.tok_begin, sg.tok_end);
        si[1] = make_int4(sg.slot, ctx, p, 0);
        if (N >= G && x == lo_w) {
          // every range is non-empty: this segment opens workgroup w's range
          int4* h = reinterpret_cast<int4*>(a.wg_head + 16 * static_cast<int64_t>(w));
          h[0] = make_int4(pb + j, b, g, sg.tok_begin);
          h[1] = make_int4(sg.tok_end, sg.slot, ctx, p);
          h[3] = make_int4(0, 0, 0, 0);
          if (w > 0)
            reinterpret_cast<int4*>(a.wg_head + 16 * static_cast<int64_t>(w - 1))[2] =
                make_int4(pb + j, 0, 0, 0);
          a.wg_begin[w] = x;
          a.wg_seg_begin[w] = pb + j;
        }
      }
      a.items[x] = it;
      if (++k == n && x + 1 < x1) {  // next pair: next kv head, or the next sequence
        k = 0;
        A += n;
        if (++g == H) {
          g = 0;
          ++b;
          ctx = t.context(b);
          n = items_of(ctx);
        }
        p = b * H + g;
        ns = nseg_at(p, A, n);
        sb = t.sbase[p];
        pb = t.pbase[p];
      }
    }
  }
}

// kPairs: pairs the LDS tables hold (0: tables in the workspace)
template <int kPairs>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  constexpr bool kLds = kPairs > 0;
  // segment counts: read back from the small LDS tables; elsewhere
  // recomputed where needed (cheaper than a dependent global load), but
  // still written to the workspace
  constexpr bool kNseg = kLds && kPairs <= kLdsPairsSmall;
  constexpr bool kStoreNseg = kNseg || !kLds;
  constexpr bool kCtx = kNseg;  // context lengths in LDS
  constexpr int NS = !kLds ? 1 : kNseg ? kLdsSeqsSmall : kLdsSeqsBig, NP = kLds ? kPairs : 1;
  __shared__ int2 wsum[kPlanWaves];
  __shared__ int32_t bad;
  __shared__ int32_t l_ctx[kCtx ? NS : 1], l_base[NS + 1];
  __shared__ int32_t l_nseg[kNseg ? NP : 1], l_sbase[NP], l_pbase[NP];
  const int tid = threadIdx.x;
  // this block's share of the per-item, per-workgroup and per-table writes
  const int32_t nblk = kLds ? static_cast<int32_t>(gridDim.x) : 1;
  const int32_t blk = kLds ? static_cast<int32_t>(blockIdx.x) : 0;
  const int32_t gtid = blk * kPlanThreads + tid, gstride = nblk * kPlanThreads;
  const int32_t B = a.batch, H = a.num_kv_heads, P = a.partition, G = a.grid;
  const int32_t pairs = B * H;
  Tables<kCtx> t;
  if constexpr (kLds) {
    t = {kCtx ? l_ctx : nullptr, l_base, kNseg ? l_nseg : nullptr, l_sbase, l_pbase, a.context_lens,
         a.ctx_offset};
  } else {
    t = {nullptr, a.batch_base, a.nseg, a.seg_base, a.pseg_base, a.context_lens, a.ctx_offset};
  }
  const Div byP(P), byH(H);
  auto items_of = [&](int32_t ctx) { return byP(static_cast<int64_t>(ctx) + P - 1); };
  if (tid == 0) bad = 0;

  // 1. thread t owns sequences [b_lo, b_hi): validate, count items; the
  //    first item of each sequence comes from a prefix sum
  const int32_t per_b = (B + kPlanThreads - 1) / kPlanThreads;
  const int32_t b_lo = min(B, tid * per_b), b_hi = min(B, b_lo + per_b);
  int32_t sum = 0;
  bool my_bad = false;
  for (int32_t b = b_lo; b < b_hi; ++b) {
    const int32_t c = a.context_lens[b];
    const bool ok = c >= max(1, a.q_check) && c <= a.capacity;
    my_bad |= !ok;
    if constexpr (kCtx) t.ctx[b] = c - a.ctx_offset;
    sum += ok ? H * items_of(c - a.ctx_offset) : 0;
  }
  __syncthreads();  // bad = 0 is visible
  if (my_bad) bad = 1;
  int2 tot;
  const int32_t first = block_exclusive_scan2<kPlanWaves>(make_int2(sum, 0), wsum, &tot).x;
  const int32_t N = tot.x;
  if (bad) {
    for (int i = gtid; i <= G; i += gstride) { a.wg_begin[i] = 0; a.wg_seg_begin[i] = 0; }
    for (int i = gtid; i < 16 * G; i += gstride) a.wg_head[i] = 0;
    for (int i = gtid; i < pairs; i += gstride) {
      a.nseg[i] = 0;
      a.counters[i] = 0;
    }
    for (int i = gtid; i <= pairs; i += gstride) { a.seg_base[i] = 0; a.pseg_base[i] = 0; }
    for (int i = gtid; i <= B; i += gstride) a.batch_base[i] = 0;
    if (gtid == 0) {
      a.status[ST_BITS] = PA_DEV_BAD_CONTEXT;
      a.status[ST_ITEMS] = 0;
      a.status[ST_SEGS] = 0;
    }
    return;
  }
  const Sched sc(N, G);
  // segments of the pair whose n items start at item A: closed form
  auto nseg_of = [&](int32_t A, int32_t n) { return sc.seg_index(A + n - 1, A) + 1; };
  // pair p's segment count: stored, or recomputed (first item A, n items)
  auto nseg_at = [&](int32_t p, int32_t A, int32_t n) {
    if constexpr (kNseg) return t.nseg[p];
    return nseg_of(A, n);
  };
  {
    int32_t A = first;
    for (int32_t b = b_lo; b < b_hi; ++b) {
      t.base[b] = A;
      A += H * items_of(t.context(b));
    }
    if (tid == 0) t.base[B] = N;
  }
  __syncthreads();

  // 2. thread t owns pairs [p_lo, p_hi): segment counts, then split-slot and
  //    segment bases by a prefix sum
  const int32_t per_p = (pairs + kPlanThreads - 1) / kPlanThreads;
  const int32_t p_lo = min(pairs, tid * per_p), p_hi = min(pairs, p_lo + per_p);
  int2 cnt = make_int2(0, 0);  // (split slots, segments)
  if (p_lo < p_hi) {
    int32_t b = byH(p_lo), g = p_lo - b * H;
    int32_t n = items_of(t.context(b));
    for (int32_t p = p_lo; p < p_hi; ++p) {
      const int32_t ns = nseg_of(t.base[b] + g * n, n);
      if constexpr (kStoreNseg) t.nseg[p] = ns;
      cnt.x += ns > 1 ? ns : 0;
      cnt.y += ns;
      if (++g == H && p + 1 < p_hi) {
        g = 0;
        n = items_of(t.context(++b));
      }
    }
  }
  const int2 run0 = block_exclusive_scan2<kPlanWaves>(cnt, wsum, &tot);
  const int32_t slots = tot.x, S = tot.y;
  if (p_lo < p_hi) {
    int2 run = run0;
    int32_t b = byH(p_lo), g = p_lo - b * H;
    int32_t n = items_of(t.context(b));
    for (int32_t p = p_lo; p < p_hi; ++p) {
      const int32_t ns = nseg_at(p, t.base[b] + g * n, n);
      t.sbase[p] = run.x;
      t.pbase[p] = run.y;
      run.x += ns > 1 ? ns : 0;
      run.y += ns;
      if (++g == H && p + 1 < p_hi) {
        g = 0;
        n = items_of(t.context(++b));
      }
    }
  }
  __syncthreads();

  // 3. this block's items, unless the items kernel writes them
  if (!a.items_apart) {
    const Div byBlk(nblk);
    const int32_t X0 = byBlk(static_cast<int64_t>(blk) * N);
    const int32_t X1 = byBlk(static_cast<int64_t>(blk + 1) * N);
    write_items<kCtx, kNseg>(a, t, sc, byP, N, X0, X1, tid);
  }

  // 4. per workgroup: its item range, its first segment (the one holding item
  //    lo(w), found from the sequence and pair tables) and its header: the
  //    first segment's index and decode record, and the segment range end
  auto first_segment = [&](int32_t w, int4& r0, int4& r1) {
    const int32_t x = sc.wg_lo(w);
    if (w >= G || x >= N) return S;
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (t.base[mid] <= x) lo = mid; else hi = mid;
    }
    const int32_t ctx = t.context(lo);
    const int32_t n = items_of(ctx);
    const int32_t g = Div(n)(x - t.base[lo]);
    const int32_t A = t.base[lo] + g * n;
    const int32_t p = lo * H + g;
    const int32_t j = sc.seg_index(x, A);
    const int32_t last = min(A + n, sc.wg_lo(sc.owner(x) + 1)) - 1;
    const int32_t ns = nseg_at(p, A, n);
    r0 = make_int4(lo, g, (x - A) * P, min((last - A + 1) * P, ctx));
    r1 = make_int4(ns > 1 ? t.sbase[p] + j : -1, ctx, p, 0);
    return t.pbase[p] + j;
  };
  // header of workgroup w: (begin, record[7], end, 0...); the thread of w
  // writes w's begin and record, and the end of w - 1 (its own begin). When
  // N >= G the segment that opens each range wrote them already.
  if (N >= G) {
    if (gtid == 0) {
      a.wg_begin[G] = N;
      a.wg_seg_begin[G] = S;
      reinterpret_cast<int4*>(a.wg_head + 16 * static_cast<int64_t>(G - 1))[2] = make_int4(S, 0, 0, 0);
    }
  } else for (int32_t w = gtid; w <= G; w += gstride) {
    int4 r0 = make_int4(0, 0, 0, 0), r1 = make_int4(0, 0, 0, 0);
    const int32_t first_seg = first_segment(w, r0, r1);
    a.wg_begin[w] = sc.wg_lo(w);
    a.wg_seg_begin[w] = first_seg;
    if (w < G) {
      int4* h = reinterpret_cast<int4*>(a.wg_head + 16 * static_cast<int64_t>(w));
      h[0] = make_int4(first_seg, r0.x, r0.y, r0.z);
      h[1] = make_int4(r0.w, r1.x, r1.y, r1.z);
      h[3] = make_int4(0, 0, 0, 0);
    }
    if (w > 0)
      reinterpret_cast<int4*>(a.wg_head + 16 * static_cast<int64_t>(w - 1))[2] =
          make_int4(first_seg, 0, 0, 0);
  }

  // 5. the fused reduce's arrival counters, cleared; the tables the decode
  //    and the tests read, copied out of LDS
  for (int32_t p = gtid; p < pairs; p += gstride) a.counters[p] = 0;
  if constexpr (kLds) {
    for (int32_t b = gtid; b <= B; b += gstride) a.batch_base[b] = t.base[b];
    for (int32_t p = gtid; p < pairs; p += gstride) {
      if constexpr (kNseg) {
        a.nseg[p] = t.nseg[p];
      } else {
        const int32_t b = byH(p), n = items_of(t.context(b));
        a.nseg[p] = nseg_of(t.base[b] + (p - b * H) * n, n);
      }
      a.seg_base[p] = t.sbase[p];
      a.pseg_base[p] = t.pbase[p];
    }
  }
  if (gtid == 0) {
    a.seg_base[pairs] = slots;
    a.pseg_base[pairs] = S;
    a.status[ST_BITS] = 0;
    a.status[ST_ITEMS] = N;
    a.status[ST_SEGS] = S;
  }
}

// Items of a batch whose tables live in the workspace, written by
// plan_kernel<0> just before on the same stream: every workgroup writes its
// slice of the list. Nothing to do when that kernel found a bad context
// length (it emptied the list).
__global__ __launch_bounds__(kPlanThreads) void plan_items_kernel(PlanArgs a) {
  if (a.status[ST_BITS] != 0) return;
  const int32_t N = a.batch_base[a.batch];
  const Sched sc(N, a.grid);
  const Tables<false> t = {nullptr,    a.batch_base,    a.nseg,       a.seg_base,
                           a.pseg_base, a.context_lens, a.ctx_offset};
  const Div byP(a.partition), byBlk(gridDim.x);
  const int32_t X0 = byBlk(static_cast<int64_t>(blockIdx.x) * N);
  const int32_t X1 = byBlk(static_cast<int64_t>(blockIdx.x + 1) * N);
  write_items<false, false>(a, t, sc, byP, N, X0, X1, threadIdx.x);
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, int64_t max_items, hipStream_t s) {
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_kv_heads;
  // about two items per thread at the largest possible item count
  const int64_t want = (max_items + 2 * kPlanThreads - 1) / (2 * kPlanThreads);
  const int blocks = static_cast<int>(want < 1 ? 1 : (want > kPlanMaxBlocks ? kPlanMaxBlocks : want));
  PlanArgs b = a;
  b.items_apart = 0;
  if (a.batch <= kLdsSeqsSmall && pairs <= kLdsPairsSmall) {
    hipLaunchKernelGGL(plan_kernel<kLdsPairsSmall>, dim3(blocks), dim3(kPlanThreads), 0, s, b);
  } else if (a.batch <= kLdsSeqsBig && pairs <= kLdsPairsBig) {
    hipLaunchKernelGGL(plan_kernel<kLdsPairsBig>, dim3(blocks), dim3(kPlanThreads), 0, s, b);
  } else {
    // one workgroup builds the tables in the workspace, then every workgroup
    // of the items kernel writes its slice of the list
    b.items_apart = 1;
    hipLaunchKernelGGL(plan_kernel<0>, dim3(1), dim3(kPlanThreads), 0, s, b);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_items_kernel, dim3(blocks), dim3(kPlanThreads), 0, s, b);
  }
  return hipGetLastError();
}

}  // namespace pa

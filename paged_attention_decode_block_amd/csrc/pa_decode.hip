// Paged-attention decode kernels for gfx950: the persistent partition pass,
// the log-sum-exp reduce of split pairs, and (test support) the partition
// pass's page loader run alone.
//
// What the pages fix: the KV cache is read page by page through a block
// table (Ascend/RecSDK issue #1281, section "背景与优化特性", background);
// overlapping the next chunk's page loads with the work on the current one
// is the optimisation that issue makes (section "优化方案": K/V double
// buffering); the decode is persistent over a metadata work list and split
// pieces are merged by a reduction kernel, with per-token or per-tensor fp8 KV
// scales ("[Kernel][Perf] Optimize paged-attention metadata decode", ROCm/
// FlyDSL PR #910, "Pull request overview"); grouped query heads share a kv
// head ("h16_kv1", hw-native-sys/simpler issue #998, table "Same-Shape
// Side-by-Side"). The arithmetic is scaled-dot-product softmax attention, the
// plainest reading of "paged attention decode".
//
// Partition pass, one workgroup of NW waves per persistent slot:
//   * the workgroup walks its segments (token ranges of one (sequence, kv
//     head) pair); the waves form NW / RS chunk streams of RS waves each;
//     inside a segment stream s takes chunks s, s + NW / RS, ... of
//     TC = 16 * NB tokens, and each of its RS waves computes RT 16-row tiles
//     of the pair's query rows on them (RS > 1 splits many rows over waves
//     so that each wave's registers allow two waves per SIMD)
//   * each wave runs an NS-stage software pipeline over its chunk stream:
//     the K/V rows of chunk i + NS - 1 (16-byte non-temporal buffer loads,
//     each wave instruction reading 1 KB contiguous) are issued while chunk i
//     is computed, and the block-table entries that address them were loaded
//     NS - 1 chunks before that, so no wait for an entry ever drains the K/V
//     loads in flight; the rows then go through LDS into MFMA operand order
//   * S^T = K Q^T on MFMA 16x16x32 bf16 (K rows are the A operand as loaded;
//     fp8 K is decoded to bf16 exactly); fp32 online softmax in the exp2
//     domain with the causal mask of the appended tokens; O^T += V^T P^T on
//     MFMA, where P^T comes lane-locally from S^T and V^T is read from a
//     wave-private LDS tile (V rows written row-major, read transposed)
//   * 64-row fp8 pairs (RS = 2, SH): a stream's two waves share each chunk
//     through LDS instead: one loads and widens K, the other V, into
//     double-buffered bf16 tiles of the stream, and the workgroup meets one
//     barrier per step (every stream takes the same number of entries)
//   * at a segment's end the NW waves merge their (max, sum, O) through LDS;
//     an unsplit pair writes bf16 output, a split pair writes its partial O
//     and log-sum-exp to its slot
#include <type_traits>

#include "pa_common.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.f;  // lazy-rescale slack of the running max (log2 units)

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Load of wave-uniform, read-only metadata (segments, context lengths,
// block-table entries, per-tensor scales) through the constant address space:
// the compiler issues it as a scalar load, counted apart from the K/V vector
// loads, so waiting for it never drains the K/V prefetch.
template <typename T>
__device__ __forceinline__ T ldu(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)(p))[i];
}

// 8 E4M3FN bytes -> 8 bf16, two per instruction (gfx950 scaled conversion
// with scale 1). Exact: every finite E4M3FN value is a bf16 value. (The
// conversion's scale operand is a power-of-two block scale: only its exponent
// takes part, so general per-token scales are applied to scores and
// probabilities instead.)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), 1.0f, true);
  return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// s_waitcnt with vmcnt = 0 (gfx9 encoding; expcnt and lgkmcnt left at their
// maxima): the wave's vector memory operations, stores included, are done.
constexpr int kWaitVmcnt0 = 0x0F70;

// Cache policy of a buffer access at agent scope (gfx950 sc1): a store is
// written through to where every XCD sees it, a load does not hit a stale L2
// line. The fused reduce's partials move between workgroups this way.
constexpr int kSc1 = 16;

// Lane i of each lane quad's value, to every lane of the quad (DPP
// quad_perm [i, i, i, i]).
__device__ __forceinline__ float quad_bcast(float x, int i) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (i) {
    case 0: r = __builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, true); break;
    case 1: r = __builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, true); break;
    case 2: r = __builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, true); break;
    default: r = __builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, true); break;
  }
  return __builtin_bit_cast(float, r);
}

// Reduction over the four 16-lane rows of a wave: every lane gets the result
// for its column (lane % 16). gfx950 permlane swaps exchange rows in VALU:
// with both operands a copy of x, the 16-lane swap leaves rows (0, 0, 2, 2)
// in one result and (1, 1, 3, 3) in the other, the 32-lane swap halves
// (lo, lo) and (hi, hi). MED3 takes the maximum of two as the median of
// (a, b, FLT_MAX): one v_med3_f32 instead of a compare and a select, but the
// constant holds a scalar register, which the shared-tile kernels can spare
// and the others cannot without spilling more (with +inf the compiler
// rewrites the median as a maximum that first quiets each operand).
template <bool MED3>
__device__ __forceinline__ float pick_max(float a, float b) {
  if constexpr (MED3) return __builtin_amdgcn_fmed3f(a, b, 3.40282347e38f);
  return a > b ? a : b;
}

template <bool kMax, bool MED3 = false>
__device__ __forceinline__ float rows_reduce(float x) {
  // (each element is copied to a scalar before the bit cast: a bit cast of a
  // vector element in place reads element 0)
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0u = r16[0], a1u = r16[1];
  const float a0 = __builtin_bit_cast(float, a0u), a1 = __builtin_bit_cast(float, a1u);
  x = kMax ? pick_max<MED3>(a0, a1) : a0 + a1;
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t b0u = r32[0], b1u = r32[1];
  const float b0 = __builtin_bit_cast(float, b0u), b1 = __builtin_bit_cast(float, b1u);
  return kMax ? pick_max<MED3>(b0, b1) : b0 + b1;
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group,
// lane i receives halfword i % 4 of the 8 bytes addressed by lane
// 4 e + i / 4, as its element e (e = 0..3). With lane c of a group
// addressing the 4 dims starting at 4 (c % 4) of token row r0 + c / 4 of a
// row-major tile, lane c gets tokens r0 .. r0+3 of dim c: an MFMA operand
// whose k index runs over tokens.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(
          (__attribute__((address_space(3))) uint8_t*)(const_cast<uint8_t*>(p))));
  return __builtin_bit_cast(bf16x4, v);
}

template <int D, bool FP8, int RT, int NB, int NW, bool LIN = false>
struct Cfg {
  static constexpr int KVB = FP8 ? 1 : 2;      // bytes per cache element
  static constexpr int ROWB = D * KVB;         // bytes per cache row
  static constexpr int LPB = ROWB / 64;        // 16-B loads per lane per 16-token block
  static constexpr int KC = D / 32;            // MFMA k-steps over head_dim
  static constexpr int DT = D / 16;            // 16-dim tiles of the output
  static constexpr int TC = 16 * NB;           // tokens per chunk
  static constexpr int VROW = 2 * D + 32;      // bytes per V row in LDS: 16-B aligned rows,
                                               // 8-dword bank shift per row
  static constexpr int VBYTES = TC * VROW;
  static constexpr int OROW = D + 4;           // floats per row of the merge tile
  static constexpr int OBYTES = 16 * OROW * 4;
  // a wave's private LDS: its V tile (and, with linear loads, its K tile in
  // front of it), which the merge's O tile reuses
  static constexpr int TBYTES = (LIN ? 2 : 1) * VBYTES;
  static constexpr int WBYTES = TBYTES > OBYTES ? TBYTES : OBYTES;
  static constexpr int THREADS = NW * 64;
  static_assert(ROWB % 64 == 0, "row must be a multiple of 64 bytes");
  static_assert(NB == 1 || NB % 2 == 0, "blocks per chunk: 1 or even");
};

// head_dim index of the first of the 8 contiguous dims that lane group j
// feeds to QK^T k-step kc. bf16 rows are loaded 16 B = 8 dims at a time; fp8
// rows 16 B = 16 dims, split into two k-steps. The same map orders Q.
template <bool FP8>
__device__ __forceinline__ constexpr int qk_dim(int kc, int j) {
  return FP8 ? 64 * (kc >> 1) + 16 * j + 8 * (kc & 1) : 32 * kc + 8 * j;
}

// Buffer resources. A raw (unswizzled) buffer load returns zeros for bytes at
// or past num_records without touching memory; the decode sizes each block's
// resource to its live rows, so dead rows and dead blocks read as zeros and
// every step issues the same number of loads.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int32_t kRsrcWord3 = 0x00020000;  // gfx9 family: 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// Values the compiler cannot prove wave-uniform (they pass a per-lane branch)
// but are: pin them to scalar registers so buffer resources stay scalar.
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// 16-byte buffer load. STREAM sets the non-temporal cache policy (each K/V
// byte is read once). In the rows layout it was 1-4% faster for bf16 caches
// and 7-8% slower for fp8 ones; in the linear layout both dtypes take it.
template <bool STREAM = false>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, STREAM ? 2 : 0));
}

// Two lane layouts of a 16-row block of ROWB-byte cache rows, for the
// 16-byte K/V loads:
//  * rows layout: load i of lane (c = lane % 16, j = lane / 16) covers bytes
//    [64 i + 16 j, +16) of row c, so each lane holds MFMA operand pieces of
//    one token row; one load touches 64 bytes of each of 16 rows;
//  * linear layout (LIN): load i of lane l covers bytes [1024 i + 16 l, +16)
//    of the block, row (64 i + l) / (ROWB / 16), so one load reads 1 KB
//    contiguous. HBM serves this layout markedly faster (a streaming probe on
//    MI355X: 7.0-7.2 TB/s with non-temporal loads, against 6.0-6.3 TB/s for
//    the rows layout), and LDS puts the rows in operand order afterwards.
template <int ROWB>
__device__ __forceinline__ int lin_row(int i, int lane) { return (64 * i + lane) / (ROWB / 16); }
template <int ROWB>
__device__ __forceinline__ int lin_col(int i, int lane) { return (16 * (64 * i + lane)) % ROWB; }

// The rows of block blk of a chunk, as loaded in the linear layout, into a
// bf16 LDS tile of VROW-byte rows (fp8 widened exactly to bf16).
template <bool FP8, int ROWB, int LPB, int VROW>
__device__ __forceinline__ void lin_to_tile(uint8_t* tile, int blk, const u32x4 (&w)[LPB], int lane) {
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    uint8_t* dst = tile + (16 * blk + lin_row<ROWB>(i, lane)) * VROW;
    const int col = lin_col<ROWB>(i, lane);
    if constexpr (FP8) {
      *reinterpret_cast<bf16x8*>(dst + 2 * col) = fp8x8_to_bf16(w[i].x, w[i].y);
      *reinterpret_cast<bf16x8*>(dst + 2 * col + 16) = fp8x8_to_bf16(w[i].z, w[i].w);
    } else {
      *reinterpret_cast<u32x4*>(dst + col) = w[i];
    }
  }
}

template <int D, bool FP8, int NB, int SM, int SHR = 0>
struct Stage {
  static constexpr int LPB = D * (FP8 ? 1 : 2) / 64;
  static constexpr int NS = SM == PA_SCALE_PER_TOKEN_HEAD ? NB : 1;
  // blocks of one array this wave loads when SHR waves share the chunk
  static constexpr int NBL = SHR ? 2 * NB / SHR : NB;
  // rows of K and V; with tiles shared by a stream's SHR waves, k holds this
  // wave's share of the chunk (wave r: blocks (r / 2) NBL .. + NBL - 1 of K
  // for even r, of V for odd r) and v is unused
  u32x4 k[NBL][LPB];
  u32x4 v[SHR ? 1 : NB][SHR ? 1 : LPB];
  // per-token scales: lane (c, j) holds those of token 4 j + c % 4 of each
  // block; the four tokens of its S^T column come from its lane quad
  float ks[NS];
  float vs[NS];
};

// One entry of a wave's chunk stream (wave-uniform values). 2 NS - 1 of them
// are in flight per wave, all in scalar registers, so they are kept small:
// the four flags and the kv head share one word, and the context length is
// kept as ctx - q_len (the last key position the first query row sees).
struct Entry {
  // bit 0: the entry exists; 1 / 2: first / last entry of this wave in its
  // segment; 3: the chunk holds tokens (else: merge only); bits 4..: kv head
  int32_t fg;
  int32_t b, cq, te, slot, tc0;
  __device__ __forceinline__ bool live() const { return fg & 1; }
  __device__ __forceinline__ bool first() const { return fg & 2; }
  __device__ __forceinline__ bool last() const { return fg & 4; }
  __device__ __forceinline__ bool data() const { return fg & 8; }
  __device__ __forceinline__ int32_t g() const { return fg >> 4; }
};

struct Cursor {
  int32_t s, s_end, k;
  int32_t b, g, ctx, tb, te, slot;
  int32_t live;
};

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// The live context length of sequence b, read at decode time, replaces the
// plan's snapshot `ctx` of a segment [.., te): the pair's last segment (the
// one ending at the snapshot) runs to the live length, and every segment's
// causal bound follows it. Partitions only set where the work may split, so
// a plan stays valid while sequences grow. A live length below the snapshot
// or past the block table's capacity is reported, and the snapshot kept.
__device__ __forceinline__ void live_context(const DecodeArgs& a, int32_t b, int32_t& te,
                                             int32_t& ctx) {
  const int32_t raw = ldu(a.context_lens, b);
  const int32_t live = raw - a.ctx_offset;
  if (live >= ctx && raw <= a.capacity) {
    if (te == ctx) te = live;
    ctx = live;
  } else {
    atomicOr(a.status + ST_BITS, PA_DEV_BAD_CONTEXT);
  }
}

// Segment record (b, g, tok_begin, tok_end, slot, ctx, pair, 0), one scalar
// load, then the live context length.
__device__ __forceinline__ void cursor_set(Cursor& c, const i32x8& r, int wave, const DecodeArgs& a) {
  c.b = r[0];
  c.g = r[1];
  c.tb = r[2];
  c.te = r[3];
  c.slot = r[4];
  c.ctx = r[5];
  c.k = wave;
  live_context(a, c.b, c.te, c.ctx);
}

__device__ __forceinline__ void cursor_load(Cursor& c, const DecodeArgs& a, int wave) {
  cursor_set(c, ldu(reinterpret_cast<const i32x8*>(a.seg_info), c.s), wave, a);
}

// With SH every stream takes the same number of entries per segment,
// ceil(chunks / NW), the missing chunks as entries without data: the waves
// then meet one workgroup barrier per step.
template <int TC, int NW, bool SH = false>
__device__ __forceinline__ Entry cursor_take(Cursor& c, const DecodeArgs& a, int wave) {
  Entry e;
  if (!c.live) {
    e.fg = e.b = e.cq = e.te = e.slot = e.tc0 = 0;
    return e;
  }
  e.b = c.b;
  e.cq = c.ctx - a.q_len;
  e.te = c.te;
  e.slot = c.slot;
  e.tc0 = c.tb + TC * c.k;
  const bool data = e.tc0 < c.te;
  const bool last = SH ? c.tb + TC * (c.k - wave + NW) >= c.te : !data || c.tb + TC * (c.k + NW) >= c.te;
  e.fg = 1 | (c.k == wave ? 2 : 0) | (last ? 4 : 0) | (data ? 8 : 0) | (c.g << 4);
  if (!last) {
    c.k += NW;
  } else if (++c.s < c.s_end) {
    cursor_load(c, a, wave);
  } else {
    c.live = 0;
  }
  return e;
}

// Block-table entries of an entry's 16-token blocks (one per block: a block
// never crosses a page), or a single entry when the whole chunk lies in one
// page (OPC). Vector loads of a uniform address, issued steps before the K/V
// loads that use them; entries past the row read as 0.
template <int NB, bool OPC>
__device__ __forceinline__ void load_pages(const DecodeArgs& a, const Entry& e, uint32_t (&pg)[NB]) {
  const bool live = e.live() && e.data();
  const rsrc_t r = make_rsrc(a.block_table + static_cast<int64_t>(e.b) * a.max_pages,
                             live ? static_cast<uint32_t>(a.max_pages) * 4u : 0u);
#pragma unroll
  for (int blk = 0; blk < (OPC ? 1 : NB); ++blk) {
    const uint32_t idx = static_cast<uint32_t>(max(e.tc0 + 16 * blk, 0)) >> a.ps_log2;
    pg[blk] = __builtin_amdgcn_raw_buffer_load_b32(r, idx * 4u, 0, 0);
  }
}

template <int D, bool FP8, int NB, int SM, bool OPC, int SHR = 0, bool LIN = false>
__device__ __forceinline__ void issue_kv(const DecodeArgs& a, const Entry& e, const uint32_t (&pgv)[NB],
                                         Stage<D, FP8, NB, SM, SHR>& st, int lane, int rsub = 0) {
  constexpr bool SH = SHR != 0;
  constexpr int ROWB = D * (FP8 ? 1 : 2);
  // non-temporal policy (each byte is read once): bf16 caches always, fp8
  // ones with the linear layout
  constexpr bool NT = !FP8 || LIN;
  // byte offset of load i of this lane inside a 16-row block
  const auto lo = [&](int i) -> uint32_t {
    return LIN ? static_cast<uint32_t>(1024 * i + 16 * lane)
               : static_cast<uint32_t>((lane & 15) * ROWB + 16 * (lane >> 4) + 64 * i);
  };
  constexpr int NBL = Stage<D, FP8, NB, SM, SHR>::NBL;
  // SH: wave r of the stream loads NBL blocks of K (even r) or V (odd r),
  // starting at block (r / 2) NBL
  const uint8_t* const kbase = SH && (rsub & 1) ? a.v_cache : a.k_cache;
  const int blk0 = SH ? (rsub >> 1) * NBL : 0;
  constexpr int LPB = ROWB / 64;
  const int c = lane & 15, j = lane >> 4;
  const int ps_mask = (1 << a.ps_log2) - 1;
  if constexpr (OPC) {
    // the chunk's 16 NB rows are consecutive rows of one page: one resource
    // per array, sized to the rows before the segment end
    int32_t nl = (e.live() && e.data()) ? min(max(e.te - e.tc0, 0), 16 * NB) : 0;
    int32_t page = static_cast<int32_t>(__builtin_amdgcn_readfirstlane(pgv[0]));
    if (a.debug_bounds && nl > 0 && (page < 0 || page >= a.num_pages)) {
      nl = 0;
      atomicOr(a.status + ST_BITS, PA_DEV_BAD_PAGE);
    }
    nl = uni(nl);
    if (nl == 0) page = 0;
    const uint64_t row0 = uni64(cache_row(page, e.g(), e.tc0 & ps_mask, a.num_kv_heads, a.ps_log2));
    const rsrc_t rk = make_rsrc(kbase + row0 * ROWB, static_cast<uint32_t>(nl * ROWB));
    const rsrc_t rv = make_rsrc(a.v_cache + row0 * ROWB, static_cast<uint32_t>(nl * ROWB));
#pragma unroll
    for (int b = 0; b < NBL; ++b)
#pragma unroll
      for (int i = 0; i < LPB; ++i) st.k[b][i] = bload16<NT>(rk, 16 * ROWB * (blk0 + b) + lo(i));
    if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
      const rsrc_t rks = make_rsrc(a.kv_scales + row0, static_cast<uint32_t>(nl * 4));
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
        st.ks[blk] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rks, 4u * (16 * blk + 4 * j + (c & 3)), 0, 0));
    }
    if constexpr (!SH) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < LPB; ++i) st.v[blk][i] = bload16<NT>(rv, 16 * ROWB * blk + lo(i));
    }
    if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
      const uint64_t vplane = static_cast<uint64_t>(a.num_pages) * a.num_kv_heads << a.ps_log2;
      const rsrc_t rvs = make_rsrc(a.kv_scales + vplane + row0, static_cast<uint32_t>(nl * 4));
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
        st.vs[blk] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rvs, 4u * (16 * blk + 4 * j + (c & 3)), 0, 0));
    }
    return;
  }
  // Each 16-token block's resource covers only its rows before the segment
  // end; loads follow the lane layout (rows or linear).
  rsrc_t rk[NB], rv[NB];
  uint64_t row0[NB];
  int32_t nlive[NB];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int32_t t0 = e.tc0 + 16 * blk;
    int32_t nl = (e.live() && e.data()) ? min(max(e.te - t0, 0), 16) : 0;
    int32_t page = static_cast<int32_t>(__builtin_amdgcn_readfirstlane(pgv[blk]));
    if (a.debug_bounds && nl > 0 && (page < 0 || page >= a.num_pages)) {
      nl = 0;
      atomicOr(a.status + ST_BITS, PA_DEV_BAD_PAGE);
    }
    nl = uni(nl);
    if (nl == 0) page = 0;
    row0[blk] = uni64(cache_row(page, e.g(), t0 & ps_mask, a.num_kv_heads, a.ps_log2));
    nlive[blk] = nl;
    rk[blk] = make_rsrc(kbase + row0[blk] * ROWB, static_cast<uint32_t>(nl * ROWB));
    rv[blk] = make_rsrc(a.v_cache + row0[blk] * ROWB, static_cast<uint32_t>(nl * ROWB));
  }
  // K first, then its scales, then V and its scales: the score math waits for
  // K alone while V is still in flight.
#pragma unroll
  for (int b = 0; b < NBL; ++b)
#pragma unroll
    for (int i = 0; i < LPB; ++i) st.k[b][i] = bload16<NT>(rk[SH ? blk0 + b : b], lo(i));
  if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const rsrc_t rks = make_rsrc(a.kv_scales + row0[blk], static_cast<uint32_t>(nlive[blk] * 4));
      st.ks[blk] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, 4u * (4 * j + (c & 3)), 0, 0));
    }
  }
  if constexpr (!SH) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < LPB; ++i) st.v[blk][i] = bload16<NT>(rv[blk], lo(i));
  }
  if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
    const uint64_t vplane = static_cast<uint64_t>(a.num_pages) * a.num_kv_heads << a.ps_log2;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const rsrc_t rvs = make_rsrc(a.kv_scales + vplane + row0[blk], static_cast<uint32_t>(nlive[blk] * 4));
      st.vs[blk] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, 4u * (4 * j + (c & 3)), 0, 0));
    }
  }
}

template <int D, bool FP8, int RT>
__device__ __forceinline__ void load_q(const DecodeArgs& a, const Entry& e, int lane, int row0,
                                       bf16x8 (&qr)[RT * (D / 32)]) {
  constexpr int KC = D / 32;
  const int c = lane & 15, j = lane >> 4;
  const int64_t seq_stride = static_cast<int64_t>(a.q_total) * a.num_q_heads * D;
  const int64_t blk_elems = static_cast<int64_t>(a.q_len) * a.num_q_heads * D;
  const rsrc_t rq = make_rsrc(a.q + e.b * seq_stride, static_cast<uint32_t>(blk_elems * 2));
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // rows past R (MFMA padding) reuse the last real row: finite values whose
    // results are never written
    const int r = min(row0 + 16 * rt + c, a.rows - 1);
    const int i = r / a.group;
    const int h = e.g() * a.group + (r - i * a.group);
    const uint32_t off = static_cast<uint32_t>((i * a.num_q_heads + h) * D) * 2u;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qr[rt * KC + kc] = __builtin_bit_cast(bf16x8, bload16(rq, off + 2u * qk_dim<FP8>(kc, j)));
  }
}

// Log-sum-exp merge of one (row r, 8 dims from d0) unit of split pair (b, g),
// whose n partials (O_s, lse_s) sit in slots base .. base + n - 1: M = max
// lse_s, w_s = exp(lse_s - M), out = sum w_s O_s / sum w_s ("[Kernel][Perf]
// Optimize paged-attention metadata decode", ROCm/FlyDSL PR #910, overview:
// the split reduction kernel), read in slot order. It is latency-bound, so
// the loads of 8 slots go out at once and fold in with a running maximum:
// one round trip for pairs of up to 8 segments. The reduce kernel and the
// fused reduce of the partition pass both call it, so the two give the same
// bits.
constexpr int kReduceBatch = 8;

// COH: the partials were written by other workgroups of the same launch, so
// they are read with agent-scope coherent loads (sc1: past any stale L2 line).
template <int D, bool COH = false>
__device__ __forceinline__ void reduce_unit(const DecodeArgs& a, int base, int n, int b, int g, int r,
                                            int d0) {
  const int R = a.rows;
  const float* lse = a.partial_lse + static_cast<int64_t>(base) * R + r;
  const float* po = a.partial_o + (static_cast<int64_t>(base) * R + r) * D + d0;
  const int64_t so = static_cast<int64_t>(R) * D;  // slot stride in floats
  // COH: resources over the pair's n slots
  const rsrc_t rl = make_rsrc(a.partial_lse + static_cast<int64_t>(base) * R,
                              static_cast<uint32_t>(n * R * 4));
  const rsrc_t ro = make_rsrc(a.partial_o + static_cast<int64_t>(base) * R * D,
                              static_cast<uint32_t>(n * R * D * 4));
  float M = neg_inf(), W = 0.f;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  for (int s0 = 0; s0 < n; s0 += kReduceBatch) {
    float lv[kReduceBatch];
    f32x4 x0[kReduceBatch], x1[kReduceBatch];
#pragma unroll
    for (int t = 0; t < kReduceBatch; ++t) {
      lv[t] = neg_inf();
      x0[t] = x1[t] = f32x4{0, 0, 0, 0};
      if (s0 + t < n) {
        if constexpr (COH) {
          const uint32_t oo = static_cast<uint32_t>(((s0 + t) * R + r) * D + d0) * 4u;
          lv[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                rl, static_cast<uint32_t>((s0 + t) * R + r) * 4u, 0, kSc1));
          x0[t] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, oo, 0, kSc1));
          x1[t] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, oo + 16, 0, kSc1));
        } else {
          lv[t] = lse[(s0 + t) * R];
          x0[t] = *reinterpret_cast<const f32x4*>(po + (s0 + t) * so);
          x1[t] = *reinterpret_cast<const f32x4*>(po + (s0 + t) * so + 4);
        }
      }
    }
    float mb = M;
#pragma unroll
    for (int t = 0; t < kReduceBatch; ++t) mb = fmaxf(mb, lv[t]);
    if (mb == neg_inf()) continue;  // every slot so far is empty for this row
    const float rescale = M == neg_inf() ? 0.f : __builtin_amdgcn_exp2f((M - mb) * kLog2e);
    W *= rescale;
    acc0 *= rescale;
    acc1 *= rescale;
    M = mb;
#pragma unroll
    for (int t = 0; t < kReduceBatch; ++t) {
      const float wgt = __builtin_amdgcn_exp2f((lv[t] - M) * kLog2e);  // 0 for empty slots
      W += wgt;
      acc0 += wgt * x0[t];
      acc1 += wgt * x1[t];
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  acc0 *= inv;
  acc1 *= inv;
  const int qi = r / a.group;
  const int h = g * a.group + (r - qi * a.group);
  const f32x8 f8 = {acc0.x, acc0.y, acc0.z, acc0.w, acc1.x, acc1.y, acc1.z, acc1.w};
  *reinterpret_cast<bf16x8*>(a.out + ((static_cast<int64_t>(b) * a.q_total + qi) * a.num_q_heads + h) *
                                         D + d0) = __builtin_convertvector(f8, bf16x8);
}

// Reduce kernel: one workgroup per (pair, block of 16 query rows); pairs with
// a single segment were finished by the partition pass.
constexpr int kReduceThreads = 256;
constexpr int kReduceRows = 16;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(DecodeArgs a) {
  const int p = blockIdx.x;
  // both loads go out before the first wait
  const int n = ldu(a.nseg, p);
  const int base = ldu(a.seg_base, p);
  if (n <= 1) return;
  const int b = p / a.num_kv_heads;
  const int g = p - b * a.num_kv_heads;
  constexpr int U = D / 8;  // 8-dim units per row
  for (int u = threadIdx.x; u < kReduceRows * U; u += kReduceThreads) {
    const int r = blockIdx.y * kReduceRows + u / U;
    if (r < a.rows) reduce_unit<D>(a, base, n, b, g, r, (u % U) * 8);
  }
}

template <int D, bool FP8, int SM, int RT, int NB, int NW, int NS, int RS, bool OPC, bool SH,
          bool FUSED, bool LIN>
__global__ __launch_bounds__(NW * 64, (NW + 3) / 4) void partition_kernel(DecodeArgs a) {
  // LIN: K/V loaded in the linear lane layout and put in operand order
  // through LDS (private K and V tiles per wave, or the stream's shared tiles)
  using C = Cfg<D, FP8, RT, NB, NW, LIN && !SH>;
  constexpr int ROWB = D * (FP8 ? 1 : 2);
  constexpr int KC = C::KC, DT = C::DT, TC = C::TC, LPB = C::LPB;
  constexpr int NST = NW / RS;  // chunk streams
  static_assert(NS == 2 || NS == 3, "2 or 3 K/V register stages");
  static_assert(NW % RS == 0, "waves split evenly over streams");
  // SH: the RS waves of a stream share the chunk through LDS. Each loads its
  // share of it (wave r: 2 NB / RS blocks of K for even r, of V for odd r),
  // widens fp8 to bf16, and writes it into the stream's bf16 K and V tiles;
  // after a workgroup barrier every wave reads K and V from the tiles for its
  // own rows. So one K/V read serves RS * RT * 16 query rows (up to 256: the
  // long queries of a chunked prefill read the cache once). The tiles
  // alternate between two buffers by step; a segment merge puts the waves' O
  // tiles in the stream's two buffers (its first barrier follows every read
  // of them).
  static_assert(!SH || (RS % 2 == 0 && (2 * NB) % RS == 0 && NB % 2 == 0),
                "shared tiles: an even number of waves, each loading whole blocks");
  constexpr int SHR = SH ? RS : 0;
  constexpr int NBL = Stage<D, FP8, NB, SM, SHR>::NBL;
  constexpr int SHBUF = 2 * C::VBYTES;  // one buffer: K tile, then V tile
  static_assert(!SH || RS * C::OBYTES <= 2 * SHBUF, "merge tiles fit the stream's buffers");
  // Prefetch the next segment's Q into registers when they are affordable.
  constexpr bool QPF = RT == 1 || (RT == 2 && NW <= 4);
  // Shared-tile kernels are bound by instruction issue, so their row sums
  // come out of the PV MFMAs: one more output tile whose V rows are all ones
  // (the matrix cores idle most of the step) instead of a VALU add per
  // probability. The sums are then those of the bf16 probabilities the PV
  // products take, the values O is the weighted sum of.
  constexpr bool ONES = SH;

  __shared__ __attribute__((aligned(16))) uint8_t lds_waves[SH ? NST * 2 * SHBUF : NW * C::WBYTES];
  __shared__ float st_m[NW][RT * 16];
  __shared__ float st_l[NW][RT * 16];
  __shared__ int32_t s_last[2];  // fused reduce: this workgroup arrived last at pend[0] / pend[1]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stream = wave / RS, rsub = wave - stream * RS;
  const int qrow0 = 16 * RT * rsub;  // first query row of this wave
  const int c = lane & 15, j = lane >> 4;
  const int w = blockIdx.x;

  // the workgroup's header: segment range and first segment, one load
  Cursor cur;
  // FUSED: the split pairs this workgroup writes partials of (-1: none). Only
  // a range's first and last segments can belong to split pairs (a segment
  // between them holds a whole pair), and the plan has both records.
  int32_t pend0 = -1, pend1 = -1;
  {
    const i32x8 h0 = ldu(reinterpret_cast<const i32x8*>(a.wg_head), 2 * w);
    const i32x8 h1 = ldu(reinterpret_cast<const i32x8*>(a.wg_head), 2 * w + 1);
    cur.s = h0[0];
    cur.s_end = h1[0];
    if (cur.s >= cur.s_end) return;
    cur.live = 1;
    const i32x8 r = {h0[1], h0[2], h0[3], h0[4], h0[5], h0[6], h0[7], 0};
    if constexpr (FUSED) {
      const i32x8 rl = ldu(reinterpret_cast<const i32x8*>(a.seg_info), cur.s_end - 1);
      if (r[4] >= 0) pend0 = r[6];                            // first segment: slot, pair
      if (cur.s_end - 1 > cur.s && rl[4] >= 0) {               // a last segment of its own
        if (pend0 < 0) pend0 = rl[6]; else pend1 = rl[6];
      }
    }
    cursor_set(cur, r, stream, a);
  }

  // Softmax scale in the exp2 domain; per-tensor scales are folded in here
  // (K scale into the scores, V scale into the output).
  float qk_f = a.qk_scale_log2;
  float out_f = a.out_scale;
  if constexpr (SM == PA_SCALE_PER_TENSOR) {
    qk_f *= ldu(a.kv_scales, 0);
    out_f = ldu(a.kv_scales, 1);
  }

  // Query index of each of this lane's rows (rows past R see every key).
  int row_q[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = qrow0 + 16 * rt + c;
    row_q[rt] = r < a.rows ? r / a.group : a.q_len;
  }

  uint8_t* const wlds = lds_waves + (SH ? 0 : wave * C::WBYTES);
  // SH: buffer p of stream s; the step's buffer alternates (par)
  const auto sh_buf = [&](int s_, int p) { return lds_waves + (s_ * 2 + p) * SHBUF; };
  int par = 0;

  // The wave's chunk stream: ev[0] is computed, ev[1 .. NS-1] have K/V in
  // flight, ev[NS .. 2NS-2] have block-table pages in flight. Pages are
  // loaded NS-1 steps before the K/V loads that use them: vector loads
  // retire in order, so waiting for a page then never waits for K/V loads
  // that are still ahead of the math.
  constexpr int NE = 2 * NS - 1;
  Entry ev[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) ev[k] = cursor_take<TC, NST, SH>(cur, a, stream);

  bf16x8 q[RT * KC];
  bf16x8 qn[QPF ? RT * KC : 1];
  Stage<D, FP8, NB, SM, SHR> st[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) st[k] = {};
  // pages of stream entry m live in pg[(m + 2) % NS] (NS = 3) / pg[m % 2]
  uint32_t pg[NS][NB];
  constexpr auto pslot = [](int m) { return ((m - 2 * NS + 2) % NS + NS) % NS; };

  // prologue, in the steady state's issue order (so that every later wait
  // has the same number of younger loads on every path): the pages of the
  // first NS-1 entries, Q of entry 0, then for k = 0 .. NS-2 the pages of
  // entry NS-1+k and the K/V of entry k
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) load_pages<NB, OPC>(a, ev[k], pg[pslot(k)]);
  if constexpr (QPF) load_q<D, FP8, RT>(a, ev[0], lane, qrow0, qn);
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {
    load_pages<NB, OPC>(a, ev[NS - 1 + k], pg[pslot(NS - 1 + k)]);
    issue_kv<D, FP8, NB, SM, OPC, SHR, LIN>(a, ev[k], pg[pslot(k)], st[k], lane, rsub);
  }

  float m[RT], l[RT];
  f32x4 o[DT][RT];
  f32x4 ol[ONES ? RT : 1];  // ONES: the row sums, in every element
  const bf16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};

  // One step of a wave's pipeline, computing ev[0] from stage CUR. Issue
  // order: pages of ev[NE-1], Q of ev[1] if it opens a segment, K/V of
  // ev[NS-1] into the stage before CUR; then the math on ev[0], whose K/V
  // were issued NS-1 steps earlier.
  auto step = [&](auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr int ISS = (CUR + NS - 1) % NS;
    Stage<D, FP8, NB, SM, SHR>& cs = st[CUR];
    const Entry& e0 = ev[0];
    if (e0.first()) {
      if constexpr (QPF) {
#pragma unroll
        for (int x = 0; x < RT * KC; ++x) q[x] = qn[x];
      } else {
        load_q<D, FP8, RT>(a, e0, lane, qrow0, q);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        m[rt] = neg_inf();
        l[rt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][rt] = f32x4{0, 0, 0, 0};
        if constexpr (ONES) ol[rt] = f32x4{0, 0, 0, 0};
      }
    }
    load_pages<NB, OPC>(a, ev[NE - 1], pg[CUR]);
    if constexpr (QPF) {
      if (ev[1].live() && ev[1].first()) load_q<D, FP8, RT>(a, ev[1], lane, qrow0, qn);
    }
    issue_kv<D, FP8, NB, SM, OPC, SHR, LIN>(a, ev[NS - 1], pg[(CUR + 1) % NS], st[ISS], lane, rsub);

    // SH: this wave's share of the chunk, widened, into the stream's tiles;
    // every wave meets the barrier once per step
    uint8_t* const ktile = SH ? sh_buf(stream, par) : wlds;
    uint8_t* const vtile = SH ? sh_buf(stream, par) + C::VBYTES : (LIN ? wlds + C::VBYTES : wlds);
    if constexpr (!SH && LIN) {
      // this wave's chunk, in operand order, into its private K and V tiles
      // (a wave's LDS accesses complete in order: no barrier)
      if (e0.data()) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          lin_to_tile<FP8, ROWB, LPB, C::VROW>(ktile, blk, cs.k[blk], lane);
          lin_to_tile<FP8, ROWB, LPB, C::VROW>(vtile, blk, cs.v[blk], lane);
        }
      }
    }
    if constexpr (SH) {
      if (e0.data()) {
        uint8_t* const mine = sh_buf(stream, par) + (rsub & 1) * C::VBYTES;
        const int blk0 = (rsub >> 1) * NBL;
        if constexpr (LIN) {
#pragma unroll
          for (int b = 0; b < NBL; ++b) lin_to_tile<FP8, ROWB, LPB, C::VROW>(mine, blk0 + b, cs.k[b], lane);
        } else
#pragma unroll
        for (int b = 0; b < NBL; ++b) {
          uint8_t* row = mine + (16 * (blk0 + b) + c) * C::VROW;
#pragma unroll
          for (int i = 0; i < LPB; ++i) {
            const u32x4 wv = cs.k[b][i];
            if constexpr (FP8) {
              *reinterpret_cast<bf16x8*>(row + 128 * i + 32 * j) = fp8x8_to_bf16(wv.x, wv.y);
              *reinterpret_cast<bf16x8*>(row + 128 * i + 32 * j + 16) = fp8x8_to_bf16(wv.z, wv.w);
            } else {
              *reinterpret_cast<u32x4*>(row + 64 * i + 16 * j) = wv;
            }
          }
        }
      }
      __syncthreads();
    }

    if (e0.data()) {
      constexpr bool per_tok = SM == PA_SCALE_PER_TOKEN_HEAD;
      // ---- S^T = K Q^T: lane holds tokens 16 blk + 4 j + i of row 16 rt + c
      f32x4 s[NB][RT];
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) s[blk][rt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          bf16x8 kf;
          if constexpr (SH || LIN) {
            kf = *reinterpret_cast<const bf16x8*>(ktile + (16 * blk + c) * C::VROW +
                                                  2 * qk_dim<FP8>(kc, j));
          } else if constexpr (FP8) {
            const u32x4 wv = cs.k[blk][kc >> 1];
            kf = (kc & 1) ? fp8x8_to_bf16(wv.z, wv.w) : fp8x8_to_bf16(wv.x, wv.y);
          } else {
            kf = __builtin_bit_cast(bf16x8, cs.k[blk][kc]);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            s[blk][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, q[rt * KC + kc], s[blk][rt], 0, 0, 0);
        }
      }

      // ---- scale, causal mask, online softmax (exp2 domain). Keys past the
      // segment end were read as zeros; the mask drops them.
      // Token 16 blk + 4 j + i of the chunk is visible to a row when
      // 16 blk + i <= lim - tc0 - 4 j: one compare per score, skipped (a
      // wave-uniform branch) in chunks that no row masks.
      const bool full = (e0.tc0 + TC <= e0.te) && (e0.tc0 + TC - 1 <= e0.cq);
      // score factor per block: the softmax scale, times the lane quad's
      // per-token K scales
      float qk[NB];
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) qk[blk] = per_tok ? cs.ks[blk] * qk_f : qk_f;
      float pv[NB][RT][4];
      float pl[ONES && per_tok ? NB : 1][RT][4];  // ONES, per-token: p before the V scale
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float x[NB][4];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[blk][i] = s[blk][rt][i] * (per_tok ? quad_bcast(qk[blk], i) : qk[blk]);
        }
        if (!full) {
          const int vis = min(e0.te - 1, e0.cq + row_q[rt]) - e0.tc0 - 4 * j;
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[blk][i] = 16 * blk + i <= vis ? x[blk][i] : neg_inf();
          }
        }
        float cm = neg_inf();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) cm = fmaxf(cm, x[blk][i]);
        }
        cm = rows_reduce<true, SH>(cm);
        // Lazy rescale: keep the running max m while every row's chunk max
        // stays within 2^kSlack of it (then p <= 2^kSlack, exact enough in
        // fp32 and bf16); move it, rescaling l and O, only when some row of
        // the wave exceeds that (a wave-uniform branch).
        if (__builtin_amdgcn_ballot_w64(cm > m[rt] + kSlack) != 0) {
          const float mn = fmaxf(m[rt], cm);
          const float alpha = __builtin_amdgcn_exp2f(m[rt] - (mn == neg_inf() ? 0.f : mn));
          l[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
          if constexpr (ONES) ol[rt] *= alpha;
          m[rt] = mn;
        }
        const float mu = m[rt] == neg_inf() ? 0.f : m[rt];
        float ps = 0.f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[blk][i] - mu);
            if constexpr (!ONES) ps += p;
            if constexpr (ONES && per_tok) pl[blk][rt][i] = p;
            pv[blk][rt][i] = per_tok ? p * quad_bcast(cs.vs[blk], i) : p;
          }
        }
        if constexpr (!ONES) l[rt] += ps;
      }

      // ---- V rows -> wave-private LDS tile (row-major bf16); SH, LIN:
      // already in the tile
      if constexpr (!SH && !LIN) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          uint8_t* vrow = wlds + (16 * blk + c) * C::VROW;
#pragma unroll
          for (int i = 0; i < LPB; ++i) {
            const u32x4 wv = cs.v[blk][i];
            if constexpr (FP8) {
              uint8_t* dst = vrow + 128 * i + 32 * j;
              *reinterpret_cast<bf16x8*>(dst + 0) = fp8x8_to_bf16(wv.x, wv.y);
              *reinterpret_cast<bf16x8*>(dst + 16) = fp8x8_to_bf16(wv.z, wv.w);
            } else {
              *reinterpret_cast<u32x4*>(vrow + 64 * i + 16 * j) = wv;
            }
          }
        }
      }

      // ---- O^T += V^T P^T (token order inside a k-step is the S^T lane
      // order). Lane (c, j) addresses token row 4 j + c / 4 (+16 per block),
      // dims 16 dt + 4 (c % 4): the transpose read hands it tokens
      // 4 j .. 4 j + 3 of dim 16 dt + c.
      const uint8_t* vt = vtile + (4 * j + (c >> 2)) * C::VROW + 8 * (c & 3);
      if constexpr (NB == 1) {
        bf16x4 bp[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const f32x4 f = {pv[0][rt][0], pv[0][rt][1], pv[0][rt][2], pv[0][rt][3]};
          bp[rt] = __builtin_convertvector(f, bf16x4);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x4 A = lds_read_tr(vt + 32 * dt);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, bp[rt], o[dt][rt], 0, 0, 0);
        }
      } else {
        bf16x8 bp[NB / 2][RT];
#pragma unroll
        for (int qq = 0; qq < NB / 2; ++qq) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f32x8 f = {pv[2 * qq][rt][0], pv[2 * qq][rt][1], pv[2 * qq][rt][2], pv[2 * qq][rt][3],
                             pv[2 * qq + 1][rt][0], pv[2 * qq + 1][rt][1], pv[2 * qq + 1][rt][2],
                             pv[2 * qq + 1][rt][3]};
            bp[qq][rt] = __builtin_convertvector(f, bf16x8);
          }
        }
        if constexpr (ONES) {
          // row sums: ones^T P^T (per-token: the probabilities before the V
          // scale)
#pragma unroll
          for (int qq = 0; qq < NB / 2; ++qq) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              bf16x8 b = bp[qq][rt];
              if constexpr (per_tok) {
                const f32x8 f = {pl[2 * qq][rt][0], pl[2 * qq][rt][1], pl[2 * qq][rt][2], pl[2 * qq][rt][3],
                                 pl[2 * qq + 1][rt][0], pl[2 * qq + 1][rt][1], pl[2 * qq + 1][rt][2],
                                 pl[2 * qq + 1][rt][3]};
                b = __builtin_convertvector(f, bf16x8);
              }
              ol[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, b, ol[rt], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int qq = 0; qq < NB / 2; ++qq) {
            const bf16x4 lo = lds_read_tr(vt + (32 * qq) * C::VROW + 32 * dt);
            const bf16x4 hi = lds_read_tr(vt + (32 * qq + 16) * C::VROW + 32 * dt);
            const bf16x8 A = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bp[qq][rt], o[dt][rt], 0, 0, 0);
          }
        }
      }
    }

    if (e0.last()) {
      // ---- merge the NW waves' (max, sum, O) of this segment
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float v = l[rt];
        if constexpr (ONES) v = ol[rt][0];  // the full row sum, in every lane of column c
        else v = rows_reduce<false>(v);
        if (j == 0) {
          st_m[wave][16 * rt + c] = m[rt];
          st_l[wave][16 * rt + c] = v;
        }
      }
      // SH: the O tiles overwrite the stream's K/V tiles, which the stream's
      // other waves may still be reading. Otherwise each wave's O tile takes
      // its own V tile, whose reads it has issued already (a wave's LDS
      // accesses complete in order): one barrier per row tile then publishes
      // maxima, sums and O together.
      if constexpr (SH) __syncthreads();
      const int pair_rows = a.rows;
      // rows are merged over the NST waves that hold them: waves s RS + rsub;
      // each wave's O is stored unscaled and weighted by exp2(m_s - M) below
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float* ob = reinterpret_cast<float*>(SH ? sh_buf(stream, 0) + rsub * C::OBYTES : wlds);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(ob + c * C::OROW + 16 * dt + 4 * j) = o[dt][rt];
        __syncthreads();
        constexpr int UNITS = 16 * (D / 8);  // (row, 8 dims) units of one wave's tile
        for (int u = threadIdx.x; u < RS * UNITS; u += C::THREADS) {
          const int rs = u / UNITS;
          const int row = (u - rs * UNITS) / (D / 8);
          const int d0 = (u - rs * UNITS - row * (D / 8)) * 8;
          const int lr = 16 * rt + row;  // row inside the waves' tiles
          const int r = 16 * RT * rs + lr;
          if (r < pair_rows) {
            float Mr = neg_inf();
#pragma unroll
            for (int s = 0; s < NST; ++s) Mr = fmaxf(Mr, st_m[s * RS + rs][lr]);
            const float Mru = Mr == neg_inf() ? 0.f : Mr;
            float L = 0.f;
            f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < NST; ++s) {
              const int ww = s * RS + rs;
              const float wgt = __builtin_amdgcn_exp2f(st_m[ww][lr] - Mru);
              L += st_l[ww][lr] * wgt;
              const uint8_t* obw = SH ? sh_buf(s, 0) + rs * C::OBYTES : lds_waves + ww * C::WBYTES;
              const float* src = reinterpret_cast<const float*>(obw) + row * C::OROW + d0;
              acc0 += *reinterpret_cast<const f32x4*>(src) * wgt;
              acc1 += *reinterpret_cast<const f32x4*>(src + 4) * wgt;
            }
            const float inv = L > 0.f ? out_f / L : 0.f;
            acc0 *= inv;
            acc1 *= inv;
            if (e0.slot < 0) {
              const int qi = r / a.group;
              const int h = e0.g() * a.group + (r - qi * a.group);
              const f32x8 f8 = {acc0.x, acc0.y, acc0.z, acc0.w, acc1.x, acc1.y, acc1.z, acc1.w};
              const bf16x8 ob8 = __builtin_convertvector(f8, bf16x8);
              *reinterpret_cast<bf16x8*>(a.out + ((static_cast<int64_t>(e0.b) * a.q_total + qi) *
                                                      a.num_q_heads + h) * D + d0) = ob8;
            } else if constexpr (FUSED) {
              // agent-scope stores: the pair's last workgroup reads them
              const rsrc_t ro = make_rsrc(a.partial_o + static_cast<int64_t>(e0.slot) * pair_rows * D,
                                          static_cast<uint32_t>(pair_rows * D * 4));
              const uint32_t oo = static_cast<uint32_t>(r * D + d0) * 4u;
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc0), ro, oo, 0, kSc1);
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc1), ro, oo + 16, 0, kSc1);
              if (d0 == 0) {
                const rsrc_t rl = make_rsrc(a.partial_lse + static_cast<int64_t>(e0.slot) * pair_rows,
                                            static_cast<uint32_t>(pair_rows * 4));
                const float lse = L > 0.f ? (Mru + __log2f(L)) * kLn2 : neg_inf();
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int32_t, lse), rl,
                                                      static_cast<uint32_t>(r) * 4u, 0, kSc1);
              }
            } else {
              float* dst = a.partial_o + (static_cast<int64_t>(e0.slot) * pair_rows + r) * D + d0;
              *reinterpret_cast<f32x4*>(dst) = acc0;
              *reinterpret_cast<f32x4*>(dst + 4) = acc1;
              if (d0 == 0)
                a.partial_lse[static_cast<int64_t>(e0.slot) * pair_rows + r] =
                    L > 0.f ? (Mru + __log2f(L)) * kLn2 : neg_inf();
            }
          }
        }
        __syncthreads();
      }
    }

#pragma unroll
    for (int k = 0; k < NE - 1; ++k) ev[k] = ev[k + 1];
    ev[NE - 1] = cursor_take<TC, NST, SH>(cur, a, stream);
    if constexpr (SH) par ^= 1;
  };

  for (;;) {
    step(std::integral_constant<int, 0>{});
    if (!ev[0].live()) break;
    step(std::integral_constant<int, 1>{});
    if (!ev[0].live()) break;
    if constexpr (NS == 3) {
      step(std::integral_constant<int, 2>{});
      if (!ev[0].live()) break;
    }
  }

  // Fused reduce (PA_FLAG_FUSED_REDUCE, the FUSED instantiations). The
  // workgroup wrote its split pairs' partials with agent-scope stores (sc1:
  // written through to where every XCD sees them). Once its loads are over,
  // every wave waits for its stores; then wave 0 counts the workgroup's
  // arrival at each such pair with a device-scope vector atomic add. The
  // workgroup that arrives last at a pair merges the pair's partials, read
  // with agent-scope loads (sc1: never a stale L2 line), with the reduce
  // kernel's arithmetic in slot order, and clears the pair's counter for the
  // next decode on the same plan. No cache-wide write-back or invalidation is
  // needed, and the waits sit after the last K/V loads.
  if constexpr (FUSED) {
    if (pend0 < 0) return;
    // segment counts and slot bases of the pending pairs: scalar loads whose
    // latency overlaps the wait for the partial stores
    const int n0 = ldu(a.nseg, pend0), base0 = ldu(a.seg_base, pend0);
    const int n1 = pend1 >= 0 ? ldu(a.nseg, pend1) : 0, base1 = pend1 >= 0 ? ldu(a.seg_base, pend1) : 0;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (wave == 0) {
      const int npend = pend1 >= 0 ? 2 : 1;
      if (lane < npend) {
        const int32_t pair = lane == 0 ? pend0 : pend1;
        const int32_t before = __hip_atomic_fetch_add(a.counters + pair, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        s_last[lane] = before == (lane == 0 ? n0 : n1) - 1 ? 1 : 0;
      }
    }
    __syncthreads();
    for (int k = 0; k < 2; ++k) {
      const int32_t pair = k == 0 ? pend0 : pend1;
      if (pair < 0 || !s_last[k]) continue;
      const int b = pair / a.num_kv_heads;
      const int g = pair - b * a.num_kv_heads;
      const int n = k == 0 ? n0 : n1;
      const int base = k == 0 ? base0 : base1;
      constexpr int U = D / 8;
      for (int u = threadIdx.x; u < a.rows * U; u += C::THREADS)
        reduce_unit<D, true>(a, base, n, b, g, u / U, (u % U) * 8);
      if (threadIdx.x == 0) a.counters[pair] = 0;
    }
  }
}

// Test support: the partition pass's own page loader, alone. Workgroup
// (s, y) takes segment s of the plan (with the live context length, as the
// partition pass does) and its chunks y, y + gridDim.y, ...; for each it runs
// load_pages and issue_kv of one instantiation, exactly as a chunk stream
// entry would, and writes the registers back out by the lane layout the math
// takes them in (load i of a lane holds the row and bytes lin_row / lin_col
// give, or in the rows layout bytes [64 i + 16 j, +16) of row 16 blk + c),
// and per-token scales of token 16 blk + 4 j + c % 4.
// Rows t < te go to [pair][t] of k_out / v_out / scales_out; rows past the
// segment's end must have loaded as zeros, and any that did not set
// PA_DEV_DEBUG_DEAD_ROW. With shared tiles (SHR waves per stream) wave r of
// the workgroup loads its share: K (even r) or V (odd r), blocks from
// (r / 2) * NBL.
template <int D, bool FP8, int SM, int NB, bool OPC, int SHR, bool LIN>
__global__ __launch_bounds__(64 * (SHR ? SHR : 1)) void loader_kernel(DecodeArgs a, uint8_t* k_out,
                                                                      uint8_t* v_out, float* s_out) {
  constexpr int ROWB = D * (FP8 ? 1 : 2);
  constexpr int LPB = ROWB / 64;
  constexpr int TC = 16 * NB;
  constexpr bool SH = SHR != 0;
  constexpr int NBL = Stage<D, FP8, NB, SM, SHR>::NBL;
  const int lane = threadIdx.x & 63;
  const int rsub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int32_t seg = blockIdx.x;
  if (seg >= ldu(a.status, ST_SEGS)) return;
  const i32x8 r = ldu(reinterpret_cast<const i32x8*>(a.seg_info), seg);
  int32_t te = r[3], ctx = r[5];
  live_context(a, r[0], te, ctx);
  const int64_t base = static_cast<int64_t>(r[6]) * a.capacity;  // pair's first output row
  const int64_t plane = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.capacity;
  for (int32_t k = blockIdx.y;; k += gridDim.y) {
    Entry e;
    e.tc0 = r[2] + TC * k;
    if (e.tc0 >= te) break;
    e.fg = 1 | 8 | (r[1] << 4);
    e.b = r[0];
    e.cq = ctx - a.q_len;
    e.te = te;
    e.slot = r[4];
    uint32_t pg[NB];
    load_pages<NB, OPC>(a, e, pg);
    Stage<D, FP8, NB, SM, SHR> st = {};
    issue_kv<D, FP8, NB, SM, OPC, SHR, LIN>(a, e, pg, st, lane, rsub);
    // load i of this lane: row and byte of the block (rows or linear layout)
    const auto put = [&](uint8_t* out, int blk, const u32x4 (&w)[LPB]) {
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        const int row = LIN ? lin_row<ROWB>(i, lane) : c;
        const int col = LIN ? lin_col<ROWB>(i, lane) : 64 * i + 16 * j;
        const int32_t t = e.tc0 + 16 * blk + row;
        if (t < te) {
          *reinterpret_cast<u32x4*>(out + (base + t) * ROWB + col) = w[i];
        } else if (w[i].x | w[i].y | w[i].z | w[i].w) {
          atomicOr(a.status + ST_BITS, PA_DEV_DEBUG_DEAD_ROW);
        }
      }
    };
    if constexpr (SH) {
      uint8_t* const out = (rsub & 1) ? v_out : k_out;
      const int blk0 = (rsub >> 1) * NBL;
#pragma unroll
      for (int b = 0; b < NBL; ++b) put(out, blk0 + b, st.k[b]);
    } else {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        put(k_out, blk, st.k[blk]);
        put(v_out, blk, st.v[blk]);
      }
    }
    if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
      if (rsub == 0 && c < 4) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          const int32_t t = e.tc0 + 16 * blk + 4 * j + c;
          if (t < te) {
            s_out[base + t] = st.ks[blk];
            s_out[plane + base + t] = st.vs[blk];
          } else if ((__builtin_bit_cast(uint32_t, st.ks[blk]) | __builtin_bit_cast(uint32_t, st.vs[blk])) != 0) {
            atomicOr(a.status + ST_BITS, PA_DEV_DEBUG_DEAD_ROW);
          }
        }
      }
    }
  }
}

template <int D, bool FP8, int SM, int NB, bool OPC, int SHR, bool LIN>
hipError_t launch_loader_t(const DecodeArgs& a, int max_segs, uint8_t* k_out, uint8_t* v_out,
                           float* s_out, hipStream_t s) {
  const int chunks = (a.capacity + 16 * NB - 1) / (16 * NB);
  const dim3 grid(max_segs, chunks < 1024 ? chunks : 1024);
  hipLaunchKernelGGL((loader_kernel<D, FP8, SM, NB, OPC, SHR, LIN>), grid, dim3(64 * (SHR ? SHR : 1)),
                     0, s, a, k_out, v_out, s_out);
  return hipGetLastError();
}

template <int D, bool FP8, int SM, int RT, int NB, int NW, int NS, int RS, bool OPC, bool SH, bool LIN>
hipError_t launch_partition_t(const DecodeArgs& a, int grid, hipStream_t s) {
  // the fused reduce is an instantiation of its own, so the separate-reduce
  // kernels carry none of its code
  if (a.counters != nullptr)
    hipLaunchKernelGGL((partition_kernel<D, FP8, SM, RT, NB, NW, NS, RS, OPC, SH, true, LIN>),
                       dim3(grid), dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((partition_kernel<D, FP8, SM, RT, NB, NW, NS, RS, OPC, SH, false, LIN>),
                       dim3(grid), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const DecodeArgs&, int, hipStream_t);
using LoaderFn = hipError_t (*)(const DecodeArgs&, int, uint8_t*, uint8_t*, float*, hipStream_t);

struct VariantEntry {
  Variant v;
  LaunchFn fn;
  LoaderFn loader;  // the same instantiation's page loader, alone (test support)
};

// K/V lane layout of every instantiation: linear (1 KB contiguous per load).
// Building with -DPA_LINEAR_LOADS=0 selects the rows layout instead, for
// measuring one against the other; the library's build and its tests use the
// linear layout only.
#ifndef PA_LINEAR_LOADS
#define PA_LINEAR_LOADS 1
#endif
constexpr bool kLin = PA_LINEAR_LOADS != 0;
#define PA_V(D, F, SM, RT, NB, NW, NS, RS, OPC)                                                  \
  {{D, F, SM, RT * RS, NB, NW, NS, OPC, 0},                                                      \
   launch_partition_t<D, F != 0, SM, RT, NB, NW, NS, RS, OPC != 0, false, kLin>,                \
   launch_loader_t<D, F != 0, SM, NB, OPC != 0, 0, kLin>}
#define PA_VS(D, F, SM, RT, NB, NW, NS, RS, OPC)                                                 \
  {{D, F, SM, RT * RS, NB, NW, NS, OPC, RS},                                                     \
   launch_partition_t<D, F != 0, SM, RT, NB, NW, NS, RS, OPC != 0, true, kLin>,                 \
   launch_loader_t<D, F != 0, SM, NB, OPC != 0, RS, kLin>}
const VariantEntry kVariants[] = {
    // head dim, fp8, scale mode, row tiles per wave, 16-token blocks per
    // chunk, waves, K/V stages, waves per chunk stream, one page per chunk;
    // PA_VS: the stream's two waves share the chunk's K and V tiles in LDS
    PA_V(128, 0, 0, 1, 2, 4, 3, 1, 0), PA_V(128, 0, 0, 2, 2, 4, 3, 1, 0), PA_V(128, 0, 0, 4, 2, 4, 2, 1, 0),
    PA_V(128, 0, 0, 1, 2, 4, 3, 1, 1), PA_V(128, 0, 0, 2, 2, 4, 3, 1, 1), PA_V(128, 0, 0, 4, 2, 4, 2, 1, 1),
    PA_V(256, 0, 0, 1, 1, 4, 3, 1, 0), PA_V(256, 0, 0, 2, 1, 4, 2, 1, 0),
    PA_V(128, 1, 1, 1, 2, 8, 2, 1, 0), PA_V(128, 1, 1, 2, 2, 8, 2, 1, 0), PA_VS(128, 1, 1, 2, 2, 8, 2, 2, 0),
    PA_V(128, 1, 1, 1, 2, 8, 2, 1, 1), PA_V(128, 1, 1, 2, 2, 8, 2, 1, 1), PA_VS(128, 1, 1, 2, 2, 8, 2, 2, 1),
    PA_V(128, 1, 2, 1, 2, 8, 2, 1, 0), PA_V(128, 1, 2, 2, 2, 8, 2, 1, 0), PA_VS(128, 1, 2, 2, 2, 8, 2, 2, 0),
    PA_V(128, 1, 2, 1, 2, 8, 2, 1, 1), PA_V(128, 1, 2, 2, 2, 8, 2, 1, 1), PA_VS(128, 1, 2, 2, 2, 8, 2, 2, 1),
    PA_V(256, 1, 1, 1, 2, 4, 3, 1, 0), PA_V(256, 1, 1, 2, 1, 4, 2, 1, 0),
    PA_V(256, 1, 2, 1, 2, 4, 3, 1, 0), PA_V(256, 1, 2, 2, 1, 4, 2, 1, 0),
    // long queries (chunked prefill): 128 or 256 rows per kv head at head
    // dim 128, 64 at 256, all sharing one read of each chunk
    PA_VS(128, 0, 0, 2, 2, 8, 2, 4, 0), PA_VS(128, 0, 0, 2, 2, 8, 2, 4, 1),
    PA_VS(128, 0, 0, 2, 4, 8, 2, 8, 0), PA_VS(128, 0, 0, 2, 4, 8, 2, 8, 1),
    PA_VS(128, 1, 1, 2, 2, 8, 2, 4, 0), PA_VS(128, 1, 1, 2, 2, 8, 2, 4, 1),
    PA_VS(128, 1, 1, 2, 4, 8, 2, 8, 0), PA_VS(128, 1, 1, 2, 4, 8, 2, 8, 1),
    PA_VS(128, 1, 2, 2, 2, 8, 2, 4, 0), PA_VS(128, 1, 2, 2, 2, 8, 2, 4, 1),
    PA_VS(128, 1, 2, 2, 4, 8, 2, 8, 0), PA_VS(128, 1, 2, 2, 4, 8, 2, 8, 1),
    PA_VS(256, 0, 0, 1, 2, 8, 2, 4, 0), PA_VS(256, 1, 1, 1, 2, 8, 2, 4, 0),
    PA_VS(256, 1, 2, 1, 2, 8, 2, 4, 0),
};
#undef PA_V
#undef PA_VS

}  // namespace

int num_variants() { return static_cast<int>(sizeof(kVariants) / sizeof(kVariants[0])); }

const Variant& variant(int i) { return kVariants[i].v; }

int pick_variant(int head_dim, int fp8, int scale_mode, int rows, int page_size, int partition) {
  const int rt = (rows + 15) / 16;
  int best = -1;
  for (int i = 0; i < num_variants(); ++i) {
    const Variant& v = kVariants[i].v;
    if (v.head_dim != head_dim || v.fp8 != fp8 || v.scale_mode != scale_mode || v.row_tiles < rt)
      continue;
    // one page per chunk: chunks start at multiples of the chunk length (a
    // partition is a whole number of chunks) and a page holds whole chunks
    const int tc = 16 * v.blocks;
    if (v.one_page && (page_size < tc || partition % tc != 0)) continue;
    if (best < 0 || v.row_tiles < kVariants[best].v.row_tiles ||
        (v.row_tiles == kVariants[best].v.row_tiles && v.one_page > kVariants[best].v.one_page))
      best = i;
  }
  return best;
}

hipError_t launch_partition(int vi, const DecodeArgs& a, int grid, hipStream_t s) {
  return kVariants[vi].fn(a, grid, s);
}

hipError_t launch_reduce(const DecodeArgs& a, int head_dim, int num_pairs, hipStream_t s) {
  const dim3 grid(num_pairs, (a.rows + kReduceRows - 1) / kReduceRows);
  if (head_dim == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(kReduceThreads), 0, s, a);
  else
    hipLaunchKernelGGL(reduce_kernel<256>, grid, dim3(kReduceThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_loader(int vi, const DecodeArgs& a, int max_segs, uint8_t* k_out,
                         uint8_t* v_out, float* scales_out, hipStream_t s) {
  return kVariants[vi].loader(a, max_segs, k_out, v_out, scales_out, s);
}

}  // namespace pa

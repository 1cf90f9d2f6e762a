// KV-cache append: the write side of the paged cache the decode reads.
//
// The decode reads K and V page by page through the block table (Ascend/
// RecSDK issue #1281, "背景与优化特性") from an fp8 cache quantised per token
// and head or per tensor ("[Kernel][Perf] Optimize paged-attention metadata
// decode", ROCm/FlyDSL PR #910, "Pull request overview"). This kernel puts the
// appended tokens there: token i of sequence b, at position
// t = ctx_b - q_len + i, goes to page block_table[b, t / ps], slot t % ps, of
// its kv head. fp8 rows are stored as e4m3fn(clamp(x / scale, +-448)),
// rounded to nearest even, with scale = max |x| / 448 per token and head (1
// for an all-zero row) or the caller's per-tensor scale; every float step is
// float32 and correctly rounded, so the codes are exactly those of that rule.
//
// Each row (sequence, token, kv head) is handled by D / 8 lanes, one 16-byte
// piece of bf16 (8 elements) of K and of V per lane; a workgroup covers
// kRowPasses groups of rows and issues all their loads before any math, so
// that each lane has 2 kRowPasses 16-byte loads in flight. The row maximum is
// a reduction over the row's lanes. At decode sizes (q_len rows per
// sequence) the launch is latency-bound; prefill-sized appends are HBM-bound
// (read 2 D bf16 and write 2 D elements per row).
#include "pa_cache.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr int kRowPasses = 4;
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two float32 values -> two E4M3FN bytes in the low 16 bits (gfx950
// conversion, round to nearest even; inputs are already within +-448).
__device__ __forceinline__ uint32_t to_e4m3x2(float lo, float hi) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false)) & 0xFFFFu;
}

// x / s rounded to nearest float32 for a positive finite scale s, from
// r = RN(1 / s): q0 = RN(x r) is within a couple of ulps of x / s, each step
// q + RN(x - s q) r (the remainder is exact with an FMA) brings it closer, and
// once q is a faithful rounding the next step gives RN(x / s) (Markstein's
// theorem; quotients small enough to underflow encode to 0 either way). Two
// steps from q0. The sign is x's (the steps would turn -0 into +0), and a
// quotient past 2^100 keeps q0: it clamps to +-448 like the exact one.
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
  q = __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
  return __builtin_copysignf(fabsf(q0) < 0x1p100f ? q : q0, x);
}

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -kE4m3Max), kE4m3Max); }

// 8 bf16 -> 8 E4M3FN bytes of e4m3fn(clamp(x / scale, +-448)); rcp = RN(1 / scale).
__device__ __forceinline__ uint2 quantise8(const u32x4 w, float scale, float rcp) {
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  uint32_t b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = clamp448(div_rn(bf16_to_f32(in[k] & 0xFFFFu), scale, rcp));
    const float hi = clamp448(div_rn(bf16_to_f32(in[k] >> 16), scale, rcp));
    b[k] = to_e4m3x2(lo, hi);
  }
  return make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

__device__ __forceinline__ float absmax8(const u32x4 w) {
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(in[k] & 0xFFFFu)), fabsf(bf16_to_f32(in[k] >> 16))));
  return m;
}

// DPP move of v (bound_ctrl: every lane reads a lane of its own row).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Maximum over the TPR lanes of a row (aligned groups of 16 or 32 lanes):
// quad swaps, then the half-row and row mirrors (each pairs a lane with one
// of the other quad / half), then for 32 lanes the neighbouring row.
template <int TPR>
__device__ __forceinline__ float row_max(float v) {
  static_assert(TPR == 16 || TPR == 32, "rows of 16 or 32 lanes");
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  if constexpr (TPR == 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}

template <int D, bool FP8, int SM, int U>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  constexpr int TPR = D / 8;                    // lanes per row
  constexpr int RPP = kAppendThreads / TPR;     // rows per pass
  constexpr int ELT = FP8 ? 1 : 2;
  const int part = threadIdx.x % TPR;           // this lane's 8 elements: [8 part, 8 part + 8)
  const int32_t row0 = static_cast<int32_t>(blockIdx.x) * (U * RPP) + threadIdx.x / TPR;
  // Every load of every pass is issued before any result is used: the
  // context lengths first (vector loads retire in order, so the page lookups
  // then wait for them alone), the new K/V rows (they depend on the row index
  // only), then the block-table entries. Rows past the end or invalid read
  // in-range addresses and are dropped at the stores.
  int32_t row[U], b[U], i[U], g[U], ctx[U];
  u32x4 k[U], v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    row[u] = row0 + u * RPP;
    const int32_t r = min(row[u], a.rows - 1);
    const int32_t bi = r / a.num_kv_heads;
    g[u] = r - bi * a.num_kv_heads;
    b[u] = bi / a.q_len;
    i[u] = bi - b[u] * a.q_len;
    ctx[u] = a.context_lens[b[u]];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = min(row[u], a.rows - 1);
    k[u] = *reinterpret_cast<const u32x4*>(a.new_k + r * D + 8 * part);
    v[u] = *reinterpret_cast<const u32x4*>(a.new_v + r * D + 8 * part);
  }
  int32_t t[U], page[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    ok[u] = row[u] < a.rows && ctx[u] >= max(1, a.q_len) && ctx[u] <= a.capacity;
    t[u] = ok[u] ? ctx[u] - a.q_len + i[u] : 0;
    page[u] = a.block_table[static_cast<int64_t>(b[u]) * a.max_pages + (t[u] >> a.ps_log2)];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bool live = ok[u] && page[u] >= 0 && page[u] < a.num_pages;
    if (part == 0 && a.status && row[u] < a.rows && !live)
      atomicOr(a.status, ok[u] ? PA_DEV_BAD_PAGE : PA_DEV_BAD_CONTEXT);
    const int64_t dst = live ? static_cast<int64_t>(cache_row(page[u], g[u], t[u] & ((1 << a.ps_log2) - 1),
                                                              a.num_kv_heads, a.ps_log2))
                             : 0;
    if constexpr (!FP8) {
      // bf16 cache: the rows as they are
      if (live) {
        *reinterpret_cast<u32x4*>(a.k_cache + (dst * D + 8 * part) * ELT) = k[u];
        *reinterpret_cast<u32x4*>(a.v_cache + (dst * D + 8 * part) * ELT) = v[u];
      }
    } else {
      float ks, vs;
      if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
        // every lane of the row takes part in the reduction
        const float km = row_max<TPR>(absmax8(k[u]));
        const float vm = row_max<TPR>(absmax8(v[u]));
        ks = km > 0.f ? km / kE4m3Max : 1.f;
        vs = vm > 0.f ? vm / kE4m3Max : 1.f;
        if (live && part == 0) {
          const uint64_t plane = static_cast<uint64_t>(a.num_pages) * a.num_kv_heads << a.ps_log2;
          a.kv_scales[dst] = ks;
          a.kv_scales[plane + dst] = vs;
        }
      } else {
        ks = a.kv_scales[0];
        vs = a.kv_scales[1];
      }
      if (live) {
        *reinterpret_cast<uint2*>(a.k_cache + dst * D + 8 * part) = quantise8(k[u], ks, 1.f / ks);
        *reinterpret_cast<uint2*>(a.v_cache + dst * D + 8 * part) = quantise8(v[u], vs, 1.f / vs);
      }
    }
  }
}

template <int D, bool FP8, int SM>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  constexpr int RPP = kAppendThreads / (D / 8);
  // few rows (a decode step): one pass per workgroup, spread over CUs;
  // many rows: kRowPasses passes per workgroup for loads in flight
  if (a.rows <= 256 * RPP) {
    const int64_t blocks = (static_cast<int64_t>(a.rows) + RPP - 1) / RPP;
    hipLaunchKernelGGL((append_kernel<D, FP8, SM, 1>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kAppendThreads), 0, s, a);
  } else {
    constexpr int64_t per_block = kRowPasses * RPP;
    const int64_t blocks = (static_cast<int64_t>(a.rows) + per_block - 1) / per_block;
    hipLaunchKernelGGL((append_kernel<D, FP8, SM, kRowPasses>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kAppendThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int head_dim, int fp8, int scale_mode, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (head_dim == 128) {
    if (!fp8) return launch_append_t<128, false, PA_SCALE_NONE>(a, s);
    if (scale_mode == PA_SCALE_PER_TENSOR) return launch_append_t<128, true, PA_SCALE_PER_TENSOR>(a, s);
    return launch_append_t<128, true, PA_SCALE_PER_TOKEN_HEAD>(a, s);
  }
  if (!fp8) return launch_append_t<256, false, PA_SCALE_NONE>(a, s);
  if (scale_mode == PA_SCALE_PER_TENSOR) return launch_append_t<256, true, PA_SCALE_PER_TENSOR>(a, s);
  return launch_append_t<256, true, PA_SCALE_PER_TOKEN_HEAD>(a, s);
}

}  // namespace pa

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
// piece of bf16 (8 elements) of K and of V per lane, one row per lane group:
// many small workgroups keep several generations of waves resident, so that
// one wave's loads overlap another's arithmetic and stores (four rows per
// lane, all loads issued first, measured 13% slower on an fp8 prefill). The
// row maximum is a reduction over the row's lanes. At decode sizes (q_len
// rows per sequence) the launch is latency-bound; prefill-sized appends are
// HBM-bound (read 2 D bf16 and write 2 D elements per row).
#include "pa_cache.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// x / s rounded to nearest float32 for a positive normal scale s, from
// r = RN(1 / s): q0 = RN(x r) is within a couple of ulps of x / s, each step
// q + RN(x - s q) r (the remainder is exact with an FMA) brings it closer, and
// once q is a faithful rounding the next step gives RN(x / s) (Markstein's
// theorem; quotients small enough to underflow encode to 0 either way). Two
// steps from q0. The remainder is formed as s q - x and subtracted, so an
// exact zero keeps the sign of the quotient (a zero x gives a zero of x's
// sign). GUARD (per-tensor scales, where x / s is unbounded): a quotient past
// 2^100 keeps q0, which clamps to +-448 like the exact one; with per-token
// scales |x / s| <= 448 (1 + 2^-23).
template <bool GUARD>
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  float q = __builtin_fmaf(-__builtin_fmaf(q0, s, -x), r, q0);
  q = __builtin_fmaf(-__builtin_fmaf(q, s, -x), r, q);
  if constexpr (GUARD) return fabsf(q0) < 0x1p100f ? q : q0;
  return q;
}

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -kE4m3Max), kE4m3Max); }

// 8 bf16 -> 8 E4M3FN bytes of e4m3fn(clamp(x / s, +-448)), r = RN(1 / s), with
// the gfx950 conversion (round to nearest even, two codes per instruction,
// inputs already within +-448). TINY:
// x and s arrive multiplied by 2^64 (exact: powers of two), which leaves the
// quotient as it was.
template <bool GUARD, bool TINY>
__device__ __forceinline__ uint2 quantise8_t(const u32x4 w, float s, float r) {
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  float y[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float lo = bf16_to_f32(in[k] & 0xFFFFu), hi = bf16_to_f32(in[k] >> 16);
    if constexpr (TINY) {
      lo *= 0x1p64f;
      hi *= 0x1p64f;
    }
    y[2 * k] = clamp448(div_rn<GUARD>(lo, s, r));
    y[2 * k + 1] = clamp448(div_rn<GUARD>(hi, s, r));
  }
  // two codes into the low, then the high half of each output word
  int32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
}

// A scale below 2^-60 (a row of tiny values, or a tiny per-tensor scale)
// would make 1 / s overflow or the remainders subnormal: such rows take x 2^64
// and s 2^64 instead (only lanes that need it run that path).
template <bool GUARD>
__device__ __forceinline__ uint2 quantise8(const u32x4 w, float scale) {
  if (scale < 0x1p-60f) {
    const float s = scale * 0x1p64f;
    return quantise8_t<GUARD, true>(w, s, 1.f / s);
  }
  return quantise8_t<GUARD, false>(w, scale, 1.f / scale);
}

// max |x| / 448 rounded to nearest float32 for the maximum m of a row (a
// bf16 value): two Markstein steps with the constant RN(1 / 448), as div_rn,
// for m >= 2^-90 (the quotient and remainders are then normal numbers); the
// correctly rounded division otherwise.
__device__ __forceinline__ float row_scale(float m) {
  if (m == 0.f) return 1.f;
  if (m < 0x1p-90f) return m / kE4m3Max;
  constexpr float r = 1.0f / kE4m3Max;
  const float q0 = m * r;
  float q = __builtin_fmaf(-__builtin_fmaf(q0, kE4m3Max, -m), r, q0);
  return __builtin_fmaf(-__builtin_fmaf(q, kE4m3Max, -m), r, q);
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

template <int D, bool FP8, int SM>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  constexpr int TPR = D / 8;                    // lanes per row
  constexpr int RPW = kAppendThreads / TPR;     // rows per workgroup
  constexpr int ELT = FP8 ? 1 : 2;
  const int part = threadIdx.x % TPR;           // this lane's 8 elements: [8 part, 8 part + 8)
  const int32_t row = static_cast<int32_t>(blockIdx.x) * RPW + threadIdx.x / TPR;
  // The context length first, then the new K/V pieces (they depend on the
  // row index only), then the block-table entry: vector loads retire in
  // order, so the page lookup waits for the context length alone. A row past
  // the end reads in-range addresses and is dropped at the stores.
  const int32_t r = min(row, a.rows - 1);
  const int32_t bi = r / a.num_kv_heads;
  const int32_t g = r - bi * a.num_kv_heads;
  const int32_t b = bi / a.q_len;
  const int32_t i = bi - b * a.q_len;
  const int32_t ctx = a.context_lens[b];
  const u32x4 k = *reinterpret_cast<const u32x4*>(a.new_k + static_cast<int64_t>(r) * D + 8 * part);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.new_v + static_cast<int64_t>(r) * D + 8 * part);
  const bool ok = row < a.rows && ctx >= max(1, a.q_len) && ctx <= a.capacity;
  const int32_t t = ok ? ctx - a.q_len + i : 0;
  const int32_t page = a.block_table[static_cast<int64_t>(b) * a.max_pages + (t >> a.ps_log2)];
  const bool live = ok && page >= 0 && page < a.num_pages;
  if (part == 0 && a.status && row < a.rows && !live)
    atomicOr(a.status, ok ? PA_DEV_BAD_PAGE : PA_DEV_BAD_CONTEXT);
  const int64_t dst =
      live ? static_cast<int64_t>(cache_row(page, g, t & ((1 << a.ps_log2) - 1), a.num_kv_heads, a.ps_log2))
           : 0;
  if constexpr (!FP8) {
    // bf16 cache: the rows as they are
    if (live) {
      *reinterpret_cast<u32x4*>(a.k_cache + (dst * D + 8 * part) * ELT) = k;
      *reinterpret_cast<u32x4*>(a.v_cache + (dst * D + 8 * part) * ELT) = v;
    }
  } else {
    float ks, vs;
    if constexpr (SM == PA_SCALE_PER_TOKEN_HEAD) {
      // every lane of the row takes part in the reduction
      ks = row_scale(row_max<TPR>(absmax8(k)));
      vs = row_scale(row_max<TPR>(absmax8(v)));
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
      constexpr bool GUARD = SM != PA_SCALE_PER_TOKEN_HEAD;
      *reinterpret_cast<uint2*>(a.k_cache + dst * D + 8 * part) = quantise8<GUARD>(k, ks);
      *reinterpret_cast<uint2*>(a.v_cache + dst * D + 8 * part) = quantise8<GUARD>(v, vs);
    }
  }
}

template <int D, bool FP8, int SM>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  constexpr int RPW = kAppendThreads / (D / 8);
  const int64_t blocks = (static_cast<int64_t>(a.rows) + RPW - 1) / RPW;
  hipLaunchKernelGGL((append_kernel<D, FP8, SM>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kAppendThreads), 0, s, a);
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

// Internal declarations of the KV-cache append (pa_cache.hip), used by the
// C-ABI wrappers. gfx950 (CDNA4) only.
#pragma once

#include "pa_common.h"

namespace pa {

// KV-cache append: new tokens' K/V rows into their pages.
struct AppendArgs {
  const uint16_t* new_k;        // bf16 bits [B, q_len, Hkv, D]
  const uint16_t* new_v;
  const int32_t* block_table;   // [B, max_pages]
  const int32_t* context_lens;  // [B], including the appended tokens
  uint8_t* k_cache;             // [num_pages, Hkv, ps, D] elements
  uint8_t* v_cache;
  float* kv_scales;             // per token: [2][num_pages][Hkv][ps] (written); per tensor: [2] (read)
  int32_t* status;              // device status bits (PA_DEV_*), may be null
  int32_t rows;                 // B * q_len * Hkv (< 2^31)
  int32_t q_len, num_kv_heads, ps_log2, max_pages, num_pages, capacity;
};

hipError_t launch_append(const AppendArgs& a, int head_dim, int fp8, int scale_mode, hipStream_t s);

}  // namespace pa

// Internal declarations shared by the HIP kernels and the C-ABI wrappers.
// gfx950 (CDNA4) only: wave64, MFMA bf16 16x16x32 / 16x16x16, OCP fp8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// One work item or one segment: a token range [tok_begin, tok_end) of one
// (sequence, kv head) pair, and its partial slot (-1: the pair is finished
// in one workgroup, which writes the output itself).
struct Span {
  int32_t pair, tok_begin, tok_end, slot;
};

// Device status word layout in the workspace (int32[4]).
enum { ST_BITS = 0, ST_ITEMS = 1, ST_SEGS = 2 };

struct DecodeArgs {
  const uint16_t* q;            // bf16 bits [B, q_len, Hq, D]
  const uint8_t* k_cache;       // [num_pages, Hkv, ps, D] elements
  const uint8_t* v_cache;
  const int32_t* block_table;   // [B, maxp]
  const int32_t* context_lens;  // [B]
  const int32_t* seg_info;      // [segs][8] b, g, tok_begin, tok_end, slot, ctx, pair, 0
  const int32_t* wg_head;       // [grid][16] segment begin, first seg_info record, segment end
  const int32_t* nseg;
  const int32_t* seg_base;
  const float* kv_scales;       // per-token: [2][num_pages][Hkv][ps]
  uint16_t* out;                // bf16 bits [B, q_len, Hq, D]
  float* partial_o;             // [slots][rows][D]
  float* partial_lse;           // [slots][rows]
  int32_t* status;
  int32_t* counters;            // [pairs] arrivals per split pair (fused reduce), or null
  int32_t batch, q_len, num_q_heads, num_kv_heads, group, rows;
  int32_t q_total;               // queries per sequence in q and out; q and out point at this
                                 // launch's block of q_len of them
  int32_t ps_log2, max_pages, num_pages;
  int32_t ctx_offset;           // queries after this launch's block: its keys end at
                                // context_lens[b] - ctx_offset
  int32_t capacity;             // max_pages * page size
  int32_t scale_mode;           // PA_SCALE_*
  int32_t debug_bounds;
  float qk_scale_log2;          // softmax scale * log2(e) (* per-tensor K scale)
  float out_scale;              // per-tensor V scale, else 1
};

// Row index of (physical page, kv head, slot) in a [num_pages, Hkv, ps, D]
// cache: the one page-addressing rule, used by the decode kernel and by the
// debug gather alike.
__device__ __forceinline__ uint64_t cache_row(int32_t page, int32_t kv_head, int32_t slot,
                                              int32_t num_kv_heads, int32_t ps_log2) {
  return ((static_cast<uint64_t>(page) * static_cast<uint64_t>(num_kv_heads) +
           static_cast<uint64_t>(kv_head))
          << ps_log2) + static_cast<uint64_t>(slot);
}

// Decode kernel instantiations: head dim, KV element type, scale mode,
// 16-row tiles of query rows, 16-token blocks per chunk, waves per
// workgroup, K/V register stages of the load pipeline.
struct Variant {
  int head_dim;
  int fp8;
  int scale_mode;
  int row_tiles;
  int blocks;
  int waves;
  int stages;
  int one_page;  // every chunk lies in one page: one block-table entry per chunk
  int shared;    // waves of a chunk stream sharing its K/V tiles in LDS (0: none)
};

int num_variants();
const Variant& variant(int i);
// Returns the index of the instantiation for (head_dim, fp8, scale mode,
// rows per kv head), or -1.
int pick_variant(int head_dim, int fp8, int scale_mode, int rows, int page_size, int partition);

hipError_t launch_partition(int variant, const DecodeArgs& a, int grid, hipStream_t s);
hipError_t launch_reduce(const DecodeArgs& a, int head_dim, int num_pairs, hipStream_t s);
// Test support: the page loader of instantiation `variant` over every chunk
// of every segment of the plan in `a`, its registers written out row-major.
hipError_t launch_loader(int variant, const DecodeArgs& a, int max_segs, uint8_t* k_out,
                         uint8_t* v_out, float* scales_out, hipStream_t s);

// Measurement support (pa_probe.hip): read num_blocks / (grid * waves)
// (rounded down to even) blocks of 16 rows of row_bytes bytes per wave, in the
// linear or the rows lane layout; block indices clamped to [0, nbuf).
hipError_t launch_read_probe(const uint8_t* buf, int32_t nbuf, const int32_t* blocks, int32_t num_blocks,
                             int row_bytes, bool linear, int grid, int waves, float* sink, hipStream_t s);

}  // namespace pa

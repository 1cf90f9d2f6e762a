// Internal declarations of the work-list builder (pa_plan.hip), used by the
// C-ABI wrappers. gfx950 (CDNA4) only.
#pragma once

#include "pa_common.h"

namespace pa {

struct PlanArgs {
  const int32_t* context_lens;
  int32_t* status;
  int32_t* wg_begin;
  int32_t* wg_seg_begin;
  Span* items;
  Span* segs;
  int32_t* nseg;
  int32_t* seg_base;
  int32_t* pseg_base;
  int32_t* batch_base;
  int32_t* seg_info;  // [max_segs][8] (b, g, tok_begin, tok_end, slot, ctx, pair, 0)
  int32_t* wg_head;   // [grid][16] (segment begin, first seg_info record, segment end, 0...)
  int32_t* counters;  // [pairs] arrival counters of the fused reduce, zeroed by the plan
  int32_t batch, num_kv_heads, q_len, partition, grid;
  int32_t capacity;  // max_pages_per_seq * page_size
  // A block of q_len queries out of q_check per sequence: context lengths
  // are validated against q_check, and the work list covers the keys the
  // block sees, ctx - ctx_offset of them (ctx_offset = the queries after it).
  int32_t q_check, ctx_offset;
  // Set by launch_plan: the items are written by a second kernel (batches
  // whose tables live in the workspace), not by the plan kernel.
  int32_t items_apart;
};

// Launches the plan kernel on s (and, past the LDS tables, the items kernel
// after it); max_items bounds the item count (it sizes the grids).
hipError_t launch_plan(const PlanArgs& a, int64_t max_items, hipStream_t s);

}  // namespace pa

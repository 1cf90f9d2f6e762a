/*
 * pa.h — paged-attention decode for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * A few query tokens per sequence attend over a KV cache that lives in
 * fixed-size physical pages reached through a block table, with grouped query
 * heads, an online softmax, causal masking of the appended query tokens,
 * optional fp8 (OCP E4M3FN) KV with per-token-head or per-tensor scales, a
 * split-KV partition pass with a log-sum-exp reduce, and a persistent grid
 * that walks a work list built by pa_plan().
 *
 * Where each operation is defined (the pages give names and behaviour, not
 * formulas; the plainest reading is stated beside each call):
 *   [P1] "Benchmark high-perf Paged Attention (#899) vs PA unroll on a2a3",
 *        hw-native-sys/simpler issue #998, table "Same-Shape Side-by-Side"
 *        (shape keys b/h/kv/s/bs/hd: batch, query heads, kv heads, context,
 *        page size, head dim).
 *   [P2] Ascend/RecSDK issue #1281, HSTU paged attention: section "背景与优化
 *        特性" (background: history K/V read page by page from the paged KV
 *        cache), "优化方案" (double-buffered page copies), "其他相关讨论"
 *        (correctness vs a CPU FP32 reference at rtol = atol = 8e-3) and
 *        "接口、兼容性与回退" (interface unchanged).
 *   [P3] "[Kernel][Perf] Optimize paged-attention metadata decode", ROCm/FlyDSL
 *        PR #910: "Pull request overview" (metadata scheduler, persistent
 *        decode, split reduction kernel, per-token KV scales, rejection of
 *        unsupported block sizes and dtypes), the code excerpt (grid = CU
 *        count x multiplier; the cache's leading dimension is the block
 *        count), "Summary" (one grid per CU by default) and "Breaking Changes".
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller (for example
 *     PyTorch tensors); the library allocates no device memory and keeps no
 *     state beyond a cached CU count per device.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream). Every call except pa_plan_status is asynchronous on it.
 *   - Return value: PA_OK (0) or a negative PA_ERR_* code; pa_last_error()
 *     gives a thread-local text for the last failure. Argument errors are
 *     found on the host before any HIP call. Nothing throws across the ABI.
 *
 * Layouts (row-major, contiguous):
 *   q, out          [batch, q_len, num_q_heads, head_dim]      bf16
 *   k_cache,v_cache [num_pages, num_kv_heads, page_size, head_dim]
 *                   bf16, or one E4M3FN byte per element
 *   block_table     [batch, max_pages_per_seq]                 int32
 *   context_lens    [batch]                                    int32
 *   kv_scales       per tensor: [2] float32 (K scale, V scale)
 *                   per token and head: [2][num_pages][num_kv_heads][page_size]
 *                   float32 (K scales, then V scales)
 * context_lens[b] counts the q_len appended tokens, whose K/V are already in
 * the cache; query i of sequence b sees keys t <= context_lens[b] - q_len + i.
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,          /* a required pointer is NULL                  */
  PA_ERR_ALIGN = -2,         /* a pointer is not aligned as documented      */
  PA_ERR_DIMS = -3,          /* non-positive size, Hq % Hkv != 0, ...       */
  PA_ERR_UNSUPPORTED = -4,   /* page size / head dim / dtype / row count the
                                kernels do not handle ([P3] overview: such
                                shapes are rejected, not run)               */
  PA_ERR_WORKSPACE = -5,     /* workspace NULL, too small or misaligned     */
  PA_ERR_PLAN_MISMATCH = -6, /* plan not built, or q_len / scale mode differ */
  PA_ERR_SCALE_MODE = -7,    /* bf16 KV with scales, fp8 KV without, or the
                                scale pointer disagrees with the mode       */
  PA_ERR_HIP = -8,           /* a HIP runtime call or launch failed         */
  PA_ERR_DEVICE = -9         /* no usable gfx950 device                     */
};

/* Bits of the device status word (pa_plan_status). */
enum {
  PA_DEV_BAD_CONTEXT = 1,    /* pa_plan: some context_lens[b] outside
                                [max(1, q_len), max_pages_per_seq * page_size];
                                the plan is then empty and decode writes
                                nothing. pa_decode: some context_lens[b] below
                                the length the plan was built with or past
                                max_pages_per_seq * page_size; that sequence
                                is then decoded over the plan's length       */
  PA_DEV_BAD_PAGE = 2,       /* a block-table entry outside [0, num_pages)
                                (checked only with PA_FLAG_DEBUG_BOUNDS; such
                                tokens are then read as zeros)               */
  PA_DEV_DEBUG_DEAD_ROW = 4  /* pa_debug_gather only: a row past a segment's
                                end did not load as zeros                   */
};

enum { PA_KV_BF16 = 0, PA_KV_FP8_E4M3FN = 1 };
enum { PA_SCALE_NONE = 0, PA_SCALE_PER_TENSOR = 1, PA_SCALE_PER_TOKEN_HEAD = 2 };
enum {
  PA_FLAG_DEBUG_BOUNDS = 1,    /* check every block-table entry the decode reads */
  PA_FLAG_FUSED_REDUCE = 2,    /* merge split pairs inside the partition pass: the
                                  last workgroup of a pair to finish (a per-pair
                                  arrival counter) merges its partials, in slot
                                  order, with the reduce kernel's arithmetic;
                                  the output is bitwise that of the separate
                                  reduce ([P3] overview: split reduction)     */
  PA_FLAG_SEPARATE_REDUCE = 4  /* merge them in a reduce kernel of its own.
                                  With neither reduce flag, pa_plan takes the
                                  tuned choice for the shape (pa_plan_choice),
                                  else the separate reduce                   */
};

/* Problem description. Zero in partition_size / grid_multiplier, and neither
 * reduce flag, select the tuned choice for the shape class when the library's
 * tuning table has one (pa_plan_choice), else the defaults: 256 tokens, one
 * persistent workgroup per CU ([P3] "Summary": the safe default) and the
 * separate reduce. */
typedef struct pa_dims {
  int32_t batch;
  int32_t q_len;               /* appended query tokens per sequence, >= 1.
                                  Up to 256 rows per kv head, q_len *
                                  (num_q_heads / num_kv_heads), at head_dim 128
                                  (64 at 256) run in one kernel, which reads
                                  each K/V chunk once for all of them; past
                                  that the queries go in blocks of q_block
                                  (each block a work list and launches of its
                                  own); one query's rows must fit, else
                                  PA_ERR_UNSUPPORTED                         */
  int32_t num_q_heads;
  int32_t num_kv_heads;        /* divides num_q_heads                        */
  int32_t head_dim;            /* 128 or 256                                 */
  int32_t page_size;           /* power of two in [16, 1024]                 */
  int32_t num_pages;           /* k_cache.shape[0] ([P3] code excerpt)       */
  int32_t max_pages_per_seq;   /* block_table row stride                     */
  int32_t kv_dtype;            /* PA_KV_*                                    */
  int32_t kv_scale_mode;       /* PA_SCALE_*                                 */
  int32_t partition_size;      /* tokens per work item, multiple of 16; 0:
                                  tuned or 256                               */
  int32_t grid_multiplier;     /* persistent workgroups per CU, 1..16; 0:
                                  tuned or 1                                 */
  int32_t flags;               /* PA_FLAG_*                                  */
} pa_dims;

/* A built plan: caller-owned plain data, filled by pa_plan(). It points into
 * the caller's workspace, which must stay alive and must not be shared by
 * two streams until the decode that uses it has finished. */
typedef struct pa_plan_t {
  uint32_t magic;              /* set by pa_plan                             */
  int32_t device;              /* HIP device the plan was built on           */
  pa_dims dims;                /* validated copy, defaults applied           */
  int32_t num_cus;             /* hipDeviceAttributeMultiprocessorCount      */
  int32_t grid;                /* num_cus * grid_multiplier                  */
  int32_t rows;                /* q_block * (num_q_heads / num_kv_heads)     */
  int32_t num_pairs;           /* batch * num_kv_heads                       */
  int32_t max_items;           /* capacity of the item list                  */
  int32_t max_segs;            /* capacity of the segment list (= max slots) */
  int32_t variant;             /* decode kernel instantiation chosen         */
  int32_t q_block;             /* queries per block (q_len when they fit)    */
  void* workspace;
  uint64_t workspace_bytes;
  /* byte offsets into the workspace (all 256-byte aligned) */
  uint64_t off_status;         /* int32[4]: status bits, N items, N segments */
  uint64_t off_wg_begin;       /* int32[grid + 1]: item range per workgroup  */
  uint64_t off_wg_seg_begin;   /* int32[grid + 1]: segment range per wg      */
  uint64_t off_items;          /* int32[max_items][4]: pair, tok_begin,
                                  tok_end, slot                              */
  uint64_t off_segs;           /* int32[max_segs][4]: same fields, one per
                                  segment, in workgroup order                */
  uint64_t off_nseg;           /* int32[num_pairs]                           */
  uint64_t off_seg_base;       /* int32[num_pairs + 1] (split pairs' slots)  */
  uint64_t off_pseg_base;      /* int32[num_pairs + 1] (all segments)        */
  uint64_t off_batch_base;     /* int32[batch + 1]: first item of sequence b */
  uint64_t off_partial_lse;    /* float[max_segs][rows]                      */
  uint64_t off_partial_o;      /* float[max_segs][rows][head_dim]            */
  uint64_t off_seg_info;       /* int32[max_segs][8]: each segment as
                                  (b, g, tok_begin, tok_end, slot, ctx_b,
                                  pair, 0), read by the decode               */
  uint64_t off_wg_head;        /* int32[grid][16]: workgroup w's first
                                  segment, that segment's seg_info record,
                                  its segment range end, then zeros          */
  uint64_t block_bytes;        /* workspace per block: block j's regions are
                                  at the offsets above plus j * block_bytes  */
  uint64_t off_counters;       /* int32[num_pairs]: arrivals per split pair
                                  (fused reduce), zeroed by pa_plan          */
} pa_plan_t;

#define PA_PLAN_MAGIC 0x50414450u

/* Number of compute units of HIP device `device` (cached after the first
 * call). Errors: PA_ERR_NULL, PA_ERR_DEVICE. */
int pa_query_device(int32_t device, int32_t* num_cus);

/* The settings pa_plan would use for `dims` on a device with `num_cus` CUs:
 * *chosen = dims with partition_size, grid_multiplier and the reduce flag
 * filled in (exactly one of PA_FLAG_FUSED_REDUCE / PA_FLAG_SEPARATE_REDUCE
 * set). Fields the caller set are kept. The rest come from the library's
 * tuning table ([P3] overview: a tuned per-shape persistent grid, with a
 * lookup that keeps the defaults when a shape has no entry), keyed by the
 * shape class (num_cus, head_dim, kv_dtype, kv_scale_mode, ceil(rows / 16)
 * with rows = q_len * num_q_heads / num_kv_heads, page_size,
 * floor(log2(batch * num_kv_heads)), floor(log2(max_pages_per_seq *
 * page_size))); with no entry, from the defaults (pa_dims). Host-only.
 * Errors: as pa_workspace_bytes. */
int pa_plan_choice(const pa_dims* dims, int32_t num_cus, pa_dims* chosen);

/* Workspace bytes a plan for `dims` on a device with `num_cus` CUs needs.
 * Host-only; validates dims exactly as pa_plan does. Errors: PA_ERR_NULL,
 * PA_ERR_DIMS, PA_ERR_UNSUPPORTED, PA_ERR_SCALE_MODE. */
int pa_workspace_bytes(const pa_dims* dims, int32_t num_cus, uint64_t* bytes);

/* Build the persistent work list on the current HIP device ([P3] overview:
 * "metadata scheduler"; code excerpt: grid = CUs x multiplier). Launches one
 * kernel (up to 256 workgroups) or, past 8192 sequences or 16336 (sequence,
 * kv head) pairs, two (one workgroup builds the per-sequence and per-pair
 * tables in the workspace, then up to 256 write the items) that read
 * context_lens (device
 * int32[batch]) and writes into `workspace` (device, 256-byte aligned,
 * >= pa_workspace_bytes):
 *   items   for b, then kv head g, then partition k < ceil(ctx_b / P):
 *           (b * Hkv + g, k * P, min((k + 1) * P, ctx_b), slot)
 *   ranges  workgroup w owns items [floor(w N / G), floor((w + 1) N / G))
 *   segments maximal same-pair runs inside one range; a pair with one
 *           segment is finished by its workgroup, the segments of a split
 *           pair get partial slots seg_base[pair] + their index
 * plus, for the decode, each segment as one 32-byte record (off_seg_info)
 * and each workgroup's segment range and first record (off_wg_head),
 * and fills *plan. Invalid context lengths set PA_DEV_BAD_CONTEXT in the
 * device status word and give an empty plan. When the queries go in blocks
 * (see pa_dims.q_len), one such list is built per block, in its own
 * block_bytes of the workspace, over the keys up to the block's last query
 * (ctx_b - (q_len - end of the block)); one kernel launch per block.
 * Asynchronous. Errors:
 * PA_ERR_NULL, PA_ERR_DIMS, PA_ERR_UNSUPPORTED, PA_ERR_SCALE_MODE,
 * PA_ERR_WORKSPACE, PA_ERR_ALIGN, PA_ERR_DEVICE, PA_ERR_HIP. */
int pa_plan(const pa_dims* dims, const int32_t* context_lens, void* workspace,
            uint64_t workspace_bytes, pa_plan_t* plan, void* stream);

/* Decode attention for every (sequence, query, head): the partition pass
 * over the plan's segments, then the log-sum-exp reduce of split pairs
 * ([P3] overview: persistent decode + "reduction kernel"; [P2] background:
 * K/V read from the paged cache through the block table). out (device bf16)
 * receives softmax(scale * q K^T) V rounded to nearest even, with fp8 K/V
 * dequantised as byte value x scale. q_len and kv_scale_mode must equal the
 * plan's; kv_scales must be NULL iff the mode is PA_SCALE_NONE. q, k_cache,
 * v_cache, out and per-token kv_scales must be 16-byte aligned; block_table,
 * context_lens and per-tensor kv_scales 4-byte aligned. With query blocks,
 * each block is decoded in turn (its rows of q and out). Asynchronous.
 *
 * Context lengths are read again here, on the device: sequence b is decoded
 * over its live context_lens[b] keys, not the length pa_plan saw. The plan
 * only says where a pair's work may split; its last segment runs to the live
 * length and the causal mask follows it. So one plan serves later decode
 * steps while every sequence only grows (pa_cache_append, then pa_decode on
 * the same plan), up to max_pages_per_seq * page_size; re-plan to rebalance
 * the work. A live length below the plan's, or past that capacity, sets
 * PA_DEV_BAD_CONTEXT, and that sequence is decoded over the plan's length.
 *
 * A plan built with PA_FLAG_FUSED_REDUCE (or so tuned) launches the
 * partition pass only; it merges the split pairs itself.
 *
 * Errors: PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_PLAN_MISMATCH, PA_ERR_SCALE_MODE,
 * PA_ERR_HIP. */
int pa_decode(const pa_plan_t* plan, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* context_lens, int32_t q_len,
              float scale, int32_t kv_scale_mode, const float* kv_scales, void* out,
              void* stream);

/* The two launches of pa_decode, separately: the partition pass (writes the
 * output of unsplit pairs and the partials of split ones) and the reduce
 * (merges the partials). pa_decode == pa_decode_partition then
 * pa_decode_reduce on the same stream; same arguments and errors. When
 * partition_size >= max_pages_per_seq * page_size no pair can be split, and
 * pa_decode_reduce validates its arguments and launches nothing; likewise
 * for a fused-reduce plan, whose partition pass merges the split pairs. */
int pa_decode_partition(const pa_plan_t* plan, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* block_table,
                        const int32_t* context_lens, int32_t q_len, float scale,
                        int32_t kv_scale_mode, const float* kv_scales, void* out,
                        void* stream);
int pa_decode_reduce(const pa_plan_t* plan, int32_t q_len, int32_t kv_scale_mode, void* out,
                     void* stream);

/* Synchronise `stream` and copy the device status word (PA_DEV_* bits; the
 * OR over query blocks) to *device_status. The only blocking call. Errors: PA_ERR_NULL,
 * PA_ERR_PLAN_MISMATCH, PA_ERR_HIP. */
int pa_plan_status(const pa_plan_t* plan, int32_t* device_status, void* stream);

/* Test support: the partition pass's own page loader, run alone. For every
 * segment of the plan (the last query block's, whose keys reach the end of
 * each context) and every chunk of it, the loader of the plan's decode
 * instantiation (block-table entries, then 16-byte buffer loads sized to the
 * segment's live rows) loads the chunk's K and V rows, and per-token scales in
 * PA_SCALE_PER_TOKEN_HEAD mode, into registers exactly as pa_decode does;
 * they are written back out in the order the math reads them:
 *   k_out, v_out  [batch * num_kv_heads][max_pages_per_seq * page_size]
 *                 [head_dim] elements of the cache's type; row t of pair
 *                 (b, g) is the row the decode loaded for key t < ctx_b
 *   scales_out    [2][batch * num_kv_heads][max_pages_per_seq * page_size]
 *                 float32 (K, then V scales of the same rows); per-token mode
 *                 only, else may be NULL
 * Rows t >= ctx_b are not written. Rows a chunk holds past its segment's end
 * must load as zeros; any that does not sets PA_DEV_DEBUG_DEAD_ROW in the
 * status word. The context lengths are the live ones, as in pa_decode.
 * Asynchronous. Errors: as pa_decode. */
int pa_debug_gather(const pa_plan_t* plan, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* context_lens,
                    const float* kv_scales, void* k_out, void* v_out, float* scales_out,
                    void* stream);

/* KV-cache append, the write side of the cache the decode reads ([P2]
 * background: K/V live page by page in the paged cache behind the block
 * table; [P3] overview: the fp8 cache is quantised per token and head or per
 * tensor). For every sequence b and appended token i < q_len, at position
 * t = context_lens[b] - q_len + i (context_lens counts the appended tokens,
 * as in pa_decode), the K and V rows of every kv head g are written to
 * page block_table[b][t / page_size], slot t % page_size:
 *   bf16 cache    the rows as they are;
 *   fp8, per token and head   scale = max_d |x_d| / 448 (1 for an all-zero
 *                 row) is written to kv_scales[0 or 1][page][g][slot] and the
 *                 bytes are e4m3fn(clamp(x_d / scale, -448, 448)), rounded to
 *                 nearest even, every step in float32;
 *   fp8, per tensor           the same bytes with scale = kv_scales[0] (K) or
 *                 kv_scales[1] (V), which are read, not written (positive
 *                 and finite; other scales give unspecified bytes).
 * new_k, new_v: device bf16 [batch, q_len, num_kv_heads, head_dim], 16-byte
 * aligned. dims as for pa_plan, except that q_len may be any length (a
 * prefill appends the whole prompt); num_q_heads, partition_size and
 * grid_multiplier are validated but not used. k_cache, v_cache, kv_scales,
 * block_table and context_lens as in pa_decode; kv_scales is NULL exactly
 * when kv_scale_mode is PA_SCALE_NONE. device_status (optional, device
 * int32, may be NULL) gets PA_DEV_BAD_CONTEXT for a sequence whose context
 * length is outside [max(1, q_len), max_pages_per_seq * page_size] and
 * PA_DEV_BAD_PAGE for a row whose page entry is outside [0, num_pages), OR-ed
 * in; such rows are not written. No other memory is touched. Asynchronous.
 * Errors: PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_DIMS, PA_ERR_UNSUPPORTED,
 * PA_ERR_SCALE_MODE, PA_ERR_DEVICE, PA_ERR_HIP. */
int pa_cache_append(const pa_dims* dims, const void* new_k, const void* new_v,
                    const int32_t* block_table, const int32_t* context_lens, void* k_cache,
                    void* v_cache, float* kv_scales, int32_t* device_status, void* stream);

/* pa_plan followed by pa_decode, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The caller passes inputs and outputs only; the work list
 * and split partials live in a static scratch array of
 * pa_static_scratch_bytes() (32 MiB) that the library holds on each device it
 * runs on until the process ends. Nothing is allocated or freed: no hipMalloc,
 * no hipFree, no allocating library call. Arguments are those of pa_plan
 * (dims, context_lens) and pa_decode (the rest), with the same layouts and
 * errors; a problem whose workspace (pa_workspace_bytes) exceeds the scratch
 * is rejected with PA_ERR_WORKSPACE before any launch. If plan_out is not
 * NULL it receives the plan, which points into the scratch (for
 * pa_plan_status) and stays valid only until the next pa_decode_static call
 * on that device. Every call on one device shares that device's scratch:
 * calls that overlap on one device (two streams, or two host threads)
 * race and must be ordered by the caller. Asynchronous. */
int pa_decode_static(const pa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* context_lens, int32_t q_len,
                     float scale, int32_t kv_scale_mode, const float* kv_scales, void* out,
                     pa_plan_t* plan_out, void* stream);

/* Size in bytes of pa_decode_static's per-device scratch. */
uint64_t pa_static_scratch_bytes(void);

/* Measurement support: the HBM read rate of the partition pass's K/V load
 * layouts, alone. Reads blocks of 16 rows of row_bytes bytes (a 16-token block
 * of one cache page and kv head: 128 = fp8 at head_dim 128, 256 = bf16 at
 * 128 or fp8 at 256, 512 = bf16 at 256) from `buffer` with 16-byte
 * non-temporal loads, in the linear lane layout (linear != 0: each load
 * instruction reads 1 KB contiguous) or the rows layout (64 bytes of each of
 * 16 rows). The grid has one workgroup of `waves` waves per CU; wave w reads
 * blocks[w * per + k] for k < per = num_blocks / (CUs * waves), rounded down
 * to even, two blocks at a time. Block indices are clamped to the buffer's
 * blocks. sink (device float[CUs * waves * 64]) receives one value per lane
 * so the loads are kept. buffer, blocks (device int32[num_blocks]) and sink
 * are device memory. Asynchronous; time it with events on `stream`. Errors:
 * PA_ERR_NULL, PA_ERR_UNSUPPORTED (row_bytes), PA_ERR_DIMS (waves outside
 * [1, 16], buffer smaller than one block), PA_ERR_ALIGN, PA_ERR_DEVICE,
 * PA_ERR_HIP. */
int pa_debug_read_probe(const void* buffer, uint64_t buffer_bytes, const int32_t* blocks,
                        int32_t num_blocks, int32_t row_bytes, int32_t linear, int32_t waves,
                        float* sink, void* stream);

/* Static text for a PA_* status code. */
const char* pa_status_string(int status);

/* Thread-local text describing the last failed call on this thread. */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */

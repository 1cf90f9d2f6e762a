// C-ABI of the paged-attention decode library (declared in include/pa.h).
//
// Host work only: argument validation (before any HIP call, so every
// argument error is reported without a device), workspace layout, the
// per-device CU count, and kernel launches on the caller's stream. The
// library allocates no device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "pa_cache.h"
#include "pa_plan.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

constexpr int kDefaultPartition = 256;
constexpr int kMaxKernelRows = 256;  // query rows per kv head the widest instantiation holds
constexpr int kMaxGridMultiplier = 16;
constexpr int kMaxDevices = 64;

std::mutex g_dev_mu;
int g_cu_cache[kMaxDevices] = {0};

// Tuned settings per shape class ([P3] overview: the persistent grid is
// looked up per shape in a tuned table, with the one-grid-per-CU default
// where a shape has none). The rows are generated at build time from the
// committed CSV table (tuning.csv beside the package, written by
// `bench.py --tune`); a row of -1 ends the list.
struct TuneEntry {
  int32_t num_cus, head_dim, kv_dtype, kv_scale_mode, row_tiles, page_size, pairs_log2,
      capacity_log2;
  int32_t grid_multiplier, partition_size, fused;
};
const TuneEntry kTuned[] = {
#include "pa_tuning_table.inc"
    {-1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}};

int floor_log2(int64_t x) {
  int r = -1;
  while (x > 0) {
    x >>= 1;
    ++r;
  }
  return r;
}

const TuneEntry* tuned(const pa_dims& d, int num_cus) {
  const int64_t rows = static_cast<int64_t>(d.q_len) * (d.num_q_heads / d.num_kv_heads);
  const int rt = static_cast<int>(std::min<int64_t>((rows + 15) / 16, 1 << 20));
  const int pl = floor_log2(static_cast<int64_t>(d.batch) * d.num_kv_heads);
  const int cl = floor_log2(static_cast<int64_t>(d.max_pages_per_seq) * d.page_size);
  for (const TuneEntry* e = kTuned; e->num_cus >= 0; ++e)
    if (e->num_cus == num_cus && e->head_dim == d.head_dim && e->kv_dtype == d.kv_dtype &&
        e->kv_scale_mode == d.kv_scale_mode && e->row_tiles == rt && e->page_size == d.page_size &&
        e->pairs_log2 == pl && e->capacity_log2 == cl)
      return e;
  return nullptr;
}

// Workspace of pa_decode_static, for callers that cannot allocate device
// memory: one array per device, held until the process ends. Host code never
// uses the array's name as an address (on the host it is a stand-in); it
// uses the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
constexpr uint64_t kStaticScratchBytes = uint64_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
void* g_scratch_ptr[kMaxDevices] = {nullptr};

constexpr int kReduceFlags = PA_FLAG_FUSED_REDUCE | PA_FLAG_SEPARATE_REDUCE;

// Validates dims and applies the tuned choice (num_cus > 0) and the defaults
// into *out. Host-only. need_decode: the rows per kv head must fit a decode
// instantiation (not for the append, which takes any q_len).
int check_dims(const pa_dims* in, pa_dims* out, int* variant, bool need_decode = true,
               int* q_block = nullptr, int num_cus = 0) {
  if (!in) return fail(PA_ERR_NULL, "dims is NULL");
  pa_dims d = *in;
  if (d.batch < 1 || d.q_len < 1 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.num_pages < 1 ||
      d.max_pages_per_seq < 1)
    return fail(PA_ERR_DIMS, "batch, q_len, heads, num_pages and max_pages_per_seq must be >= 1");
  if (d.num_q_heads % d.num_kv_heads != 0)
    return fail(PA_ERR_DIMS, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                d.num_q_heads, d.num_kv_heads);
  if (d.flags & ~(PA_FLAG_DEBUG_BOUNDS | kReduceFlags))
    return fail(PA_ERR_DIMS, "unknown flag bits 0x%x", d.flags);
  if ((d.flags & kReduceFlags) == kReduceFlags)
    return fail(PA_ERR_DIMS, "PA_FLAG_FUSED_REDUCE and PA_FLAG_SEPARATE_REDUCE are exclusive");
  if (num_cus > 0 && (d.partition_size == 0 || d.grid_multiplier == 0 || !(d.flags & kReduceFlags))) {
    if (const TuneEntry* e = tuned(d, num_cus)) {
      if (d.partition_size == 0) d.partition_size = e->partition_size;
      if (d.grid_multiplier == 0) d.grid_multiplier = e->grid_multiplier;
      if (!(d.flags & kReduceFlags))
        d.flags |= e->fused ? PA_FLAG_FUSED_REDUCE : PA_FLAG_SEPARATE_REDUCE;
    }
  }
  if (d.partition_size == 0) d.partition_size = kDefaultPartition;
  if (d.grid_multiplier == 0) d.grid_multiplier = 1;
  if (!(d.flags & kReduceFlags)) d.flags |= PA_FLAG_SEPARATE_REDUCE;
  if (d.grid_multiplier < 1 || d.grid_multiplier > kMaxGridMultiplier)
    return fail(PA_ERR_DIMS, "grid_multiplier %d outside [1, %d]", d.grid_multiplier,
                kMaxGridMultiplier);
  if (d.head_dim != 128 && d.head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (128 or 256)", d.head_dim);
  if (!pow2(d.page_size) || d.page_size < 16 || d.page_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "page_size %d not supported (power of two in [16, 1024])",
                d.page_size);
  if (d.partition_size < 16 || d.partition_size % 16 != 0 || d.partition_size > (1 << 20))
    return fail(PA_ERR_UNSUPPORTED, "partition_size %d must be a positive multiple of 16",
                d.partition_size);
  if (d.kv_dtype != PA_KV_BF16 && d.kv_dtype != PA_KV_FP8_E4M3FN)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype %d not supported", d.kv_dtype);
  if (d.kv_dtype == PA_KV_BF16 && d.kv_scale_mode != PA_SCALE_NONE)
    return fail(PA_ERR_SCALE_MODE, "bf16 KV takes no scales (kv_scale_mode must be NONE)");
  if (d.kv_dtype == PA_KV_FP8_E4M3FN && d.kv_scale_mode != PA_SCALE_PER_TENSOR &&
      d.kv_scale_mode != PA_SCALE_PER_TOKEN_HEAD)
    return fail(PA_ERR_SCALE_MODE, "fp8 KV needs PER_TENSOR or PER_TOKEN_HEAD scales");
  const int64_t capacity = static_cast<int64_t>(d.max_pages_per_seq) * d.page_size;
  if (capacity > (int64_t(1) << 30)) return fail(PA_ERR_DIMS, "max_pages_per_seq * page_size too large");
  const int64_t rows = static_cast<int64_t>(d.q_len) * (d.num_q_heads / d.num_kv_heads);
  int v = pa::pick_variant(d.head_dim, d.kv_dtype == PA_KV_FP8_E4M3FN, d.kv_scale_mode,
                                 static_cast<int>(rows > 4096 ? 4096 : rows), d.page_size,
                                 d.partition_size);
  int qb = d.q_len;
  if (need_decode && (rows > 4096 || v < 0)) {
    // more rows than one kernel holds: the queries go in blocks of the most
    // whose rows one does, each block decoded as its own work list
    const int64_t group = d.num_q_heads / d.num_kv_heads;
    qb = 0;
    for (int q = static_cast<int>(std::min<int64_t>(d.q_len, kMaxKernelRows)); q >= 1 && qb == 0; --q) {
      if (q * group > kMaxKernelRows) continue;
      v = pa::pick_variant(d.head_dim, d.kv_dtype == PA_KV_FP8_E4M3FN, d.kv_scale_mode,
                           static_cast<int>(q * group), d.page_size, d.partition_size);
      if (v >= 0) qb = q;
    }
    if (qb == 0)
      return fail(PA_ERR_UNSUPPORTED,
                  "num_q_heads / num_kv_heads = %lld rows of one query are more than the kernels "
                  "hold for head_dim %d",
                  static_cast<long long>(group), d.head_dim);
  }
  if (q_block) *q_block = qb;
  const int64_t pairs = static_cast<int64_t>(d.batch) * d.num_kv_heads;
  const int64_t items = pairs * ((capacity + d.partition_size - 1) / d.partition_size);
  if (pairs > (1 << 24) || items > (int64_t(1) << 30))
    return fail(PA_ERR_DIMS, "too many work items (%lld)", static_cast<long long>(items));
  *out = d;
  *variant = v;
  return PA_OK;
}

struct Layout {
  uint64_t status, wg_begin, wg_seg_begin, items, segs, nseg, seg_base, pseg_base, batch_base,
      partial_lse, partial_o, seg_info, wg_head, counters, total;
  int32_t grid, pairs, rows, max_items, max_segs;
};

uint64_t round256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

Layout layout(const pa_dims& d, int num_cus) {
  Layout L;
  L.grid = num_cus * d.grid_multiplier;
  L.pairs = d.batch * d.num_kv_heads;
  L.rows = d.q_len * (d.num_q_heads / d.num_kv_heads);
  const int64_t capacity = static_cast<int64_t>(d.max_pages_per_seq) * d.page_size;
  L.max_items = static_cast<int32_t>(L.pairs * ((capacity + d.partition_size - 1) / d.partition_size));
  L.max_segs = L.grid + L.pairs;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = round256(off + bytes);
    return o;
  };
  L.status = take(16);
  L.wg_begin = take(4ull * (L.grid + 1));
  L.wg_seg_begin = take(4ull * (L.grid + 1));
  L.items = take(16ull * L.max_items);
  L.segs = take(16ull * L.max_segs);
  L.nseg = take(4ull * L.pairs);
  L.seg_base = take(4ull * (L.pairs + 1));
  L.pseg_base = take(4ull * (L.pairs + 1));
  L.batch_base = take(4ull * (d.batch + 1));
  L.partial_lse = take(4ull * L.max_segs * L.rows);
  L.partial_o = take(4ull * L.max_segs * L.rows * d.head_dim);
  L.seg_info = take(32ull * L.max_segs);
  L.wg_head = take(64ull * L.grid);
  L.counters = take(4ull * L.pairs);
  L.total = off;
  return L;
}

// The work list of one block of queries (all of them when they fit one
// kernel), and the blocks: block j holds queries [j qb, min((j+1) qb, q_len)),
// each with its own block_bytes of workspace.
struct Geometry {
  Layout L;
  int qb, nblk;
  uint64_t block_bytes, total;
};

Geometry geometry(const pa_dims& d, int num_cus, int qb) {
  Geometry g;
  pa_dims db = d;
  db.q_len = qb;
  g.L = layout(db, num_cus);
  g.qb = qb;
  g.nblk = (d.q_len + qb - 1) / qb;
  g.block_bytes = round256(g.L.total);
  g.total = g.block_bytes * static_cast<uint64_t>(g.nblk);
  return g;
}

int block_q_len(const pa_plan_t* p, int j) { return std::min(p->q_block, p->dims.q_len - j * p->q_block); }
int num_blocks(const pa_plan_t* p) { return (p->dims.q_len + p->q_block - 1) / p->q_block; }

int current_device(int* dev) {
  const hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  return PA_OK;
}

template <typename T>
T* at(const pa_plan_t* p, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(p->workspace) + off);
}

int check_plan(const pa_plan_t* plan) {
  if (!plan) return fail(PA_ERR_NULL, "plan is NULL");
  if (plan->magic != PA_PLAN_MAGIC) return fail(PA_ERR_PLAN_MISMATCH, "plan was not built by pa_plan");
  int dev = -1;
  if (int rc = current_device(&dev)) return rc;
  if (dev != plan->device)
    return fail(PA_ERR_PLAN_MISMATCH, "plan was built on device %d, current device is %d",
                plan->device, dev);
  return PA_OK;
}

int check_decode_args(const pa_plan_t* plan, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* context_lens, int32_t q_len,
                      int32_t kv_scale_mode, const float* kv_scales, const void* out) {
  if (!plan) return fail(PA_ERR_NULL, "plan is NULL");
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out)
    return fail(PA_ERR_NULL, "q, k_cache, v_cache, block_table, context_lens and out are required");
  if (plan->magic != PA_PLAN_MAGIC) return fail(PA_ERR_PLAN_MISMATCH, "plan was not built by pa_plan");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(PA_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_ALIGN, "block_table and context_lens must be 4-byte aligned");
  if (q_len != plan->dims.q_len)
    return fail(PA_ERR_PLAN_MISMATCH, "q_len %d differs from the plan's %d", q_len, plan->dims.q_len);
  if (kv_scale_mode != plan->dims.kv_scale_mode)
    return fail(PA_ERR_PLAN_MISMATCH, "kv_scale_mode %d differs from the plan's %d", kv_scale_mode,
                plan->dims.kv_scale_mode);
  if ((kv_scale_mode == PA_SCALE_NONE) != (kv_scales == nullptr))
    return fail(PA_ERR_SCALE_MODE, "kv_scales must be NULL exactly when kv_scale_mode is NONE");
  if (kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD && !aligned(kv_scales, 16))
    return fail(PA_ERR_ALIGN, "per-token kv_scales must be 16-byte aligned");
  if (kv_scale_mode == PA_SCALE_PER_TENSOR && !aligned(kv_scales, 4))
    return fail(PA_ERR_ALIGN, "per-tensor kv_scales must be 4-byte aligned");
  return check_plan(plan);
}

// Kernel arguments of query block blk (its queries' rows of q and out, its
// part of the workspace).
pa::DecodeArgs decode_args(const pa_plan_t* plan, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, float scale, const float* kv_scales,
                           void* out, int blk = 0) {
  const pa_dims& d = plan->dims;
  const uint64_t wb = plan->block_bytes * static_cast<uint64_t>(blk);
  const int64_t q0 = static_cast<int64_t>(blk) * plan->q_block * d.num_q_heads * d.head_dim;
  const int group = d.num_q_heads / d.num_kv_heads;
  pa::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q) + q0;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.seg_info = at<const int32_t>(plan, plan->off_seg_info + wb);
  a.wg_head = at<const int32_t>(plan, plan->off_wg_head + wb);
  a.nseg = at<const int32_t>(plan, plan->off_nseg + wb);
  a.seg_base = at<const int32_t>(plan, plan->off_seg_base + wb);
  a.kv_scales = kv_scales;
  a.out = static_cast<uint16_t*>(out) + q0;
  a.partial_o = at<float>(plan, plan->off_partial_o + wb);
  a.partial_lse = at<float>(plan, plan->off_partial_lse + wb);
  a.status = at<int32_t>(plan, plan->off_status + wb);
  a.counters = (d.flags & PA_FLAG_FUSED_REDUCE) ? at<int32_t>(plan, plan->off_counters + wb) : nullptr;
  a.batch = d.batch;
  a.q_len = block_q_len(plan, blk);
  a.q_total = d.q_len;
  a.num_q_heads = d.num_q_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.group = group;
  a.rows = a.q_len * group;
  a.ps_log2 = log2i(d.page_size);
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.ctx_offset = d.q_len - (blk * plan->q_block + a.q_len);
  a.capacity = d.max_pages_per_seq * d.page_size;
  a.scale_mode = d.kv_scale_mode;
  a.debug_bounds = (d.flags & PA_FLAG_DEBUG_BOUNDS) ? 1 : 0;
  a.qk_scale_log2 = scale * 1.4426950408889634f;
  a.out_scale = 1.0f;
  return a;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_query_device(int32_t device, int32_t* num_cus) {
  if (!num_cus) return fail(PA_ERR_NULL, "num_cus is NULL");
  if (device < 0 || device >= kMaxDevices) return fail(PA_ERR_DEVICE, "device %d out of range", device);
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_cu_cache[device] > 0) {
      *num_cus = g_cu_cache[device];
      return ok();
    }
  }
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device >= count)
    return fail(PA_ERR_DEVICE, "no HIP device %d", device);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(PA_ERR_DEVICE, "hipGetDeviceProperties(%d) failed", device);
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(PA_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", device,
                prop.gcnArchName);
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n < 1)
    return fail(PA_ERR_DEVICE, "cannot read the CU count of device %d", device);
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_cu_cache[device] = n;
  }
  *num_cus = n;
  return ok();
}

int pa_plan_choice(const pa_dims* dims, int32_t num_cus, pa_dims* chosen) {
  if (!chosen) return fail(PA_ERR_NULL, "chosen is NULL");
  if (num_cus < 1 || num_cus > 65536) return fail(PA_ERR_DIMS, "num_cus %d out of range", num_cus);
  pa_dims d;
  int v = -1, qb = 0;
  if (int rc = check_dims(dims, &d, &v, true, &qb, num_cus)) return rc;
  *chosen = d;
  return ok();
}

int pa_workspace_bytes(const pa_dims* dims, int32_t num_cus, uint64_t* bytes) {
  if (!bytes) return fail(PA_ERR_NULL, "bytes is NULL");
  if (num_cus < 1 || num_cus > 65536) return fail(PA_ERR_DIMS, "num_cus %d out of range", num_cus);
  pa_dims d;
  int v = -1, qb = 0;
  if (int rc = check_dims(dims, &d, &v, true, &qb, num_cus)) return rc;
  *bytes = geometry(d, num_cus, qb).total;
  return ok();
}

int pa_plan(const pa_dims* dims, const int32_t* context_lens, void* workspace,
            uint64_t workspace_bytes, pa_plan_t* plan, void* stream) {
  pa_dims d;
  int v = -1, qb = 0;
  // argument errors first, before any HIP call; the tuned choice needs the
  // device's CU count, so the dims are checked again with it below
  if (int rc = check_dims(dims, &d, &v, true, &qb)) return rc;
  if (!context_lens || !plan) return fail(PA_ERR_NULL, "context_lens and plan are required");
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(PA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(context_lens, 4)) return fail(PA_ERR_ALIGN, "context_lens must be 4-byte aligned");
  int dev = -1;
  if (int rc = current_device(&dev)) return rc;
  int32_t cus = 0;
  if (int rc = pa_query_device(dev, &cus)) return rc;
  if (int rc = check_dims(dims, &d, &v, true, &qb, cus)) return rc;
  const Geometry gm = geometry(d, cus, qb);
  const Layout& L = gm.L;
  if (workspace_bytes < gm.total)
    return fail(PA_ERR_WORKSPACE, "workspace of %llu bytes, %llu needed",
                static_cast<unsigned long long>(workspace_bytes),
                static_cast<unsigned long long>(gm.total));
  pa_plan_t p;
  memset(&p, 0, sizeof(p));
  p.magic = PA_PLAN_MAGIC;
  p.device = dev;
  p.dims = d;
  p.num_cus = cus;
  p.grid = L.grid;
  p.rows = L.rows;
  p.num_pairs = L.pairs;
  p.max_items = L.max_items;
  p.max_segs = L.max_segs;
  p.variant = v;
  p.q_block = gm.qb;
  p.block_bytes = gm.block_bytes;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.off_status = L.status;
  p.off_wg_begin = L.wg_begin;
  p.off_wg_seg_begin = L.wg_seg_begin;
  p.off_items = L.items;
  p.off_segs = L.segs;
  p.off_nseg = L.nseg;
  p.off_seg_base = L.seg_base;
  p.off_pseg_base = L.pseg_base;
  p.off_batch_base = L.batch_base;
  p.off_partial_lse = L.partial_lse;
  p.off_partial_o = L.partial_o;
  p.off_seg_info = L.seg_info;
  p.off_wg_head = L.wg_head;
  p.off_counters = L.counters;

  // one work list per block of queries; block j sees the keys up to its
  // last query, ctx - (q_len - its end) of them
  for (int j = 0; j < gm.nblk; ++j) {
    const uint64_t wb = gm.block_bytes * static_cast<uint64_t>(j);
    const int qj = block_q_len(&p, j);
    pa::PlanArgs a;
    a.context_lens = context_lens;
    a.status = at<int32_t>(&p, p.off_status + wb);
    a.wg_begin = at<int32_t>(&p, p.off_wg_begin + wb);
    a.wg_seg_begin = at<int32_t>(&p, p.off_wg_seg_begin + wb);
    a.items = at<pa::Span>(&p, p.off_items + wb);
    a.segs = at<pa::Span>(&p, p.off_segs + wb);
    a.nseg = at<int32_t>(&p, p.off_nseg + wb);
    a.seg_base = at<int32_t>(&p, p.off_seg_base + wb);
    a.pseg_base = at<int32_t>(&p, p.off_pseg_base + wb);
    a.batch_base = at<int32_t>(&p, p.off_batch_base + wb);
    a.seg_info = at<int32_t>(&p, p.off_seg_info + wb);
    a.wg_head = at<int32_t>(&p, p.off_wg_head + wb);
    a.counters = at<int32_t>(&p, p.off_counters + wb);
    a.batch = d.batch;
    a.num_kv_heads = d.num_kv_heads;
    a.q_len = qj;
    a.partition = d.partition_size;
    a.grid = L.grid;
    a.capacity = d.max_pages_per_seq * d.page_size;
    a.q_check = d.q_len;
    a.ctx_offset = d.q_len - (j * gm.qb + qj);
    if (int rc = hip_check(pa::launch_plan(a, L.max_items, static_cast<hipStream_t>(stream)),
                           "plan launch"))
      return rc;
  }
  *plan = p;
  return ok();
}

int pa_decode_partition(const pa_plan_t* plan, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* block_table,
                        const int32_t* context_lens, int32_t q_len, float scale,
                        int32_t kv_scale_mode, const float* kv_scales, void* out, void* stream) {
  if (int rc = check_decode_args(plan, q, k_cache, v_cache, block_table, context_lens, q_len,
                                 kv_scale_mode, kv_scales, out))
    return rc;
  for (int j = 0; j < num_blocks(plan); ++j) {
    const pa::DecodeArgs a =
        decode_args(plan, q, k_cache, v_cache, block_table, context_lens, scale, kv_scales, out, j);
    if (int rc = hip_check(pa::launch_partition(plan->variant, a, plan->grid,
                                                static_cast<hipStream_t>(stream)),
                           "partition launch"))
      return rc;
  }
  return ok();
}

int pa_decode_reduce(const pa_plan_t* plan, int32_t q_len, int32_t kv_scale_mode, void* out,
                     void* stream) {
  if (!plan || !out) return fail(PA_ERR_NULL, "plan and out are required");
  if (plan->magic != PA_PLAN_MAGIC) return fail(PA_ERR_PLAN_MISMATCH, "plan was not built by pa_plan");
  if (!aligned(out, 16)) return fail(PA_ERR_ALIGN, "out must be 16-byte aligned");
  if (q_len != plan->dims.q_len || kv_scale_mode != plan->dims.kv_scale_mode)
    return fail(PA_ERR_PLAN_MISMATCH, "q_len / kv_scale_mode differ from the plan's");
  if (int rc = check_plan(plan)) return rc;
  // A context never longer than one partition (partition_size >= the block
  // table's capacity) makes every pair a single item, hence a single
  // segment, written out by the partition pass: nothing is left to merge.
  // A fused-reduce plan's partition pass merged the split pairs itself.
  if (plan->max_items <= plan->num_pairs || (plan->dims.flags & PA_FLAG_FUSED_REDUCE)) return ok();
  for (int j = 0; j < num_blocks(plan); ++j) {
    pa::DecodeArgs a = decode_args(plan, out, out, out, nullptr, nullptr, 1.0f, nullptr, out, j);
    if (int rc = hip_check(pa::launch_reduce(a, plan->dims.head_dim, plan->num_pairs,
                                             static_cast<hipStream_t>(stream)),
                           "reduce launch"))
      return rc;
  }
  return ok();
}

int pa_decode(const pa_plan_t* plan, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* context_lens, int32_t q_len, float scale,
              int32_t kv_scale_mode, const float* kv_scales, void* out, void* stream) {
  if (int rc = pa_decode_partition(plan, q, k_cache, v_cache, block_table, context_lens, q_len,
                                   scale, kv_scale_mode, kv_scales, out, stream))
    return rc;
  return pa_decode_reduce(plan, q_len, kv_scale_mode, out, stream);
}

int pa_plan_status(const pa_plan_t* plan, int32_t* device_status, void* stream) {
  if (!device_status) return fail(PA_ERR_NULL, "device_status is NULL");
  if (int rc = check_plan(plan)) return rc;
  if (int rc = hip_check(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize"))
    return rc;
  int32_t all = 0;
  for (int j = 0; j < num_blocks(plan); ++j) {
    int32_t st = 0;
    const uint64_t wb = plan->block_bytes * static_cast<uint64_t>(j);
    if (int rc = hip_check(hipMemcpy(&st, at<int32_t>(plan, plan->off_status + wb), sizeof(st),
                                     hipMemcpyDeviceToHost),
                           "hipMemcpy status"))
      return rc;
    all |= st;
  }
  *device_status = all;
  return ok();
}

int pa_debug_gather(const pa_plan_t* plan, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* context_lens,
                    const float* kv_scales, void* k_out, void* v_out, float* scales_out,
                    void* stream) {
  if (!plan || !k_cache || !v_cache || !block_table || !context_lens || !k_out || !v_out)
    return fail(PA_ERR_NULL, "plan, caches, block_table, context_lens, k_out and v_out are required");
  if (plan->magic != PA_PLAN_MAGIC) return fail(PA_ERR_PLAN_MISMATCH, "plan was not built by pa_plan");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(PA_ERR_ALIGN, "caches and outputs must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_ALIGN, "block_table and context_lens must be 4-byte aligned");
  const pa_dims& d = plan->dims;
  const bool per_tok = d.kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD;
  if ((d.kv_scale_mode == PA_SCALE_NONE) != (kv_scales == nullptr))
    return fail(PA_ERR_SCALE_MODE, "kv_scales must be NULL exactly when kv_scale_mode is NONE");
  if (per_tok && (!scales_out || !aligned(kv_scales, 16) || !aligned(scales_out, 4)))
    return fail(!scales_out ? PA_ERR_NULL : PA_ERR_ALIGN,
                "per-token mode needs scales_out (4-byte aligned) and 16-byte aligned kv_scales");
  if (int rc = check_plan(plan)) return rc;
  // the last query block's list: its keys reach the end of every context
  const int last = num_blocks(plan) - 1;
  pa::DecodeArgs a = decode_args(plan, k_cache, k_cache, v_cache, block_table, context_lens, 1.0f,
                                 kv_scales, k_out, last);
  return hip_check(pa::launch_loader(plan->variant, a, plan->max_segs, static_cast<uint8_t*>(k_out),
                                     static_cast<uint8_t*>(v_out), per_tok ? scales_out : nullptr,
                                     static_cast<hipStream_t>(stream)),
                   "loader launch") ?: ok();
}

int pa_cache_append(const pa_dims* dims, const void* new_k, const void* new_v,
                    const int32_t* block_table, const int32_t* context_lens, void* k_cache,
                    void* v_cache, float* kv_scales, int32_t* device_status, void* stream) {
  pa_dims d;
  int v = -1;
  if (int rc = check_dims(dims, &d, &v, false)) return rc;
  if (!new_k || !new_v || !block_table || !context_lens || !k_cache || !v_cache)
    return fail(PA_ERR_NULL, "new_k, new_v, block_table, context_lens, k_cache and v_cache are required");
  if (!aligned(new_k, 16) || !aligned(new_v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_ALIGN, "new_k, new_v, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(device_status, 4))
    return fail(PA_ERR_ALIGN, "block_table, context_lens and device_status must be 4-byte aligned");
  if ((d.kv_scale_mode == PA_SCALE_NONE) != (kv_scales == nullptr))
    return fail(PA_ERR_SCALE_MODE, "kv_scales must be NULL exactly when kv_scale_mode is NONE");
  if (kv_scales && !aligned(kv_scales, 4)) return fail(PA_ERR_ALIGN, "kv_scales must be 4-byte aligned");
  // element offsets of the new rows stay below 2^31
  const int64_t rows = static_cast<int64_t>(d.batch) * d.q_len * d.num_kv_heads;
  if (rows >= (int64_t(1) << 31) / d.head_dim)
    return fail(PA_ERR_DIMS, "batch * q_len * num_kv_heads = %lld rows is too many for one append",
                static_cast<long long>(rows));
  int dev = -1;
  if (int rc = current_device(&dev)) return rc;
  int32_t cus = 0;
  if (int rc = pa_query_device(dev, &cus)) return rc;
  pa::AppendArgs a;
  a.new_k = static_cast<const uint16_t*>(new_k);
  a.new_v = static_cast<const uint16_t*>(new_v);
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.kv_scales = kv_scales;
  a.status = device_status;
  a.rows = static_cast<int32_t>(rows);
  a.q_len = d.q_len;
  a.num_kv_heads = d.num_kv_heads;
  a.ps_log2 = log2i(d.page_size);
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.capacity = d.max_pages_per_seq * d.page_size;
  return hip_check(pa::launch_append(a, d.head_dim, d.kv_dtype == PA_KV_FP8_E4M3FN, d.kv_scale_mode,
                                     static_cast<hipStream_t>(stream)),
                   "append launch") ?: ok();
}

int pa_decode_static(const pa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* context_lens, int32_t q_len,
                     float scale, int32_t kv_scale_mode, const float* kv_scales, void* out,
                     pa_plan_t* plan_out, void* stream) {
  pa_dims d;
  int v = -1, qb = 0;
  if (int rc = check_dims(dims, &d, &v, true, &qb)) return rc;
  int dev = -1;
  if (int rc = current_device(&dev)) return rc;
  int32_t cus = 0;
  if (int rc = pa_query_device(dev, &cus)) return rc;
  if (int rc = check_dims(dims, &d, &v, true, &qb, cus)) return rc;
  const uint64_t need = geometry(d, cus, qb).total;
  if (need > kStaticScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_static: this problem needs %llu bytes of workspace; the static scratch "
                "holds %llu (use pa_plan with a caller workspace)",
                static_cast<unsigned long long>(need),
                static_cast<unsigned long long>(kStaticScratchBytes));
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  // the plan kernel writes every table and status word the decode reads, so
  // nothing left in the scratch by an earlier call needs clearing
  pa_plan_t plan;
  if (int rc = pa_plan(dims, context_lens, ws, kStaticScratchBytes, &plan, stream)) return rc;
  if (int rc = pa_decode(&plan, q, k_cache, v_cache, block_table, context_lens, q_len, scale,
                         kv_scale_mode, kv_scales, out, stream))
    return rc;
  if (plan_out) *plan_out = plan;
  return ok();
}

uint64_t pa_static_scratch_bytes(void) { return kStaticScratchBytes; }

int pa_debug_read_probe(const void* buffer, uint64_t buffer_bytes, const int32_t* blocks,
                        int32_t num_blocks, int32_t row_bytes, int32_t linear, int32_t waves,
                        float* sink, void* stream) {
  if (!buffer || !blocks || !sink) return fail(PA_ERR_NULL, "buffer, blocks and sink are required");
  if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512)
    return fail(PA_ERR_UNSUPPORTED, "row_bytes %d is not 128, 256 or 512", row_bytes);
  if (waves < 1 || waves > 16) return fail(PA_ERR_DIMS, "waves %d outside [1, 16]", waves);
  if (!aligned(buffer, 16) || !aligned(blocks, 4) || !aligned(sink, 4))
    return fail(PA_ERR_ALIGN, "buffer must be 16-byte aligned, blocks and sink 4-byte aligned");
  const uint64_t nbuf = buffer_bytes / (16ull * row_bytes);
  if (nbuf < 1 || nbuf > (1ull << 31) - 1 || num_blocks < 0)
    return fail(PA_ERR_DIMS, "buffer holds %llu blocks; 1 to 2^31 - 1 are supported",
                static_cast<unsigned long long>(nbuf));
  int dev = -1;
  if (int rc = current_device(&dev)) return rc;
  int32_t cus = 0;
  if (int rc = pa_query_device(dev, &cus)) return rc;
  return hip_check(pa::launch_read_probe(static_cast<const uint8_t*>(buffer), static_cast<int32_t>(nbuf),
                                         blocks, num_blocks, row_bytes, linear != 0, cus, waves, sink,
                                         static_cast<hipStream_t>(stream)),
                   "read probe launch") ?: ok();
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a pointer is misaligned";
    case PA_ERR_DIMS: return "PA_ERR_DIMS: invalid dimensions";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_PLAN_MISMATCH: return "PA_ERR_PLAN_MISMATCH: call does not match the plan";
    case PA_ERR_SCALE_MODE: return "PA_ERR_SCALE_MODE: kv dtype and scale mode disagree";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime error";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE: no usable gfx950 device";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

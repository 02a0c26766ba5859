// C ABI of the paged MLA decode library: argument checks, workspace layout and
// launches on the caller's stream.  The operation and the error rules are
// documented in include/mla_decode.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/mla_decode.h"
#include "mla_internal.h"
#include "mla_plan.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int device) {
  if (device < 0 || device >= kMaxDevices) return 0;
  int v = g_cu_count[device].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || c <= 0) return 0;
  g_cu_count[device].store(c, std::memory_order_relaxed);
  return c;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WorkspaceLayout {
  size_t tile_md, num_splits, part_lse, part_scale, part_o, total;
};

// [plan][partial lse][partial row scales][partial O].  The caller's workspace
// is sized for fp32 partial rows whichever kernel runs; `compact` sizes the
// partial O for the kernel that runs instead (the wide kernel keeps fp16
// tiles), which is what the static scratch of the no-allocation call holds.
WorkspaceLayout layout(int64_t batch, int64_t rows, int64_t dv, int64_t num_parts, bool compact = false,
                       bool wide = false) {
  WorkspaceLayout w;
  const int64_t slots = batch + num_parts;
  w.tile_md = 0;
  w.num_splits = align256((size_t)num_parts * mla::kTileMdInts * 4);
  w.part_lse = w.num_splits + align256((size_t)(batch + 1) * 4);
  w.part_scale = w.part_lse + align256((size_t)(slots * rows) * 4);
  w.part_o = w.part_scale + align256((size_t)(slots * rows) * 4);
  const size_t o_bytes = compact && wide ? (size_t)slots * (size_t)mla::partial_slot_bytes(rows)
                                         : (size_t)(slots * rows * dv) * 4;
  w.total = w.part_o + align256(o_bytes);
  return w;
}

// ---- the no-allocation call's scratch: plan and partials in a file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// never uses the array's name as an address: the first call on a device,
// with that device current, looks up its address there and keeps it.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<uint8_t*> g_scratch[64];
std::mutex g_scratch_mu;

mla_status scratch_address(int device, uint8_t** out) {
  if (device < 0 || device >= 64) return MLA_ERR_HIP;
  uint8_t* ptr = g_scratch[device].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[device].load(std::memory_order_relaxed);
    if (!ptr) {
      void* sym = nullptr;
      if (hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)) != hipSuccess || sym == nullptr) return MLA_ERR_HIP;
      ptr = (uint8_t*)sym;
      g_scratch[device].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int default_parts(int device, int rows) {
  const int cus = cu_count(device);
  if (cus <= 0) return -1;
  const int per = cus / mla::row_blocks(rows);
  return per < 1 ? 1 : per;
}

mla_status check_plan_args(int32_t batch, int32_t q_rows, int32_t h_kv, int32_t num_parts) {
  if (batch < 0 || q_rows <= 0 || h_kv <= 0 || num_parts <= 0) return MLA_ERR_BAD_SHAPE;
  if (q_rows % h_kv) return MLA_ERR_BAD_SHAPE;
  if (q_rows / h_kv > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
  if (num_parts > (1 << 20)) return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

// The 128-row decode kernel of a bf16 cache has an instance that plans in
// its prologue (every wave scans the lengths; the split counts are listed in
// LDS), used for at most kPlanInKernelMaxBatch sequences and when the plan's
// costs, with lengths clamped to the table's width, sum below 2^31.  (Built
// with the plan code, the 16-row kernel ran 20% slower even when given a
// plan, and the fp8 one spilled registers; they keep the plan kernel.)
bool plan_fits_kernel(int64_t batch, int c, int64_t max_blocks) {
  const int64_t units = c + (max_blocks > 1 ? max_blocks : 1);
  return batch >= 1 && batch <= mla::kPlanInKernelMaxBatch && batch * units < ((int64_t)1 << 31);
}

// Checks, plan and launches of one decode call.  With no_alloc the plan and the
// partials go to the static scratch instead of the caller's workspace (whose
// fields are then ignored).
mla_status decode_call(const mla_decode_params* p, void* stream, bool no_alloc) {
  if (!p) return MLA_ERR_NULL_POINTER;
  if (p->batch < 0 || p->s_q <= 0 || p->h_q <= 0 || p->h_kv <= 0 || p->num_blocks < 0 ||
      p->max_blocks_per_seq < 0 || p->block_size <= 0 || p->d <= 0 || p->dv <= 0)
    return MLA_ERR_BAD_SHAPE;
  if (p->d != 576 || p->dv != 512 || p->block_size != 64 || p->h_kv != 1) return MLA_ERR_UNSUPPORTED;
  if (p->h_q % p->h_kv) return MLA_ERR_BAD_SHAPE;
  const int64_t rows = (int64_t)p->s_q * p->h_q / p->h_kv;
  if (rows > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
  if (!(p->softmax_scale == p->softmax_scale) || isinf(p->softmax_scale)) return MLA_ERR_BAD_ARGUMENT;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_BAD_ARGUMENT;
  const bool kv8 = p->kv_dtype == MLA_KV_FP8_E4M3;
  if (kv8 && !(p->kv_scale > 0.f && isfinite(p->kv_scale))) return MLA_ERR_BAD_ARGUMENT;
  const int64_t kelem = kv8 ? 1 : 2;  // bytes per cache element
  if (p->batch == 0) return MLA_OK;
  if (!p->q || !p->k_cache || !p->block_table || !p->cache_seqlens || !p->out || !p->lse ||
      (!no_alloc && !p->workspace))
    return MLA_ERR_NULL_POINTER;
  if ((p->tile_md == nullptr) != (p->num_splits == nullptr)) return MLA_ERR_NULL_POINTER;
  // strides and alignment (elements; 16-byte vector loads and stores)
  if (!aligned16(p->q) || !aligned16(p->k_cache) || !aligned16(p->out)) return MLA_ERR_BAD_STRIDE;
  if (!no_alloc && ((uintptr_t)p->workspace & 255) != 0) return MLA_ERR_BAD_STRIDE;
  if (p->q_batch_stride % 8 || p->q_seq_stride % 8 || p->q_head_stride % 8) return MLA_ERR_BAD_STRIDE;
  if (p->out_batch_stride % 8 || p->out_seq_stride % 8 || p->out_head_stride % 8) return MLA_ERR_BAD_STRIDE;
  if ((p->k_block_stride * kelem) % 16 || (p->k_row_stride * kelem) % 16 || p->k_row_stride < p->d)
    return MLA_ERR_BAD_STRIDE;
  if (p->k_block_stride < 0 || p->q_batch_stride < 0 || p->q_seq_stride < 0 || p->q_head_stride < 0 ||
      p->out_batch_stride < 0 || p->out_seq_stride < 0 || p->out_head_stride < 0 ||
      p->lse_batch_stride < 0 || p->lse_seq_stride < 0 || p->lse_head_stride < 0)
    return MLA_ERR_BAD_STRIDE;
  if (p->block_table_stride < p->max_blocks_per_seq) return MLA_ERR_BAD_STRIDE;
  // a page's 64 rows lie inside one block stride (the copy reads rows 0..63 of a block)
  if (p->k_block_stride < (int64_t)(p->block_size - 1) * p->k_row_stride + p->d) return MLA_ERR_BAD_STRIDE;
  if ((int64_t)64 * p->k_row_stride * kelem > INT32_MAX) return MLA_ERR_BAD_STRIDE;
  if ((int64_t)p->max_blocks_per_seq * 64 > INT32_MAX) return MLA_ERR_BAD_SHAPE;

  int num_parts = p->num_parts;
  if (p->tile_md) {
    if (num_parts <= 0) return MLA_ERR_BAD_SHAPE;
  } else if (num_parts <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    num_parts = default_parts(dev, (int)rows);
    if (num_parts < 0) return MLA_ERR_HIP;
  }
  if (num_parts > (1 << 20)) return MLA_ERR_BAD_SHAPE;
  const bool wide = kv8 || mla::rows_per_block((int)rows) == mla::kRowsPerWorkgroup;
  const WorkspaceLayout w = layout(p->batch, rows, p->dv, num_parts, no_alloc, wide);
  uint8_t* ws = (uint8_t*)p->workspace;
  if (no_alloc) {
    if (w.total > kScratchBytes) return MLA_ERR_SCRATCH_TOO_SMALL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    const mla_status st = scratch_address(dev, &ws);
    if (st != MLA_OK) return st;
  } else if (p->workspace_bytes < w.total) {
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  }

  hipStream_t s = (hipStream_t)stream;
  const int32_t* tile_md = p->tile_md;
  const int32_t* num_splits = p->num_splits;
  // No metadata: the decode workgroups plan their own parts when the batch is
  // small enough for every wave to scan the lengths; otherwise the plan
  // kernel runs first.  Either way the plan lands in the workspace.
  const int plan_c = mla::segment_cost(mla::rows_per_block((int)rows));
  int32_t* plan_md = (int32_t*)(ws + w.tile_md);
  int32_t* plan_ns = (int32_t*)(ws + w.num_splits);
  const bool plan_in_kernel = !tile_md && !kv8 && mla::rows_per_block((int)rows) == mla::kRowsPerWorkgroup &&
                              plan_fits_kernel(p->batch, plan_c, p->max_blocks_per_seq);
  if (!tile_md) {
    if (!plan_in_kernel) {
      if (p->batch > mla::kMaxPlanBatch) return MLA_ERR_UNSUPPORTED;
      if (mla::launch_plan(p->cache_seqlens, p->batch, (int)rows, num_parts, plan_md, plan_ns, s) != hipSuccess)
        return MLA_ERR_HIP;
    }
    tile_md = plan_md;
    num_splits = plan_ns;
  }

  mla::DecodeArgs a;
  a.q = (const uint16_t*)p->q;
  a.q_sb = p->q_batch_stride;
  a.q_ss = p->q_seq_stride;
  a.q_sh = p->q_head_stride;
  a.k = (const uint8_t*)p->k_cache;
  a.k_block_bytes = p->k_block_stride * kelem;
  a.k_row_bytes = p->k_row_stride * kelem;
  a.num_blocks = p->num_blocks;
  a.block_table = p->block_table;
  a.bt_stride = p->block_table_stride;
  a.max_blocks = p->max_blocks_per_seq;
  a.seqlens = p->cache_seqlens;
  a.batch = p->batch;
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.rows = (int32_t)rows;
  a.causal = p->causal ? 1 : 0;
  a.scale_log2 = kv8 ? (float)((double)p->softmax_scale * (double)p->kv_scale * 1.4426950408889634)
                    : p->softmax_scale * 1.4426950408889634f;
  a.kv8 = kv8 ? 1 : 0;
  a.kv_scale = kv8 ? p->kv_scale : 1.f;
  a.tile_md = tile_md;
  a.num_splits = num_splits;
  a.num_parts = num_parts;
  a.plan_in_kernel = plan_in_kernel ? 1 : 0;
  a.plan_c = plan_c;
  a.plan_md = plan_in_kernel ? plan_md : nullptr;
  a.plan_ns = plan_in_kernel ? plan_ns : nullptr;
  a.row_blocks = mla::row_blocks((int)rows);
  a.part_lse = (float*)(ws + w.part_lse);
  a.part_o = (float*)(ws + w.part_o);
  a.part_scale = (float*)(ws + w.part_scale);
  a.out = (uint16_t*)p->out;
  a.o_sb = p->out_batch_stride;
  a.o_ss = p->out_seq_stride;
  a.o_sh = p->out_head_stride;
  a.lse = p->lse;
  a.l_sb = p->lse_batch_stride;
  a.l_ss = p->lse_seq_stride;
  a.l_sh = p->lse_head_stride;

  if (mla::launch_decode(a, s) != hipSuccess) return MLA_ERR_HIP;
  if (mla::launch_combine(a, s) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

static_assert(sizeof(mla_status) == sizeof(int), "mla_status is an int");

extern "C" {

const char* mla_status_string(mla_status status) {
  // A C caller may pass any int; in C++ reading an enum object outside the
  // enumerators' range is undefined, so read its bytes as an int instead.
  int code;
  memcpy(&code, &status, sizeof code);
  switch (code) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "invalid or inconsistent size";
    case MLA_ERR_BAD_STRIDE: return "stride or alignment not supported";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration (needs d=576, dv=512, block_size=64, h_kv=1)";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_BAD_ARGUMENT: return "invalid argument";
    case MLA_ERR_SCRATCH_TOO_SMALL: return "the call needs more than the library's 64 MiB static scratch";
    default: return "unknown status";
  }
}

size_t mla_decode_params_size(void) { return sizeof(mla_decode_params); }

mla_status mla_default_num_parts(int device, int32_t q_rows, int32_t h_kv, int32_t* num_parts) {
  if (!num_parts) return MLA_ERR_NULL_POINTER;
  if (q_rows <= 0 || h_kv <= 0 || q_rows % h_kv) return MLA_ERR_BAD_SHAPE;
  const int p = default_parts(device, q_rows / h_kv);
  if (p < 0) return MLA_ERR_HIP;
  *num_parts = p;
  return MLA_OK;
}

mla_status mla_plan_host(const int32_t* cache_seqlens_h, int32_t batch, int32_t q_rows, int32_t h_kv,
                  int32_t num_parts, int32_t* tile_md_h, int32_t* num_splits_h) {
  if ((!cache_seqlens_h && batch > 0) || !tile_md_h || !num_splits_h) return MLA_ERR_NULL_POINTER;
  const mla_status st = check_plan_args(batch, q_rows, h_kv, num_parts);
  if (st != MLA_OK) return st;
  std::vector<int64_t> prefix((size_t)batch + 1);
  mla::plan_split_kv_host(cache_seqlens_h, batch, q_rows / h_kv, num_parts, tile_md_h, num_splits_h,
                          prefix.data());
  return MLA_OK;
}

mla_status mla_get_metadata(const int32_t* cache_seqlens_d, int32_t batch, int32_t q_rows, int32_t h_kv,
                     int32_t num_parts, int32_t* tile_md_d, int32_t* num_splits_d, void* stream) {
  if ((!cache_seqlens_d && batch > 0) || !tile_md_d || !num_splits_d) return MLA_ERR_NULL_POINTER;
  const mla_status st = check_plan_args(batch, q_rows, h_kv, num_parts);
  if (st != MLA_OK) return st;
  if (batch > mla::kMaxPlanBatch) return MLA_ERR_UNSUPPORTED;
  if (mla::launch_plan(cache_seqlens_d, batch, q_rows / h_kv, num_parts, tile_md_d, num_splits_d,
                       (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_workspace_size(int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t dv,
                       int32_t num_parts, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL_POINTER;
  if (batch < 0 || s_q <= 0 || h_q <= 0 || h_kv <= 0 || dv <= 0 || h_q % h_kv) return MLA_ERR_BAD_SHAPE;
  const int64_t rows = (int64_t)s_q * h_q / h_kv;
  if (rows > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
  if (num_parts <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    num_parts = default_parts(dev, (int)rows);
    if (num_parts < 0) return MLA_ERR_HIP;
  }
  *bytes = layout(batch, rows, dv, num_parts).total;
  return MLA_OK;
}

mla_status mla_decode_with_kvcache(const mla_decode_params* p, void* stream) {
  return decode_call(p, stream, false);
}

mla_status mla_decode_with_kvcache_noalloc(const mla_decode_params* p, void* stream) {
  return decode_call(p, stream, true);
}

}  // extern "C"

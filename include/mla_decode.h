/*
 * Paged Multi-head Latent Attention (MLA) decode on MI355X (gfx950).
 *
 * A C ABI over a HIP library (libmla_decode.so).  Plain pointers and sizes
 * only; a hipStream_t is passed as void* (NULL = the default stream).
 *
 * The operation.  Each cached token is one 576-element bf16 latent row shared
 * by every query head: K is the whole row (512 latent + 64 rope elements) and
 * V is its first 512 elements.  Tokens live in 64-token pages that a block
 * table maps (the PAI FlashMLA tutorial on segmentfault, "云上玩转DeepSeek系列之五：
 * 实测优化16%, 体验FlashMLA加速DeepSeek-V2-Lite推理", section 二.4, builds q,
 * block_table and blocked_k this way and returns (out, lse)).  For sequence b
 * with n = cache_seqlens[b] tokens, query token i < s_q and head h:
 *     s_t = softmax_scale * <q[b,i,h,:], k_t>,   t visible
 *     lse[b,i,h] = ln(sum_t exp(s_t))
 *     out[b,i,h,:] = sum_t exp(s_t - lse) * v_t
 * where t < n is visible, or, with causal masking, t < n - (s_q - 1 - i)
 * (the query tokens are the last s_q positions).  No visible key gives
 * out = 0 and lse = -inf.
 *
 * The work is split along the key length and the pieces merged by their lse
 * (Flash-Decoding, as the Hacker News discussion of the FlashMLA release
 * describes it).  The same tutorial, section 二.2 (FlashMLA as a vLLM
 * attention backend), names the two calls a serving engine makes: a metadata
 * builder prepares the forward's metadata with get_mla_metadata, and the
 * attention implementation runs the forward with flash_mla_with_kvcache.
 * mla_get_metadata and mla_decode_with_kvcache follow that split; since the
 * plan depends only on the lengths, one plan serves every layer of a step
 * (our reading).
 *
 * Cache entries may be stored at the dense 576-element pitch or at the
 * 256-byte-aligned 640-element pitch of vLLM pull request "[Perf] Mem align
 * KV caches for CUDA devices (MLA perf improvement) #12676" (a padded
 * allocation viewed through its first 576 elements); the pitch is the row
 * stride below.  Pad elements are never read.
 *
 * Errors.  Every function returns an mla_status.  All argument checks happen
 * on the host before anything is enqueued; on error nothing is launched and
 * no output is touched.  The library never allocates, frees or synchronises,
 * and never reads device memory from the host; it keeps no state besides a
 * per-device cache of the compute-unit count, so calls from several threads
 * are safe.  Launch failures are reported as MLA_ERR_HIP.
 *
 * Device-side preconditions (not checkable on the host without a copy):
 * 0 <= cache_seqlens[b] <= max_blocks_per_seq * 64 (larger values are clamped
 * to the table's width, negative ones read as an empty sequence),
 * block_table entries of used pages lie in [0, num_blocks) (a page outside
 * that range is never read; its sequence's rows come out NaN instead), and
 * no input is written while a call that reads it is in flight.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,         /* a required pointer is NULL */
  MLA_ERR_BAD_SHAPE = 2,            /* a size is negative, zero where it must not be, or inconsistent */
  MLA_ERR_BAD_STRIDE = 3,           /* a stride or base address breaks the alignment rules */
  MLA_ERR_UNSUPPORTED = 4,          /* d != 576, dv != 512, block_size != 64, h_kv != 1, too many rows */
  MLA_ERR_WORKSPACE_TOO_SMALL = 5,  /* workspace_bytes < mla_workspace_size(...) */
  MLA_ERR_HIP = 6,                  /* the HIP runtime reported an error */
  MLA_ERR_BAD_ARGUMENT = 7,         /* any other invalid scalar (e.g. non-finite softmax_scale) */
  MLA_ERR_SCRATCH_TOO_SMALL = 8     /* mla_decode_with_kvcache_noalloc: the call needs more than the
                                       library's static scratch (MLA_NOALLOC_SCRATCH_BYTES) */
} mla_status;

/* int32 values per part in the tile-scheduler metadata. */
#define MLA_TILE_MD_INTS 8
/* Rows (s_q * h_q / h_kv) handled by one workgroup; more rows use several. */
#define MLA_ROWS_PER_WORKGROUP 128
/* Upper bound on s_q * h_q / h_kv. */
#define MLA_MAX_ROWS 1024
/* Bytes of static device scratch behind mla_decode_with_kvcache_noalloc, per GPU. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Static, NUL-terminated description of a status. */
const char* mla_status_string(mla_status status);

/* sizeof(mla_decode_params) as compiled into the library, so that foreign-language
   bindings can check their mirror of the struct. */
size_t mla_decode_params_size(void);

/*
 * Number of parts the planner should cut the key work into on `device` for
 * q_rows = s_q * h_q query rows over h_kv kv heads: one workgroup per compute
 * unit, shared among the row blocks.  Advisory; any value >= 1 is valid.
 */
mla_status mla_default_num_parts(int device, int32_t q_rows, int32_t h_kv, int32_t* num_parts);

/*
 * The split-KV plan (tile-scheduler metadata), enqueued on `stream`.
 *
 * cache_seqlens_d : device int32 [batch], read only.
 * q_rows          : s_q * h_q (the rows that share one kv head after dividing by h_kv).
 * num_parts       : number of work ranges (>= 1); see mla_default_num_parts.
 * tile_md_d       : device int32 [num_parts][MLA_TILE_MD_INTS], written.  Part p covers
 *                   pages (seq_begin, page_begin) .. (seq_last, page_end - 1) of the
 *                   flattened (sequence, page) order; entry 4 is the split index of its
 *                   first sequence.  An idle part has seq_begin == batch.
 * num_splits_d    : device int32 [batch + 1], written: prefix sums of the number of
 *                   parts that touch each sequence (num_splits[0] = 0).
 * batch <= 16384 (MLA_ERR_UNSUPPORTED otherwise; mla_plan_host has no limit).
 * The plan depends only on (cache_seqlens, batch, q_rows, h_kv, num_parts), so one plan
 * serves every layer's decode of one step.  Asynchronous; the caller owns all buffers.
 */
mla_status mla_get_metadata(const int32_t* cache_seqlens_d, int32_t batch, int32_t q_rows,
                     int32_t h_kv, int32_t num_parts, int32_t* tile_md_d,
                     int32_t* num_splits_d, void* stream);

/* The same plan computed on the host from host arrays; bit-identical to mla_get_metadata. */
mla_status mla_plan_host(const int32_t* cache_seqlens_h, int32_t batch, int32_t q_rows, int32_t h_kv,
                  int32_t num_parts, int32_t* tile_md_h, int32_t* num_splits_h);

/*
 * Workspace bytes mla_decode_with_kvcache needs for these sizes: room for an internal
 * plan (used when no plan is passed) and for the per-split partial results
 * ((batch + num_parts) slots of rows * (dv + 2) fp32).  num_parts <= 0 means
 * mla_default_num_parts of the current device.
 */
mla_status mla_workspace_size(int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t dv,
                       int32_t num_parts, size_t* bytes);

typedef struct mla_decode_params {
  /* queries: bf16 [batch][s_q][h_q][d]; strides in elements, last dimension contiguous */
  const void* q;
  int64_t q_batch_stride, q_seq_stride, q_head_stride;
  int32_t batch, s_q, h_q;

  /* paged latent cache: bf16 [num_blocks][block_size][h_kv][d] viewed with these element
     strides; k_row_stride is the entry pitch (576 dense, 640 for 256-byte-aligned entries) */
  const void* k_cache;
  int64_t k_block_stride, k_row_stride, k_head_stride;
  int32_t num_blocks, block_size, h_kv, d;

  /* block table: int32 [batch][max_blocks_per_seq] with this row stride (elements) */
  const int32_t* block_table;
  int64_t block_table_stride;
  int32_t max_blocks_per_seq;

  /* cached tokens per sequence: int32 [batch] */
  const int32_t* cache_seqlens;

  int32_t dv;            /* value width: 512 */
  float softmax_scale;   /* required; e.g. 1/sqrt(192) for DeepSeek-V2/V3 */
  int32_t causal;        /* nonzero: bottom-right causal mask over the s_q query tokens */

  /* optional plan from mla_get_metadata for the same seqlens / q_rows / h_kv;
     NULL tile_md: the call plans internally with num_parts parts (num_parts <= 0: the
     device default), and the workspace then starts with that plan: tile_md
     [num_parts][MLA_TILE_MD_INTS] at byte 0, num_splits [batch + 1] at the next 256-byte
     boundary.  For a bf16 cache with more than 64 query rows per kv head (s_q * h_q /
     h_kv > 64) and at most 256 sequences, the decode kernel plans for itself in its first
     instructions instead of after a separate plan launch; its plan is mla_get_metadata's
     except that lengths past max_blocks_per_seq * 64 count as that many tokens. */
  const int32_t* tile_md;
  const int32_t* num_splits;
  int32_t num_parts;

  /* device scratch of at least mla_workspace_size(...) bytes, 256-byte aligned */
  void* workspace;
  size_t workspace_bytes;

  /* outputs: bf16 out [batch][s_q][h_q][dv] and fp32 lse [batch][s_q][h_q] (natural log) */
  void* out;
  int64_t out_batch_stride, out_seq_stride, out_head_stride;
  float* lse;
  int64_t lse_batch_stride, lse_seq_stride, lse_head_stride;

  /* cache element type (0 in a zero-initialised struct: bf16).  MLA_KV_FP8_E4M3: every
     element is one OCP FP8 E4M3 byte whose value is its decode times kv_scale (one scale per
     cache, finite and > 0; ignored for bf16).  k_*_stride count elements of this type. */
  int32_t kv_dtype;
  float kv_scale;
} mla_decode_params;

/* mla_decode_params.kv_dtype values */
#define MLA_KV_BF16 0
#define MLA_KV_FP8_E4M3 1

/*
 * Enqueue the decode (plan if needed, split-KV attention, lse merge) on `stream` and
 * return.  Alignment rules (MLA_ERR_BAD_STRIDE otherwise): q, k_cache and out 16-byte
 * aligned; q_*_stride and out_*_stride multiples of 8 elements; k_*_stride multiples of
 * 16 bytes (8 bf16 or 16 fp8 elements); k_row_stride >= d; k_block_stride >= 63 *
 * k_row_stride + d (a page's rows inside one block stride); workspace 256-byte aligned.
 *
 * An fp8 cache (kv_dtype MLA_KV_FP8_E4M3) is our reading of the FP8 latent cache the
 * Hacker News discussion of the FlashMLA release links to (vLLM's MLA and FP8 work): K is
 * the 576 decoded elements times kv_scale and V their first 512, exactly as for bf16; the
 * queries and out stay bf16.  It runs on the 128-row kernel whatever the row count.
 */
mla_status mla_decode_with_kvcache(const mla_decode_params* params, void* stream);

/*
 * The same decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The caller still passes every input and output in params; workspace and
 * workspace_bytes are ignored.  The plan (when params->tile_md is NULL) and
 * the per-split partial results go to a static device array inside the
 * library instead: MLA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, placed when
 * the library's code is loaded on that GPU and held until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  A call that needs more scratch than that returns
 * MLA_ERR_SCRATCH_TOO_SMALL before anything is enqueued; b = 128 sequences of
 * 128 query rows at the default part count of a 256-CU GPU need about 49 MB.
 * Every call on one GPU uses that GPU's one array: calls whose executions
 * overlap on one GPU (two streams, two threads) race and give undefined
 * results, so serialise them.  Nothing needs clearing between calls: every
 * scratch byte a call reads is written earlier by the same call.
 */
mla_status mla_decode_with_kvcache_noalloc(const mla_decode_params* params, void* stream);

/* ---- Writes into the paged cache (the steps before a decode).
 *
 * A cache view is (base, num_blocks, block_stride, row_stride) in elements:
 * row r of page k starts at base + k * block_stride + r * row_stride and its
 * first 576 elements are the entry.  Rules: base 16-byte aligned, both
 * strides multiples of 8, row_stride >= 576 (576 dense, 640 for vLLM pull
 * request "[Perf] Mem align KV caches for CUDA devices (MLA perf
 * improvement) #12676"'s 256-byte-aligned entries), block_stride >=
 * 63 * row_stride + 576; otherwise MLA_ERR_BAD_STRIDE.  Elements past the
 * 576th of a row are never read or written.  All pointers are device
 * pointers (or host memory the device can access); the caller owns them.
 *
 * mla_append_kv: token t's entry (kv_c[t, 0:512] followed by k_pe[t, 0:64],
 * bf16, rows kv_c_stride / k_pe_stride elements apart, 16-byte aligned) is
 * written to row slot % 64 of page slot / 64, slot = slot_mapping[t] (int64).
 * A negative slot (a padding token) or one past num_blocks * 64 is skipped.
 * Two tokens with the same slot race (precondition: distinct slots).
 * num_tokens = 0 launches nothing.
 *
 * mla_copy_blocks: for each pair k of block_mapping (int64 [num_pairs][2],
 * device memory), the 64 entries of page mapping[k][0] of the source cache
 * are copied to page mapping[k][1] of the destination cache.  The two views
 * may be the same cache (a block copy) or different caches of either pitch
 * (a swap or re-layout).  A pair naming a page outside its pool is skipped.
 * Pairs must not write a page another pair of the same call reads or writes.
 */
mla_status mla_append_kv(const void* kv_c, int64_t kv_c_stride, const void* k_pe, int64_t k_pe_stride,
                  const int64_t* slot_mapping, int32_t num_tokens, void* k_cache, int32_t num_blocks,
                  int64_t k_block_stride, int64_t k_row_stride, void* stream);

mla_status mla_copy_blocks(const void* src_cache, int32_t src_num_blocks, int64_t src_block_stride,
                    int64_t src_row_stride, void* dst_cache, int32_t dst_num_blocks, int64_t dst_block_stride,
                    int64_t dst_row_stride, const int64_t* block_mapping, int32_t num_pairs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */

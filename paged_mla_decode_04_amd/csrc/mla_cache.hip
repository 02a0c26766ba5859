// Writes into the paged latent cache: the steps before a decode.
//
// mla_append_kv stores each new token's latent row (512 compressed elements
// followed by the 64 rope elements, the 576-element entry the decode reads)
// at the cache slot its slot mapping names.  mla_copy_blocks copies whole
// pages between caches of either entry pitch.  vLLM pull request "[Perf] Mem
// align KV caches for CUDA devices (MLA perf improvement) #12676" pads each
// entry to 640 elements (256 bytes x 5) and then needs block copies and swaps
// that know the padded layout (its copy_blocks_mla and swap-blocks commits);
// here the pitch is just the row stride of each cache, and pad elements are
// neither read nor written.
//
// Both kernels move 16-byte pieces: a row is 72 of them (64 latent + 8 rope).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_decode.h"
#include "mla_internal.h"

namespace {

constexpr int kPiecesPerRow = 576 / 8;     // 16-byte pieces per cache entry
constexpr int kLatentPieces = 512 / 8;     // ... of which the compressed latent part
constexpr int kAppendThreads = 128;        // one workgroup per token (72 busy lanes)
constexpr int kCopyThreads = 256;          // one workgroup per 16 rows of a page pair

struct Piece {
  uint32_t x, y, z, w;
};

// Token t of the batch: latent row into page slot / 64, row slot % 64.
__global__ __launch_bounds__(kAppendThreads) void append_kv_kernel(const uint16_t* kv_c, int64_t kv_c_stride,
                                                                    const uint16_t* k_pe, int64_t k_pe_stride,
                                                                    const int64_t* slots, int64_t cache_slots,
                                                                    uint16_t* cache, int64_t block_stride,
                                                                    int64_t row_stride) {
  const int t = blockIdx.x, p = threadIdx.x;
  if (p >= kPiecesPerRow) return;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= cache_slots) return;  // padding token, or a slot past the pool
  const uint16_t* src = p < kLatentPieces ? kv_c + (int64_t)t * kv_c_stride + 8 * p
                                          : k_pe + (int64_t)t * k_pe_stride + 8 * (p - kLatentPieces);
  uint16_t* dst = cache + (slot / 64) * block_stride + (slot % 64) * row_stride + 8 * p;
  *(Piece*)dst = *(const Piece*)src;
}

// Pair k = (src page, dst page) of the mapping; workgroup y copies rows
// 16 y .. 16 y + 15 of it (16 x 72 pieces over 256 threads).
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const uint16_t* src, int64_t src_blocks,
                                                                    int64_t src_block_stride, int64_t src_row_stride,
                                                                    uint16_t* dst, int64_t dst_blocks,
                                                                    int64_t dst_block_stride, int64_t dst_row_stride,
                                                                    const int64_t* mapping) {
  const int k = blockIdx.x;
  const int64_t a = mapping[2 * k], b = mapping[2 * k + 1];
  if (a < 0 || a >= src_blocks || b < 0 || b >= dst_blocks) return;  // a pair outside the pools is skipped
  for (int i = threadIdx.x; i < 16 * kPiecesPerRow; i += kCopyThreads) {
    const int row = 16 * (int)blockIdx.y + i / kPiecesPerRow, p = i % kPiecesPerRow;
    *(Piece*)(dst + b * dst_block_stride + row * dst_row_stride + 8 * p) =
        *(const Piece*)(src + a * src_block_stride + row * src_row_stride + 8 * p);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The layout rules a cache view must follow (elements; 16-byte pieces).
mla_status check_cache(const void* cache, int64_t num_blocks, int64_t block_stride, int64_t row_stride) {
  if (num_blocks < 0) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(cache) || block_stride % 8 || row_stride % 8 || row_stride < 576) return MLA_ERR_BAD_STRIDE;
  if (block_stride < 63 * row_stride + 576) return MLA_ERR_BAD_STRIDE;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_append_kv(const void* kv_c, int64_t kv_c_stride, const void* k_pe, int64_t k_pe_stride,
                  const int64_t* slot_mapping, int32_t num_tokens, void* k_cache, int32_t num_blocks,
                  int64_t k_block_stride, int64_t k_row_stride, void* stream) {
  if (num_tokens < 0) return MLA_ERR_BAD_SHAPE;
  if (num_tokens == 0) return MLA_OK;
  if (!kv_c || !k_pe || !slot_mapping || !k_cache) return MLA_ERR_NULL_POINTER;
  const mla_status st = check_cache(k_cache, num_blocks, k_block_stride, k_row_stride);
  if (st != MLA_OK) return st;
  if (!aligned16(kv_c) || !aligned16(k_pe) || kv_c_stride % 8 || k_pe_stride % 8 || kv_c_stride < 512 ||
      k_pe_stride < 64)
    return MLA_ERR_BAD_STRIDE;
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)num_tokens), dim3(kAppendThreads), 0, (hipStream_t)stream,
                     (const uint16_t*)kv_c, kv_c_stride, (const uint16_t*)k_pe, k_pe_stride, slot_mapping,
                     (int64_t)num_blocks * 64, (uint16_t*)k_cache, k_block_stride, k_row_stride);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_copy_blocks(const void* src_cache, int32_t src_num_blocks, int64_t src_block_stride,
                    int64_t src_row_stride, void* dst_cache, int32_t dst_num_blocks, int64_t dst_block_stride,
                    int64_t dst_row_stride, const int64_t* block_mapping, int32_t num_pairs, void* stream) {
  if (num_pairs < 0) return MLA_ERR_BAD_SHAPE;
  if (num_pairs == 0) return MLA_OK;
  if (!src_cache || !dst_cache || !block_mapping) return MLA_ERR_NULL_POINTER;
  mla_status st = check_cache(src_cache, src_num_blocks, src_block_stride, src_row_stride);
  if (st != MLA_OK) return st;
  st = check_cache(dst_cache, dst_num_blocks, dst_block_stride, dst_row_stride);
  if (st != MLA_OK) return st;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, 4), dim3(kCopyThreads), 0, (hipStream_t)stream,
                     (const uint16_t*)src_cache, (int64_t)src_num_blocks, src_block_stride, src_row_stride,
                     (uint16_t*)dst_cache, (int64_t)dst_num_blocks, dst_block_stride, dst_row_stride,
                     block_mapping);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

// Internal interface between the C ABI (mla_api.hip) and the kernels (mla_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeArgs {
  const uint16_t* q;           // bf16 bits
  int64_t q_sb, q_ss, q_sh;    // element strides
  const uint8_t* k;            // cache base
  int64_t k_block_bytes, k_row_bytes;
  int32_t num_blocks;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t max_blocks;
  const int32_t* seqlens;
  int32_t batch, s_q, h_q, rows, causal;
  float scale_log2;            // softmax_scale * log2(e)
  const int32_t* tile_md;
  const int32_t* num_splits;
  int32_t num_parts, row_blocks;
  float* part_lse;             // [slots][rows]
  float* part_o;               // [slots][rows][512]
  uint16_t* out;               // bf16 bits
  int64_t o_sb, o_ss, o_sh;
  float* lse;
  int64_t l_sb, l_ss, l_sh;
};

hipError_t launch_plan(const int32_t* seqlens, int batch, int rows, int num_parts, int32_t* tile_md,
                       int32_t* num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream);

}  // namespace mla

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
  float scale_log2;            // softmax_scale * log2(e) (* kv_scale for an fp8 cache)
  int32_t kv8;                 // the cache holds E4M3 bytes (the wide kernel converts them to bf16)
  float kv_scale;              // value of a cache element per unit of its stored number (1 for bf16)
  const int32_t* tile_md;
  const int32_t* num_splits;   // read by the merge (and by the decode unless it plans)
  int32_t num_parts, row_blocks;
  float* part_lse;             // [slots][rows]
  float* part_o;               // narrow kernel: fp32 [slots][rows][512]; wide kernel: fp16 tiles (below)
  float* part_scale;           // wide kernel: [slots][rows] power-of-two factor of each partial row
  uint16_t* out;               // bf16 bits
  int64_t o_sb, o_ss, o_sh;
  float* lse;
  int64_t l_sb, l_ss, l_sh;
  // No metadata given: each decode workgroup derives its part from the
  // lengths (plan cost c per sequence), writes its record to plan_md and the
  // split counts it owns to plan_ns (== num_splits, for the merge).
  int32_t plan_in_kernel, plan_c;
  int32_t* plan_md;
  int32_t* plan_ns;
};

// Wide kernel partials: per slot, ceil(rows / 32) tiles of 32 rows x 512
// columns in fp16 (32 KB), stored in the accumulator layout: [tile][column
// tile ct (16)][element pair gp (2)][lane (64)][8 fp16].  A lane (j = lane & 31,
// h = lane >> 5) holds row j, columns 32 ct + 8 g + 4 h + e for g = 2 gp,
// 2 gp + 1 and e = 0..3.  Row r of slot s holds (O / l) * 2^-e_r with 2^e_r the
// smallest power of two above the row's largest magnitude, so that every
// element lies in (-1, 1) and keeps fp16's 11 significant bits;
// part_scale[s][r] = 2^e_r undoes it.
constexpr int kPartialTileBytes = 32 * 512 * 2;
__host__ __device__ inline int64_t partial_slot_bytes(int rows) {
  return (int64_t)((rows + 31) / 32) * kPartialTileBytes;
}

// The tile merge reads a sequence's splits one batch after another; when the
// splits per sequence average seven or more (a few long sequences over many
// parts), the split-parallel merge spreads them over four waves instead.
inline bool many_splits(int64_t num_parts, int64_t batch) { return num_parts + batch >= 8 * batch; }

hipError_t launch_plan(const int32_t* seqlens, int batch, int rows, int num_parts, int32_t* tile_md,
                       int32_t* num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream);

}  // namespace mla

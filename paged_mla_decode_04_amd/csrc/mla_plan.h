// Split-KV work planner for paged MLA decode (host and device).
//
// Flash-Decoding adds the key length as a parallel dimension so that a small
// batch still fills the GPU, then merges the pieces (Hacker News discussion of
// the FlashMLA release, the Flash-Decoding description).  The PAI FlashMLA
// tutorial (segmentfault, "云上玩转DeepSeek系列之五", section 二.2) names a
// metadata step, get_mla_metadata, computed once per decode step ahead of the
// per-layer forward; its contents are not given there.  This is our reading:
//
//   * work unit = one 64-token page of one sequence; a sequence with no
//     tokens still owns one (empty) unit so that some part writes its
//     result (out = 0, lse = -inf);
//   * the flattened (sequence, page) order is cut into num_parts contiguous
//     ranges of near-equal cost, cost = pages + segment_cost per
//     (part, sequence) pair: a piece of a sequence pays for loading its
//     queries and for writing (and later merging) its result;
//   * part p is [seq_begin, page_begin, seq_last, page_end, split_first,
//     0, 0, 0]: pages from (seq_begin, page_begin) to (seq_last,
//     page_end - 1); split_first is how many earlier parts touched
//     seq_begin; an idle part has seq_begin = batch;
//   * num_splits[b + 1] - num_splits[b] is the number of parts that touch
//     sequence b (num_splits[0] = 0); a sequence touched once needs no merge.
//
// The same function runs in the host mirror and in the one-thread plan
// kernel, so both produce identical plans.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define MLA_HD __host__ __device__
#else
#define MLA_HD
#endif

namespace mla {

constexpr int kPageTokens = 64;
constexpr int kTileMdInts = 8;
constexpr int kRowsPerWorkgroup = 64;

// Rows one workgroup handles when the kv head has `rows` query rows (16 per
// compute wave, up to 4 compute waves).
MLA_HD inline int rows_per_block(int rows) {
  if (rows <= 16) return 16;
  if (rows <= 32) return 32;
  return kRowsPerWorkgroup;
}

MLA_HD inline int row_blocks(int rows) {
  const int r = rows_per_block(rows);
  return (rows + r - 1) / r;
}

// Fixed cost of one (part, sequence) segment, in pages.  A page is
// 64 * 576 * 2 = 73728 B of cache; a segment reads rows * 1152 B of queries
// and writes rows * 1024 B of output, or rows * 2052 B of fp32 partial that
// the merge reads again (these mostly stay in L2 / the memory-side cache).
MLA_HD inline int segment_cost(int rows_in_block) {
  const int c = (rows_in_block + 27) / 28;
  return c < 1 ? 1 : c;
}

MLA_HD inline int seq_units(int32_t n) {
  if (n <= 0) return 1;
  const int64_t u = ((int64_t)n + kPageTokens - 1) / kPageTokens;
  return (int)u;
}

MLA_HD inline void plan_split_kv(const int32_t* seqlens, int batch, int q_rows_per_kv_head,
                                 int num_parts, int32_t* tile_md, int32_t* num_splits) {
  const int c = segment_cost(rows_per_block(q_rows_per_kv_head));
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) total += seq_units(seqlens[b]) + c;
  // Each cut inside a sequence costs one more segment; at most num_parts - 1 cuts.
  int64_t target = (total + (int64_t)(num_parts - 1) * c + num_parts - 1) / num_parts;
  if (target < c + 1) target = c + 1;

  num_splits[0] = 0;
  int part = 0;
  int b = 0, pg = 0, touched = 0;  // next unit; parts that already touched sequence b
  while (part < num_parts && b < batch) {
    const bool last = (part == num_parts - 1);
    const int start_b = b, start_pg = pg, first_split = touched;
    int end_b = b, end_pg = pg;
    int64_t budget = target;
    while (b < batch) {
      const int units = seq_units(seqlens[b]);
      const int rem = units - pg;
      if (last || rem + c <= budget) {
        budget -= rem + c;
        num_splits[b + 1] = num_splits[b] + touched + 1;
        end_b = b;
        end_pg = units;
        ++b;
        pg = 0;
        touched = 0;
        if (!last && budget <= c) break;
      } else {
        const int64_t take = budget - c;
        if (take >= 1) {
          pg += (int)take;
          ++touched;
          end_b = b;
          end_pg = pg;
        }
        break;
      }
    }
    int32_t* md = tile_md + (int64_t)part * kTileMdInts;
    md[0] = start_b;
    md[1] = start_pg;
    md[2] = end_b;
    md[3] = end_pg;
    md[4] = first_split;
    md[5] = 0;
    md[6] = 0;
    md[7] = 0;
    ++part;
  }
  for (; part < num_parts; ++part) {
    int32_t* md = tile_md + (int64_t)part * kTileMdInts;
    md[0] = batch;
    md[1] = 0;
    md[2] = batch;
    md[3] = 0;
    md[4] = 0;
    md[5] = 0;
    md[6] = 0;
    md[7] = 0;
  }
}

}  // namespace mla

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
//   * every sequence also carries a fixed cost c: a piece of a sequence
//     loads its queries and writes (and later merges) its result;
//   * lay the sequences end to end on a cost axis: sequence b occupies
//     positions [S_b, S_{b+1}) with S_{b+1} = S_b + c + units_b (its c
//     overhead positions first, then one position per page); W = S_batch;
//   * part p owns positions [p T, (p+1) T) with T = max(c + 1, ceil(W / P)),
//     so parts are contiguous, in order, and never empty;
//   * part p is [seq_begin, page_begin, seq_last, page_end, split_first,
//     0, 0, 0]: pages (seq_begin, page_begin) .. (seq_last, page_end - 1);
//     split_first is the number of earlier parts that touched seq_begin;
//     an idle part (p T >= W) has seq_begin = batch;
//   * num_splits[b + 1] - num_splits[b] is the number of parts that touch
//     sequence b (num_splits[0] = 0); a sequence touched once needs no merge.
//
// Everything is closed-form integer arithmetic on prefix sums, so the host
// mirror below and the one-workgroup device kernel (a block scan plus one
// binary search per part) produce identical plans.
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
constexpr int kRowsPerWorkgroup = 128;
constexpr int kMaxPlanBatch = 16384;  // device plan keeps the prefix sums in LDS
constexpr int kPlanInKernelMaxBatch = 256;  // the 128-row decode plans for itself up to this batch

// Rows one workgroup handles when the kv head has `rows` query rows: 16, 32
// or 64 (the narrow kernel, up to 4 score tiles of 16 rows), else 128 (the
// wide kernel).
MLA_HD inline int rows_per_block(int rows) {
  if (rows <= 16) return 16;
  if (rows <= 32) return 32;
  if (rows <= 64) return 64;
  return kRowsPerWorkgroup;
}

MLA_HD inline int row_blocks(int rows) {
  const int r = rows_per_block(rows);
  return (rows + r - 1) / r;
}

// Fixed cost of one (part, sequence) segment, in pages.  A page is
// 64 * 576 * 2 = 73728 B of cache; a segment reads rows * 1152 B of queries
// and writes rows * 1024 B of output, or a partial the merge reads again
// (rows * 1032 B of fp16 tiles from the wide kernel, rows * 2052 B of fp32
// from the narrow one), and spends a few steps outside the pipelined loop.
// For the wide kernel's 128-row blocks, per-workgroup timers at b = 128,
// h_q = 128, seqlens ~ N(4096, 1024) fit about 3850 cycles per 32-token chunk
// and 17600 per segment, i.e. 2.3 pages; of charges 2 to 5, 3 gave the
// shortest calls there and with two query tokens.  The narrow kernel keeps
// ceil(rows / 28).
MLA_HD inline int segment_cost(int rows_in_block) {
  if (rows_in_block >= kRowsPerWorkgroup) return 3;
  const int c = (rows_in_block + 27) / 28;
  return c < 1 ? 1 : c;
}

MLA_HD inline int seq_units(int32_t n) {
  if (n <= 0) return 1;
  const int64_t u = ((int64_t)n + kPageTokens - 1) / kPageTokens;
  return (int)u;
}

MLA_HD inline int64_t plan_stride(int64_t total, int num_parts, int c) {
  int64_t t = (total + num_parts - 1) / num_parts;
  return t < c + 1 ? c + 1 : t;
}

// Largest b in [0, batch) with prefix[b] <= x (prefix[0] = 0 <= x).
MLA_HD inline int locate(const int64_t* prefix, int batch, int64_t x) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Part p's record from the prefix sums (prefix has batch + 1 entries).
MLA_HD inline void plan_part(const int64_t* prefix, int batch, int c, int64_t T,
                             int p, int32_t* md) {
  const int64_t W = prefix[batch];
  const int64_t x = (int64_t)p * T;
  for (int i = 0; i < kTileMdInts; ++i) md[i] = 0;
  if (x >= W) {
    md[0] = batch;
    md[2] = batch;
    return;
  }
  const int b = locate(prefix, batch, x);
  const int64_t off = x - prefix[b] - c;
  const int pg = off > 0 ? (int)off : 0;
  int eb, epg;
  const int64_t xn = x + T;
  // (sequence e's units are prefix[e + 1] - prefix[e] - c: no second read of
  // the lengths)
  if (xn >= W) {
    eb = batch - 1;
    epg = (int)(prefix[batch] - prefix[batch - 1] - c);
  } else {
    const int nb = locate(prefix, batch, xn);
    const int64_t noff = xn - prefix[nb] - c;
    if (noff > 0) {
      eb = nb;
      epg = (int)noff;
    } else {
      eb = nb - 1;
      epg = (int)(prefix[nb] - prefix[nb - 1] - c);
    }
  }
  md[0] = b;
  md[1] = pg;
  md[2] = eb;
  md[3] = epg;
  // parts before p that touched b: those from the one owning b's first page
  md[4] = pg > 0 ? (int)(p - (prefix[b] + c) / T) : 0;
}

// Number of parts that touch sequence b.
MLA_HD inline int32_t plan_touches(const int64_t* prefix, int b, int c, int64_t T) {
  return (int32_t)((prefix[b + 1] - 1) / T - (prefix[b] + c) / T + 1);
}

// Host mirror (the device kernel computes the same with a parallel scan).
inline void plan_split_kv_host(const int32_t* seqlens, int batch, int q_rows_per_kv_head, int num_parts,
                               int32_t* tile_md, int32_t* num_splits, int64_t* prefix /* batch + 1 */) {
  const int c = segment_cost(rows_per_block(q_rows_per_kv_head));
  prefix[0] = 0;
  for (int b = 0; b < batch; ++b) prefix[b + 1] = prefix[b] + c + seq_units(seqlens[b]);
  const int64_t T = plan_stride(prefix[batch], num_parts, c);
  for (int p = 0; p < num_parts; ++p) plan_part(prefix, batch, c, T, p, tile_md + (int64_t)p * kTileMdInts);
  num_splits[0] = 0;
  for (int b = 0; b < batch; ++b) num_splits[b + 1] = num_splits[b] + plan_touches(prefix, b, c, T);
}

}  // namespace mla

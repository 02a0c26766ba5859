// The merge of a split sequence's partial results by their log-sum-exp:
// the online fold all three merge kernels use, and the row-tile merge of the
// wide kernel's fp16 tile partials.
//
// Flash-Decoding splits the key length of a sequence across workgroups and
// rescales the pieces by their log-sum-exp when it combines them (Hacker News
// discussion of the FlashMLA release, the Flash-Decoding description).  For
// pieces i with lse_i and normalised output O_i:
//   lse = log(sum_i exp(lse_i)),  out = sum_i exp(lse_i - lse) O_i.
#pragma once
#include "mla_device.h"

namespace mla {

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// The merge runs in one pass over the splits, online: a running maximum m of
// the lse seen so far, the sum of exp(lse_i - m) and the sum of
// exp(lse_i - m) * scale_i * O_i, both rescaled when m grows;
// out = (weighted sum) / (sum of weights), lse = m + log(sum).  Many splits'
// loads go out together, so that a row's merge takes a round trip to memory
// per batch of splits, not per split.  An empty partial (lse = -inf) weighs
// nothing; a row with only empty partials gets out = 0 and lse = -inf; a NaN
// partial lse makes the row's out and lse NaN.
struct OnlineLse {
  float m = -INFINITY, sum = 0.f;
  bool nan = false;
  // Folds a batch of lse values in; returns the factor the running sums were
  // scaled by and leaves the batch's weights exp(x - m) in x.
  template <int B>
  __device__ __forceinline__ float fold(float (&x)[B]) {
    float mn = m;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (x[u] != x[u]) nan = true;
      else mn = fmaxf(mn, x[u]);
    }
    const float f = (m == -INFINITY || mn == -INFINITY) ? (mn == -INFINITY ? 1.f : 0.f)
                                                        : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
    sum *= f;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float w = (x[u] == -INFINITY || x[u] != x[u]) ? 0.f : __builtin_amdgcn_exp2f((x[u] - mn) * kLog2e);
      sum += w;
      x[u] = w;
    }
    m = mn;
    return f;
  }
  __device__ __forceinline__ float lse() const {
    if (nan) return __builtin_nanf("");
    return m == -INFINITY ? -INFINITY : m + __builtin_amdgcn_logf(sum) * kLn2;
  }
};

constexpr int kTileMergeBatch = 4;    // splits whose loads are in flight together (tile merge)
constexpr int kSplitMergeBatch = 8;   // ... per wave (split-parallel merge)
constexpr int kMergeTileStride = kDv / 2 + 8;  // bf16 elements per row of the merge's LDS half tile

// Merges the ns >= 2 partials in slots base .. base + ns - 1 of row tile rt
// (32 rows) of sequence b into out and lse, for column half hf (256 columns,
// column tiles 8 hf .. 8 hf + 7), with 256 threads (4 waves).  Wave v merges
// column tiles 8 hf + 2 v and 8 hf + 2 v + 1 of the 32 rows in the
// accumulator layout the partials keep; the half tile then goes through LDS
// (`tile`, 32 rows of kMergeTileStride bf16) so that every output row is
// written as 512 contiguous bytes.  Half 0 writes the lse.  Ends with a
// barrier, so the LDS tile may be reused at once.
__device__ __forceinline__ void merge_row_tile(const DecodeArgs& a, int b, int rt, int hf, int base, int ns,
                                               lds_u16* tile) {
  const int v = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int row = 32 * rt + j;
  const bool ok = row < a.rows;
  const float* lse_p = a.part_lse + (int64_t)base * a.rows + row;
  const float* scale_p = a.part_scale + (int64_t)base * a.rows + row;
  const uint8_t* src0 = (const uint8_t*)a.part_o + (int64_t)base * partial_slot_bytes(a.rows) +
                        (int64_t)rt * kPartialTileBytes + 2048 * (8 * hf + 2 * v) + 16 * lane;
  float acc[4][8];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[p][e] = 0.f;
  OnlineLse ol;
  for (int i0 = 0; i0 < ns; i0 += kTileMergeBatch) {
    float x[kTileMergeBatch], sc[kTileMergeBatch];
    f16x8 pv[kTileMergeBatch][4];
#pragma unroll
    for (int u = 0; u < kTileMergeBatch; ++u) {
      const int i = i0 + u;
      const bool in = i < ns;
      x[u] = (in && ok) ? lse_p[(int64_t)i * a.rows] : -INFINITY;
      sc[u] = (in && ok) ? scale_p[(int64_t)i * a.rows] : 0.f;
      const uint8_t* src = src0 + (int64_t)(in ? i : 0) * partial_slot_bytes(a.rows);
#pragma unroll
      for (int p = 0; p < 4; ++p) pv[u][p] = in ? *(const f16x8*)(src + 1024 * p) : f16x8{};
    }
    const float f = ol.fold(x);
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[p][e] *= f;
#pragma unroll
    for (int u = 0; u < kTileMergeBatch; ++u) {
      const float wgt = x[u] * sc[u];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[p][e] += wgt * (float)pv[u][p][e];
    }
  }
  const float Lo = ol.lse();
  const float inv = (ol.nan || !(ol.sum > 0.f)) ? (ol.nan ? __builtin_nanf("") : 0.f) : 1.f / ol.sum;
  // pair p of wave v: column tile 2 v + (p >> 1) of the half, elements of g = 2 (p & 1) + (e >> 2)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int ct = 2 * v + (p >> 1);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int col = 32 * ct + 8 * (2 * (p & 1) + gg) + 4 * h;
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[p][4 * gg + e] * inv);
      *(__attribute__((address_space(3))) bf16x4*)(tile + j * kMergeTileStride + col) = o4;
    }
  }
  if (hf == 0 && v == 0 && h == 0 && ok) {
    const int qi = row / a.h_q, hh = row - qi * a.h_q;
    a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)hh * a.l_sh] = Lo;
  }
  __syncthreads();
  // wave v writes rows 8 v .. 8 v + 7, two at a time: 32 lanes x 16 bytes each
#pragma unroll
  for (int r = 0; r < 8; r += 2) {
    const int jr = 8 * v + r + h, orow = 32 * rt + jr;
    if (orow < a.rows) {
      const int qi = orow / a.h_q, hh = orow - qi * a.h_q;
      uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)hh * a.o_sh + 256 * hf + 8 * j;
      *(bf16x8*)op = *(const lds_bf16x8*)(tile + jr * kMergeTileStride + 8 * j);
    }
  }
  __syncthreads();
}

}  // namespace mla

// Device helpers shared by the decode kernels: operand types, the chunk
// descriptors of the page walk and the LDS-direct copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "mla_plan.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) int32_t lds_i32;

constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kPageBytes = 64 * kD * 2;  // 73728
constexpr int kKSteps = kD / 32;          // 18 MFMA k-steps of 32 for the scores
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 16.0f;    // log2 units: p = 2^(x - m) stays <= 65536
constexpr int32_t kBufferFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x7FFFF000u;

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float wave_max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Opaque copy of an LDS pointer: keeps base + constant address arithmetic from
// being re-associated (and hoisted) so the constant lands in the instruction
// offset field.
__device__ __forceinline__ lds_u8* launder(lds_u8* p) {
  asm volatile("" : "+v"(p));
  return p;
}

// Workgroup barrier for LDS hand-offs.  The page copies are waited for
// explicitly (vmcnt) before it; unlike __syncthreads it does not also wait for
// the next page's copies still in flight.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int kChunk = 32;  // tokens per pipeline step (half a page)

typedef const __attribute__((address_space(4))) int32_t cint32;  // read-only, uniform: scalar loads
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

// 16-byte LDS-direct buffer load: lane l's 16 bytes land at lds_addr + 16 l.
// Written as inline assembly so that the compiler does not track the LDS
// write: it would otherwise make every later LDS read wait for all copies in
// flight.  Completion is awaited explicitly (vmcnt) before the barrier that
// hands a chunk over, and a copy only targets a tile no wave reads any more.
// An LDS-direct load reads M0, which the compiler writes (a scalar
// instruction) right before the assembly; the load needs one wait state after
// that write, which the compiler's hazard check does not see through inline
// assembly, so the s_nop is part of the block.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}
// Position of the page-bookkeeping cursor: one 32-token chunk of the part's
// (sequence, chunk) order.
struct Cursor {
  int seq, chunk;  // sequence, chunk within the sequence (page chunk / 2)
  int n;           // cached tokens of seq as stored (clamp_len applies the cap)
  int phys;        // block-table entry of the chunk's page (-1 past the row)
  bool valid;      // inside the part
};

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int n) {
  const int cap = a.max_blocks * kPageTokens;
  return n < 0 ? 0 : (n > cap ? cap : n);
}
__device__ __forceinline__ int load_len(const DecodeArgs& a, int b) { return ((cint32*)a.seqlens)[b]; }
__device__ __forceinline__ int load_phys(const DecodeArgs& a, int b, int page) {
  return page < a.max_blocks ? ((cint32*)a.block_table)[(int64_t)b * a.bt_stride + page] : -1;
}
// chunks a sequence of n tokens occupies; an empty sequence owns one empty chunk
__device__ __forceinline__ int chunk_count(int n) { return n <= 0 ? 1 : (n + kChunk - 1) / kChunk; }

// The chunk after c in the part.  Uses c.n, fetched at least a step earlier;
// starts the fetch of a new sequence's length and of a new page's table entry.
__device__ __forceinline__ Cursor next_chunk(const DecodeArgs& a, const Cursor& c, int seq_last, int page_end) {
  Cursor d = c;
  if (!c.valid) return d;
  int end = chunk_count(clamp_len(a, c.n));
  if (c.seq == seq_last && 2 * page_end < end) end = 2 * page_end;
  if (c.chunk + 1 < end) {
    d.chunk = c.chunk + 1;
    if ((d.chunk & 1) == 0) d.phys = load_phys(a, d.seq, d.chunk >> 1);
  } else if (c.seq < seq_last) {
    d.seq = c.seq + 1;
    d.chunk = 0;
    d.n = load_len(a, d.seq);
    d.phys = load_phys(a, d.seq, 0);
  } else {
    d.valid = false;
  }
  return d;
}

// What every wave needs to know about one chunk.  Wave 4 walks the part with a
// Cursor and publishes these, six chunks ahead, in a ring of eight LDS slots
// (16 bytes each), so that the page bookkeeping costs the CU's scalar unit one
// wave's work instead of eight.
struct Chunk {
  int seq;     // -1: past the end of the part
  int chunk;   // within the sequence
  int tok;     // tokens in the chunk (0 for an empty sequence's chunk)
  int phys;    // block-table entry of its page
  bool first;  // first chunk of its segment (the part's piece of one sequence)
  bool last;   // last chunk of its segment
  bool bad;    // the entry lies outside the pool
  __device__ bool valid() const { return seq >= 0; }
};

__device__ __forceinline__ i32x4 pack_chunk(const DecodeArgs& a, const Cursor& c, const Cursor& next, bool first) {
  i32x4 d;
  if (!c.valid) {
    d = i32x4{-1, 0, 0, -1};
    return d;
  }
  int tok = clamp_len(a, c.n) - kChunk * c.chunk;
  tok = tok < 0 ? 0 : (tok > kChunk ? kChunk : tok);
  const bool last = !next.valid || next.seq != c.seq;
  const bool bad = tok > 0 && !(c.phys >= 0 && c.phys < a.num_blocks);
  d = i32x4{c.seq, c.chunk, tok | (first ? 256 : 0) | (last ? 512 : 0) | (bad ? 1024 : 0), c.phys};
  return d;
}

__device__ __forceinline__ Chunk unpack_chunk(const i32x4 d) {
  Chunk c;
  c.seq = uniform(d[0]);
  c.chunk = uniform(d[1]);
  const int z = uniform(d[2]);
  c.phys = uniform(d[3]);
  c.tok = z & 255;
  c.first = (z & 256) != 0;
  c.last = (z & 512) != 0;
  c.bad = (z & 1024) != 0;
  return c;
}

// Source of one chunk's copy: a buffer resource over the chunk's valid rows
// (zero records for a page outside the pool, so it reads as zeros): rows at or
// past the chunk's token count read as zeros through the range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const DecodeArgs& a, const Chunk& c) {
  const bool ok = !c.bad;
  const uint32_t rb = (uint32_t)a.k_row_bytes;
  const uint64_t base =
      (uint64_t)(a.k + (ok ? (int64_t)c.phys * a.k_block_bytes + (int64_t)(c.chunk & 1) * kChunk * rb : 0));
  // the descriptor fields are wave-uniform; say so, so the resource lands in scalar registers
  const uint64_t ubase = ((uint64_t)(uint32_t)uniform((int)(base >> 32)) << 32) | (uint32_t)uniform((int)base);
  const int32_t records = uniform(ok ? (int32_t)(c.tok * rb) : 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)ubase, (short)0, records, kBufferFlags);
}

// What a workgroup knows about its plan part.
struct PartInfo {
  int seq_begin, page_begin, seq_last, page_end, split_first;
  int blk_row0;
};

// ---- The plan inside the decode kernels, used when the caller passes no
// metadata (at most kPlanInKernelMaxBatch sequences).  It is the plan of
// mla_plan.h (plan_part, plan_touches), with lengths past the block table's
// width counted as clamped.  Every wave loads the lengths once (four per
// lane) and:
//   * sums the sequence costs c + pages for the stride T;
//   * scans them into the prefix sums and finds the sequences holding the
//     part's first unit x = p T and its end x + T (plan_part's searches);
//   * scans touches(j) = floor((prefix[j+1] - 1) / T) - floor((prefix[j] + c)
//     / T) + 1 into num_splits.  Wave 0 lists num_splits in LDS (the segment
//     bookkeeping reads it there) and, in row block 0, publishes for the merge
//     each sequence's split count from the part that holds its last unit,
//     which is the last part touching it.
// The host checks that the costs sum below 2^31, so 32-bit arithmetic holds.

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS round
// trips): shifts right by 1, 2, 4 and 8 lanes inside each row of 16 (lanes
// shifted in from outside the row read 0), then row 0's total added to row 1
// and row 2's to row 3 (row_bcast:15), then lane 31's total to rows 2 and 3
// (row_bcast:31).  All lanes must be active.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return (uint32_t)x;
}
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int k) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, k);
}

// Part `part` from the lengths: fills pi's plan fields and len (lane l of
// len[k]: the stored length of sequence 64 k + l); wave 0 fills split_tab[j] =
// num_splits[j] for every sequence j <= batch.  Row block 0's wave 0 also
// writes the part's record to plan_md and the split counts it owns to
// plan_ns.  Returns false for an idle part.
constexpr int kPlanBlocks = (kPlanInKernelMaxBatch + 63) / 64;  // lengths per lane

__device__ __forceinline__ bool plan_in_kernel(const DecodeArgs& a, int part, int mblock, PartInfo& pi,
                                               lds_i32* split_tab, int (&len)[kPlanBlocks]) {
  constexpr int kBlocks = kPlanBlocks;
  const int lane = threadIdx.x & 63;
  const int B = a.batch, c = a.plan_c;
  const bool wave0 = (threadIdx.x >> 6) == 0;
  const bool writer = mblock == 0 && wave0;
  const int cap = a.max_blocks * kPageTokens;
  // the lengths, four per lane, loaded together (an index past the batch
  // reads the last length again and counts nothing), with one wait
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) len[k] = a.seqlens[64 * k + lane < B ? 64 * k + lane : B - 1];
  uint32_t u[kBlocks];
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) {
    const int n = len[k] > cap ? cap : len[k];
    u[k] = 64 * k + lane < B ? (uint32_t)(c + seq_units(n)) : 0u;
  }
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) acc += u[k];
  const uint32_t W = lane_value(wave_incl_scan_u32(acc), 63);
  const uint32_t T = (uint32_t)plan_stride((int64_t)W, a.num_parts, c);
  const int64_t x = (int64_t)part * T, xn = x + T;
  int32_t* md = a.plan_md + (int64_t)part * kTileMdInts;
  if (x >= (int64_t)W) {
    if (writer && lane < kTileMdInts) md[lane] = lane == 0 || lane == 2 ? B : 0;
    return false;
  }
  uint32_t carry = 0, pre_b = 0, pre_nb = 0, u_nbm1 = 0, u_last = 0;
  int b = 0, nb = 0, ns_carry = 0;
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) {
    if (64 * k < B) {
      const int i = 64 * k + lane;
      const bool in = i < B;
      const uint32_t incl = carry + wave_incl_scan_u32(u[k]);  // prefix[i + 1]
      const uint32_t excl = incl - u[k];                       // prefix[i]
      const uint64_t hx = __ballot(in && (int64_t)excl <= x && x < (int64_t)incl);
      const uint64_t hn = __ballot(in && (int64_t)excl <= xn && xn < (int64_t)incl);
      if (hx) {
        const int h = __ffsll((unsigned long long)hx) - 1;
        b = 64 * k + h;
        pre_b = lane_value(excl, h);
      }
      if (hn) {
        const int h = __ffsll((unsigned long long)hn) - 1;
        nb = 64 * k + h;
        pre_nb = lane_value(excl, h);
        u_nbm1 = h > 0 ? lane_value(u[k], h - 1) : u_last;
      }
      const int last = B - 1 - 64 * k < 63 ? B - 1 - 64 * k : 63;
      u_last = lane_value(u[k], last);
      carry = lane_value(incl, last);
      if (wave0) {
        const int last_part = in ? (int)((incl - 1u) / T) : 0;
        const int touch = in ? last_part - (int)((excl + (uint32_t)c) / T) + 1 : 0;
        const int ns_incl = ns_carry + (int)wave_incl_scan_u32((uint32_t)touch);  // num_splits[i + 1]
        if (in) {
          split_tab[i] = ns_incl - touch;
          if (i == B - 1) split_tab[B] = ns_incl;
          if (writer && last_part == part) a.plan_ns[i + 1] = ns_incl;
        }
        ns_carry = (int)lane_value((uint32_t)ns_incl, last);
      }
    }
  }
  const int64_t off = x - (int64_t)pre_b - c;
  const int pg = off > 0 ? (int)off : 0;
  int eb, epg;
  if (xn >= (int64_t)W) {
    eb = B - 1;
    epg = (int)u_last - c;
  } else {
    const int64_t noff = xn - (int64_t)pre_nb - c;
    if (noff > 0) {
      eb = nb;
      epg = (int)noff;
    } else {
      eb = nb - 1;
      epg = (int)u_nbm1 - c;
    }
  }
  pi.seq_begin = b;
  pi.page_begin = pg;
  pi.seq_last = eb;
  pi.page_end = epg;
  pi.split_first = pg > 0 ? part - (int)((pre_b + (uint32_t)c) / T) : 0;
  if (writer && lane < kTileMdInts) {
    const int v = lane == 0 ? b : lane == 1 ? pg : lane == 2 ? eb : lane == 3 ? epg : lane == 4 ? pi.split_first : 0;
    md[lane] = v;
  }
  if (writer && part == 0 && lane == 0) a.plan_ns[0] = 0;
  return true;
}

// Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
// run of (part, row block) pairs so that the row blocks of one part, and
// neighbouring parts of one sequence, share that XCD's L2.  The part's record
// comes from the plan's metadata, or from the lengths in a kernel instance
// that plans (kPlan; then wave 0 also fills split_tab, read after the
// prologue's barrier, and len holds the lengths).  Returns false for an idle
// part.
template <bool kPlan>
__device__ __forceinline__ bool load_part(const DecodeArgs& a, int rows_per_block, PartInfo& pi, lds_i32* split_tab,
                                          int (&len)[kPlanBlocks]) {
  const int G = gridDim.x, hw = blockIdx.x;
  const int xcd = hw & 7, pos = hw >> 3;
  const int logical = xcd * (G >> 3) + min(xcd, G & 7) + pos;
  const int part = logical / a.row_blocks;
  const int mblock = logical - part * a.row_blocks;
  if constexpr (kPlan) {
    pi.blk_row0 = mblock * rows_per_block;
    return plan_in_kernel(a, part, mblock, pi, split_tab, len);
  } else {
    cint32* md = (cint32*)a.tile_md + (int64_t)part * kTileMdInts;
    pi.seq_begin = md[0];
    if (pi.seq_begin >= a.batch) return false;
    pi.page_begin = md[1];
    pi.seq_last = md[2];
    pi.page_end = md[3];
    pi.split_first = md[4];
    pi.blk_row0 = mblock * rows_per_block;
    return true;
  }
}

// The stored length of sequence s (per lane, 0 <= s < 64 kPlanBlocks) from
// the lengths the in-kernel plan loaded: lane s % 64 of len[s / 64].  A
// cross-lane read: call it with every lane of the wave active.
__device__ __forceinline__ int planned_length(const int (&len)[kPlanBlocks], int s) {
  int v = 0;
#pragma unroll
  for (int k = 0; k < kPlanBlocks; ++k) {
    const int x = __shfl(len[k], s & 63);
    v = (s >> 6) == k ? x : v;
  }
  return v;
}

// A segment of sequence s of the part starts: the first partial slot of s
// and the number of parts that touch it, from the plan's num_splits or, when
// the kernel plans, from its copy in LDS.
template <bool kPlan>
__device__ __forceinline__ void segment_splits(const DecodeArgs& a, int s, const lds_i32* split_tab, int& slot0,
                                               int& nsplit) {
  if constexpr (kPlan) {
    const int s0 = uniform(split_tab[s]);
    slot0 = s0;
    nsplit = uniform(split_tab[s + 1]) - s0;
  } else {
    const int s0 = ((cint32*)a.num_splits)[s];
    slot0 = s0;
    nsplit = ((cint32*)a.num_splits)[s + 1] - s0;
  }
}

}  // namespace mla

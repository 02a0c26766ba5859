// Split-KV decode for the wide-head shape: up to 128 query rows per kv head in
// one workgroup, so that every cached token is read from HBM once per part.
//
// What is computed is the same as for the narrow kernel (mla_kernels.hip):
// for each query row r = (query token i, head h), softmax(scale * q_r . k_t)
// over the sequence's visible cached latent rows k_t (576 bf16; V is the first
// 512 elements of the same row), out = P . V and the natural-log lse.  The PAI
// FlashMLA tutorial (segmentfault, "云上玩转DeepSeek系列之五", section 二.4)
// states the inputs and prices the work as (d + dv) multiply-adds per
// query-key pair and one d-element read per cached token.
//
// Layout of the work on gfx950 (one workgroup of 4 waves per CU, one wave per
// SIMD, each wave with the SIMD's whole register file):
//   * wave w holds the queries of rows 32 w .. 32 w + 31 (two 16-row tiles,
//     144 registers) and computes their scores S^T = K . Q^T for all 32 tokens
//     of a chunk on 16x16x32 bf16 MFMA -- every 16-byte K fragment read from
//     LDS feeds two MFMAs;
//   * wave w owns the softmax state of those rows.  It sees every score of a
//     row, so it moves the row's reference max itself when a chunk passes it
//     and writes P (bf16) to LDS already in the B-operand layout of the value
//     product;
//   * wave w also owns output columns 128 w .. 128 w + 127 of all 128 rows
//     (256 accumulator registers) and accumulates O^T += V^T . P^T, reading
//     V^T with the transposing LDS read ds_read_b64_tr_b16, so V is read from
//     LDS once per workgroup;
//   * when a wave moved the reference of its rows it leaves the rescale
//     factors in LDS and a flag; the next step every wave rescales those rows
//     of its accumulators before adding the next chunk.
// In step t the waves compute the scores and P of chunk t + 1 and the values
// of chunk t; the copy of chunk t + 2 lands and that of chunk t + 3 is issued.
// A chunk's latent part (32 tokens x 512 columns) lives in one of four 32 KB
// slots (read for the scores one step, for the values the next), its rope
// part (32 x 64) in one of three 4 KB slots (read for the scores only).
// One workgroup barrier per step.
//
// LDS slot layout: latent block (r, q) = tokens 8r..8r+7 x columns 64q..64q+63
// at 8192 r + 1024 q, rope block r at 1024 r; inside a block token a sits at
// 128 a and its 16-byte column chunk c at slot (c ^ a ^ 2 (r & 1)), the same
// conflict-free swizzle as the narrow kernel.
#include <type_traits>

#include "mla_device.h"

namespace mla {
namespace {

constexpr int kThreadsW = 256;                          // 4 waves, one per SIMD
constexpr int kRowsW = 128;                             // query rows per workgroup
constexpr int kRowTiles = kRowsW / 16;                  // 8
constexpr int kLatBytes = kChunk * kDv * 2;             // 32768
constexpr int kRopeBytes = kChunk * (kD - kDv) * 2;     // 4096
constexpr int kLatSlots = 4, kRopeSlots = 3;
constexpr int kRopeOff = kLatSlots * kLatBytes;                 // 131072
constexpr int kPOff = kRopeOff + kRopeSlots * kRopeBytes;       // P^T: [parity][row tile][lane] x 16 B
constexpr int kFacOff = kPOff + 2 * kRowTiles * 1024;           // rescale factors: [parity][row] f32
constexpr int kFinOff = kFacOff + 2 * kRowsW * 4;               // segment results: [segment parity][inv, lse][row]
constexpr int kFlagOff = kFinOff + 2 * 2 * kRowsW * 4;          // reference moved: [parity][wave] int
constexpr int kSmemW = kFlagOff + 2 * 4 * 4;
static_assert(kSmemW <= 160 * 1024, "LDS budget");
static_assert(kKSteps == 18, "16 latent k-steps + 2 rope k-steps");
constexpr int kCopyLoadsW = 9;  // 1 KB LDS-direct loads per wave per chunk
constexpr int kKAheadW = 2;     // k-steps of K fragments in flight

// Wave w copies the blocks of its own value columns, latent blocks (r, 2w) and
// (r, 2w + 1) for r = 0..3, and rope block w: 9 KB of the chunk's 36 KB, as
// nine 1 KB LDS-direct loads.
// Lane l moves 16 bytes of token row 8 r + (l >> 3); its byte offset is
// A[r & 1] + 8 r * row_bytes (+ 128 for the second column block), with the
// lane constants A[p] = (l >> 3) * row_bytes + 16 ((l & 7) ^ (l >> 3) ^ 2p) +
// 256 w -- the swizzled source chunk that lands at the lane's LDS slot.
struct CopyPlan {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lat, rope;  // LDS destinations: this wave's latent blocks, its rope block
  uint32_t rb8;        // 8 rows in bytes
  bool on;             // the chunk has keys to copy
};

__device__ __forceinline__ CopyPlan copy_plan(const DecodeArgs& a, const Chunk& c, uint32_t lat, uint32_t rope,
                                              int w) {
  CopyPlan p;
  p.on = c.valid() && c.tok > 0;
  p.rsrc = chunk_rsrc(a, c);
  p.lat = lat + 2048u * w;
  p.rope = rope + 1024u * w;
  p.rb8 = 8u * (uint32_t)a.k_row_bytes;
  return p;
}

// Load k (0..8) of the wave's share: latent block (k >> 1, 2w + (k & 1)), or
// for k = 8 the rope block.
template <int K>
__device__ __forceinline__ void copy_one(const CopyPlan& p, int w, uint32_t a0, uint32_t a1) {
  if constexpr (K < 8) {
    constexpr int r = K >> 1, h = K & 1;
    const uint32_t v = ((r & 1) ? a1 : a0) + (uint32_t)r * p.rb8 + 128u * h;
    lds_dma16(p.rsrc, v, p.lat + 8192u * r + 1024u * h);
  } else {
    // rope block w: row 8 w + (l >> 3), byte 1024 + 16 (swizzled chunk)
    const uint32_t v = ((w & 1) ? a1 : a0) + (uint32_t)w * (p.rb8 - 256u) + 1024u;
    lds_dma16(p.rsrc, v, p.rope);
  }
}

__device__ __forceinline__ bool wide_copy(const DecodeArgs& a, const Chunk& c, uint32_t lat, uint32_t rope, int w,
                                          uint32_t a0, uint32_t a1) {
  const CopyPlan p = copy_plan(a, c, lat, rope, w);
  if (!p.on) return false;
  copy_one<0>(p, w, a0, a1);
  copy_one<1>(p, w, a0, a1);
  copy_one<2>(p, w, a0, a1);
  copy_one<3>(p, w, a0, a1);
  copy_one<4>(p, w, a0, a1);
  copy_one<5>(p, w, a0, a1);
  copy_one<6>(p, w, a0, a1);
  copy_one<7>(p, w, a0, a1);
  copy_one<8>(p, w, a0, a1);
  return true;
}

// An opaque copy of the lane index: lane-derived offsets computed from it in
// one section of the step are not merged with (and kept live until) those of
// another.
__device__ __forceinline__ int fresh_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// Per-lane offsets of the operand reads and of the copy.  Rebuilt from the
// lane index every step: the loop keeps the queries (144 VGPRs) and the value
// accumulators (256 AGPRs) resident and cannot afford to hold these too.
struct LaneMap {
  int g, r16;
  uint32_t kx, k_lat, k_rope;  // score K fragment: token 16 tt + r16, column chunk 4 ks + g
  uint32_t vy, v_lane;         // value V^T fragment (transposing read)
  uint32_t cp0, cp1;           // copy source offsets A[0], A[1]
  __device__ __forceinline__ LaneMap(int lane, int w, uint32_t row_bytes) {
    g = lane >> 4;
    r16 = lane & 15;
    const int ka = r16 & 7, kr = r16 >> 3;
    kx = (uint32_t)(g ^ ka ^ (2 * kr));
    k_lat = 8192u * kr + 128u * ka;
    k_rope = 1024u * kr + 128u * ka;
    const int va = 4 * (g & 1) + (r16 >> 2);
    vy = (uint32_t)(((r16 & 3) >> 1) ^ va ^ (2 * ((g >> 1) & 1)));
    v_lane = 8192u * (g >> 1) + 1024u * (2 * w) + 128u * va + 8u * (r16 & 1);
    const int ta = lane >> 3, te = lane & 7;
    cp0 = (uint32_t)ta * row_bytes + 16u * (uint32_t)(te ^ ta) + 256u * w;
    cp1 = (uint32_t)ta * row_bytes + 16u * (uint32_t)(te ^ ta ^ 2) + 256u * w;
  }
};

// f(std::integral_constant<int, I>{}) for I = B .. E - 1, unrolled by construction
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Compiler fence between the sections of a step: the next section's LDS reads
// (and the registers they fill) stay behind it instead of being hoisted ahead
// of the previous section's MFMAs.
__device__ __forceinline__ void section_fence() { asm volatile("" ::: "memory"); }

// One k-step of the scores, s[tt][rl] += K_tt . Q_rl^T, as four MFMAs with
// VGPR accumulators.  Written as assembly so that the score accumulators stay
// in VGPRs while the value accumulators fill all 256 AGPRs (the compiler puts
// every MFMA result of a function in one register file).  The k-step
// fragments come straight from LDS and global loads; the first k-step starts
// from zero (no VALU write feeds an MFMA here), and consecutive MFMAs on one
// accumulator are three MFMAs apart.
__device__ __forceinline__ void score_mfma(f32x4 (&s)[2][2], bf16x8 k0, bf16x8 k1, bf16x8 q0, bf16x8 q1,
                                           bool first) {
  if (first)
    asm("s_nop 4\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %6, 0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %4, %7, 0\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %5, %6, 0\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %5, %7, 0"
        : "=&v"(s[0][0]), "=&v"(s[0][1]), "=&v"(s[1][0]), "=&v"(s[1][1])
        : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
  else
    asm("v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3"
        : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1])
        : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
}

// The score accumulators are read by VALU instructions next: wait out the
// MFMA result latency (more than the 8-pass requirement) first.
__device__ __forceinline__ void score_done(f32x4 (&s)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}

// One MFMA of the values, o += V^T_ct . P^T_rt, accumulating in AGPRs.
// Assembly for the same reason as the scores.  A new V fragment may have been
// assembled by VALU moves, hence the wait states before its first MFMA.  Each
// accumulator gets one MFMA per step.
__device__ __forceinline__ void value_mfma1(f32x4& o, bf16x8 v, bf16x8 p, bool new_v) {
  if (new_v)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
  else
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}

// The accumulators of one row tile are about to be read or written by VALU
// instructions: wait out the result latency of the MFMAs that wrote them.
__device__ __forceinline__ void acc_ready(f32x4 (&o)[8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]));
}

// Chunk descriptors in batches of 64.  Every wave computes the descriptors of
// the next 64 chunks of its part lane-parallel (lane i: chunk position + i),
// packed as in the narrow kernel ({seq, chunk, tok | first << 8 | last << 9 |
// bad << 10, phys}; {-1, 0, 0, -1} past the part's end), and takes one per step
// with v_readlane: no page walk, no scalar loads and no LDS hand-off in the
// loop.  (A batch refill waits for the vector memory work in flight; it comes
// once per 64 chunks.)
struct BatchPos {
  int seq, chunk;  // part position of the batch's first chunk
  bool more;       // the part has chunks from there on
};

__device__ __forceinline__ i32x4 desc_batch(const DecodeArgs& a, const PartInfo& pi, BatchPos& pos, int lane) {
  i32x4 out = i32x4{-1, 0, 0, -1};
  if (!pos.more) return out;
  // lengths of the sequences the batch may touch: lane k holds sequence pos.seq + k
  const int sk = pos.seq + lane;
  const int nk = sk <= pi.seq_last ? clamp_len(a, a.seqlens[sk]) : 0;
  int rem = lane;  // chunks still to skip before this lane's own
  bool found = false;
  int my_seq = -1, my_chunk = 0, my_n = 0, my_lo = 0, my_hi = 0;
  int sq = pos.seq, lo = pos.chunk;
#pragma unroll 1
  for (int k = 0; k < 64 && sq <= pi.seq_last; ++k) {
    const int n = __builtin_amdgcn_readlane(nk, k);
    int hi = chunk_count(n);
    if (sq == pi.seq_last && 2 * pi.page_end < hi) hi = 2 * pi.page_end;
    const int seg_lo = sq == pi.seq_begin ? 2 * pi.page_begin : 0;
    const int cnt = hi - lo;
    if (!found) {
      if (rem < cnt) {
        my_seq = sq;
        my_chunk = lo + rem;
        my_n = n;
        my_lo = seg_lo;
        my_hi = hi;
        found = true;
      } else {
        rem -= cnt;
      }
    }
    ++sq;
    lo = 0;
    if (__builtin_amdgcn_ballot_w64(!found) == 0) break;
  }
  int phys = -1;
  if (found) {
    const int page = my_chunk >> 1;
    if (page < a.max_blocks) phys = a.block_table[(int64_t)my_seq * a.bt_stride + page];
    int tok = my_n - kChunk * my_chunk;
    tok = tok < 0 ? 0 : (tok > kChunk ? kChunk : tok);
    const bool bad = tok > 0 && !(phys >= 0 && phys < a.num_blocks);
    out = i32x4{my_seq, my_chunk,
                tok | (my_chunk == my_lo ? 256 : 0) | (my_chunk == my_hi - 1 ? 512 : 0) | (bad ? 1024 : 0), phys};
  }
  // where the next batch starts: after lane 63's chunk
  const int s63 = __builtin_amdgcn_readlane(my_seq, 63);
  if (s63 < 0) {
    pos.more = false;
  } else {
    const int c63 = __builtin_amdgcn_readlane(my_chunk, 63), h63 = __builtin_amdgcn_readlane(my_hi, 63);
    if (c63 + 1 < h63) {
      pos.seq = s63;
      pos.chunk = c63 + 1;
    } else if (s63 < pi.seq_last) {
      pos.seq = s63 + 1;
      pos.chunk = 0;
    } else {
      pos.more = false;
    }
  }
  return out;
}

// Descriptor i (0..63, wave-uniform) of a batch.
__device__ __forceinline__ Chunk batch_get(const i32x4& b, int i) {
  Chunk c;
  c.seq = __builtin_amdgcn_readlane(b[0], i);
  c.chunk = __builtin_amdgcn_readlane(b[1], i);
  const int z = __builtin_amdgcn_readlane(b[2], i);
  c.phys = __builtin_amdgcn_readlane(b[3], i);
  c.tok = z & 255;
  c.first = (z & 256) != 0;
  c.last = (z & 512) != 0;
  c.bad = (z & 1024) != 0;
  return c;
}

__global__ __launch_bounds__(kThreadsW, 1) void decode_wide_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemW];
  const int w = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  PartInfo pi;
  if (!load_part(a, kRowsW, pi)) return;

  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  lds_f32* const fac = (lds_f32*)(lds + kFacOff);
  lds_f32* const fin = (lds_f32*)(lds + kFinOff);
  lds_i32* const flags = (lds_i32*)(lds + kFlagOff);
  const uint32_t row_bytes = (uint32_t)a.k_row_bytes;
  const float sc = a.scale_log2;

  // ---- scores and softmax: rows 32 w + 16 rl + r16 (reference max m_ref in
  // log2 units, running sum of 2^(x - m_ref) per lane over its tokens)
  bf16x8 qf[2][kKSteps];
  float m_ref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  int lim_min = 0;  // smallest visible-key limit among this wave's rows
  int seg_n = 0;    // cached tokens of the scores' segment (after the cap)
  // ---- values: columns 128 w + 16 ct + 4 g + j of rows 16 rt + r16
  f32x4 o[kRowTiles][8];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool seg_bad = false;
  int seg_slot = 0, seg_nsplit = 1;

  // Queries of this wave's rows for the segment of chunk c, and the
  // visible-key limits.  Waits for the loads here, before the next copy is
  // issued, so that no later wait for them also waits for that copy.
  auto load_queries = [&](const Chunk& c, int g, int r16) {
    const int n = clamp_len(a, load_len(a, c.seq));
#pragma unroll
    for (int rl = 0; rl < 2; ++rl) {
      const int row = pi.blk_row0 + 32 * w + 16 * rl + r16;
      const bool ok = row < a.rows;
      const int rr = ok ? row : 0;  // rows past the last one score row 0's query, all masked
      const int qi = rr / a.h_q, h = rr - qi * a.h_q;
      const uint16_t* qp = a.q + (int64_t)c.seq * a.q_sb + (int64_t)qi * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[rl][ks] = *(const bf16x8*)(qp + 32 * ks);
    }
    // chunks below every row's limit need no masking; a wave with rows past
    // the last one masks every chunk
    lim_min = pi.blk_row0 + 32 * w + 32 > a.rows ? 0 : (a.causal ? n - (a.s_q - 1) : n);
    seg_n = n;
    // waits here for the loads; the queries stay in VGPRs (the accumulators fill the AGPRs)
#pragma unroll
    for (int rl = 0; rl < 2; ++rl)
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qf[rl][ks]));
  };

  // ---- prologue: the first descriptor batch; copies of chunks 0 and 1;
  // queries of the first segment
  BatchPos bpos;
  bpos.seq = pi.seq_begin;
  bpos.chunk = 2 * pi.page_begin;
  bpos.more = true;
  i32x4 batch = desc_batch(a, pi, bpos, lane);
  int c0 = 0;  // chunk ordinal of the batch's first descriptor
  Chunk D0 = unpack_chunk(i32x4{-1, 0, 0, -1});  // chunk t: values
  Chunk D1 = batch_get(batch, 0);                // chunk t + 1: scores
  Chunk D2 = batch_get(batch, 1);                // chunk t + 2: landing
  Chunk D3 = batch_get(batch, 2);                // chunk t + 3: copied this step
  {
    const LaneMap lm(lane, w, row_bytes);
    wide_copy(a, D1, lds_addr, lds_addr + kRopeOff, w, lm.cp0, lm.cp1);
    wide_copy(a, D2, lds_addr + kLatBytes, lds_addr + kRopeOff + kRopeBytes, w, lm.cp0, lm.cp1);
    if (D1.valid()) load_queries(D1, lm.g, lm.r16);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int rs1 = 0;    // rope slot of chunk t + 1 (chunk ordinal mod 3)
  int s_seg = 0;  // segments whose results the score side has published
  int v_seg = 0;  // segments the value side has closed

  for (int t = -1;; ++t) {
    if (!D0.valid() && !D1.valid()) break;
    const int par = t & 1, par1 = (t + 1) & 1;
    const bool v_has = D0.valid() && D0.tok > 0;
    const bool s_has = D1.valid() && D1.tok > 0;
    bool drain = false;  // this step issued other vector memory work: wait for all of it
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int g = ln >> 4, r16 = ln & 15;

    // ---- chunk t + 1 starts a segment: its queries (the first ones were
    // loaded in the prologue) and a fresh softmax state
    if (D1.valid() && D1.first) {
      if (t >= 0) {
        load_queries(D1, g, r16);
        drain = true;
      }
#pragma unroll
      for (int rl = 0; rl < 2; ++rl) {
        m_ref[rl] = -INFINITY;
        lsum[rl] = 0.f;
      }
    }
    // ---- copy chunk t + 3 into the slots of chunks t - 1 (latent) and t (rope)
    const int rs3 = rs1 == 0 ? 2 : rs1 - 1;
    bool issued;
    {
      const LaneMap lm(fresh_lane(lane), w, row_bytes);
      issued = wide_copy(a, D3, lds_addr + (uint32_t)((t + 3) & 3) * kLatBytes,
                         lds_addr + kRopeOff + (uint32_t)rs3 * kRopeBytes, w, lm.cp0, lm.cp1);
    }
    // ---- the values enter a new segment
    if (D0.valid() && D0.first) {
      const int split = D0.seq == pi.seq_begin ? pi.split_first : 0;
      const int s0 = ((cint32*)a.num_splits)[D0.seq];
      seg_slot = s0 + split;
      seg_nsplit = ((cint32*)a.num_splits)[D0.seq + 1] - s0;
      seg_bad = false;
    }
    if (D0.valid()) seg_bad |= D0.bad;

    // ---- scores of chunk t + 1: 32 rows x 32 tokens, two MFMAs per K read
    f32x4 s[2][2] = {};  // [token tile][row tile]
    if (s_has) {
      const LaneMap lm(fresh_lane(lane), w, row_bytes);
      lds_u8* const lat = lds + (uint32_t)((t + 1) & 3) * kLatBytes;
      lds_u8* const rope = lds + kRopeOff + (uint32_t)rs1 * kRopeBytes;
      lds_u8* const kb0 = launder(lat + lm.k_lat + 16u * lm.kx);
      lds_u8* const kb1 = launder(lat + lm.k_lat + 16u * (lm.kx ^ 4u));
      lds_u8* const rb0 = launder(rope + lm.k_rope + 16u * lm.kx);
      lds_u8* const rb1 = launder(rope + lm.k_rope + 16u * (lm.kx ^ 4u));
      auto kfrag = [&](int ks, int tt) -> bf16x8 {
        if (ks < 16) return *(const lds_bf16x8*)(((ks & 1) ? kb1 : kb0) + 16384u * tt + 1024u * (ks >> 1));
        return *(const lds_bf16x8*)(((ks & 1) ? rb1 : rb0) + 2048u * tt);
      };
      // K fragments in flight: a ring of kKAheadW + 1 pairs
      bf16x8 kf[kKAheadW + 1][2];
#pragma unroll
      for (int ks = 0; ks < kKAheadW; ++ks) {
        kf[ks][0] = kfrag(ks, 0);
        kf[ks][1] = kfrag(ks, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        constexpr int R = kKAheadW + 1;
        if (ks + kKAheadW < kKSteps) {
          kf[(ks + kKAheadW) % R][0] = kfrag(ks + kKAheadW, 0);
          kf[(ks + kKAheadW) % R][1] = kfrag(ks + kKAheadW, 1);
        }
        score_mfma(s, kf[ks % R][0], kf[ks % R][1], qf[0][ks], qf[1][ks], ks == 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // without a value product behind it, the softmax would read the scores
      // right away
      if (!v_has) score_done(s);
    }
    section_fence();

    // ---- rows whose reference moved at chunk t: rescale what they have
    // accumulated so far
    const i32x4 fl = *(const lds_i32x4*)(flags + 4 * par);
    if (v_has && uniform(fl[0] | fl[1] | fl[2] | fl[3])) {
      const lds_f32* fp = fac + par * kRowsW + r16;
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        if (uniform(fl[rt >> 1])) {
          const float f = fp[16 * rt];
          acc_ready(o[rt]);
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) o[rt][ct] *= f;
        }
      }
    }

    section_fence();
    // ---- values of chunk t, O^T[columns 128 w ..] += V^T . P^T, in 16 groups
    // of four MFMAs; the softmax of chunk t + 1 runs in the VALU between them
    lds_u8* vb[4];
    lds_u8* pp;
    bf16x8 pf[4];  // P^T fragments of four row tiles (the first, then the second half)
    bf16x8 vr[3];  // V^T fragments in flight: group k uses vr[k % 3], read two groups ahead
    auto vfrag = [&](int ct) -> bf16x8 {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct & 3] + 1024u * (ct >> 2)));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct & 3] + 1024u * (ct >> 2) + 16384u));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto v_setup = [&]() {
      const LaneMap lm(fresh_lane(lane), w, row_bytes);
      lds_u8* const lat = lds + (uint32_t)(t & 3) * kLatBytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) vb[u] = launder(lat + lm.v_lane + 16u * ((2u * u) ^ lm.vy));
      pp = lds + kPOff + 16u * fresh_lane(lane) + (uint32_t)par * (kRowTiles * 1024);
#pragma unroll
      for (int i = 0; i < 4; ++i) pf[i] = *(const lds_bf16x8*)(pp + 1024u * i);
      vr[0] = vfrag(0);
      vr[1] = vfrag(1);
    };
    // softmax state of this step (lane holds tokens 32 chunk + 16 tt + 4 g + j
    // of row 16 rl + r16, as x[rl][4 tt + j], in log2 units less mu[rl])
    float x[2][8];
    float mu[2], mx[2];
    bf16x8 pv[2];
    bool moved = false;
    // 64 single MFMAs (row tiles 0..3 over the eight column tiles, then 4..7:
    // V read twice, half of P held); group q works on column tile (q >> 2) & 7,
    // row tile 4 (q >> 5) + (q & 3)
    auto v_group = [&](auto qc) {
      constexpr int q = decltype(qc)::value;
      const int cg = q >> 2, ct = cg & 7, i = q & 3, half = q >> 5;
      if constexpr (i == 0 && cg + 2 < 16) vr[(cg + 2) % 3] = vfrag((cg + 2) & 7);
      value_mfma1(o[4 * half + i][ct], vr[cg % 3], pf[i], i == 0);
      // the second half's P fragments, each right after its last use
      if constexpr (half == 0 && ct == 7) pf[i] = *(const lds_bf16x8*)(pp + 1024u * (4 + i));
    };
    // the softmax of chunk t + 1 in small pieces, one after each MFMA
    auto s_piece = [&](auto qc) {
      constexpr int q = decltype(qc)::value;
      if constexpr (q >= 4 && q < 8) {
        const int rl = (q - 4) >> 1, tt = (q - 4) & 1;
        if (tt == 0) mu[rl] = m_ref[rl] == -INFINITY ? 0.f : m_ref[rl];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[rl][4 * tt + j] = __builtin_fmaf(s[tt][rl][j], sc, -mu[rl]);
      } else if constexpr (q == 8) {
        // mask keys past each row's limit (only chunks that reach a limit)
        const int tok0 = kChunk * D1.chunk;
        if (!s_has || tok0 + kChunk > lim_min) {
#pragma unroll
          for (int rl = 0; rl < 2; ++rl) {
            // the row's visible-key limit (rows past the last one see nothing)
            const int row = pi.blk_row0 + 32 * w + 16 * rl + r16;
            const int qi = row / a.h_q;
            const int lim = row < a.rows ? seg_n - (a.causal ? a.s_q - 1 - qi : 0) : 0;
            const int vis = s_has ? lim - tok0 - 4 * g : 0;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (16 * tt + j >= vis) x[rl][4 * tt + j] = -INFINITY;
          }
        }
      } else if constexpr (q == 9 || q == 10) {
        const int rl = q - 9;
        mx[rl] = fmaxf(fmaxf(fmaxf(x[rl][0], x[rl][1]), fmaxf(x[rl][2], x[rl][3])),
                       fmaxf(fmaxf(x[rl][4], x[rl][5]), fmaxf(x[rl][6], x[rl][7])));
      } else if constexpr (q == 11) {
        bool over = false;
#pragma unroll
        for (int rl = 0; rl < 2; ++rl)
          over |= m_ref[rl] == -INFINITY ? mx[rl] > -INFINITY : mx[rl] > kRescaleSlack;
        moved = __builtin_amdgcn_ballot_w64(over) != 0;
        if (moved) {
          // a chunk max passed the reference by more than 2^16 (or the
          // segment just started): move every row's reference to its max
#pragma unroll
          for (int rl = 0; rl < 2; ++rl) {
            const float rowmax = wave_max16(mx[rl]) + mu[rl];
            const float m_new = fmaxf(m_ref[rl], rowmax);
            const float f = m_ref[rl] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[rl] - m_new);
            const float mu_new = m_new == -INFINITY ? 0.f : m_new;
            lsum[rl] *= f;
            m_ref[rl] = m_new;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[rl][i] += mu[rl] - mu_new;
            mu[rl] = mu_new;
            if (g == 0) fac[par1 * kRowsW + 32 * w + 16 * rl + r16] = f;
          }
        }
      } else if constexpr (q >= 12 && q < 28) {
        const int rl = (q - 12) >> 3, i = (q - 12) & 7;
        x[rl][i] = __builtin_amdgcn_exp2f(x[rl][i]);
      } else if constexpr (q >= 28 && q < 36) {
        const int rl = (q - 28) >> 2, i = 2 * ((q - 28) & 3);
        lsum[rl] += x[rl][i] + x[rl][i + 1];
      } else if constexpr (q >= 36 && q < 44) {
        const int rl = (q - 36) >> 2, i = 2 * ((q - 36) & 3);
        pv[rl][i] = (__bf16)x[rl][i];
        pv[rl][i + 1] = (__bf16)x[rl][i + 1];
      } else if constexpr (q == 44 || q == 45) {
        const int rl = q - 44;
        *(lds_bf16x8*)(lds + kPOff + 16u * fresh_lane(lane) + par1 * (kRowTiles * 1024) + 1024u * (2 * w + rl)) =
            pv[rl];
        if (rl == 1 && lane == 0) flags[4 * par1 + w] = moved ? 1 : 0;
      }
    };
    // (a chunk without keys runs the softmax fully masked: no state changes,
    // P = 0)
    if (v_has) {
      v_setup();
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, 64>([&](auto qc) {
        v_group(qc);
        s_piece(qc);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      static_for<0, 64>([&](auto qc) { s_piece(qc); });
    }
    // ---- chunk t + 1 ends its segment: publish 1 / (sum of p) and lse of the rows
    if (D1.valid() && D1.last) {
      lds_f32* const fs = fin + (s_seg & 1) * (2 * kRowsW);
#pragma unroll
      for (int rl = 0; rl < 2; ++rl) {
        const float l = wave_sum16(lsum[rl]);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse = l > 0.f ? (m_ref[rl] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
        if (g == 0) {
          fs[32 * w + 16 * rl + r16] = inv;
          fs[kRowsW + 32 * w + 16 * rl + r16] = lse;
        }
      }
      ++s_seg;
    }

    // ---- chunk t ends its segment: write this wave's columns of every row
    if (D0.valid() && D0.last) {
      const lds_f32* const fs = fin + (v_seg & 1) * (2 * kRowsW) + r16;
      const bool final_out = seg_nsplit == 1;
      int row0 = pi.blk_row0 + r16;  // opaque: keeps the address arithmetic in this block
      asm volatile("" : "+v"(row0));
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        float inv = fs[16 * rt];
        float lse = fs[kRowsW + 16 * rt];
        acc_ready(o[rt]);
        if (seg_bad) {
          inv = __builtin_nanf("");
          lse = __builtin_nanf("");
        }
        const int row = row0 + 16 * rt;
        if (row < a.rows) {
          const int qi = row / a.h_q, h = row - qi * a.h_q;
          const int col0 = 128 * w + 4 * g;
          if (final_out) {
            uint16_t* op = a.out + (int64_t)D0.seq * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + col0;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
              const f32x4 v = o[rt][ct] * inv;
              *(bf16x4*)(op + 16 * ct) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            }
            if (w == 0 && g == 0)
              a.lse[(int64_t)D0.seq * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = lse;
          } else {
            float* pp = a.part_o + ((int64_t)seg_slot * a.rows + row) * kDv + col0;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) *(f32x4*)(pp + 16 * ct) = o[rt][ct] * inv;
            if (w == 0 && g == 0) a.part_lse[(int64_t)seg_slot * a.rows + row] = lse;
          }
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      ++v_seg;
      drain = true;
    }

    // ---- end of step: this wave's share of chunk t + 2 has landed (that of
    // chunk t + 3 may still be in flight); all LDS reads have returned
    static_assert(kCopyLoadsW == 9, "vmcnt below");
    if (issued && !drain)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    block_sync();
    D0 = D1;
    D1 = D2;
    D2 = D3;
    // the descriptor of chunk t + 4 (a new batch every 64 chunks)
    if (t + 4 - c0 >= 64) {
      batch = desc_batch(a, pi, bpos, lane);
      c0 += 64;
    }
    D3 = batch_get(batch, t + 4 - c0);
    rs1 = rs1 == 2 ? 0 : rs1 + 1;
  }
}

}  // namespace

hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_parts * a.row_blocks));
  hipLaunchKernelGGL(decode_wide_kernel, grid, dim3(kThreadsW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

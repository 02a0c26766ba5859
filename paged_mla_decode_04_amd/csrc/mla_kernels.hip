// Paged MLA decode kernels for gfx950 (MI355X): plan, split-KV decode, lse merge.
//
// What is computed: for each sequence, query rows r = (query token i, head h)
// attend over the sequence's cached latent rows k_t (576 bf16: K is the whole
// row, V its first 512 elements) fetched through the block table, with
// softmax(scale * q.k) over the visible keys, returning out (bf16) and the
// natural-log lse (fp32).  The PAI FlashMLA tutorial (segmentfault,
// "云上玩转DeepSeek系列之五", section 二.4) fixes the inputs this way and prices
// the work as (d + dv) multiply-adds per query-key pair and one d-element read
// per cached token -- K and V come out of the same row, read once.
//
// Design on gfx950 (256 CUs in 8 XCDs, 160 KB LDS, 64-wide waves, bf16 MFMA):
//   * one workgroup (8 waves, 2 per SIMD) per CU processes one plan part for
//     one block of up to 64 query rows: a contiguous run of 64-token pages,
//     possibly spanning several sequences;
//   * a page (64 x 576 bf16 = 72 KB) is copied HBM -> LDS with 16-byte buffer
//     loads that write LDS directly (no register staging), double buffered;
//   * scores are computed transposed, S^T = K . Q^T, on 16x16x32 bf16 MFMA,
//     with the query tile held in registers, so every lane holds whole query
//     rows and row max / row sum need two cross-lane steps;
//   * P . V is computed as O^T = V^T . P^T; V^T comes from LDS through the
//     gfx950 transposing read ds_read_b64_tr_b16 (4 consecutive tokens per
//     lane), P^T through LDS in exactly the layout the scores leave it in;
//   * online softmax in the log2 domain against a reference max per row that
//     only moves when a page's max passes it by more than 2^16;
//   * a part that covers only a piece of a sequence writes an fp32 partial
//     (O / l, lse); the merge kernel combines them by lse (Flash-Decoding, as
//     the Hacker News discussion of the FlashMLA release describes it).
//
// LDS page tile: 9 x 8 blocks of 1 KB; block (r, q) holds tokens 8r..8r+7 x
// 16-byte chunks 8q..8q+7 (columns 64q..64q+63), token a of the block at
// 128 a, its chunk c at slot (c % 8) ^ a ^ (r & 1).  The swizzle keeps both
// the 16-byte K reads (16 tokens x one chunk) and the 8-byte transposing V
// reads (4 tokens x 2 chunks x 2 halves per 16 lanes) free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "mla_internal.h"
#include "mla_plan.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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

// ---------------------------------------------------------------------------
// Split-KV decode.
//
// One workgroup of 8 waves (2 per SIMD) handles one row block (up to 64 query
// rows, NRT row tiles of 16) of one plan part.  Per page:
//   scores   wave w computes S^T = K . Q^T for row tile w % NRT and 16-token
//            tiles (w / NRT) * TT .. + TT - 1 (TT = 2 for 4 row tiles, else 1),
//            keeping the query tile in registers;
//   softmax  log2 domain, against a per-row reference max shared by the whole
//            workgroup; p is rounded to bf16 and written to LDS already in
//            the operand layout of the next product;
//   values   wave w owns output columns 64 w .. 64 w + 63 for every row and
//            accumulates O^T += V^T . P^T, reading V^T with the transposing
//            LDS read.
// Only wave w reads column block w of the values, so right after its own
// products it may start the copy of the page two steps ahead into that block
// (and into one rope block, free since the score step): the copy of the next
// page is always in flight behind the arithmetic, with two barriers per page.
//
// Page bookkeeping runs three pages ahead on the scalar unit: the sequence
// length and the block-table entry of a page are fetched one step before the
// page's copy is issued, so no dependent load sits on the copy path.
// ---------------------------------------------------------------------------

constexpr int kThreads = 512;
constexpr int kPOffset = 2 * kPageBytes;          // P^T operands: [row tile][32-token half][lane] x 16 B
constexpr int kMaxOffset = kPOffset + 8 * 1024;   // page row max per (token group, row): f32 [4][64]
constexpr int kSumOffset = kMaxOffset + 1024;     // row sums of rounded p per (token group, row)
constexpr int kSumExOffset = kSumOffset + 1024;   // row sums of unrounded p per (token group, row)
constexpr int kFlagOffset = kSumExOffset + 1024;  // per wave: a row max passed the reference
constexpr int kSmemBytes = kFlagOffset + 8 * 4;
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");

typedef const __attribute__((address_space(4))) int32_t cint32;  // read-only, uniform: scalar loads
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

// 16-byte LDS-direct buffer load: lane l's 16 bytes land at lds_addr + 16 l.
// Written as inline assembly so that the compiler does not track the LDS
// write: it would otherwise make every later LDS read wait for all copies in
// flight.  Completion is awaited explicitly (vmcnt) before the barrier that
// hands a page over, and a copy only targets LDS that no wave reads any more.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

// Block table position of one page of the part and what is known about it.
struct Cursor {
  int seq, page;  // sequence, page within the sequence
  int n;          // cached tokens of seq as stored (clamp_len applies the cap)
  int phys;       // block-table entry (-1 past the row)
  bool valid;     // inside the part
};

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int n) {
  const int cap = a.max_blocks * kPageTokens;
  return n < 0 ? 0 : (n > cap ? cap : n);
}
__device__ __forceinline__ int load_len(const DecodeArgs& a, int b) { return ((cint32*)a.seqlens)[b]; }
__device__ __forceinline__ int load_phys(const DecodeArgs& a, int b, int page) {
  return page < a.max_blocks ? ((cint32*)a.block_table)[(int64_t)b * a.bt_stride + page] : -1;
}
__device__ __forceinline__ int page_tokens(const DecodeArgs& a, const Cursor& c) {
  if (!c.valid) return 0;
  const int t = clamp_len(a, c.n) - kPageTokens * c.page;
  return t > kPageTokens ? kPageTokens : t;
}

// The page after c in the part's (sequence, page) order.  Uses c.n, fetched a
// step earlier; starts the fetch of the new page's length (on a sequence
// change) and table entry.
__device__ __forceinline__ Cursor next_page(const DecodeArgs& a, const Cursor& c, int seq_last, int page_end) {
  Cursor d = c;
  if (!c.valid) return d;
  const int end = c.seq == seq_last ? page_end : seq_units(clamp_len(a, c.n));
  if (c.page + 1 < end) {
    d.page = c.page + 1;
  } else if (c.seq < seq_last) {
    d.seq = c.seq + 1;
    d.page = 0;
    d.n = load_len(a, d.seq);
  } else {
    d.valid = false;
    return d;
  }
  d.phys = load_phys(a, d.seq, d.page);
  return d;
}

// Start this wave's share of the copy of page c into the tile at LDS address
// `tile`: column block `wave` of every row (8 x 1 KB) and the rope block of
// token octet `wave` (1 KB) -- 9 loads per wave, 72 KB per workgroup.  Rows at
// or past the page's token count, and pages whose table entry lies outside
// the pool, read as zeros through the buffer range check.
__device__ __forceinline__ bool issue_copy(const DecodeArgs& a, const Cursor& c, uint32_t tile, int wave,
                                           int lane) {
  const int tok = page_tokens(a, c);
  if (tok <= 0) return false;
  const bool ok = c.phys >= 0 && c.phys < a.num_blocks;
  const uint8_t* base = a.k + (ok ? (int64_t)c.phys * a.k_block_bytes : 0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)base, (short)0, ok ? (int32_t)(kPageTokens * a.k_row_bytes) : 0, kBufferFlags);
  const int ta = lane >> 3, e = lane & 7;
  const uint32_t rb = (uint32_t)a.k_row_bytes;
  {
    const int t = 8 * wave + ta;
    const uint32_t voff = t < tok ? t * rb + 16u * (64 + (e ^ ta ^ (wave & 1))) : kOutOfRange;
    lds_dma16(rsrc, voff, tile + 1024u * (9 * wave + 8));
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int t = 8 * r + ta;
    const uint32_t voff = t < tok ? t * rb + 16u * (8 * wave + (e ^ ta ^ (r & 1))) : kOutOfRange;
    lds_dma16(rsrc, voff, tile + 1024u * (9 * r + wave));
  }
  return true;
}

constexpr int kAheadK = 3;  // score k-steps whose K fragments are read ahead

template <int NRT>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  constexpr int TT = NRT == 4 ? 2 : 1;  // 16-token score tiles per scoring wave
  constexpr int NG = 4 / TT;            // token groups a row's scores are split into
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
  // run of (part, row block) pairs so that the row blocks of one part, and
  // neighbouring parts of one sequence, share that XCD's L2.
  const int G = gridDim.x, hw = blockIdx.x;
  const int xcd = hw & 7, pos = hw >> 3;
  const int logical = xcd * (G >> 3) + min(xcd, G & 7) + pos;
  const int part = logical / a.row_blocks;
  const int mblock = logical - part * a.row_blocks;

  cint32* md = (cint32*)a.tile_md + (int64_t)part * kTileMdInts;
  const int seq_begin = md[0];
  if (seq_begin >= a.batch) return;
  const int page_begin = md[1];
  const int seq_last = md[2];
  const int page_end = md[3];
  const int split_first = md[4];

  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  // this lane's row r16 in the per-row statistics: [token group][row tile][r16]
  lds_f32* const stats = (lds_f32*)launder(lds + kMaxOffset + 4u * r16);
  constexpr int kSumAt = (kSumOffset - kMaxOffset) / 4, kSumExAt = (kSumExOffset - kMaxOffset) / 4;

  // score role
  const bool scorer = wave < NRT * NG;
  const int rt1 = wave % NRT;
  const int tg = wave / NRT;
  const int blk_row0 = mblock * NRT * 16;
  const int own_row = blk_row0 + 16 * rt1 + r16;
  // per-lane LDS offsets in a page tile (layout at the top of this file)
  const int ka = r16 & 7, kr = r16 >> 3;
  const uint32_t kx = (uint32_t)(g ^ ka ^ kr);
  const uint32_t k_lane = 9216u * kr + 128u * ka + 18432u * (tg * TT);
  const int va = 4 * (g & 1) + (r16 >> 2);
  const uint32_t vy = (uint32_t)(((r16 & 3) >> 1) ^ va ^ ((g >> 1) & 1));
  const uint32_t v_lane = 9216u * (g >> 1) + 128u * va + 8u * (r16 & 1) + 1024u * wave;
  lds_u8* const pfrag = launder(lds + kPOffset + 16u * lane);

  bf16x8 qf[kKSteps];
  f32x4 o[NRT][4];
  float mref[NRT];           // reference max of row 16 rt + r16 (log2 units)
  float m_own = -INFINITY;   // mref of the scoring row
  float lsum = 0.f, lex = 0.f;
  int lim = 0;               // visible tokens of the scoring row
  bool bad = false;
  int slot = 0, nsplit = 1;

  auto begin_segment = [&](const Cursor& c) {
    const int b = c.seq;
    const int n = clamp_len(a, c.n);
    const int split = b == seq_begin ? split_first : 0;
    const int s0 = ((cint32*)a.num_splits)[b];
    slot = s0 + split;
    nsplit = ((cint32*)a.num_splits)[b + 1] - s0;
    if (scorer) {
      const bool ok = own_row < a.rows;
      const int rr = ok ? own_row : 0;
      const int qi = rr / a.h_q, h = rr - qi * a.h_q;
      lim = ok ? (a.causal ? n - (a.s_q - 1 - qi) : n) : 0;
      const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)qi * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8 v = *(const bf16x8*)(qp + 32 * ks);
        qf[ks] = ok ? v : bf16x8{};
      }
      // wait for the queries here, before the next copy is issued, so that no
      // later wait for them also waits for that copy
      asm volatile("" ::"v"(qf[kKSteps - 1]), "v"(qf[0]));
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      mref[rt] = -INFINITY;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    m_own = -INFINITY;
    lsum = 0.f;
    lex = 0.f;
    bad = false;
  };

  // ---- prologue: copies of the first two pages, queries of the first segment
  Cursor c0;
  c0.seq = seq_begin;
  c0.page = page_begin;
  c0.n = load_len(a, seq_begin);
  c0.phys = load_phys(a, seq_begin, page_begin);
  c0.valid = true;
  issue_copy(a, c0, lds_addr, wave, lane);
  Cursor c1 = next_page(a, c0, seq_last, page_end);
  issue_copy(a, c1, lds_addr + kPageBytes, wave, lane);
  begin_segment(c0);  // waits for the queries, and with them for both copies
  bool c1_copy = false;
  Cursor c2 = next_page(a, c1, seq_last, page_end);

  for (int s = 0;; ++s) {
    // ---- B1: page s (buffer s & 1) has landed; page s + 1 may be in flight
    if (c1_copy)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    block_sync();
    const Cursor c3 = next_page(a, c2, seq_last, page_end);

    const int tok0 = page_tokens(a, c0);
    const uint32_t tile_off = (uint32_t)(s & 1) * kPageBytes;
    lds_u8* const tile = lds + tile_off;
    if (tok0 > 0) {
      bad |= !(c0.phys >= 0 && c0.phys < a.num_blocks);
      f32x4 sc[TT];
      float psum = 0.f, psumx = 0.f;
      if (scorer) {
        // ---- scores of row tile rt1, token tiles tg * TT .. (16 x 16 per tile)
#pragma unroll
        for (int u = 0; u < TT; ++u) sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        lds_u8* const kb0 = launder(tile + k_lane + 16u * kx);
        lds_u8* const kb1 = launder(tile + k_lane + 16u * (kx ^ 4u));
        bf16x8 kf[kKSteps][TT];
        auto load_k = [&](int ks) {
#pragma unroll
          for (int u = 0; u < TT; ++u)
            kf[ks][u] = *(const lds_bf16x8*)(((ks & 1) ? kb1 : kb0) + 18432u * u + 1024u * (ks >> 1));
        };
#pragma unroll
        for (int ks = 0; ks < kAheadK; ++ks) load_k(ks);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + kAheadK < kKSteps) load_k(ks + kAheadK);
#pragma unroll
          for (int u = 0; u < TT; ++u)
            sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][u], qf[ks], sc[u], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- mask, scale, page row max; token 16 (tg TT + u) + 4 g + j
        const int vis = lim - kPageTokens * c0.page - 16 * tg * TT - 4 * g;
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < TT; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = (16 * u + j < vis) ? sc[u][j] * a.scale_log2 : -INFINITY;
            sc[u][j] = x;
            mx = fmaxf(mx, x);
          }
        mx = wave_max16(mx);
        const bool over = mx > m_own + kRescaleSlack;
        const float mu = m_own == -INFINITY ? 0.f : m_own;
        // probabilities against the current reference (recomputed below if
        // any row of the workgroup passed its reference)
        bf16x8 pv;
#pragma unroll
        for (int u = 0; u < TT; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float e = __builtin_amdgcn_exp2f(sc[u][j] - mu);
            const __bf16 p = (__bf16)e;
            psum += (float)p;
            psumx += e;
            pv[4 * u + j] = p;
          }
        if constexpr (TT == 2) {
          *(lds_bf16x8*)(pfrag + 1024u * (2 * rt1 + tg)) = pv;
        } else {
          *(lds_bf16x4*)(pfrag + 1024u * (2 * rt1 + (tg >> 1)) + 8u * (tg & 1)) =
              bf16x4{pv[0], pv[1], pv[2], pv[3]};
        }
        if (g == 0) stats[64 * tg + 16 * rt1] = mx;
        const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
        if (lane == 0) ((lds_i32*)(lds + kFlagOffset))[wave] = wave_over ? 1 : 0;
      } else if (lane == 0) {
        ((lds_i32*)(lds + kFlagOffset))[wave] = 0;
      }
      block_sync();  // ---- B2: P, page row maxima and flags visible

      const i32x4 f0 = *(const lds_i32x4*)(lds + kFlagOffset);
      const i32x4 f1 = *(const lds_i32x4*)(lds + kFlagOffset + 16);
      const i32x4 fo = f0 | f1;
      const int any = uniform(fo[0] | fo[1] | fo[2] | fo[3]);
      if (any) {
        // Rare: some row's page max passed its reference by more than the
        // slack (always on a segment's first page).  Every row moves its
        // reference to max(reference, page max) and rescales what it has
        // accumulated; the scorers redo their probabilities.
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          float m_new = mref[rt];
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) m_new = fmaxf(m_new, stats[64 * gi + 16 * rt]);
          const float f = mref[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref[rt] - m_new);
          mref[rt] = m_new;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) o[rt][ct] *= f;
          if (scorer && rt == rt1) {
            lsum *= f;
            lex *= f;
            m_own = m_new;
          }
        }
        if (scorer) {
          const float mu = m_own == -INFINITY ? 0.f : m_own;
          bf16x8 pv;
          psum = 0.f;
          psumx = 0.f;
#pragma unroll
          for (int u = 0; u < TT; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float e = __builtin_amdgcn_exp2f(sc[u][j] - mu);
              const __bf16 p = (__bf16)e;
              psum += (float)p;
              psumx += e;
              pv[4 * u + j] = p;
            }
          if constexpr (TT == 2) {
            *(lds_bf16x8*)(pfrag + 1024u * (2 * rt1 + tg)) = pv;
          } else {
            *(lds_bf16x4*)(pfrag + 1024u * (2 * rt1 + (tg >> 1)) + 8u * (tg & 1)) =
                bf16x4{pv[0], pv[1], pv[2], pv[3]};
          }
        }
        block_sync();  // ---- B3: redone P visible
      }
      lsum += psum;
      lex += psumx;

      // ---- O^T[column block wave] += V^T . P^T, both 32-token halves
      lds_u8* vb[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) vb[ct] = launder(tile + v_lane + 16u * ((2u * ct) ^ vy));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 pf[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) pf[rt] = *(const lds_bf16x8*)(pfrag + 1024u * (2 * rt + kb));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct] + 36864u * kb));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct] + 36864u * kb + 18432u));
          const bf16x8 vf = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], o[rt][ct], 0, 0, 0);
        }
      }
    }

    // ---- segment epilogue after its last page
    const bool seg_last = !c1.valid || c1.seq != c0.seq;
    if (seg_last) {
      if (scorer) {
        const float l = wave_sum16(lsum), le = wave_sum16(lex);
        if (g == 0) {
          stats[kSumAt + 64 * tg + 16 * rt1] = l;
          stats[kSumExAt + 64 * tg + 16 * rt1] = le;
        }
      }
      block_sync();  // ---- E1: row sums visible
      const int b = c0.seq;
      const bool final_out = nsplit == 1;
      // opaque copy: keeps the output address arithmetic inside this rarely
      // taken block instead of hoisted (and held in registers) across the loop
      int row0 = blk_row0 + r16;
      asm volatile("" : "+v"(row0));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        float L = 0.f, LE = 0.f;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          L += stats[kSumAt + 64 * gi + 16 * rt];
          LE += stats[kSumExAt + 64 * gi + 16 * rt];
        }
        float inv = L > 0.f ? 1.f / L : 0.f;
        float lse = LE > 0.f ? (mref[rt] + __builtin_amdgcn_logf(LE)) * kLn2 : -INFINITY;
        if (bad) {
          inv = __builtin_nanf("");
          lse = __builtin_nanf("");
        }
        const int row = row0 + 16 * rt;
        if (row < a.rows) {
          const int qi = row / a.h_q, h = row - qi * a.h_q;
          const int col0 = 64 * wave + 4 * g;
          if (final_out) {
            uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + col0;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
              const f32x4 v = o[rt][ct] * inv;
              *(bf16x4*)(op + 16 * ct) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            }
            if (wave == 0 && g == 0) a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = lse;
          } else {
            float* pp = a.part_o + ((int64_t)slot * a.rows + row) * kDv + col0;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) *(f32x4*)(pp + 16 * ct) = o[rt][ct] * inv;
            if (wave == 0 && g == 0) a.part_lse[(int64_t)slot * a.rows + row] = lse;
          }
        }
      }
      if (c1.valid) begin_segment(c1);
    }

    // ---- copy page s + 2 into this page's buffer: this wave's value block
    // and rope block are no longer read by anyone (the rope block since B2,
    // the value block since this wave's own products above)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    c1_copy = issue_copy(a, c2, lds_addr + tile_off, wave, lane);
    c0 = c1;
    c1 = c2;
    c2 = c3;
    if (!c0.valid) break;
  }
}

// Merge the partials of every sequence that more than one part touched:
// L = log(sum_i exp(lse_i)), out = sum_i exp(lse_i - L) * O_i (empty partials,
// lse = -inf, weigh nothing; all empty gives out = 0, lse = -inf).
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int b = blockIdx.x;
  const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int base = a.num_splits[b];
  const int ns = a.num_splits[b + 1] - base;
  if (ns <= 1 || r >= a.rows) return;
  float mx = -INFINITY;
  bool nan = false;
  for (int i = 0; i < ns; ++i) {
    const float x = a.part_lse[(int64_t)(base + i) * a.rows + r];
    nan |= (x != x);
    mx = fmaxf(mx, x);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int i = 0; i < ns; ++i) {
      const float x = a.part_lse[(int64_t)(base + i) * a.rows + r];
      sum += __builtin_amdgcn_exp2f((x - mx) * kLog2e);
    }
    L = mx + __builtin_amdgcn_logf(sum) * kLn2;
    for (int i = 0; i < ns; ++i) {
      const float x = a.part_lse[(int64_t)(base + i) * a.rows + r];
      const float w = __builtin_amdgcn_exp2f((x - L) * kLog2e);
      const f32x4* src = (const f32x4*)(a.part_o + ((int64_t)(base + i) * a.rows + r) * kDv + 8 * lane);
      const f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += w * v0[j];
        acc[4 + j] += w * v1[j];
      }
    }
  }
  if (nan) {
    L = __builtin_nanf("");
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_nanf("");
  }
  const int qi = r / a.h_q, h = r - qi * a.h_q;
  uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + 8 * lane;
  bf16x8 w;
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = (__bf16)acc[j];
  *(bf16x8*)op = w;
  if (lane == 0) a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = L;
}

// Block-wide inclusive scan step over one 1024-entry chunk (16 waves).
template <typename T>
__device__ __forceinline__ T block_inclusive_scan(T v, T* wave_tot, T* carry) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  if (lane == 63) wave_tot[wv] = v;
  __syncthreads();
  T add = *carry;
  for (int w = 0; w < wv; ++w) add += wave_tot[w];
  __syncthreads();
  if (tid == 1023) *carry = add + v;
  return add + v;
}

// The plan of mla_plan.h on one workgroup: prefix sums of the per-sequence
// costs in LDS, one binary search per part, a scan of the per-sequence touch
// counts.  Identical to the host mirror by construction (same integer math).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* seqlens, int batch, int rows, int num_parts,
                                                    int32_t* tile_md, int32_t* num_splits) {
  __shared__ int64_t prefix[kMaxPlanBatch + 1];
  __shared__ int64_t wave_tot64[16];
  __shared__ int64_t carry64;
  __shared__ int32_t wave_tot32[16];
  __shared__ int32_t carry32;
  const int tid = threadIdx.x;
  const int c = segment_cost(rows_per_block(rows));
  if (tid == 0) {
    prefix[0] = 0;
    carry64 = 0;
    carry32 = 0;
    num_splits[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < batch; base += 1024) {
    const int i = base + tid;
    const int64_t v = i < batch ? (int64_t)(c + seq_units(seqlens[i])) : 0;
    const int64_t incl = block_inclusive_scan<int64_t>(v, wave_tot64, &carry64);
    if (i < batch) prefix[i + 1] = incl;
    __syncthreads();
  }
  const int64_t T = plan_stride(prefix[batch], num_parts, c);
  for (int p = tid; p < num_parts; p += 1024)
    plan_part(prefix, seqlens, batch, c, T, p, tile_md + (int64_t)p * kTileMdInts);
  for (int base = 0; base < batch; base += 1024) {
    const int i = base + tid;
    const int32_t v = i < batch ? plan_touches(prefix, i, c, T) : 0;
    const int32_t incl = block_inclusive_scan<int32_t>(v, wave_tot32, &carry32);
    if (i < batch) num_splits[i + 1] = incl;
    __syncthreads();
  }
}

hipError_t launch_plan(const int32_t* seqlens, int batch, int rows, int num_parts, int32_t* tile_md,
                       int32_t* num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, seqlens, batch, rows, num_parts, tile_md,
                     num_splits);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_parts * a.row_blocks));
  const int rpb = rows_per_block(a.rows);
  if (rpb == 16)
    hipLaunchKernelGGL((decode_kernel<1>), grid, dim3(kThreads), 0, stream, a);
  else if (rpb == 32)
    hipLaunchKernelGGL((decode_kernel<2>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<4>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.batch, (unsigned)((a.rows + 3) / 4));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

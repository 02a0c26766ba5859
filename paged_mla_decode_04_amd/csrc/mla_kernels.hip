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
// LDS chunk tile (32 tokens): 9 x 4 blocks of 1 KB; block (r, q) holds tokens
// 8r..8r+7 x 16-byte column chunks 8q..8q+7 (columns 64q..64q+63), token a of
// the block at 128 a, its chunk c at slot (c % 8) ^ a ^ 2 (r & 1).  The swizzle
// keeps both the 16-byte K reads (16 tokens x one chunk per 16 lanes, two
// such groups per 512 bytes of banks) and the 8-byte transposing V reads
// (4 tokens x 2 chunks x 2 halves per 16 lanes) free of bank conflicts.
#include <utility>

#include "mla_merge.h"

namespace mla {


// ---------------------------------------------------------------------------
// Split-KV decode.
//
// One workgroup of 8 waves handles one row block (up to 64 query rows, NRT row
// tiles of 16) of one plan part, stepping through its keys 32 tokens (half a
// page) at a time.  Waves w and w + 4 share a SIMD; the roles are split so
// that each SIMD always has matrix work from one wave while the other waits:
//   score waves 0..3   wave i holds the queries of row tiles 2(i&1), 2(i&1)+1
//                      (32 rows) and computes S^T = K . Q^T for token tile
//                      i >> 1 (16 tokens) of a chunk: every 16-byte K read
//                      from LDS feeds two MFMAs.  It then masks, scales and
//                      exponentiates against the per-row reference max and
//                      writes P (bf16) to LDS already in the operand layout of
//                      the value product;
//   value waves 4..7   wave 4 + j owns output columns 128 j .. 128 j + 127 of
//                      all rows and accumulates O^T += V^T . P^T, reading V^T
//                      with the transposing LDS read.
// In step t the score waves work on chunk t + 1 while the value waves work on
// chunk t, the copy of chunk t + 2 lands and that of chunk t + 3 is issued,
// into four 36 KB chunk tiles; one workgroup barrier per step.
//
// Online softmax in the log2 domain: p = 2^(x - m) against a reference m per
// row that only moves when a chunk's max passes it by more than 2^16.  The
// score waves write P optimistically against the current reference together
// with their per-lane chunk maxima and a flag; when a flag is set (a
// segment's first chunk, and rarely later) every wave moves the reference of
// its rows at the start of the next step, the value waves rescale their
// accumulators and the score waves redo P from the scores they still hold,
// behind one extra barrier.  No cross-lane reduction is needed otherwise.
//
// Page bookkeeping runs four chunks ahead on the scalar unit: the sequence
// length and the block-table entry of a chunk are fetched a step before its
// copy is issued, so no dependent load sits on the copy path.
// ---------------------------------------------------------------------------

constexpr int kThreads = 512;
constexpr int kChunkBytes = kChunk * kD * 2;          // 36864
constexpr int kBuffers = 4;                           // chunk tiles in LDS
constexpr int kPOffset = kBuffers * kChunkBytes;      // P^T: [parity][row tile][lane] x 16 B
constexpr int kCmaxOffset = kPOffset + 2 * 4096;      // chunk maxima: [parity][token tile][lane group][row] f32
constexpr int kFlagOffset = kCmaxOffset + 2 * 2048;   // [parity][score wave] int
constexpr int kFinalOffset = kFlagOffset + 2 * 4 * 4; // [parity] segment totals (below)
constexpr int kFinalSum = 0, kFinalSumX = 128, kFinalRef = 256, kFinalFloats = 320;  // [2][64], [2][64], [64]
constexpr int kRingOffset = kFinalOffset + 2 * kFinalFloats * 4;  // 8 chunk descriptors x 16 B
constexpr int kSmemBytes = kRingOffset + 8 * 16;
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");


// The chunk tile's 36 blocks of 1 KB are copied by: score wave i the rope
// block of token octet i (block (i, 8)); value wave 4 + j the blocks
// (r, 2j + h), r = 0..3, h = 0..1 -- the columns it multiplies itself.
template <bool SCORE>
constexpr int copy_loads() { return SCORE ? 1 : 8; }

template <bool SCORE>
__device__ __forceinline__ bool issue_copy(const DecodeArgs& a, const Chunk& c, uint32_t tile, int wave, int lane) {
  if (!c.valid() || c.tok <= 0) return false;
  const __amdgpu_buffer_rsrc_t rsrc = chunk_rsrc(a, c);
  const uint32_t rb = (uint32_t)a.k_row_bytes;
  const int ta = lane >> 3, e = lane & 7;
#pragma unroll
  for (int k = 0; k < copy_loads<SCORE>(); ++k) {
    const int r = SCORE ? wave : (k >> 1);
    const int q = SCORE ? 8 : 2 * (wave - 4) + (k & 1);
    const int t = 8 * r + ta;
    const uint32_t voff = t < c.tok ? t * rb + 16u * (8 * q + (e ^ ta ^ (2 * (r & 1)))) : kOutOfRange;
    lds_dma16(rsrc, voff, tile + 1024u * (9 * r + q));
  }
  return true;
}

constexpr int kAheadK = 6;  // score k-steps whose K fragment is read ahead
constexpr int kRingAhead = 6;  // chunks the bookkeeping runs ahead of the values

// The decode loop of one role.  Both roles step through the same chunk
// descriptors and meet the same workgroup barriers in the same order (the
// rare fix-up barrier sits after the score product in the score waves and
// before the value product in the value waves): every condition around a
// barrier depends only on the descriptors or on flags read from LDS after a
// barrier.  Each role has its own copy of the loop so that the score state
// (queries) and the value state (accumulators) never occupy registers at the
// same time.  Within a step the score waves start their product at once and
// the value waves first issue the copy, so each SIMD's matrix unit has work
// while the other wave does its bookkeeping.
template <int NRT, bool SCORE>
__device__ __forceinline__ void decode_role(const DecodeArgs& a, const PartInfo& pi, lds_u8* const lds,
                                            const int wave, const int lane) {
  const int g = lane >> 4, r16 = lane & 15;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  lds_f32* const cmax = (lds_f32*)(lds + kCmaxOffset);
  lds_i32* const flags = (lds_i32*)(lds + kFlagOffset);
  lds_f32* const fin = (lds_f32*)(lds + kFinalOffset);
  lds_i32x4* const ring = (lds_i32x4*)(lds + kRingOffset);
  lds_u8* const plane = launder(lds + kPOffset + 16u * lane);
  const bool producer = wave == 4;  // a value wave: they wait for the score waves at every barrier

  // ---- score role: rows 16 (rp0 + rt) + r16, token tile tt of each chunk
  const int tt = (wave & 3) >> 1;
  const int rp0 = 2 * (wave & 1);
  const bool score_active = NRT == 4 || (wave & 1) == 0;
  const int ka = r16 & 7, kr = r16 >> 3;
  const uint32_t kx = (uint32_t)(g ^ ka ^ (2 * kr));
  const uint32_t k_lane = 9216u * (2 * tt + kr) + 128u * ka;
  bf16x8 qf[SCORE ? 2 : 1][kKSteps];
  f32x4 sc[2];
  float m_own[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f}, lsumx[2] = {0.f, 0.f};
  float psum[2] = {0.f, 0.f}, psumx[2] = {0.f, 0.f};
  int lim[2] = {0, 0};
  // ---- value role: columns 128 vj .. 128 vj + 127 of rows 16 rt + r16
  const int vj = wave & 3;
  const int va = 4 * (g & 1) + (r16 >> 2);
  const uint32_t vy = (uint32_t)(((r16 & 3) >> 1) ^ va ^ (2 * ((g >> 1) & 1)));
  const uint32_t v_lane = 9216u * (g >> 1) + 1024u * (2 * vj) + 128u * va + 8u * (r16 & 1);
  f32x4 o[SCORE ? 1 : NRT][8];
  float mref[NRT];
  if constexpr (!SCORE) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      mref[rt] = -INFINITY;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  bool seg_bad = false;
  int seg_slot = 0, seg_nsplit = 1;

  // Load the queries of the segment of chunk c and the visible-key limits of
  // the score rows.  Waits for the loads here, before the next copy is issued,
  // so that no later wait for them also waits for that copy.
  auto load_queries = [&](const Chunk& c) {
    if constexpr (SCORE) {
      const int n = clamp_len(a, load_len(a, c.seq));
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int row = pi.blk_row0 + 16 * (rp0 + rt) + r16;
        const bool ok = row < a.rows && rp0 + rt < NRT;
        const int rr = ok ? row : 0;
        const int qi = rr / a.h_q, h = rr - qi * a.h_q;
        lim[rt] = ok ? (a.causal ? n - (a.s_q - 1 - qi) : n) : 0;
        const uint16_t* qp = a.q + (int64_t)c.seq * a.q_sb + (int64_t)qi * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          const bf16x8 v = *(const bf16x8*)(qp + 32 * ks);
          qf[rt][ks] = ok ? v : bf16x8{};
        }
      }
      asm volatile("" ::"v"(qf[0][kKSteps - 1]), "v"(qf[1][kKSteps - 1]), "v"(qf[0][0]), "v"(qf[1][0]));
    }
  };

  // ---- prologue: wave 4 publishes chunks 0..4; copies of chunks 0, 1 and 2;
  // queries of the first segment (with one row tile, loaded during the walk)
  Cursor cur, nxt;  // producer: the next chunk to publish and the one after
  bool prod_first = false;
  if (producer) {
    cur.seq = pi.seq_begin;
    cur.chunk = 2 * pi.page_begin;
    cur.n = load_len(a, pi.seq_begin);
    cur.phys = load_phys(a, pi.seq_begin, pi.page_begin);
    cur.valid = true;
    prod_first = true;
#pragma unroll 1
    for (int k = 0; k < kRingAhead - 1; ++k) {
      nxt = next_chunk(a, cur, pi.seq_last, pi.page_end);
      const i32x4 d = pack_chunk(a, cur, nxt, prod_first);
      if (lane == 0) ring[k] = d;
      prod_first = !cur.valid || !nxt.valid || nxt.seq != cur.seq;
      cur = nxt;
    }
    nxt = next_chunk(a, cur, pi.seq_last, pi.page_end);
  }
  // the first segment's queries need only the part record: the score waves
  // load them while the producer walks (with one row tile; with more, the
  // registers they hold across the copies' address work spill)
  constexpr bool kEarlyQueries = SCORE && NRT == 1;
  if constexpr (kEarlyQueries) load_queries(Chunk{pi.seq_begin, 0, 0, 0, false, false, false});
  block_sync();
  Chunk D0 = unpack_chunk(i32x4{-1, 0, 0, -1});  // chunk t (values)
  Chunk D1 = unpack_chunk(ring[0]);              // chunk t + 1 (scores)
  Chunk D2 = unpack_chunk(ring[1]);              // chunk t + 2 (landing)
  Chunk D3 = unpack_chunk(ring[2]);              // chunk t + 3 (in flight)
  Chunk D4 = unpack_chunk(ring[3]);              // chunk t + 4 (copied this step)
  issue_copy<SCORE>(a, D1, lds_addr, wave, lane);
  issue_copy<SCORE>(a, D2, lds_addr + kChunkBytes, wave, lane);
  issue_copy<SCORE>(a, D3, lds_addr + 2 * kChunkBytes, wave, lane);
  if constexpr (SCORE && !kEarlyQueries) load_queries(D1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  block_sync();
  bool p_last = false;  // chunk t - 1 ended its segment (the values still have to close it)
  int p_seq = -1;
  bool iss_prev = false;  // this wave issued loads for chunk t + 3 (in the previous step)
  // value role: V^T operands of chunk t (read from its tile one step early, so
  // the tile is free for the next copy as soon as the scores are done with it)
  bf16x8 vcur[SCORE ? 1 : 8], vnext[SCORE ? 1 : 8];

  for (int t = -1;; ++t) {
    if (!D0.valid() && !D1.valid() && !p_last) break;
    const int par = t & 1;
    const bool v_has = D0.valid() && D0.tok > 0;
    // LDS reads whose latency hides behind the first work of the step:
    // chunk t's flags and the descriptor of chunk t + 5 (for the next step)
    const i32x4 fl = *(const lds_i32x4*)(flags + 4 * par);
    const i32x4 d5 = ring[(t + 5) & 7];
    // chunk t + 4 goes into the tile of chunk t, whose last reader (step t - 1) is done
    const uint32_t copy_tile = lds_addr + (uint32_t)((t + 4) & 3) * kChunkBytes;
    bool issued = false;

    if constexpr (SCORE) {
      // ---- chunk t + 1 starts a segment: its queries (the first ones were
      // loaded in the prologue)
      if (D1.valid() && D1.first && t >= 0) load_queries(D1);
      issued = issue_copy<SCORE>(a, D4, copy_tile, wave, lane);
      // the score chain (product, softmax, P) is the step's critical path: let
      // its instructions go first on the SIMD the value wave shares
      __builtin_amdgcn_s_setprio(1);
      // ---- scores of chunk t + 1: 32 rows x 16 tokens, two MFMAs per K read
      const bool s_has = score_active && D1.valid() && D1.tok > 0;
      f32x4 snew[2] = {};
      if (s_has) {
        lds_u8* const tile = lds + (uint32_t)((t + 1) & 3) * kChunkBytes;
        lds_u8* const kb0 = launder(tile + k_lane + 16u * kx);
        lds_u8* const kb1 = launder(tile + k_lane + 16u * (kx ^ 4u));
        f32x4 acc[2][2] = {};  // [row tile][k-step parity]: independent MFMA chains
        bf16x8 kf[kKSteps];
#pragma unroll
        for (int ks = 0; ks < kAheadK; ++ks) kf[ks] = *(const lds_bf16x8*)(((ks & 1) ? kb1 : kb0) + 1024u * (ks >> 1));
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + kAheadK < kKSteps)
            kf[ks + kAheadK] =
                *(const lds_bf16x8*)((((ks + kAheadK) & 1) ? kb1 : kb0) + 1024u * ((ks + kAheadK) >> 1));
          acc[0][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[0][ks], acc[0][ks & 1], 0, 0, 0);
          acc[1][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[1][ks], acc[1][ks & 1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        snew[0] = acc[0][0] + acc[0][1];
        snew[1] = acc[1][0] + acc[1][1];
      }
      // ---- chunk t's flags: move the reference max where a chunk max passed it
      if (v_has && uniform(fl[0] | fl[1] | fl[2] | fl[3])) {
        if (score_active) {
          const lds_f32* cm = cmax + par * 512 + r16;
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const int rw = 16 * (rp0 + rt);
            float m_new = m_own[rt];
#pragma unroll
            for (int gi = 0; gi < 8; ++gi)  // group gi = 4 * token tile + lane group, written by wave 2 tt + (row tile / 2)
              if (uniform(fl[2 * (gi >> 2) + (rp0 >> 1)])) m_new = fmaxf(m_new, cm[64 * gi + rw]);
            const float f = m_own[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_own[rt] - m_new);
            lsum[rt] *= f;
            lsumx[rt] *= f;
            m_own[rt] = m_new;
            const float mu = m_new == -INFINITY ? 0.f : m_new;
            bf16x4 pv;
            psum[rt] = 0.f;
            psumx[rt] = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float e = __builtin_amdgcn_exp2f(sc[rt][j] - mu);
              const __bf16 p = (__bf16)e;
              psum[rt] += (float)p;
              psumx[rt] += e;
              pv[j] = p;
            }
            *(lds_bf16x4*)(plane + par * 4096 + 1024u * (rp0 + rt) + 8u * tt) = pv;
          }
        }
        block_sync();  // ---- redone P visible (the value waves wait here before their product)
      }
      // ---- chunk t's probabilities are final: add their sums
      if (v_has) {
        lsum[0] += psum[0];
        lsum[1] += psum[1];
        lsumx[0] += psumx[0];
        lsumx[1] += psumx[1];
      }
      // ---- chunk t ended its segment: publish the row totals
      if (D0.valid() && D0.last && score_active) {
        lds_f32* fs = fin + par * kFinalFloats;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const float l = wave_sum16(lsum[rt]), lx = wave_sum16(lsumx[rt]);
          const int rw = 16 * (rp0 + rt) + r16;
          if (g == 0) {
            fs[kFinalSum + 64 * tt + rw] = l;
            fs[kFinalSumX + 64 * tt + rw] = lx;
            if (tt == 0) fs[kFinalRef + rw] = m_own[rt];
          }
        }
      }
      // ---- chunk t + 1 starts a segment: fresh softmax state
      if (D1.valid() && D1.first) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          m_own[rt] = -INFINITY;
          lsum[rt] = 0.f;
          lsumx[rt] = 0.f;
        }
      }
      if (s_has) {
        // ---- mask, scale, optimistic probabilities of chunk t + 1;
        // token 32 chunk + 16 tt + 4 g + j
        sc[0] = snew[0];
        sc[1] = snew[1];
        const int base_tok = kChunk * D1.chunk + 16 * tt + 4 * g;
        const int par1 = (t + 1) & 1;
        bool over = false;
        float cmx[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int vis = lim[rt] - base_tok;
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = j < vis ? sc[rt][j] * a.scale_log2 : -INFINITY;
            sc[rt][j] = x;
            mx = fmaxf(mx, x);
          }
          over |= mx > m_own[rt] + kRescaleSlack;
          cmx[rt] = mx;
          const float mu = m_own[rt] == -INFINITY ? 0.f : m_own[rt];
          bf16x4 pv;
          psum[rt] = 0.f;
          psumx[rt] = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float e = __builtin_amdgcn_exp2f(sc[rt][j] - mu);
            const __bf16 p = (__bf16)e;
            psum[rt] += (float)p;
            psumx[rt] += e;
            pv[j] = p;
          }
          *(lds_bf16x4*)(plane + par1 * 4096 + 1024u * (rp0 + rt) + 8u * tt) = pv;
        }
        const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
        // the chunk maxima are only read when some wave is flagged, and then
        // only those of the flagged waves
        if (wave_over) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) cmax[par1 * 512 + 64 * (4 * tt + g) + 16 * (rp0 + rt) + r16] = cmx[rt];
        }
        if (lane == 0) flags[4 * par1 + wave] = wave_over ? 1 : 0;
      } else if (lane == 0) {
        flags[4 * ((t + 1) & 1) + wave] = 0;
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
      // ---- copy chunk t + 4, first thing in the step -- unless a segment
      // closes here, whose stores go first
      if (!p_last) issued = issue_copy<SCORE>(a, D4, copy_tile, wave, lane);
      // ---- close the segment that ended with chunk t - 1
      if (p_last) {
        const lds_f32* fs = fin + ((t - 1) & 1) * kFinalFloats + r16;
        const bool final_out = seg_nsplit == 1;
        int row0 = pi.blk_row0 + r16;  // opaque: keeps the address arithmetic in this block
        asm volatile("" : "+v"(row0));
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const float L0 = fs[kFinalSum + 16 * rt] + fs[kFinalSum + 64 + 16 * rt];
          const float LE = fs[kFinalSumX + 16 * rt] + fs[kFinalSumX + 64 + 16 * rt];
          float inv = L0 > 0.f ? 1.f / L0 : 0.f;
          float lse = LE > 0.f ? (fs[kFinalRef + 16 * rt] + __builtin_amdgcn_logf(LE)) * kLn2 : -INFINITY;
          if (seg_bad) {
            inv = __builtin_nanf("");
            lse = __builtin_nanf("");
          }
          const int row = row0 + 16 * rt;
          if (row < a.rows) {
            const int qi = row / a.h_q, h = row - qi * a.h_q;
            const int col0 = 128 * vj + 4 * g;
            if (final_out) {
              uint16_t* op = a.out + (int64_t)p_seq * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + col0;
#pragma unroll
              for (int ct = 0; ct < 8; ++ct) {
                const f32x4 v = o[rt][ct] * inv;
                *(bf16x4*)(op + 16 * ct) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
              }
              if (vj == 0 && g == 0)
                a.lse[(int64_t)p_seq * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = lse;
            } else {
              float* pp = a.part_o + ((int64_t)seg_slot * a.rows + row) * kDv + col0;
#pragma unroll
              for (int ct = 0; ct < 8; ++ct) *(f32x4*)(pp + 16 * ct) = o[rt][ct] * inv;
              if (vj == 0 && g == 0) a.part_lse[(int64_t)seg_slot * a.rows + row] = lse;
            }
          }
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
          mref[rt] = -INFINITY;
        }
        issued = issue_copy<SCORE>(a, D4, copy_tile, wave, lane);
      }
      if (D0.valid() && D0.first) {  // the values enter a new segment
        const int split = D0.seq == pi.seq_begin ? pi.split_first : 0;
        int s0, nsplit;
        segment_splits<false>(a, D0.seq, nullptr, s0, nsplit);
        seg_slot = s0 + split;
        seg_nsplit = nsplit;
        seg_bad = false;
      }
      if (D0.valid()) seg_bad |= D0.bad;
      // ---- wave 4: publish chunk t + 5 (read from the ring from step t + 1 on)
      if (producer) {
        const i32x4 d = pack_chunk(a, cur, nxt, prod_first);
        if (lane == 0) ring[(t + kRingAhead) & 7] = d;
        prod_first = !cur.valid || !nxt.valid || nxt.seq != cur.seq;
        cur = nxt;
        nxt = next_chunk(a, cur, pi.seq_last, pi.page_end);
      }
      // ---- chunk t's flags: rescale what the rows whose reference moved
      // have accumulated, then wait for the redone P
      if (v_has && uniform(fl[0] | fl[1] | fl[2] | fl[3])) {
        const lds_f32* cm = cmax + par * 512 + r16;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          float m_new = mref[rt];
#pragma unroll
          for (int gi = 0; gi < 8; ++gi)
            if (uniform(fl[2 * (gi >> 2) + (rt >> 1)])) m_new = fmaxf(m_new, cm[64 * gi + 16 * rt]);
          const float f = mref[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref[rt] - m_new);
          mref[rt] = m_new;
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) o[rt][ct] *= f;
        }
        block_sync();  // ---- redone P visible
      }
      // ---- V^T operands of chunk t + 1 from its tile (the scores read it now too)
      if (D1.valid() && D1.tok > 0) {
        lds_u8* const tile = lds + (uint32_t)((t + 1) & 3) * kChunkBytes;
        lds_u8* vb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) vb[u] = launder(tile + v_lane + 16u * ((2u * u) ^ vy));
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct & 3] + 1024u * (ct >> 2)));
          const bf16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct & 3] + 1024u * (ct >> 2) + 18432u));
          vnext[ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      if (v_has) {
        // ---- O^T[columns 128 vj ..] += V^T . P^T for chunk t
        bf16x8 pf[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) pf[rt] = *(const lds_bf16x8*)(plane + par * 4096 + 1024u * rt);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur[ct], pf[rt], o[rt][ct], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) vcur[ct] = vnext[ct];
      p_seq = D0.seq;
    }

    // ---- end of step: this wave's share of chunk t + 2 has landed (the copies
    // of chunks t + 3 and t + 4, issued after it, may still be in flight) and
    // all LDS reads of the step have returned
    static_assert(copy_loads<true>() == 1 && copy_loads<false>() == 8, "vmcnt below");
    const int pending = (iss_prev ? 1 : 0) + (issued ? 1 : 0);
    if (pending == 2) {
      if constexpr (SCORE)
        asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else if (pending == 1) {
      if constexpr (SCORE)
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    block_sync();
    iss_prev = issued;
    p_last = D0.valid() && D0.last;
    D0 = D1;
    D1 = D2;
    D2 = D3;
    D3 = D4;
    D4 = unpack_chunk(d5);
  }
}

template <int NRT>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  PartInfo pi;
  int unused_len[kPlanBlocks];
  if (!load_part<false>(a, NRT * 16, pi, nullptr, unused_len)) return;
  lds_u8* const lds = (lds_u8*)smem;
  if (wave < 4)
    decode_role<NRT, true>(a, pi, lds, wave, lane);
  else
    decode_role<NRT, false>(a, pi, lds, wave, lane);
}

constexpr int kMergeUnroll = 8;  // splits whose loads are in flight together

// Merge the partials of every sequence that more than one part touched:
// L = log(sum_i exp(lse_i)), out = sum_i exp(lse_i - L) * O_i (empty partials,
// lse = -inf, weigh nothing; all empty gives out = 0, lse = -inf; a NaN lse
// gives NaN).  One wave per (sequence, row), in one online pass over the
// splits (OnlineLse), eight splits' loads at a time.
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int b = blockIdx.x;
  const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int base = a.num_splits[b];
  const int ns = a.num_splits[b + 1] - base;
  if (ns <= 1 || r >= a.rows) return;
  const float* lse_p = a.part_lse + (int64_t)base * a.rows + r;
  const f32x4* src0 = (const f32x4*)(a.part_o + ((int64_t)base * a.rows + r) * kDv + 8 * lane);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  OnlineLse ol;
  for (int i0 = 0; i0 < ns; i0 += kMergeUnroll) {
    float x[kMergeUnroll];
    f32x4 v0[kMergeUnroll], v1[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (i0 + u < ns) {
        x[u] = lse_p[(int64_t)(i0 + u) * a.rows];
        const f32x4* src = src0 + (int64_t)(i0 + u) * a.rows * (kDv / 4);
        v0[u] = src[0];
        v1[u] = src[1];
      } else {
        x[u] = -INFINITY;
        v0[u] = v1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const float f = ol.fold(x);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= f;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += x[u] * v0[u][j];
        acc[4 + j] += x[u] * v1[u][j];
      }
    }
  }
  const float L = ol.lse();
  const float inv = ol.nan ? __builtin_nanf("") : (ol.sum > 0.f ? 1.f / ol.sum : 0.f);
  const int qi = r / a.h_q, h = r - qi * a.h_q;
  uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + 8 * lane;
  bf16x8 w;
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = (__bf16)(acc[j] * inv);
  *(bf16x8*)op = w;
  if (lane == 0) a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = L;
}

// Few splits per sequence: one workgroup per (sequence, 32-row tile, column
// half).
__global__ __launch_bounds__(256) void combine_tiles_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[32 * kMergeTileStride];
  const int b = blockIdx.x, rt = blockIdx.y, hf = blockIdx.z;
  const int base = a.num_splits[b];
  const int ns = a.num_splits[b + 1] - base;
  if (ns <= 1) return;
  merge_row_tile(a, b, rt, hf, base, ns, (lds_u16*)tile);
}

// Many splits per sequence (a few long sequences over many parts): workgroup
// (hc, rt, b) merges half hc & 1 (16 columns) of column tile hc >> 1 of row
// tile rt (32 rows) of sequence b; a half is one 1 KB block of a partial tile
// (element pair gp of the accumulator layout).  Wave v folds splits v, v + 4,
// ... online, eight splits' loads at a time; the four waves' running sums are
// then combined through LDS and written as 32 rows of 32 contiguous bytes,
// lse by half 0.  Half tiles spread a long sequence's bytes over twice as
// many compute units as whole tiles would.  The sequence is the grid's
// slowest index, so a sequence's workgroups are dispatched together: with
// more workgroups than fit at once, a long sequence's (the ones that run
// longest) then do not wait behind other sequences' tiles.
__global__ __launch_bounds__(256) void combine_splits_kernel(DecodeArgs a) {
  __shared__ float red_m[4][64], red_s[4][64];
  __shared__ int red_nan[4][64];
  __shared__ float red[4][64][8];
  const int hc = blockIdx.x, rt = blockIdx.y, b = blockIdx.z;
  const int ct = hc >> 1, gp = hc & 1;
  const int v = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int base = a.num_splits[b];
  const int ns = a.num_splits[b + 1] - base;
  if (ns <= 1) return;
  const int t = threadIdx.x;
  {
    const int j = lane & 31;
    const bool ok = 32 * rt + j < a.rows;
    const float* lse_p = a.part_lse + (int64_t)base * a.rows + 32 * rt + j;
    const float* scale_p = a.part_scale + (int64_t)base * a.rows + 32 * rt + j;
    const uint8_t* src0 = (const uint8_t*)a.part_o + (int64_t)base * partial_slot_bytes(a.rows) +
                          (int64_t)rt * kPartialTileBytes + 2048 * ct + 1024 * gp + 16 * lane;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    OnlineLse ol;
    for (int i0 = v; i0 < ns; i0 += 4 * kSplitMergeBatch) {
      float x[kSplitMergeBatch], sc[kSplitMergeBatch];
      f16x8 d[kSplitMergeBatch];
#pragma unroll
      for (int u = 0; u < kSplitMergeBatch; ++u) {
        const int i = i0 + 4 * u;
        const bool in = i < ns;
        x[u] = (in && ok) ? lse_p[(int64_t)i * a.rows] : -INFINITY;
        sc[u] = (in && ok) ? scale_p[(int64_t)i * a.rows] : 0.f;
        const uint8_t* src = src0 + (int64_t)(in ? i : 0) * partial_slot_bytes(a.rows);
        d[u] = in ? *(const f16x8*)src : f16x8{};
      }
      const float f = ol.fold(x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= f;
#pragma unroll
      for (int u = 0; u < kSplitMergeBatch; ++u) {
        const float wgt = x[u] * sc[u];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)d[u][e];
      }
    }
    red_m[v][lane] = ol.m;
    red_s[v][lane] = ol.sum;
    red_nan[v][lane] = ol.nan;
#pragma unroll
    for (int e = 0; e < 8; ++e) red[v][lane][e] = acc[e];
  }
  __syncthreads();
  {
    // row j = t / 8, output columns 2 c, 2 c + 1 of the half; column i of the
    // half is accumulator 4 (i / 8) + i % 4 of lane j + 32 ((i / 4) % 2)
    const int j = t >> 3, c = t & 7;
    const int row = 32 * rt + j;
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      M = fmaxf(M, red_m[w][j]);
      nan |= red_nan[w][j] != 0;
    }
    float wv[4], S = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wv[w] = (M == -INFINITY || red_m[w][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((red_m[w][j] - M) * kLog2e);
      S += wv[w] * red_s[w][j];
    }
    const float inv = nan ? __builtin_nanf("") : (S > 0.f ? 1.f / S : 0.f);
    const float L = nan ? __builtin_nanf("") : (M == -INFINITY ? -INFINITY : M + __builtin_amdgcn_logf(S) * kLn2);
    bf16x2 o2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * c + e;
      const int ln = j + 32 * ((i >> 2) & 1), r = 4 * (i >> 3) + (i & 3);
      const float val = wv[0] * red[0][ln][r] + wv[1] * red[1][ln][r] + wv[2] * red[2][ln][r] + wv[3] * red[3][ln][r];
      o2[e] = (__bf16)(val * inv);
    }
    if (row < a.rows) {
      const int qi = row / a.h_q, hh = row - qi * a.h_q;
      uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)hh * a.o_sh + 32 * ct + 16 * gp + 2 * c;
      *(bf16x2*)op = o2;
      if (hc == 0 && c == 0) a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)hh * a.l_sh] = L;
    }
  }
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
    plan_part(prefix, batch, c, T, p, tile_md + (int64_t)p * kTileMdInts);
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
  if (rpb == kRowsPerWorkgroup || a.kv8) return launch_decode_wide(a, stream);
  if (rpb == 16)
    hipLaunchKernelGGL((decode_kernel<1>), grid, dim3(kThreads), 0, stream, a);
  else if (rpb == 32)
    hipLaunchKernelGGL((decode_kernel<2>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<4>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  if (rows_per_block(a.rows) == kRowsPerWorkgroup || a.kv8) {
    if (many_splits(a.num_parts, a.batch)) {
      const dim3 grid((unsigned)(kDv / 16), (unsigned)((a.rows + 31) / 32), (unsigned)a.batch);
      hipLaunchKernelGGL(combine_splits_kernel, grid, dim3(256), 0, stream, a);
    } else {
      const dim3 grid((unsigned)a.batch, (unsigned)((a.rows + 31) / 32), 2u);
      hipLaunchKernelGGL(combine_tiles_kernel, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.batch, (unsigned)((a.rows + 3) / 4));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

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
// Design on gfx950 (256 CUs, 160 KB LDS, 64-wide waves, bf16 MFMA):
//   * one workgroup (4 waves) per CU processes one plan part: a contiguous
//     run of 64-token pages, possibly spanning several sequences;
//   * a page (64 x 576 bf16 = 72 KB) is copied HBM -> LDS with 16-byte
//     buffer loads that write LDS directly (no VGPR staging), double
//     buffered; all 4 waves issue the copies;
//   * up to 4 compute waves own 16 or 32 query rows each (a workgroup holds
//     at most 128 rows, so every page is read once for 128 heads); the query
//     block stays in registers as MFMA operands and the fp32 output
//     accumulator (up to 32 x 512 per wave) in the accumulation registers;
//   * scores are computed transposed, S^T = K . Q^T, on 16x16x32 bf16 MFMA,
//     so every lane holds whole query rows: row max / row sum need only two
//     cross-lane steps;
//   * P . V is computed as O^T = V^T . P^T: P^T comes straight from the score
//     registers (no data movement) and V^T from LDS with the gfx950
//     transposing read ds_read_b64_tr_b16 (4 consecutive tokens per lane);
//   * online softmax in the log2 domain.  The reference max only moves when a
//     row's score exceeds it by more than 2^16; then (rarely) the wave flushes
//     its unscaled accumulator into a carry in global scratch instead of
//     rescaling it in registers, so no vector ALU op touches the accumulator
//     inside the page loop;
//   * a part that covers only a piece of a sequence writes an fp32 partial
//     (O / l, lse); the merge kernel combines them by lse (Flash-Decoding, as
//     the Hacker News discussion of the FlashMLA release describes it).
//
// LDS page tile: 9 x 8 blocks of 1 KB; block (r, q) holds tokens 8r..8r+7 x
// 16-byte chunks 8q..8q+7, token a of the block at 128 a, its chunk c at slot
// (c % 8) ^ a ^ (r & 1).  The swizzle keeps both the 16-byte K reads (16
// tokens x one chunk) and the 8-byte transposing V reads (4 tokens x 2 chunks
// x 2 halves per 16 lanes) free of bank conflicts.
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
constexpr int kThreads = 256;
constexpr int kKSteps = kD / 32;          // 18 MFMA k-steps of 32 for the scores
constexpr int kColTiles = kDv / 16;       // 32 output column tiles of 16
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

// Register-class hints (emit no instructions): the output accumulator lives
// in the accumulation registers, scores in ordinary VGPRs, so that the query
// fragments, scores and accumulator fit one wave's 512 registers.
__device__ __forceinline__ void pin_acc(f32x4& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void pin_vgpr(f32x4& x) { asm volatile("" : "+v"(x)); }

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

// Nine 16-byte LDS-direct loads: chunk octets 0..8 of one token octet.  The
// byte step between octets travels in the VGPR offset: the instruction's
// immediate offset would move the LDS destination as well.
template <int... Q>
__device__ __forceinline__ void copy_row_octet(__amdgpu_buffer_rsrc_t rsrc, uint8_t* dst, uint32_t voff,
                                               std::integer_sequence<int, Q...>) {
  (__builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * Q), 16, voff + 128u * Q, 0, 0, 0),
   ...);
}

// Copy one page's used rows into an LDS tile.  Wave w copies token octets 2w
// and 2w+1 (18 x 1 KB).  Rows at or past `tokens` and pages outside the pool
// read as zeros through the buffer range check, so no byte outside the cache
// is touched and masked rows never carry stale NaNs.
__device__ __forceinline__ void copy_page(const DecodeArgs& a, int phys, bool valid, int tokens,
                                          uint8_t* tile, int wave, int lane) {
  const uint8_t* base = a.k + (valid ? (int64_t)phys * a.k_block_bytes : 0);
  const int32_t records = valid ? (int32_t)(64 * a.k_row_bytes) : 0;
  __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, records, kBufferFlags);
  const int ta = lane >> 3, e = lane & 7;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int r = 2 * wave + rr;
    const int t = 8 * r + ta;
    const uint32_t voff = (t < tokens)
                              ? (uint32_t)(t * a.k_row_bytes + 16 * (e ^ ta ^ (r & 1)))
                              : kOutOfRange;
    copy_row_octet(rsrc, tile + 1024 * 9 * r, voff, std::make_integer_sequence<int, 9>{});
  }
}

// Per-wave state.  A compute wave owns 16 query rows for the scores and the
// softmax (lane row l % 16), and one column block of the output accumulator
// for all the workgroup's rows: NWC row tiles x (32 / NWC) column tiles of
// 16 x 16, always 128 accumulation registers.
template <int NWC>
struct WaveState {
  static constexpr int kCT = kColTiles / NWC;  // column tiles of this wave's block
  bf16x8 qf[kKSteps];       // Q^T operand fragments of the wave's 16 rows
  f32x4 o[kCT][NWC];        // O^T accumulators: [column tile][row tile]
  float m, l, le;           // own row: reference max (log2 units), sums of rounded /
                            // unrounded probabilities
  float cm, cl, cle;        // own row: the carry's reference and sums
  bool carry;               // workgroup-uniform: the carry holds a flushed accumulator
};

// Fold the accumulator into the carry: carry = carry * fc[row] + O (O unscaled),
// then O = 0.  The accumulator is only stored (from the accumulation registers),
// never operated on by vector ALU instructions, so the page loop keeps it in
// AGPRs; the dump is read back as fresh values.
template <int NWC>
__device__ __forceinline__ void fold_into_carry(WaveState<NWC>& st, float* carry, float* dump, int lane,
                                                const lds_f32* fc) {
  constexpr int kCT = WaveState<NWC>::kCT;
  constexpr int kStride = kCT * 16;
  const int g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < NWC; ++rt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
      *(f32x4*)(dump + (16 * rt + (lane & 15)) * kStride + 16 * ct + 4 * g) = st.o[ct][rt];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int rt = 0; rt < NWC; ++rt) {
    const float f = st.carry ? fc[16 * rt + (lane & 15)] : 0.f;
#pragma unroll 2
    for (int ct = 0; ct < kCT; ++ct) {
      float* cp = carry + (16 * rt + (lane & 15)) * kStride + 16 * ct + 4 * g;
      float* dp = dump + (16 * rt + (lane & 15)) * kStride + 16 * ct + 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d = __hip_atomic_load(dp + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float c = st.carry ? __hip_atomic_load(cp + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
        __hip_atomic_store(cp + j, c * f + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      st.o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      pin_acc(st.o[ct][rt]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// LDS fragments are fetched a fixed number of steps ahead into explicit
// register buffers, and consecutive MFMAs accumulate into different tiles, so
// neither LDS latency nor the MFMA dependency chain is exposed; scheduling
// barriers pin that order.
constexpr int kAheadK = 2;  // score k-steps (4 fragments each)
constexpr int kAheadV = 3;  // output column tiles (one transposed fragment each)

// LDS regions next to the two page tiles.
constexpr int kPFragOffset = 2 * kPageBytes;                   // P^T fragments [row tile][half][lane]
constexpr int kStatsOffset = kPFragOffset + 4 * 2 * 64 * 16;   // fc / wo / wc [64 rows], flags[4]
constexpr int kSmemBytes = kStatsOffset + 3 * 64 * 4 + 16;

struct Lds {
  lds_u8* base;
  __device__ lds_bf16x8* pfrag(int rt, int half) const {
    return (lds_bf16x8*)(base + kPFragOffset + (rt * 2 + half) * 1024);
  }
  __device__ lds_f32* fc() const { return (lds_f32*)(base + kStatsOffset); }
  __device__ lds_f32* wo() const { return (lds_f32*)(base + kStatsOffset + 256); }
  __device__ lds_f32* wc() const { return (lds_f32*)(base + kStatsOffset + 512); }
  __device__ lds_i32* flags() const { return (lds_i32*)(base + kStatsOffset + 768); }
};

// One 64-token page for compute wave `wave`.  Scores and softmax for the
// wave's own 16 rows; P^T fragments go through LDS to every compute wave;
// each wave then adds V^T . P^T into its column block for all the rows.
// `vis` is the own row's visible-token count relative to the page start.
// Contains one workgroup barrier that the non-computing waves match with
// page_barrier_for_idle().
template <int NWC>
__device__ __forceinline__ void compute_page(const DecodeArgs& a, WaveState<NWC>& st, const Lds& L, int wave,
                                             int lane, int vis, lds_u8* kb0, lds_u8* kb1, lds_u8* const* vb,
                                             float* carry, float* dump) {
  constexpr int kCT = WaveState<NWC>::kCT;
  const int g = lane >> 4;
  // ---- scores of the own 16 rows: 4 token tiles, 18 k-steps
  f32x4 s[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 kf[kKSteps][4];
  auto load_k = [&](int ks) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      kf[ks][tt] = *(const lds_bf16x8*)(((ks & 1) ? kb1 : kb0) + 18432u * tt + 1024u * (ks >> 1));
  };
#pragma unroll
  for (int ks = 0; ks < kAheadK; ++ks) load_k(ks);
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    if (ks + kAheadK < kKSteps) load_k(ks + kAheadK);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][tt], st.qf[ks], s[tt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) pin_vgpr(s[tt]);

  // ---- mask (token 16 tt + 4 g + j visible iff < vis), scale, row max
  const int lim = vis - 4 * g;
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = (16 * tt + j < lim) ? s[tt][j] * a.scale_log2 : -INFINITY;
      s[tt][j] = x;
      mx = fmaxf(mx, x);
    }
  mx = wave_max16(mx);
  // The reference max is set on the row's first visible key and moved only when
  // a finite reference is exceeded by more than the slack; then the whole
  // workgroup folds its accumulator into the carry (below).
  const bool over = (st.m != -INFINITY) && (mx > st.m + kRescaleSlack);
  const float fc = st.carry ? __builtin_amdgcn_exp2f(st.cm - st.m) : 0.f;  // carry factor at the old reference
  const float m_new = over ? fmaxf(st.m, mx) : (st.m == -INFINITY ? mx : st.m);
  // probabilities (bf16 P^T fragments per 32-token half) and their sums
  const float mu = (m_new == -INFINITY) ? 0.f : m_new;
  bf16x8 pf[2];
  float sum = 0.f, sum_exact = 0.f;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(s[tt][j] - mu);
      const __bf16 p = (__bf16)e;
      sum += (float)p;
      sum_exact += e;
      pf[tt >> 1][4 * (tt & 1) + j] = p;
    }
  sum = wave_sum16(sum);
  sum_exact = wave_sum16(sum_exact);
  L.pfrag(wave, 0)[lane] = pf[0];
  L.pfrag(wave, 1)[lane] = pf[1];
  if (g == 0) L.fc()[16 * wave + lane] = fc;
  const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
  if (lane == 0) L.flags()[wave] = wave_over ? 1 : 0;
  block_sync();

  bool flush = false;
#pragma unroll
  for (int w = 0; w < NWC; ++w) flush |= L.flags()[w] != 0;
  if (flush) {  // rare: fold everything accumulated so far into the carry
    fold_into_carry<NWC>(st, carry, dump, lane, L.fc());
    st.cl = st.cl * fc + st.l;
    st.cle = st.cle * fc + st.le;
    st.cm = st.m;
    st.l = sum;
    st.le = sum_exact;
    st.carry = true;
  } else {
    st.l += sum;
    st.le += sum_exact;
  }
  st.m = m_new;

  // ---- O^T[column block] += V^T . P^T over both halves, all row tiles
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8 pr[NWC];
#pragma unroll
    for (int rt = 0; rt < NWC; ++rt) pr[rt] = L.pfrag(rt, half)[lane];
    bf16x8 vf[kCT];
    auto load_v = [&](int ct) {
      lds_u8* vp = vb[ct & 3] + 9216u * (4 * half) + 1024u * (ct >> 2);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vp);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 2 * 9216u));
      vf[ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
#pragma unroll
    for (int ct = 0; ct < kAheadV && ct < kCT; ++ct) load_v(ct);
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      if (ct + kAheadV < kCT) load_v(ct + kAheadV);
#pragma unroll
      for (int rt = 0; rt < NWC; ++rt) {
        st.o[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct], pr[rt], st.o[ct][rt], 0, 0, 0);
        pin_acc(st.o[ct][rt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Segment epilogue, in two steps around a workgroup barrier (which the idle
// waves match): each row's owner turns its statistics (with the carry, if the
// workgroup flushed) into output weights and the lse; then every compute wave
// writes its column block of every row, as bf16 output or fp32 partial.
template <int NWC>
__device__ __forceinline__ void publish_row_weights(const DecodeArgs& a, const WaveState<NWC>& st, const Lds& L,
                                                    int wave, int lane, int row, int b, bool bad, bool final_out,
                                                    int slot) {
  float M = st.m, fo = 1.f, fc = 0.f;
  if (st.carry) {
    M = fmaxf(st.cm, st.m);
    fo = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - M);
    fc = st.cm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.cm - M);
  }
  const float Lr = st.l * fo + st.cl * fc;
  const float LE = st.le * fo + st.cle * fc;
  float inv = Lr > 0.f ? 1.f / Lr : 0.f;
  float lse = LE > 0.f ? (M + __builtin_amdgcn_logf(LE)) * kLn2 : -INFINITY;
  if (bad) {
    inv = __builtin_nanf("");
    lse = __builtin_nanf("");
  }
  if ((lane >> 4) == 0) {
    L.wo()[16 * wave + lane] = fo * inv;
    L.wc()[16 * wave + lane] = fc * inv;
    if (row < a.rows) {
      const int qi = row / a.h_q, h = row - qi * a.h_q;
      if (final_out)
        a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = lse;
      else
        a.part_lse[(int64_t)slot * a.rows + row] = lse;
    }
  }
}

template <int NWC>
__device__ __forceinline__ void write_block(const DecodeArgs& a, const WaveState<NWC>& st, const Lds& L,
                                            const float* carry, int wave, int lane, int blk_row0, int b,
                                            bool final_out, int slot) {
  constexpr int kCT = WaveState<NWC>::kCT;
  constexpr int kStride = kCT * 16;
  const int g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < NWC; ++rt) {
    const int r = blk_row0 + 16 * rt + (lane & 15);
    const float wo = L.wo()[16 * rt + (lane & 15)];
    const float wc = L.wc()[16 * rt + (lane & 15)];
    const bool ok = r < a.rows;
    const int rr = ok ? r : 0;
    const int qi = rr / a.h_q, h = rr - qi * a.h_q;
    const int col0 = wave * kCT * 16 + 4 * g;
    const float* cp = carry + (16 * rt + (lane & 15)) * kStride + 4 * g;
    if (final_out) {
      uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + col0;
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        f32x4 v = st.o[ct][rt] * wo;
        if (st.carry) v += *(const f32x4*)(cp + 16 * ct) * wc;
        const bf16x4 w = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        if (ok) *(bf16x4*)(op + 16 * ct) = w;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      float* pp = a.part_o + ((int64_t)slot * a.rows + rr) * kDv + col0;
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        f32x4 v = st.o[ct][rt] * wo;
        if (st.carry) v += *(const f32x4*)(cp + 16 * ct) * wc;
        if (ok) *(f32x4*)(pp + 16 * ct) = v;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// NWC compute waves (16 rows each for the scores, one column block each for
// the output); all 4 waves copy pages.
template <int NWC>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  constexpr int kBlockRows = NWC * 16;
  constexpr int kCT = WaveState<NWC>::kCT;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run
  // of parts so neighbouring pieces of one sequence share that XCD's L2.
  const int G = gridDim.x, hw = blockIdx.x;
  const int xcd = hw & 7, pos = hw >> 3;
  const int logical = xcd * (G >> 3) + min(xcd, G & 7) + pos;
  const int part = logical / a.row_blocks;
  const int mblock = logical - part * a.row_blocks;

  const int32_t* md = a.tile_md + (int64_t)part * kTileMdInts;
  const int seq_begin = uniform(md[0]);
  if (seq_begin >= a.batch) return;
  const int page_begin = uniform(md[1]);
  const int seq_last = uniform(md[2]);
  const int page_end = uniform(md[3]);
  const int split_first = uniform(md[4]);

  // per-lane LDS offsets (see the tile layout above)
  const int kt = lane & 15;
  const int ka = kt & 7, kr = kt >> 3;
  const uint32_t kx = (uint32_t)(g ^ ka ^ (kr & 1));
  const uint32_t kb_lane = 9216u * kr + 128u * ka;
  const int vs = lane & 15;
  const int va = 4 * (g & 1) + (vs >> 2);
  const int vR = (g >> 1) & 1;
  const uint32_t vy = (uint32_t)(((vs & 3) >> 1) ^ va ^ vR);
  // this wave's column block starts at column tile wave * kCT (a multiple of 4)
  const uint32_t vb_lane = 9216u * (g >> 1) + 128u * va + 8u * (vs & 1) + 1024u * (wave * kCT / 4);

  const bool computes = wave < NWC;
  const int blk_row0 = mblock * kBlockRows;
  const int own_row = blk_row0 + 16 * wave + (lane & 15);
  // this wave's flush scratch: carry, then dump, 16 * NWC rows x its columns
  float* carry = a.flush + ((int64_t)hw * 4 + wave) * (2 * 16 * kDv);
  float* dump = carry + 16 * kDv;
  const Lds L{(lds_u8*)smem};
  WaveState<NWC> st;

  for (int b = seq_begin; b <= seq_last; ++b) {
    int n = uniform(a.seqlens[b]);
    n = n < 0 ? 0 : n;
    const int cap = a.max_blocks * 64;
    n = n > cap ? cap : n;
    const int units = seq_units(n);
    const int pb = (b == seq_begin) ? page_begin : 0;
    const int pe = (b == seq_last) ? page_end : units;
    const int split = (b == seq_begin) ? split_first : 0;
    const int nsplit = uniform(a.num_splits[b + 1] - a.num_splits[b]);
    const int slot = uniform(a.num_splits[b]) + split;
    const int32_t* table = a.block_table + (int64_t)b * a.bt_stride;

    if (computes) {
      const bool ok = own_row < a.rows;
      const int rr = ok ? own_row : 0;
      const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)(rr / a.h_q) * a.q_ss +
                           (int64_t)(rr % a.h_q) * a.q_sh + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        bf16x8 v = *(const bf16x8*)(qp + 32 * ks);
        if (!ok) v = bf16x8{};
        st.qf[ks] = v;
      }
      st.m = -INFINITY;
      st.l = 0.f;
      st.le = 0.f;
      st.cm = -INFINITY;
      st.cl = 0.f;
      st.cle = 0.f;
      st.carry = false;
#pragma unroll
      for (int rt = 0; rt < NWC; ++rt)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          st.o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          pin_acc(st.o[ct][rt]);
        }
    }
    // visible keys of the own row: n, or n - (s_q - 1 - i) for query token i
    const int vis_row = a.causal ? n - (a.s_q - 1 - own_row / a.h_q) : n;
    bool bad = false;
    // page p has tokens [64 p, min(64 p + 64, n)); pages with none are skipped
    auto page_tokens = [&](int p) { int t = n - 64 * p; return t > 64 ? 64 : t; };
    auto page_phys = [&](int p) { return uniform(table[p]); };

    int buf = 0;
    bool pending = false;
    if (pb < pe && page_tokens(pb) > 0) {
      const int phys = page_phys(pb);
      const bool valid = phys >= 0 && phys < a.num_blocks;
      bad |= !valid;
      copy_page(a, phys, valid, page_tokens(pb), smem, wave, lane);
      pending = true;
    }
    for (int p = pb; p < pe; ++p) {
      const int tok = page_tokens(p);
      bool next = false;
      if (p + 1 < pe && page_tokens(p + 1) > 0) {
        const int phys = page_phys(p + 1);
        const bool valid = phys >= 0 && phys < a.num_blocks;
        bad |= !valid;
        copy_page(a, phys, valid, page_tokens(p + 1), smem + (buf ^ 1) * kPageBytes, wave, lane);
        next = true;
      }
      if (next)
        __builtin_amdgcn_s_waitcnt(0x4F72);  // vmcnt(18): this page's copies have landed
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      block_sync();
      if (tok > 0 && pending) {
        if (computes) {
          // per-page base addresses; every access adds a constant that fits the
          // LDS instruction's 16-bit offset field
          lds_u8* tile = (lds_u8*)smem + buf * kPageBytes;
          lds_u8* vb[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) vb[u] = launder(tile + vb_lane + 16u * (vy ^ (2u * u)));
          compute_page<NWC>(a, st, L, wave, lane, vis_row - 64 * p, launder(tile + kb_lane + 16u * kx),
                            launder(tile + kb_lane + 16u * (kx ^ 4u)), vb, carry, dump);
        } else {
          block_sync();  // matches the P hand-off barrier inside compute_page
        }
      }
      block_sync();
      pending = next;
      buf ^= 1;
    }

    if (computes) publish_row_weights<NWC>(a, st, L, wave, lane, own_row, b, bad, nsplit == 1, slot);
    block_sync();
    if (computes) write_block<NWC>(a, st, L, carry, wave, lane, blk_row0, b, nsplit == 1, slot);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    block_sync();
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

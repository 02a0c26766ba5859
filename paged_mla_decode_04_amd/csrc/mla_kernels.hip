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
//     at most 128 rows); the query block stays in registers as MFMA operands
//     and the 128 x 512 fp32 output accumulator in (accumulation) registers;
//   * scores are computed transposed, S^T = K . Q^T, on 16x16x32 bf16 MFMA,
//     so every lane holds whole query rows: row max / row sum need only two
//     cross-lane steps and the output rescale is lane-local;
//   * P . V is computed as O^T = V^T . P^T: P^T comes straight from the score
//     registers (no data movement) and V^T from LDS with the gfx950
//     transposing read ds_read_b64_tr_b16 (4 consecutive tokens per lane);
//   * online softmax in the log2 domain; the running max is only moved when
//     it grows by more than 2^8, so the output is rescaled rarely;
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
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kPageBytes = 64 * kD * 2;  // 73728
constexpr int kThreads = 256;
constexpr int kKSteps = kD / 32;          // 18 MFMA k-steps of 32 for the scores
constexpr int kColTiles = kDv / 16;       // 32 output column tiles of 16
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;     // log2 units: p = 2^(x - m) stays <= 256
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

// Workgroup barrier for LDS hand-offs.  The page copies are waited for
// explicitly (vmcnt) before it; unlike __syncthreads it does not also wait for
// the next page's copies still in flight.
// Register-class hints (emit no instructions): the 128 x 512 fp32 output
// accumulator lives in the accumulation registers, the query fragments in
// ordinary VGPRs, so that together they fit one wave's 512 registers.
__device__ __forceinline__ void pin_acc(f32x4& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void pin_vgpr(bf16x8& x) { asm volatile("" : "+v"(x)); }

// x *= alpha for an accumulator element kept in an accumulation register.  One
// opaque read-multiply-write, so the copy through a VGPR happens here and only
// here (the compiler would otherwise keep a VGPR copy of every accumulator
// alive across the page loop for this rarely taken path).  Callers run it far
// from the MFMAs that write or read these accumulators.
__device__ __forceinline__ void scale_acc1(float& x, float alpha) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32_e32 %1, %2, %1\n\t"
      "s_nop 1\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "+a"(x), "=&v"(t)
      : "v"(alpha));
}
__device__ __forceinline__ void scale_acc(f32x4& o, float alpha) {
  float x0 = o[0], x1 = o[1], x2 = o[2], x3 = o[3];
  scale_acc1(x0, alpha);
  scale_acc1(x1, alpha);
  scale_acc1(x2, alpha);
  scale_acc1(x3, alpha);
  o = f32x4{x0, x1, x2, x3};
  pin_acc(o);
}

// Opaque copy of a pointer: keeps base + constant address arithmetic from being
// re-associated (and hoisted) so the constant lands in the instruction offset.
__device__ __forceinline__ lds_u8* launder(lds_u8* p) {
  asm volatile("" : "+v"(p));
  return p;
}

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

constexpr int kLatentSteps = kDv / 32;  // k-steps whose Q fragments live in registers
constexpr int kRopeSteps = kKSteps - kLatentSteps;
constexpr int kQRopeOffset = 2 * kPageBytes;            // LDS bytes: after the two page tiles
constexpr int kQRopeWaveBytes = 2 * kRopeSteps * 64 * 16;  // RT <= 2 row tiles per wave
constexpr int kSmemBytes = kQRopeOffset + 4 * kQRopeWaveBytes;  // 163840

template <int RT>  // row tiles of 16 per compute wave
struct WaveState {
  bf16x8 qf[RT][kLatentSteps];  // Q^T operand fragments of the 512 latent columns
  f32x4 o[kColTiles][RT];       // O^T accumulators: lane row, columns 16 ct + 4 g + j
  float m[RT];                  // running max (log2 units of scaled scores)
  float l[RT];                  // running sum of the bf16-rounded probabilities P . V used
  float le[RT];                 // running sum of the unrounded probabilities (for lse)
};

// One page in two halves of 32 tokens.  Per half: S^T = K . Q^T (16x16x32 MFMA,
// the 64 rope columns' Q fragments read back from LDS), mask, online softmax,
// O^T += V^T . P^T.  `vis` is this lane's visible-token count per row tile,
// relative to the page start (>= 64 when nothing is masked).
template <int RT>
__device__ __forceinline__ void compute_page(const DecodeArgs& a, WaveState<RT>& st, lds_u8* qrope,
                                             int lane, const int* vis, lds_u8* kb0, lds_u8* kb1,
                                             lds_u8* const* vb) {
  const int g = lane >> 4;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    f32x4 s[2][RT];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[t2][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qr[RT][kRopeSteps];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < kRopeSteps; ++k)
        qr[rt][k] = *(const lds_bf16x8*)(qrope + (rt * kRopeSteps + k) * 1024 + lane * 16);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int tt = 2 * half + t2;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8 kf = *(const lds_bf16x8*)(((ks & 1) ? kb1 : kb0) + 18432u * tt + 1024u * (ks >> 1));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8 qv = ks < kLatentSteps ? st.qf[rt][ks < kLatentSteps ? ks : 0]
                                              : qr[rt][ks < kLatentSteps ? 0 : ks - kLatentSteps];
          s[t2][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qv, s[t2][rt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + RT * kRopeSteps, 0);
#pragma unroll
    for (int i = 0; i < 2 * kKSteps; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, RT, 0);
      if (i < 2 * kKSteps - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }

    // mask (token 32 half + 16 t2 + 4 g + j visible iff < vis), scale, row max
    float mx[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int lim = vis[rt] - 32 * half - 4 * g;
      float v = -INFINITY;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = (16 * t2 + j < lim) ? s[t2][rt][j] * a.scale_log2 : -INFINITY;
          s[t2][rt][j] = x;
          v = fmaxf(v, x);
        }
      mx[rt] = wave_max16(v);
    }
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) grow |= (mx[rt] > st.m[rt] + kRescaleSlack);
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mnew = fmaxf(st.m[rt], mx[rt]);
        const float alpha = __builtin_amdgcn_exp2f(st.m[rt] - (mnew == -INFINITY ? 0.f : mnew));
        st.m[rt] = mnew;
        st.l[rt] *= alpha;
        st.le[rt] *= alpha;
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) scale_acc(st.o[ct][rt], alpha);
      }
    }
    bf16x8 pf[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mu = (st.m[rt] == -INFINITY) ? 0.f : st.m[rt];
      float sum = 0.f, sum_exact = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = __builtin_amdgcn_exp2f(s[t2][rt][j] - mu);
          const __bf16 p = (__bf16)e;
          sum += (float)p;
          sum_exact += e;
          pf[rt][4 * t2 + j] = p;
        }
      st.l[rt] += wave_sum16(sum);
      st.le[rt] += wave_sum16(sum_exact);
    }

    // O^T += V^T . P^T over this half's 32 tokens
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      lds_u8* vp = vb[ct & 3] + 9216u * (4 * half) + 1024u * (ct >> 2);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vp);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 2 * 9216u));
      const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        st.o[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], st.o[ct][rt], 0, 0, 0);
        pin_acc(st.o[ct][rt]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
    for (int i = 0; i < kColTiles; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, RT, 1);
      if (i < kColTiles - 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
  }
}

// NWC compute waves of RT*16 rows each; all 4 waves copy pages.
template <int NWC, int RT>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  constexpr int kBlockRows = NWC * RT * 16;

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
  const uint32_t vb_lane = 9216u * (g >> 1) + 128u * va + 8u * (vs & 1);

  const bool computes = wave < NWC;
  const int row0 = mblock * kBlockRows + wave * RT * 16;  // first row of this wave
  WaveState<RT> st;

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

    lds_u8* qrope = (lds_u8*)smem + kQRopeOffset + wave * kQRopeWaveBytes;
    if (computes) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + 16 * rt + (lane & 15);
        const bool ok = r < a.rows;
        const int rr = ok ? r : 0;
        const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)(rr / a.h_q) * a.q_ss +
                             (int64_t)(rr % a.h_q) * a.q_sh + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          bf16x8 v = *(const bf16x8*)(qp + 32 * ks);
          if (!ok) v = bf16x8{};
          if (ks < kLatentSteps)
            st.qf[rt][ks < kLatentSteps ? ks : 0] = v;
          else  // rope fragments wait in this wave's LDS slice, in lane order
            *(lds_bf16x8*)(qrope + (rt * kRopeSteps + ks - kLatentSteps) * 1024 + lane * 16) = v;
        }
        st.m[rt] = -INFINITY;
        st.l[rt] = 0.f;
        st.le[rt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) {
          st.o[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          pin_acc(st.o[ct][rt]);
        }
      }
    }
    // visible keys of this lane's rows: n, or n - (s_q - 1 - i) for query token i
    int vis_row[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = row0 + 16 * rt + (lane & 15);
      vis_row[rt] = a.causal ? n - (a.s_q - 1 - r / a.h_q) : n;
    }
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
      if (computes && tok > 0 && pending) {
        int vis[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) vis[rt] = vis_row[rt] - 64 * p;
        // per-page base addresses; every access adds a constant that fits the
        // LDS instruction's 16-bit offset field
        lds_u8* tile = (lds_u8*)smem + buf * kPageBytes;
        lds_u8* vb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) vb[u] = launder(tile + vb_lane + 16u * (vy ^ (2u * u)));
        compute_page<RT>(a, st, qrope, lane, vis, launder(tile + kb_lane + 16u * kx),
                         launder(tile + kb_lane + 16u * (kx ^ 4u)), vb);
      }
      block_sync();
      pending = next;
      buf ^= 1;
    }

    // ---- epilogue: final output, or an fp32 partial for the merge
    if (computes) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + 16 * rt + (lane & 15);
        if (r >= a.rows) continue;
        const float l = st.l[rt];
        float inv = l > 0.f ? 1.f / l : 0.f;
        float lse = l > 0.f ? (st.m[rt] + __builtin_amdgcn_logf(st.le[rt])) * kLn2 : -INFINITY;
        if (bad) {
          inv = __builtin_nanf("");
          lse = __builtin_nanf("");
        }
        const int qi = r / a.h_q, h = r - qi * a.h_q;
        if (nsplit == 1) {
          uint16_t* op = a.out + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh + 4 * g;
#pragma unroll
          for (int ct = 0; ct < kColTiles; ++ct) {
            const f32x4 v = st.o[ct][rt] * inv;
            bf16x4 w = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            *(bf16x4*)(op + 16 * ct) = w;
            __builtin_amdgcn_sched_barrier(0);
          }
          if (g == 0) a.lse[(int64_t)b * a.l_sb + (int64_t)qi * a.l_ss + (int64_t)h * a.l_sh] = lse;
        } else {
          float* pp = a.part_o + ((int64_t)slot * a.rows + r) * kDv + 4 * g;
#pragma unroll
          for (int ct = 0; ct < kColTiles; ++ct) {
            *(f32x4*)(pp + 16 * ct) = st.o[ct][rt] * inv;
            __builtin_amdgcn_sched_barrier(0);
          }
          if (g == 0) a.part_lse[(int64_t)slot * a.rows + r] = lse;
        }
      }
    }
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

__global__ void plan_kernel(const int32_t* seqlens, int batch, int rows, int num_parts, int32_t* tile_md,
                            int32_t* num_splits) {
  if (threadIdx.x == 0 && blockIdx.x == 0) plan_split_kv(seqlens, batch, rows, num_parts, tile_md, num_splits);
}

hipError_t launch_plan(const int32_t* seqlens, int batch, int rows, int num_parts, int32_t* tile_md,
                       int32_t* num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, stream, seqlens, batch, rows, num_parts, tile_md,
                     num_splits);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_parts * a.row_blocks));
  const int rpb = rows_per_block(a.rows);
  if (rpb == 16)
    hipLaunchKernelGGL((decode_kernel<1, 1>), grid, dim3(kThreads), 0, stream, a);
  else if (rpb == 32)
    hipLaunchKernelGGL((decode_kernel<2, 1>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<4, 1>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.batch, (unsigned)((a.rows + 3) / 4));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

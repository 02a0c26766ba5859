// Split-KV decode for the wide-head shape: up to 128 query rows of one kv
// head per workgroup, so that every cached token is read from HBM once per
// part.
//
// What is computed is the same as for the narrow kernel (mla_kernels.hip):
// for each query row r = (query token i, head h), softmax(scale * q_r . k_t)
// over the sequence's visible cached latent rows k_t (576 bf16; V is the first
// 512 elements of the same row), out = P . V and the natural-log lse.  The PAI
// FlashMLA tutorial (segmentfault, "云上玩转DeepSeek系列之五", section 二.4)
// states the inputs and prices the work as (d + dv) multiply-adds per
// query-key pair and one d-element read per cached token.
//
// Layout of the work on gfx950: one workgroup of 4 waves per CU, one wave per
// SIMD with the SIMD's whole register file.  Wave w owns query rows
// 32 w .. 32 w + 31 from end to end:
//   * its queries stay in 144 VGPRs as the B operand of the scores
//     S^T = K . Q^T, one 32x32x16 bf16 MFMA per 16 columns of d (36 per
//     32-token chunk, one accumulator chain: the matrix core forwards the
//     accumulator, so the chain runs at the full rate);
//   * in the 32x32 result each lane holds one query row and 16 of the
//     chunk's 32 tokens, so the softmax needs no cross-lane step except when
//     the reference max moves, and P (bf16) is already the B operand of the
//     value product, lane for lane, for the token order the transposing V
//     read produces;
//   * its output rows, O^T = V^T . P^T for all 512 columns, are 16 32x32
//     tiles in the 256 accumulation registers, one MFMA per tile per 16
//     tokens (32 per chunk), V^T read with ds_read_b64_tr_b16.
// Nothing but the cached chunks goes through LDS: no wave waits for another
// except at the one barrier per step that recycles chunk slots.
//
// Step t scores chunk t + 1 and accumulates the values of chunk t, with the
// softmax of chunk t + 1 issued between the value MFMAs; the copy of chunk
// t + 3 is issued between the score MFMAs and lands by the end of step t + 1.
// A step whose score chunk starts a new sequence loads that sequence's
// queries first and runs its value product before the scores, which hides the
// load behind it.
//
// LDS: four slots of one 32-token chunk (32 x 576 bf16 = 36 KB): column block
// q (64 columns) of the chunk at 4096 q, token a at 128 a inside it, its
// 16-byte column chunk c (0..7) at slot c ^ swz(a).  The swizzle keeps the
// score reads (32 tokens x one chunk per 512 bytes) and the transposing value
// reads (4 tokens x 4 chunks per 256 bytes) at two and one pass over the
// banks.
//
// An fp8 cache (one E4M3 byte per element, one scale per cache) takes the
// same path after a widening step: its chunks (18 KB) are copied as bytes into
// a staging area, and each step converts the staged chunk t + 2 to bf16 in a
// chunk slot (three slots) before copying chunk t + 4 into the staging it just
// read.  Every E4M3 value is exact in bf16; the cache's scale multiplies the
// score scale and the output's 1 / l instead of every element.
#include <type_traits>

#include "mla_device.h"

namespace mla {
namespace {

constexpr int kThreadsW = 256;                    // 4 waves, one per SIMD
constexpr int kRowsW = 128;                       // query rows per workgroup
constexpr int kTileBytes = kChunk * kD * 2;       // 36864
constexpr int kSlots = 4;
constexpr int kSmemW = kSlots * kTileBytes;       // 147456
constexpr int kSSteps = kD / 16;                  // 36 score k-steps
constexpr int kColTiles = kDv / 32;               // 16 output column tiles
constexpr int kCopiesW = 9;                       // 1 KB copies per wave per chunk
constexpr int kKAhead = 4;                        // score K fragments in flight
constexpr int kVAhead = 7;                        // value V^T fragments in flight
static_assert(kSmemW <= 160 * 1024, "LDS budget");
static_assert(kThreadsW / 64 * kCopiesW * 1024 == kTileBytes, "copies cover the chunk");
// An fp8 cache (one E4M3 byte per element): a wave's token octet of a chunk
// (8 x 576 bytes) is staged as five 1 KB copies, then converted to bf16 into
// one of three chunk slots the score and value products read as before.
constexpr int kCopies8 = 5;
constexpr int kStageWave = kCopies8 * 1024;       // 5120
constexpr int kStageBytes = 4 * kStageWave;       // 20480
constexpr int kSlots8 = 3;
constexpr int kSmem8 = kSlots8 * kTileBytes + 2 * kStageBytes;  // 151552
static_assert(kSmem8 <= 160 * 1024, "LDS budget (fp8 cache)");
static_assert(8 * 576 <= kStageWave, "staging covers a token octet");

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Swizzle of token a's eight 16-byte chunks in a column block (uses bits 1..3
// of a, so it repeats every 16 tokens).
__device__ __forceinline__ int swz(int a) { return (((a >> 1) & 1) << 2) | ((a >> 2) & 3); }

// Copy Q (1 KB) of the wave's token octet: source at lane_off + 128 Q (the
// immediate offset), LDS at wave_base + LSTRIDE Q (the immediate offset is
// added to the LDS address too, so M0 is lowered by it).  A bf16 cache copies
// column block Q (LSTRIDE 4096, the block's place in a chunk slot), an fp8
// cache byte range 128 Q .. 128 Q + 127 of each row (LSTRIDE 1024, staging).
// (The s_nop is the wait state an LDS-direct load needs after the scalar write
// of M0 just before it; the compiler does not insert it for assembly.)
template <int Q, uint32_t LSTRIDE = 4096u>
__device__ __forceinline__ void copy_block(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, uint32_t wave_base) {
  // (M0 = wave_base + the block's constant, written here: the compiler would
  // otherwise keep nine such sums in scalar registers, spilled under pressure)
  asm volatile("s_add_u32 m0, %3, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%2 nt lds" ::"v"(lane_off),
               "s"(rsrc), "n"(128 * Q), "s"(wave_base), "n"((LSTRIDE - 128u) * Q)
               : "memory", "m0", "scc");
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s (+)= K . Q^T for one 16-column step of d; the accumulator stays in VGPRs
// (written as assembly: the compiler would put every MFMA result of the
// kernel in the register file the value accumulators fill).  One MFMA per
// statement, so that the copies' address work between them overlaps the
// matrix core.
__device__ __forceinline__ void score_mfma1(f32x16& s, bf16x8 k, bf16x8 q, bool first) {
  if (first)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
}

// ---- the output accumulators: fixed AGPRs, a[16 ct .. 16 ct + 15] for tile
// ct, touched only by the assembly below (the compiler never holds them, so
// it cannot copy or spill them; the zeroing names every one of them as
// clobbered, which reserves all 256 for the kernel).
// One value MFMA, tile CT, per statement: the softmax's VALU work goes between
// consecutive MFMAs, where it runs while the matrix core works (VALU work
// issued after two back-to-back MFMAs waits for them instead).
#define MLA_VMFMA1(L, H) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[" #L ":" #H "], %0, %1, a[" #L ":" #H "]" ::"v"(v), "v"(p))
template <int CT>
__device__ __forceinline__ void value_mfma1(bf16x8 v, bf16x8 p) {
  static_assert(CT >= 0 && CT < 16, "tile");
  if constexpr (CT == 0) MLA_VMFMA1(0, 15);
  else if constexpr (CT == 1) MLA_VMFMA1(16, 31);
  else if constexpr (CT == 2) MLA_VMFMA1(32, 47);
  else if constexpr (CT == 3) MLA_VMFMA1(48, 63);
  else if constexpr (CT == 4) MLA_VMFMA1(64, 79);
  else if constexpr (CT == 5) MLA_VMFMA1(80, 95);
  else if constexpr (CT == 6) MLA_VMFMA1(96, 111);
  else if constexpr (CT == 7) MLA_VMFMA1(112, 127);
  else if constexpr (CT == 8) MLA_VMFMA1(128, 143);
  else if constexpr (CT == 9) MLA_VMFMA1(144, 159);
  else if constexpr (CT == 10) MLA_VMFMA1(160, 175);
  else if constexpr (CT == 11) MLA_VMFMA1(176, 191);
  else if constexpr (CT == 12) MLA_VMFMA1(192, 207);
  else if constexpr (CT == 13) MLA_VMFMA1(208, 223);
  else if constexpr (CT == 14) MLA_VMFMA1(224, 239);
  else MLA_VMFMA1(240, 255);
}
#undef MLA_VMFMA1

#define MLA_AREAD4(A, B, C, D)                                                                 \
  asm volatile("v_accvgpr_read_b32 %0, a" #A "\n\tv_accvgpr_read_b32 %1, a" #B                  \
               "\n\tv_accvgpr_read_b32 %2, a" #C "\n\tv_accvgpr_read_b32 %3, a" #D             \
               : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3))
// Accumulators a[4 I .. 4 I + 3] (elements 4 g .. 4 g + 3 of tile ct at I = 4 ct + g).
template <int I>
__device__ __forceinline__ f32x4 acc_read4() {
  float x0, x1, x2, x3;
  if constexpr (I == 0) MLA_AREAD4(0, 1, 2, 3);
  else if constexpr (I == 1) MLA_AREAD4(4, 5, 6, 7);
  else if constexpr (I == 2) MLA_AREAD4(8, 9, 10, 11);
  else if constexpr (I == 3) MLA_AREAD4(12, 13, 14, 15);
  else if constexpr (I == 4) MLA_AREAD4(16, 17, 18, 19);
  else if constexpr (I == 5) MLA_AREAD4(20, 21, 22, 23);
  else if constexpr (I == 6) MLA_AREAD4(24, 25, 26, 27);
  else if constexpr (I == 7) MLA_AREAD4(28, 29, 30, 31);
  else if constexpr (I == 8) MLA_AREAD4(32, 33, 34, 35);
  else if constexpr (I == 9) MLA_AREAD4(36, 37, 38, 39);
  else if constexpr (I == 10) MLA_AREAD4(40, 41, 42, 43);
  else if constexpr (I == 11) MLA_AREAD4(44, 45, 46, 47);
  else if constexpr (I == 12) MLA_AREAD4(48, 49, 50, 51);
  else if constexpr (I == 13) MLA_AREAD4(52, 53, 54, 55);
  else if constexpr (I == 14) MLA_AREAD4(56, 57, 58, 59);
  else if constexpr (I == 15) MLA_AREAD4(60, 61, 62, 63);
  else if constexpr (I == 16) MLA_AREAD4(64, 65, 66, 67);
  else if constexpr (I == 17) MLA_AREAD4(68, 69, 70, 71);
  else if constexpr (I == 18) MLA_AREAD4(72, 73, 74, 75);
  else if constexpr (I == 19) MLA_AREAD4(76, 77, 78, 79);
  else if constexpr (I == 20) MLA_AREAD4(80, 81, 82, 83);
  else if constexpr (I == 21) MLA_AREAD4(84, 85, 86, 87);
  else if constexpr (I == 22) MLA_AREAD4(88, 89, 90, 91);
  else if constexpr (I == 23) MLA_AREAD4(92, 93, 94, 95);
  else if constexpr (I == 24) MLA_AREAD4(96, 97, 98, 99);
  else if constexpr (I == 25) MLA_AREAD4(100, 101, 102, 103);
  else if constexpr (I == 26) MLA_AREAD4(104, 105, 106, 107);
  else if constexpr (I == 27) MLA_AREAD4(108, 109, 110, 111);
  else if constexpr (I == 28) MLA_AREAD4(112, 113, 114, 115);
  else if constexpr (I == 29) MLA_AREAD4(116, 117, 118, 119);
  else if constexpr (I == 30) MLA_AREAD4(120, 121, 122, 123);
  else if constexpr (I == 31) MLA_AREAD4(124, 125, 126, 127);
  else if constexpr (I == 32) MLA_AREAD4(128, 129, 130, 131);
  else if constexpr (I == 33) MLA_AREAD4(132, 133, 134, 135);
  else if constexpr (I == 34) MLA_AREAD4(136, 137, 138, 139);
  else if constexpr (I == 35) MLA_AREAD4(140, 141, 142, 143);
  else if constexpr (I == 36) MLA_AREAD4(144, 145, 146, 147);
  else if constexpr (I == 37) MLA_AREAD4(148, 149, 150, 151);
  else if constexpr (I == 38) MLA_AREAD4(152, 153, 154, 155);
  else if constexpr (I == 39) MLA_AREAD4(156, 157, 158, 159);
  else if constexpr (I == 40) MLA_AREAD4(160, 161, 162, 163);
  else if constexpr (I == 41) MLA_AREAD4(164, 165, 166, 167);
  else if constexpr (I == 42) MLA_AREAD4(168, 169, 170, 171);
  else if constexpr (I == 43) MLA_AREAD4(172, 173, 174, 175);
  else if constexpr (I == 44) MLA_AREAD4(176, 177, 178, 179);
  else if constexpr (I == 45) MLA_AREAD4(180, 181, 182, 183);
  else if constexpr (I == 46) MLA_AREAD4(184, 185, 186, 187);
  else if constexpr (I == 47) MLA_AREAD4(188, 189, 190, 191);
  else if constexpr (I == 48) MLA_AREAD4(192, 193, 194, 195);
  else if constexpr (I == 49) MLA_AREAD4(196, 197, 198, 199);
  else if constexpr (I == 50) MLA_AREAD4(200, 201, 202, 203);
  else if constexpr (I == 51) MLA_AREAD4(204, 205, 206, 207);
  else if constexpr (I == 52) MLA_AREAD4(208, 209, 210, 211);
  else if constexpr (I == 53) MLA_AREAD4(212, 213, 214, 215);
  else if constexpr (I == 54) MLA_AREAD4(216, 217, 218, 219);
  else if constexpr (I == 55) MLA_AREAD4(220, 221, 222, 223);
  else if constexpr (I == 56) MLA_AREAD4(224, 225, 226, 227);
  else if constexpr (I == 57) MLA_AREAD4(228, 229, 230, 231);
  else if constexpr (I == 58) MLA_AREAD4(232, 233, 234, 235);
  else if constexpr (I == 59) MLA_AREAD4(236, 237, 238, 239);
  else if constexpr (I == 60) MLA_AREAD4(240, 241, 242, 243);
  else if constexpr (I == 61) MLA_AREAD4(244, 245, 246, 247);
  else if constexpr (I == 62) MLA_AREAD4(248, 249, 250, 251);
  else if constexpr (I == 63) MLA_AREAD4(252, 253, 254, 255);
  return f32x4{x0, x1, x2, x3};
}
#undef MLA_AREAD4

#define MLA_AZERO4(A, B, C, D)                                                                 \
  asm volatile("v_accvgpr_write_b32 a" #A ", 0\n\tv_accvgpr_write_b32 a" #B ", 0\n\t"            \
               "v_accvgpr_write_b32 a" #C ", 0\n\tv_accvgpr_write_b32 a" #D ", 0" ::                \
                   : "a" #A, "a" #B, "a" #C, "a" #D)
// Every accumulator to zero.
__device__ __forceinline__ void acc_zero() {
  MLA_AZERO4(0, 1, 2, 3); MLA_AZERO4(4, 5, 6, 7); MLA_AZERO4(8, 9, 10, 11); MLA_AZERO4(12, 13, 14, 15);
  MLA_AZERO4(16, 17, 18, 19); MLA_AZERO4(20, 21, 22, 23); MLA_AZERO4(24, 25, 26, 27); MLA_AZERO4(28, 29, 30, 31);
  MLA_AZERO4(32, 33, 34, 35); MLA_AZERO4(36, 37, 38, 39); MLA_AZERO4(40, 41, 42, 43); MLA_AZERO4(44, 45, 46, 47);
  MLA_AZERO4(48, 49, 50, 51); MLA_AZERO4(52, 53, 54, 55); MLA_AZERO4(56, 57, 58, 59); MLA_AZERO4(60, 61, 62, 63);
  MLA_AZERO4(64, 65, 66, 67); MLA_AZERO4(68, 69, 70, 71); MLA_AZERO4(72, 73, 74, 75); MLA_AZERO4(76, 77, 78, 79);
  MLA_AZERO4(80, 81, 82, 83); MLA_AZERO4(84, 85, 86, 87); MLA_AZERO4(88, 89, 90, 91); MLA_AZERO4(92, 93, 94, 95);
  MLA_AZERO4(96, 97, 98, 99); MLA_AZERO4(100, 101, 102, 103); MLA_AZERO4(104, 105, 106, 107); MLA_AZERO4(108, 109, 110, 111);
  MLA_AZERO4(112, 113, 114, 115); MLA_AZERO4(116, 117, 118, 119); MLA_AZERO4(120, 121, 122, 123); MLA_AZERO4(124, 125, 126, 127);
  MLA_AZERO4(128, 129, 130, 131); MLA_AZERO4(132, 133, 134, 135); MLA_AZERO4(136, 137, 138, 139); MLA_AZERO4(140, 141, 142, 143);
  MLA_AZERO4(144, 145, 146, 147); MLA_AZERO4(148, 149, 150, 151); MLA_AZERO4(152, 153, 154, 155); MLA_AZERO4(156, 157, 158, 159);
  MLA_AZERO4(160, 161, 162, 163); MLA_AZERO4(164, 165, 166, 167); MLA_AZERO4(168, 169, 170, 171); MLA_AZERO4(172, 173, 174, 175);
  MLA_AZERO4(176, 177, 178, 179); MLA_AZERO4(180, 181, 182, 183); MLA_AZERO4(184, 185, 186, 187); MLA_AZERO4(188, 189, 190, 191);
  MLA_AZERO4(192, 193, 194, 195); MLA_AZERO4(196, 197, 198, 199); MLA_AZERO4(200, 201, 202, 203); MLA_AZERO4(204, 205, 206, 207);
  MLA_AZERO4(208, 209, 210, 211); MLA_AZERO4(212, 213, 214, 215); MLA_AZERO4(216, 217, 218, 219); MLA_AZERO4(220, 221, 222, 223);
  MLA_AZERO4(224, 225, 226, 227); MLA_AZERO4(228, 229, 230, 231); MLA_AZERO4(232, 233, 234, 235); MLA_AZERO4(236, 237, 238, 239);
  MLA_AZERO4(240, 241, 242, 243); MLA_AZERO4(244, 245, 246, 247); MLA_AZERO4(248, 249, 250, 251); MLA_AZERO4(252, 253, 254, 255);
}
#undef MLA_AZERO4

#define MLA_ASCALE4(A, B, C, D)                                                                \
  asm volatile("v_accvgpr_read_b32 %0, a" #A "\n\tv_accvgpr_read_b32 %1, a" #B "\n\t"               \
               "v_accvgpr_read_b32 %2, a" #C "\n\tv_accvgpr_read_b32 %3, a" #D "\n\t"               \
               "v_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\t"                                  \
               "v_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\t"                                  \
               "v_accvgpr_write_b32 a" #A ", %0\n\tv_accvgpr_write_b32 a" #B ", %1\n\t"              \
               "v_accvgpr_write_b32 a" #C ", %2\n\tv_accvgpr_write_b32 a" #D ", %3"                    \
               : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)                                    \
               : "v"(f))
// Every accumulator times this lane's factor f.
__device__ __forceinline__ void acc_scale(float f) {
  float t0, t1, t2, t3;
  MLA_ASCALE4(0, 1, 2, 3); MLA_ASCALE4(4, 5, 6, 7); MLA_ASCALE4(8, 9, 10, 11); MLA_ASCALE4(12, 13, 14, 15);
  MLA_ASCALE4(16, 17, 18, 19); MLA_ASCALE4(20, 21, 22, 23); MLA_ASCALE4(24, 25, 26, 27); MLA_ASCALE4(28, 29, 30, 31);
  MLA_ASCALE4(32, 33, 34, 35); MLA_ASCALE4(36, 37, 38, 39); MLA_ASCALE4(40, 41, 42, 43); MLA_ASCALE4(44, 45, 46, 47);
  MLA_ASCALE4(48, 49, 50, 51); MLA_ASCALE4(52, 53, 54, 55); MLA_ASCALE4(56, 57, 58, 59); MLA_ASCALE4(60, 61, 62, 63);
  MLA_ASCALE4(64, 65, 66, 67); MLA_ASCALE4(68, 69, 70, 71); MLA_ASCALE4(72, 73, 74, 75); MLA_ASCALE4(76, 77, 78, 79);
  MLA_ASCALE4(80, 81, 82, 83); MLA_ASCALE4(84, 85, 86, 87); MLA_ASCALE4(88, 89, 90, 91); MLA_ASCALE4(92, 93, 94, 95);
  MLA_ASCALE4(96, 97, 98, 99); MLA_ASCALE4(100, 101, 102, 103); MLA_ASCALE4(104, 105, 106, 107); MLA_ASCALE4(108, 109, 110, 111);
  MLA_ASCALE4(112, 113, 114, 115); MLA_ASCALE4(116, 117, 118, 119); MLA_ASCALE4(120, 121, 122, 123); MLA_ASCALE4(124, 125, 126, 127);
  MLA_ASCALE4(128, 129, 130, 131); MLA_ASCALE4(132, 133, 134, 135); MLA_ASCALE4(136, 137, 138, 139); MLA_ASCALE4(140, 141, 142, 143);
  MLA_ASCALE4(144, 145, 146, 147); MLA_ASCALE4(148, 149, 150, 151); MLA_ASCALE4(152, 153, 154, 155); MLA_ASCALE4(156, 157, 158, 159);
  MLA_ASCALE4(160, 161, 162, 163); MLA_ASCALE4(164, 165, 166, 167); MLA_ASCALE4(168, 169, 170, 171); MLA_ASCALE4(172, 173, 174, 175);
  MLA_ASCALE4(176, 177, 178, 179); MLA_ASCALE4(180, 181, 182, 183); MLA_ASCALE4(184, 185, 186, 187); MLA_ASCALE4(188, 189, 190, 191);
  MLA_ASCALE4(192, 193, 194, 195); MLA_ASCALE4(196, 197, 198, 199); MLA_ASCALE4(200, 201, 202, 203); MLA_ASCALE4(204, 205, 206, 207);
  MLA_ASCALE4(208, 209, 210, 211); MLA_ASCALE4(212, 213, 214, 215); MLA_ASCALE4(216, 217, 218, 219); MLA_ASCALE4(220, 221, 222, 223);
  MLA_ASCALE4(224, 225, 226, 227); MLA_ASCALE4(228, 229, 230, 231); MLA_ASCALE4(232, 233, 234, 235); MLA_ASCALE4(236, 237, 238, 239);
  MLA_ASCALE4(240, 241, 242, 243); MLA_ASCALE4(244, 245, 246, 247); MLA_ASCALE4(248, 249, 250, 251); MLA_ASCALE4(252, 253, 254, 255);
}
#undef MLA_ASCALE4

// The MFMA results about to be read by VALU instructions: wait out the result
// latency of a 32x32 MFMA (more than its 18 required wait states).
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }


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

// The lengths a batch from pos may need: lane k holds that of sequence
// pos.seq + k (0 past the part's last sequence).
__device__ __forceinline__ int batch_lengths(const DecodeArgs& a, const PartInfo& pi, const BatchPos& pos, int lane) {
  const int sk = pos.seq + lane;
  return sk <= pi.seq_last ? clamp_len(a, a.seqlens[sk]) : 0;
}

// nk: batch_lengths(pos), however obtained.
__device__ __forceinline__ i32x4 desc_batch(const DecodeArgs& a, const PartInfo& pi, BatchPos& pos, int lane, int nk) {
  i32x4 out = i32x4{-1, 0, 0, -1};
  if (!pos.more) return out;
  int rem = lane;  // chunks still to skip before this lane's own
  bool found = false;
  int my_seq = -1, my_chunk = 0, my_n = 0, my_lo = 0, my_hi = 0;
  int sq = pos.seq, lo = pos.chunk;
#pragma unroll 1
  for (int k = 0; k < 64 && sq <= pi.seq_last; ++k) {
    const int n = __builtin_amdgcn_readlane(nk, k);
    int hi = chunk_count(n);
    if (sq == pi.seq_last && 2 * pi.page_end < hi) hi = 2 * pi.page_end;
    // The plan counts pages of the stored length, the walk those of the
    // length clamped to the block table: a planned segment that starts past
    // the clamp still gets one (empty) chunk, so that its split slot is
    // written and the next sequence's chunks are not skipped.
    if (hi <= lo) hi = lo + 1;
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


// PLAN: the instance that derives its part from the lengths (no metadata
// given; bf16 cache only, the fp8 instance has no registers to spare).  The
// plan code changes the register allocation of the whole kernel, so the
// instance given a plan is built without it.
template <bool KV8, bool PLAN>
__global__ __launch_bounds__(kThreadsW, 1) void decode_wide_kernel(DecodeArgs a) {
  static_assert(!(KV8 && PLAN), "the fp8 instance takes a plan");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[KV8 ? kSmem8 : kSmemW];
  __shared__ int32_t split_tab[PLAN ? kPlanInKernelMaxBatch + 1 : 1];  // in-kernel plan: num_splits
  constexpr int kCopies = KV8 ? kCopies8 : kCopiesW;
  const int w = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  PartInfo pi;
  int plan_len[kPlanBlocks];  // the in-kernel plan's lengths (PLAN)
  if (!load_part<PLAN>(a, kRowsW, pi, (lds_i32*)split_tab, plan_len)) return;

  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  const uint32_t row_bytes = (uint32_t)a.k_row_bytes;
  const float sc = a.scale_log2;

  // this lane's query row (the same in the scores and the values), rebuilt
  // from an opaque lane index where it is used
  const int hlf = lane >> 5;
  struct RowInfo {
    int row, qi, hh;
    bool ok;
  };
  auto row_info = [&]() -> RowInfo {
    RowInfo r;
    r.row = pi.blk_row0 + 32 * w + (opaque(lane) & 31);
    r.ok = r.row < a.rows;
    const int rr = r.ok ? r.row : 0;
    r.qi = rr / a.h_q;
    r.hh = rr - r.qi * a.h_q;
    return r;
  };
  const bool wave_full = pi.blk_row0 + 32 * w + 32 <= a.rows;
  const int qi_min = (pi.blk_row0 + 32 * w) / a.h_q;

  // ---- per-lane LDS offsets inside a slot
  // Score K fragment of k-step ks (u = ks & 3): token j of the lane's half,
  // 16-byte chunk 2 ks + h at slot ((2 u + h) ^ swz(j)), i.e. at byte
  // 128 j + 16 ((2 u + h) ^ swz(j)) = k_lane ^ 32 u of the column block (the u
  // part only flips bits 5..6).
  const uint32_t k_lane = [&] {
    const int j = lane & 31, hb = lane >> 5, sw = swz(j);
    return 128u * j + 16u * (uint32_t)(hb ^ (sw & 1)) + 32u * (uint32_t)(sw >> 1);
  }();
  // Value V^T half fragment (cb = ct & 1, b): 16-lane group G reads tokens
  // 8 b + 4 (G >> 1) + 0..3 of the k-step, columns 16 (G & 1) + 0..15 of the
  // tile, at v_lane ^ (64 cb + 32 b) + 1024 b (cb and b only flip bits 5..6 of
  // the swizzled chunk; 1024 b is the token octet).
  const uint32_t v_lane = [&] {
    const int G = lane >> 4, s16 = lane & 15;
    const int tl = 4 * (G >> 1) + (s16 >> 2);
    const int c = 2 * (G & 1) + ((s16 >> 1) & 1);
    return 128u * tl + 16u * (uint32_t)(c ^ swz(tl)) + 8u * (uint32_t)(s16 & 1);
  }();

  // ---- copies: wave w moves token octet w (tokens 8 w .. 8 w + 7) of the
  // chunk's nine column blocks q, 1 KB each; lane l fetches token 8 w + (l >> 3)
  // and the 16-byte chunk that lands at its LDS position.  A chunk without keys
  // (or past the part's end) copies from an empty range: the loads write zeros
  // and read nothing, and every step issues the same nine loads.  Column block
  // q is the load's immediate offset 128 q, which an LDS-direct load also adds
  // to its LDS address, so M0 is lowered by as much.
  // An fp8 cache's copy Q moves 16-byte pieces 8 Q .. 8 Q + 7 of the octet's
  // rows: lane l takes token 8 w + (l >> 3), piece 8 Q + (l & 7), so that the
  // wave's staging holds piece c of its token a at 1024 (c / 8) + 128 a +
  // 16 (c % 8).  Pieces 36..39 (copy 4, lanes with l & 7 >= 4) lie past the
  // 576 bytes of the entry: they land in staging and are never converted.
  const uint32_t cp_lane = [&] {
    const int tk = 8 * w + (lane >> 3);
    if constexpr (KV8) return (uint32_t)tk * row_bytes + 16u * (uint32_t)(lane & 7);
    return (uint32_t)tk * row_bytes + 16u * (uint32_t)((lane & 7) ^ swz(tk));
  }();
  auto copy_rsrc = [&](const Chunk& c) -> __amdgpu_buffer_rsrc_t {
    const Chunk cz = c.valid() ? c : Chunk{0, 0, 0, 0, false, false, true};
    return chunk_rsrc(a, cz);
  };
  // (slot_addr: the chunk slot for a bf16 cache, the staging slot for fp8)
  auto copy_one = [&](__amdgpu_buffer_rsrc_t rsrc, uint32_t slot_addr, auto qc) {
    if constexpr (KV8)
      copy_block<decltype(qc)::value, 1024u>(rsrc, cp_lane, slot_addr + (uint32_t)kStageWave * w);
    else
      copy_block<decltype(qc)::value>(rsrc, cp_lane, slot_addr + 1024u * w);
  };
  auto copy_chunk = [&](const Chunk& c, uint32_t slot_addr) {
    const __amdgpu_buffer_rsrc_t rsrc = copy_rsrc(c);
    static_for<0, kCopies>([&](auto qc) { copy_one(rsrc, slot_addr, qc); });
  };
  // fp8 cache: the wave's token octet of a staged chunk to bf16 in a chunk
  // slot (every E4M3 value is exact in bf16; the cache's scale is applied to
  // the scores and the output instead).  Piece c (16 elements) of token a
  // becomes bf16 chunks 2 (c % 4) and 2 (c % 4) + 1 of column block c / 4.
  auto convert_chunk = [&](uint32_t stage_off, uint32_t slot_off) {
    const int tk = 8 * w + (lane >> 3), j = lane & 7, sw = swz(tk);
    lds_u8* src = launder(lds + stage_off + (uint32_t)kStageWave * w + 16u * (uint32_t)lane);
    lds_u8* dst = launder(lds + slot_off + 128u * (uint32_t)tk);
    static_for<0, kCopies8>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      if (I < kCopies8 - 1 || j < 4) {
        const u32x4 v = *(const lds_u32x4*)(src + 1024 * I);
        const int c = 8 * I + j, h = 2 * (c & 3);
        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.f, false);
        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.f, true);
        const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.f, false);
        const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.f, true);
        const auto p4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2], 1.f, false);
        const auto p5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2], 1.f, true);
        const auto p6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[3], 1.f, false);
        const auto p7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[3], 1.f, true);
        const uint32_t blk = 4096u * (uint32_t)(c >> 2);
        *(lds_bf16x8*)(dst + blk + 16u * (uint32_t)(h ^ sw)) =
            bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        *(lds_bf16x8*)(dst + blk + 16u * (uint32_t)((h + 1) ^ sw)) =
            bf16x8{p4[0], p4[1], p5[0], p5[1], p6[0], p6[1], p7[0], p7[1]};
      }
    });
  };

  // ---- state
  bf16x8 qf[kSSteps];          // queries of the segment being scored
  f32x16 s;                    // scores of the chunk being scored
  acc_zero();                  // output rows (the accumulator AGPRs)
  // P^T of chunk t (the value product's B operand); the softmax of chunk t + 1
  // overwrites each half after the value product's last use of it
  bf16x8 pc[2];
  pc[0] = pc[1] = bf16x8{};
  float m_ref = -INFINITY;     // reference max of this lane's row (log2 units)
  float lsum = 0.f;            // running sum of 2^(x - m_ref) over this lane's tokens
  int lim = 0, lim_min = 0;    // visible keys of this row / smallest of the wave
  float pend_f = 1.f;          // pending rescale of o (the reference moved)
  bool pending = false;
  float cap_inv = 0.f, cap_lse = -INFINITY;  // results of the last segment scored
  float seg_inv = 0.f, seg_lse = -INFINITY;  // ... of the segment being accumulated
  bool seg_bad = false;
  int seg_slot = 0, seg_nsplit = 1;

  auto load_queries = [&](const Chunk& c) {
    const int n = clamp_len(a, load_len(a, c.seq));
    const RowInfo ri = row_info();
    const uint16_t* qp =
        a.q + (int64_t)c.seq * a.q_sb + (int64_t)ri.qi * a.q_ss + (int64_t)ri.hh * a.q_sh + 8 * hlf;
#pragma unroll
    for (int ks = 0; ks < kSSteps; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    lim = ri.ok ? (a.causal ? n - (a.s_q - 1 - ri.qi) : n) : 0;
    lim_min = wave_full ? (a.causal ? n - (a.s_q - 1 - qi_min) : n) : 0;
    m_ref = -INFINITY;
    lsum = 0.f;
  };
  // The query loads have landed: waits for them here (and for the older chunk
  // copies, which must land in this step anyway) and hands the registers on as
  // new values, so that no later wait for them also waits for copies issued
  // after this point.
  auto queries_ready = [&]() {
#pragma unroll
    for (int ks = 0; ks < kSSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
  };

  // ---- the score product of chunk c (in the slot at byte offset slot_off),
  // with the copies [C0, C1) of chunk cc issued between the MFMAs
  auto score_loop = [&](uint32_t slot_off, auto with_copies, const Chunk& cc, uint32_t cc_slot) {
    constexpr bool WC = decltype(with_copies)::value;
    lds_u8* kb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kb[u] = launder(lds + slot_off + (k_lane ^ (32u * u)));
    auto kfrag = [&](int ks) -> bf16x8 { return *(const lds_bf16x8*)(kb[ks & 3] + 4096u * (ks >> 2)); };
    constexpr int R = kKAhead + 2;  // the read of step k goes ahead of MFMA k
    bf16x8 kf[R];
#pragma unroll
    for (int ks = 0; ks < kKAhead; ++ks) kf[ks] = kfrag(ks);
    __amdgpu_buffer_rsrc_t rsrc;
    if constexpr (WC) rsrc = copy_rsrc(cc);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, kSSteps>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k + kKAhead < kSSteps) kf[(k + kKAhead) % R] = kfrag(k + kKAhead);
      score_mfma1(s, kf[k % R], qf[k], k == 0);
      // the copies go out over the first half of the score product (each one as
      // early as the MFMAs allow, so more of the chunk is in flight)
      if constexpr (WC && k % 2 == 1 && k < 2 * kCopies) copy_one(rsrc, cc_slot, std::integral_constant<int, k / 2>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- softmax of the scored chunk D (scores in s), in 32 pieces; piece q
  // runs between value MFMAs q and q + 1 when interleaved
  float mu = 0.f;
  // (FAST: a full chunk inside its segment that no row's limit reaches:
  // no masking and no segment results)
  auto smax_piece = [&](auto qc, const Chunk& D, auto fast_tag) {
    constexpr int q = decltype(qc)::value;
    constexpr bool FAST = decltype(fast_tag)::value;
    if constexpr (q == 0) {
      // The scores' last MFMA is followed, in a common step, by the value
      // product's first fragment reads (2 kVAhead of them, held in place by
      // the scheduling barriers), their wait and the first value MFMA: with
      // four more wait states that is past the 18 the result needs.
      if constexpr (FAST) {
        static_assert(2 * kVAhead + 2 + 4 >= 18, "wait states before the first score read");
        asm volatile("s_nop 3" ::: "memory");
      } else {
        mfma_result_wait();
      }
      // (a common step's reference is finite: its segment's first chunk had
      // visible keys in every row)
      mu = FAST ? m_ref : (m_ref == -INFINITY ? 0.f : m_ref);
    } else if constexpr (q >= 1 && q <= 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * (q - 1) + e] = __builtin_fmaf(s[4 * (q - 1) + e], sc, -mu);
    } else if constexpr (q == 5 && !FAST) {
      // keys past the row's limit (only chunks that reach the smallest limit)
      const int tok0 = kChunk * D.chunk;
      if (D.tok <= 0 || tok0 + kChunk > lim_min) {
        const int vis = (D.tok > 0 ? lim - tok0 : 0) - 4 * hlf;  // token 8 g + 4 hlf + e visible iff 8 g + e < vis
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) >= vis) s[i] = -INFINITY;
      }
    } else if constexpr (q == 6) {
      // the lane's chunk max (kept in pend_f's neighbour below)
    } else if constexpr (q == 7) {
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      const bool over = FAST ? mx > kRescaleSlack : (m_ref == -INFINITY ? mx > -INFINITY : mx > kRescaleSlack);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) {  // (rare: kept out of line)
        // a chunk max passed the reference by more than 2^16 (or the segment
        // just started): move the row's reference to its max
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
        const float rowmax = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1])) + mu;
        const float m_new = fmaxf(m_ref, rowmax);
        const float f = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        const float mu_new = m_new == -INFINITY ? 0.f : m_new;
        lsum *= f;
        m_ref = m_new;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] += mu - mu_new;
        mu = mu_new;
        if (!D.first) {
          pend_f = f;
          pending = true;
        }
      }
    } else if constexpr (q >= 8 && q < 24) {
      s[q - 8] = __builtin_amdgcn_exp2f(s[q - 8]);
    } else if constexpr (q >= 24 && q < 28) {
      const int i = 4 * (q - 24);
      lsum += (s[i] + s[i + 1]) + (s[i + 2] + s[i + 3]);
    } else if constexpr (q == 28 || q == 31) {
      // P^T half kk (value MFMAs 16 kk .. 16 kk + 15 are issued by now; the
      // last one reads the registers this overwrites, so wait a few cycles)
      const int kk = q == 28 ? 0 : 1;
      if constexpr (q == 31) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)s[8 * kk + e];
      pc[kk] = v;
    } else if constexpr (q == 30 && !FAST) {
      if (D.last) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(lsum), __float_as_int(lsum), false, false);
        const float l = __int_as_float(sw[0]) + __int_as_float(sw[1]);
        cap_inv = l > 0.f ? a.kv_scale / l : 0.f;  // (an fp8 cache's V is its bytes times kv_scale)
        cap_lse = l > 0.f ? (m_ref + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
      }
    }
  };

  // ---- the value product of chunk t (slot at slot_off), optionally with the
  // softmax of chunk D between its MFMAs
  // with_smax: 0 = values only, 1 = with the softmax of D, 2 = with the fast
  // softmax of D
  auto value_loop = [&](uint32_t slot_off, auto with_smax, const Chunk& D) {
    constexpr int WS = decltype(with_smax)::value;
    constexpr std::integral_constant<bool, WS == 2> fast_tag{};
    lds_u8* vb[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int b = 0; b < 2; ++b) vb[cb][b] = launder(lds + slot_off + (v_lane ^ (64u * cb + 32u * b)));
    auto vfrag = [&](int f) -> bf16x8 {
      const int kk = f >> 4, ct = f & 15;
      const uint32_t off = 4096u * (ct >> 1) + 2048u * kk;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct & 1][0] + off));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb[ct & 1][1] + off + 1024u));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    constexpr int R = kVAhead + 2;
    bf16x8 vf[R];
#pragma unroll
    for (int f = 0; f < kVAhead; ++f) vf[f] = vfrag(f);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 2 * kColTiles>([&](auto fc) {
      constexpr int f = decltype(fc)::value;  // fragment f: tile f & 15 of k-step f >> 4
      if constexpr (f + kVAhead < 2 * kColTiles) vf[(f + kVAhead) % R] = vfrag(f + kVAhead);
      value_mfma1<(f & 15)>(vf[f % R], pc[f >> 4]);
      if constexpr (WS != 0) smax_piece(std::integral_constant<int, f>{}, D, fast_tag);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- the end of chunk D0's segment: this wave's rows of out and lse, or,
  // for a split sequence, its fp16 partial (O / l, scaled per row) and lse;
  // then clear the accumulators.  The partial of a split keeps the accumulator layout: per
  // 32-row tile, tile ct and element pair gp, 64 lanes x 16 bytes (elements
  // 8 gp .. 8 gp + 7 of the lane's 16), so every store is 1 KB contiguous.
  auto segment_end = [&](const Chunk& D0) {
    float inv = seg_inv, lse = seg_lse;
    if (seg_bad) {
      inv = __builtin_nanf("");
      lse = __builtin_nanf("");
    }
    mfma_result_wait();
    const RowInfo ri = row_info();
    const int row = ri.row;
    if (seg_nsplit == 1) {
      if (ri.ok) {
        uint16_t* op =
            a.out + (int64_t)D0.seq * a.o_sb + (int64_t)ri.qi * a.o_ss + (int64_t)ri.hh * a.o_sh + 4 * hlf;
        static_for<0, 4 * kColTiles>([&](auto ic) {
          constexpr int I = decltype(ic)::value;  // tile I >> 2, elements 4 (I & 3) ..
          const f32x4 v = acc_read4<I>() * inv;
          *(bf16x4*)(op + 32 * (I >> 2) + 8 * (I & 3)) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        });
        if (hlf == 0) a.lse[(int64_t)D0.seq * a.l_sb + (int64_t)ri.qi * a.l_ss + (int64_t)ri.hh * a.l_sh] = lse;
      }
    } else if (pi.blk_row0 + 32 * w < a.rows) {
      // fp16 partial (O / l) * 2^-e with 2^e the smallest power of two above
      // the row's largest |O / l| (the row's two lanes agree on it), so that
      // every element keeps 11 significant bits; 2^e goes to part_scale.
      // (rows past the last one store zeros into the tile's padding)
      float mx = 0.f;
      static_for<0, 4 * kColTiles>([&](auto ic) {
        const f32x4 v = acc_read4<decltype(ic)::value>();
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
      });
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
      mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1])) * fabsf(inv);
      // mx = f 2^e with f in [0.5, 1); an empty, NaN or overflowing row keeps e = 0
      const int e = (mx > 0.f && mx < INFINITY) ? __builtin_amdgcn_frexp_expf(mx) : 0;
      const float f = inv * __builtin_ldexpf(1.f, -e);
      uint8_t* pb = (uint8_t*)a.part_o + (int64_t)seg_slot * partial_slot_bytes(a.rows) +
                    (int64_t)((pi.blk_row0 >> 5) + w) * kPartialTileBytes + 16 * opaque(lane);
      static_for<0, 2 * kColTiles>([&](auto ic) {
        constexpr int I = decltype(ic)::value;  // tile I >> 1, elements 8 (I & 1) ..
        const f32x4 v0 = acc_read4<2 * I>() * f, v1 = acc_read4<2 * I + 1>() * f;
        *(f16x8*)(pb + 1024 * I) = f16x8{(_Float16)v0[0], (_Float16)v0[1], (_Float16)v0[2], (_Float16)v0[3],
                                         (_Float16)v1[0], (_Float16)v1[1], (_Float16)v1[2], (_Float16)v1[3]};
      });
      if (ri.ok && hlf == 0) {
        a.part_lse[(int64_t)seg_slot * a.rows + row] = lse;
        a.part_scale[(int64_t)seg_slot * a.rows + row] = __builtin_ldexpf(1.f, e);
      }
    }
    acc_zero();
    asm volatile("s_nop 4" ::: "memory");
  };

  // ---- prologue.  The descriptor batch comes first: its loads (the lengths,
  // unless the plan already holds them, then the block-table entries) would
  // otherwise complete only after everything issued before them.  Then the
  // copies of the part's first two chunks, then the first sequence's queries
  // (most of the bytes a part needs before its first step, and all parts
  // start at once).  With an fp8 cache: chunks 0 and 1 copied to staging,
  // chunk 0 converted to its bf16 slot, chunk 2 copied (it lands during step
  // -1, which converts chunk 1).
  const int seq0 = pi.seq_begin;
  BatchPos bpos;
  bpos.seq = seq0;
  bpos.chunk = 2 * pi.page_begin;
  bpos.more = true;
  int nk0;
  if constexpr (PLAN) {
    // (a cross-lane read: every lane takes part, whatever it keeps)
    const int sk = seq0 + lane;
    const int n = planned_length(plan_len, sk);
    nk0 = sk <= pi.seq_last ? clamp_len(a, n) : 0;
  } else {
    nk0 = batch_lengths(a, pi, bpos, lane);
  }
  i32x4 batch = desc_batch(a, pi, bpos, lane, nk0);
  int c0 = 0;  // chunk ordinal of the batch's first descriptor
  Chunk D0 = unpack_chunk(i32x4{-1, 0, 0, -1});  // chunk t: values
  Chunk D1 = batch_get(batch, 0);                // chunk t + 1: scores
  Chunk D2 = batch_get(batch, 1);                // chunk t + 2: landing (fp8: converted this step)
  Chunk D3 = batch_get(batch, 2);                // chunk t + 3: copied this step (fp8: in flight)
  Chunk D4 = KV8 ? batch_get(batch, 3) : D3;     // fp8: chunk t + 4, copied this step
  const uint32_t stage_base = (uint32_t)kSlots8 * kTileBytes;
  copy_chunk(D1, KV8 ? lds_addr + stage_base : lds_addr);
  copy_chunk(D2, KV8 ? lds_addr + stage_base + kStageBytes : lds_addr + kTileBytes);
  load_queries(Chunk{seq0, 0, 0, 0, false, false, false});
  // fp8: bf16 slots of chunks t, t + 1, t + 2 (rotating) and the staging
  // slot of chunks t + 2 and t + 4 (alternating with that of t + 3)
  uint32_t bs0 = 2 * kTileBytes, bs1 = 0, bs2 = kTileBytes;
  queries_ready();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (KV8) {
    convert_chunk(stage_base, 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    copy_chunk(D3, lds_addr + stage_base);
  }
  __syncthreads();

  for (int t = -1;; ++t) {
    if (!D0.valid() && !D1.valid()) break;
    const bool v_has = D0.valid() && D0.tok > 0;
    const bool s_has = D1.valid() && D1.tok > 0;
    uint32_t slot0, slot1, slot3;  // (slot3: where this step's copies go)
    if constexpr (KV8) {
      slot0 = bs0;
      slot1 = bs1;
      const uint32_t stage = stage_base + (uint32_t)(t & 1) * kStageBytes;  // chunks t + 2, t + 4
      convert_chunk(stage, bs2);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      slot3 = lds_addr + stage;
    } else {
      slot0 = (uint32_t)(t & 3) * kTileBytes;
      slot1 = (uint32_t)((t + 1) & 3) * kTileBytes;
      slot3 = lds_addr + (uint32_t)((t + 3) & 3) * kTileBytes;
    }
    const Chunk& Dc = KV8 ? D4 : D3;  // the chunk this step copies

    // the common step: full chunks inside one segment, no limit reached, no
    // pending rescale -- no segment bookkeeping, no masking, no results
    const bool fast = t >= 0 && v_has && D1.valid() && D1.tok == kChunk && !D0.first && !D0.last && !D0.bad &&
                      !D1.first && !D1.last && !pending && kChunk * (D1.chunk + 1) <= lim_min;
    if (fast) {
      score_loop(slot1, std::true_type{}, Dc, slot3);
      value_loop(slot0, std::integral_constant<int, 2>{}, D1);
    } else {
      // the values enter a new segment / close one
      if (D0.valid() && D0.first) {
        const int split = D0.seq == pi.seq_begin ? pi.split_first : 0;
        int s0, nsplit;
        segment_splits<PLAN>(a, D0.seq, (const lds_i32*)split_tab, s0, nsplit);
        seg_slot = s0 + split;
        seg_nsplit = nsplit;
        seg_bad = false;
      }
      if (D0.valid()) {
        seg_bad |= D0.bad;
        if (D0.last) {
          seg_inv = cap_inv;
          seg_lse = cap_lse;
        }
      }
      // the reference max of some rows moved at chunk t: rescale their sums
      if (pending) {
        if (v_has) {
          mfma_result_wait();
          acc_scale(pend_f);
          asm volatile("s_nop 4" ::: "memory");
        }
        pending = false;
        pend_f = 1.f;
      }

      if (D1.valid() && D1.first && t >= 0) {
        // ---- a new segment is scored: queries first, values of chunk t, the
        // end of its segment, then the scores and the softmax
        load_queries(D1);
        if (v_has) value_loop(slot0, std::integral_constant<int, 0>{}, D1);
        if (D0.valid() && D0.last) segment_end(D0);
        queries_ready();
        if (s_has)
          score_loop(slot1, std::false_type{}, Dc, slot3);
        else
          s = f32x16{};
        static_for<0, 2 * kColTiles>([&](auto qc) { smax_piece(qc, D1, std::false_type{}); });
        copy_chunk(Dc, slot3);
      } else {
        // A step that closes a segment issues its copies after the segment's
        // stores: stores count in the same vector memory counter, so copies
        // issued before them would have to land by this step's end.
        const bool closes = D0.valid() && D0.last;
        if (s_has && !closes)
          score_loop(slot1, std::true_type{}, Dc, slot3);
        else if (s_has)
          score_loop(slot1, std::false_type{}, Dc, slot3);
        else
          s = f32x16{};
        if (!s_has && !closes) copy_chunk(Dc, slot3);
        if (v_has)
          value_loop(slot0, std::integral_constant<int, 1>{}, D1);
        else if (D1.valid())
          static_for<0, 2 * kColTiles>([&](auto qc) { smax_piece(qc, D1, std::false_type{}); });
        if (closes) {
          segment_end(D0);
          copy_chunk(Dc, slot3);
        }
      }
    }

    // ---- end of step: this wave's share of chunk t + 2 (fp8: t + 3) has
    // landed (that of the chunk copied this step, the last vector memory loads
    // issued, may still be in flight; loads complete in order)
    static_assert(kCopiesW == 9 && kCopies8 == 5, "vmcnt below");
    if constexpr (KV8)
      asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    block_sync();
    D0 = D1;
    D1 = D2;
    D2 = D3;
    if constexpr (KV8) {
      D3 = D4;
      const uint32_t b = bs0;
      bs0 = bs1;
      bs1 = bs2;
      bs2 = b;
    }
    // the descriptor of the chunk copied next step (a new batch every 64 chunks)
    constexpr int kAhead = KV8 ? 5 : 4;
    if (t + kAhead - c0 >= 64) {
      batch = desc_batch(a, pi, bpos, lane, batch_lengths(a, pi, bpos, lane));
      c0 += 64;
    }
    if constexpr (KV8)
      D4 = batch_get(batch, t + kAhead - c0);
    else
      D3 = batch_get(batch, t + kAhead - c0);
  }
}

}  // namespace

hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_parts * a.row_blocks));
  if (a.kv8)
    hipLaunchKernelGGL((decode_wide_kernel<true, false>), grid, dim3(kThreadsW), 0, stream, a);
  else if (a.plan_in_kernel)
    hipLaunchKernelGGL((decode_wide_kernel<false, true>), grid, dim3(kThreadsW), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_wide_kernel<false, false>), grid, dim3(kThreadsW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

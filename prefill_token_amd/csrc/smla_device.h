// Device-side building blocks shared by the gfx950 kernels of the fused sparse-MLA step
// (smla_kernels.hip and smla_hs.hip): vector types, the kernels' argument block, the
// E4M3 / UE8M0 / bf16 conversions, buffer resources and LDS DMA, the E4M3 QK^T MFMA
// chain, the q prologue (RMSNorm + RoPE + the two-term E4M3 split or bf16), the output
// epilogue (inverse RoPE + UE8M0 / E4M3 quantization) and the RoPE table.  Everything
// sits in an unnamed namespace: each translation unit gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include <cmath>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int T = kTileRows;  // 64
constexpr int NTHREADS = 512;  // main kernel: 8 waves, two per SIMD
constexpr int NWAVES = NTHREADS / 64;
constexpr int CTHREADS = 128;  // combine kernel: one (token, head) per workgroup
constexpr int HP = 64;        // heads per workgroup (padded)

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
constexpr int align16(int x) { return (x + 15) & ~15; }

template <int D, int EB>  // EB: pool element bytes (1 = E4M3 + UE8M0 scales, 2 = bf16)
struct Cfg {
  static constexpr int kD = D, kEB = EB;
  static constexpr int RB = D * EB;     // bytes per pool row
  static constexpr int NCH = RB / 16;   // 16-byte chunks per row
  static constexpr int CE = 16 / EB;    // elements per chunk
  static constexpr int NSB = D / 32;    // UE8M0 bytes per row
  // Raw tile: one DMA instruction (64 lanes x 16 B) moves G rows, lane i carrying chunk
  // i / G of row i % G; the G rows are interleaved chunk by chunk, groups padded so that
  // eight consecutive rows read at one chunk land in eight distinct 16-byte bank slots.
  static constexpr int G = 1024 / RB;
  static constexpr int GS = 1024 + 16 * G;
  static constexpr int RAW_BYTES = (T / G) * GS;
  static constexpr int SC_BYTES = (EB == 1) ? T * NSB : 16;
  static constexpr int VT_BYTES = D * T * 2;  // [D][T] bf16, 128 B per dim
  static constexpr int P_BYTES = HP * T * 2;  // [HP][T] bf16, 128 B per head
  static constexpr int KS = D / 16;           // k-steps of the bf16 QK contraction
  static constexpr int KS8 = D / 64;          // k-steps of the E4M3 QK contraction
  static constexpr int KSW = KS / 2;          // ... per wave (each wave takes half the dims)
  static constexpr int KSW8 = KS8 / 2;
  static constexpr int PVW = (D / 32) < NWAVES ? (D / 32) : NWAVES;  // waves in P.V
  static constexpr int DQ = D / PVW;          // P.V output dims per wave
  static constexpr int NB = DQ / 32;          // 32-wide n-blocks per wave
  static constexpr int OFF_RAW0 = 0;
  static constexpr int OFF_RAW1 = OFF_RAW0 + RAW_BYTES;
  static constexpr int OFF_SC0 = OFF_RAW1 + RAW_BYTES;
  static constexpr int OFF_SC1 = OFF_SC0 + SC_BYTES;
  static constexpr int RAW_END = align16(OFF_SC1 + SC_BYTES);
  static constexpr int OFF_VT = RAW_END;
  static constexpr int OFF_P = OFF_VT + VT_BYTES;
  static constexpr int OFF_SX = OFF_P + P_BYTES;  // partial S of the 4 S blocks, f32
  static constexpr int LOOP_END = OFF_SX + 4 * 32 * 32 * 4;
  // prologue q tile: E4M3 pool -> two E4M3 terms [2][HP][QS8] + UE8M0 [2][HP][NSB];
  // bf16 pool -> bf16 [HP][QS]
  static constexpr int QS8 = D + 16;
  static constexpr int OFF_QSC = 2 * HP * QS8;
  static constexpr int QS = D + 8;
  static constexpr int Q_BYTES = (EB == 1) ? OFF_QSC + 2 * HP * NSB : HP * QS * 2;
  static constexpr int OS = D + 4;  // f32 stride of the epilogue o tile
  static constexpr int O_BYTES = HP * OS * 4;
  // the prologue's q tile sits after the raw tiles, so the first tile's DMA can land
  // while the prologue runs
  static constexpr int OFF_Q = RAW_END;
  static constexpr int BIG = align16(cmax(LOOP_END, cmax(OFF_Q + Q_BYTES, O_BYTES)));
  // small area: maxx[2][HP], alpha[HP], lsum[2][HP], cos[D/2], sin[D/2]
  static constexpr int OFF_MAXX = BIG;
  static constexpr int OFF_ALPHA = OFF_MAXX + 2 * HP * 4;
  static constexpr int OFF_LSUM = OFF_ALPHA + HP * 4;
  static constexpr int OFF_COS = OFF_LSUM + 2 * HP * 4;
  static constexpr int OFF_SIN = OFF_COS + (D / 2) * 4;
  static constexpr int OFF_FLAG = OFF_SIN + (D / 2) * 4;  // rescale flags of the 2 head groups
  static constexpr int SMEM = OFF_FLAG + 16;
  static_assert(G >= 1 && G <= 8 && (T % G) == 0 && ((T / G) % NWAVES) == 0, "row size unsupported");
  static_assert(KSW8 == 1 || KSW8 == 2 || KSW8 == 4, "k-steps per wave");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

// byte offset of chunk c of row r in a raw tile
template <class C>
__device__ __forceinline__ int raw_off(int r, int c) {
  return (r / C::G) * C::GS + 16 * (C::G * c + r % C::G);
}

// The UE8M0 scales of the k-steps a wave owns (dim half qd) for one row or head: byte j
// holds the scale of block 2(ks) + h, ks = KSW8*qd + j, h = lane half (hsel picks the
// bytes 2j + h of the 8 block scales of the half).
template <class C>
__device__ __forceinline__ uint32_t scale_word(const unsigned char* row_scales, int qd, uint32_t hsel) {
  if constexpr (C::NSB == 16) {
    const uint2 s2 = *reinterpret_cast<const uint2*>(row_scales + 8 * qd);
    return __builtin_amdgcn_perm(s2.y, s2.x, hsel);
  } else {
    static_assert(C::NSB == 4, "scale layout");
    const uint32_t s1 = *reinterpret_cast<const uint32_t*>(row_scales);
    return __builtin_amdgcn_perm(s1, s1, hsel) >> (8 * qd);
  }
}

struct KArgs {
  const uint16_t* q;
  const uint8_t* pool;
  const uint8_t* scales;
  const int32_t* indices;
  const int32_t* topk_length;
  const int32_t* positions;
  const float* norm_w;
  uint8_t* out_fp8;
  uint8_t* out_scales;
  float* out_f32;
  float* ws;         // split partials (after the scheduler state)
  unsigned* sched;   // work-item scheduler: [0] next item - gridDim.x, [1] finished workgroups
  const int* order;  // item taken in scheduling slot k (written by smla_order), or null: item k
  int s_q, h_q, rope_dim, topk, num_splits, tiles_per_split;
  long long n_rows;
  float sm_scale, rms_eps, rope_theta;
  double log2_theta;  // log2(rope_theta), computed on the host
  // two-pool (nvfp4_ds_mla) calls only: the NVFP4 pool of the compressed rows and where
  // an index row switches to it (pool / scales above are then the E4M3 SWA pool)
  const uint8_t* cmp_pool;    // E2M1 pairs [n_cmp][256]
  const uint8_t* cmp_scales;  // E4M3 [n_cmp][32], one per 16 elements
  long long n_cmp;
  int swa_entries;
};

__device__ __forceinline__ uint32_t cvt_lo(uint32_t src, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, sc, false));
}
__device__ __forceinline__ uint32_t cvt_hi(uint32_t src, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, sc, true));
}
// UE8M0 byte -> the f32 scale operand of the scaled converts (the hardware reads the
// exponent field as the E8M0 value, so e = 0 means 2^-127)
__device__ __forceinline__ float ue8m0_f32(uint32_t e) { return __builtin_bit_cast(float, e << 23); }

// smallest e in [0, 254] with 448 * 2^(e-127) >= amax (amax >= 0), decided on the f32 bits
__device__ __forceinline__ int ue8m0_exp(float amax) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
  int e = (int)(bits >> 23) - 8 + (((bits & 0x7FFFFFu) > 0x600000u) ? 1 : 0);
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// two f32 -> E4M3 codes (RNE) of x / 2^(e-127), into bytes 0-1 (hi = false) or 2-3
__device__ __forceinline__ uint32_t enc2(uint32_t old, float x0, float x1, float sc, bool hi) {
  s16x2 o = __builtin_bit_cast(s16x2, old);
  o = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, x0, x1, sc, true)
         : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, x0, x1, sc, false);
  return __builtin_bit_cast(uint32_t, o);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_f32(uint32_t h) { return __builtin_bit_cast(float, h << 16); }

// XOR swizzle of the 16-byte chunk index in 128-byte LDS rows (Vt rows indexed by dim,
// P rows indexed by head).  Eight consecutive rows get eight distinct slots (P.V reads);
// rows 16c + e for the chunk pattern of the V transpose also spread over all slots
// (bits 3-5 of the row enter through r >> 3 and r >> 6).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3) ^ (r >> 6)) & 7; }

// One split's partial in the workspace of the generic kernel: the f32 accumulator of HP
// heads x d dims, row-major [head][dim] (rows of heads >= h_q unused), then m [HP] and
// l [HP].  This is also the workspace stride the host sizes for.
__device__ __forceinline__ size_t partial_floats_d(int, int d) { return (size_t)HP * (size_t)(d + 2); }

// One split's partial of smla_ws (d = 512), in floats; about half the bytes of the f32
// form, so that the split's stores and the combine's loads move half as much:
//   [0, WSP_SCL): the accumulator in the P.V waves' register order as f16, each 32-dim
//     block of a head scaled by 2^(-E) with 2^E <= its amax < 2^(E+1), so that the values
//     lie in (-2, 2) (f16 keeps 11 significant bits: the rounding error is at most 2^-11
//     of the block amax).  The 16-byte slot (((v * 2 + mb) * 4 + nb) * 2 + g2) * 64 +
//     lrow + 32 lhalf holds registers 8 g2 .. 8 g2 + 7 of acc[mb][nb] of lane lrow +
//     32 lhalf of P.V wave v: dims 128v + 32nb + 16 g2 + 4 lhalf + {0..3, 8..11} of head
//     32 mb + lrow.  Each store instruction of a wave writes 1 KB contiguously.
//   [WSP_SCL, WSP_M): the decode scale 2^E (f32) of block gb of head h at gb * HP + h;
//   [WSP_M, WSP_L): m [HP]; [WSP_L, WSP_ROPE): l [HP];
//   [WSP_ROPE, WSP_FLOATS): the token's cos [32] and sin [32] of its rotary angles (every
//     split writes the same table), for the combine's inverse RoPE.
constexpr int WSP_SCL = HP * 512 / 2, WSP_M = WSP_SCL + HP * 16, WSP_L = WSP_M + HP, WSP_ROPE = WSP_L + HP,
              WSP_FLOATS = WSP_ROPE + 64;
static_assert(WSP_FLOATS <= HP * (512 + 2), "smla_ws partials fit the host's per-split stride");

// 2^(-E) and 2^E for a block amax a >= 0 (E from the f32 exponent field, kept where both
// are normal floats)
__device__ __forceinline__ void f16_block_scale(float a, float& enc, float& dec) {
  int eb = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFFu);
  eb = eb < 1 ? 1 : (eb > 253 ? 253 : eb);
  enc = __builtin_bit_cast(float, (uint32_t)(254 - eb) << 23);
  dec = __builtin_bit_cast(float, (uint32_t)eb << 23);
}
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  const f2v v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// LDS DMA (buffer_load_dword[x4] ... lds): every lane writes its 4 / 16 bytes at
// lds_base + 4*lane / 16*lane, read at byte offset voff of a buffer resource.  An
// offset at or beyond the resource's size reads as zeros, which is how entries that are
// not read (sentinels, beyond the length) become zero rows without a branch.  Whoever
// reads the rows waits for them (vmcnt 0) before the barrier that publishes them.
// dma16 / dma4 are issued from asm (no register results; M0 saved and restored), which the
// compiler schedules as written and does not count: the tile loops use them.  Vector
// loads retire in order, so the compiler's own waits stay correct (they can only
// over-wait).  dma16c / dma4c are the compiler's own LDS-DMA loads, which it counts like
// any other: an item's prologue issues its first tile with them after its q loads, so
// that the compiler's wait for q leaves the DMA in flight.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
constexpr uint32_t kNoRow = 0xFFFFFFF0u;  // an offset past every resource: zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(uint32_t voff, __amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void dma4(uint32_t voff, __amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void dma16c(uint32_t voff, __amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(size_t)lds_base, 16, voff,
                                           0, 0, 0);
}
__device__ __forceinline__ void dma4c(uint32_t voff, __amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(size_t)lds_base, 4, voff,
                                           0, 0, 0);
}

#ifdef SMLA_DEBUG_CHECKS
// Debug build only: entries that are read (j < topk_length) but lie outside [-1, n_rows),
// and read rows whose UE8M0 scales lie outside [kScaleMin, kScaleMax], set bits 1 and 2 of
// the error word after the scheduler counters (or-ed in, never cleared here).  One wave
// covers a tile: lane l holds entry l and reads the nsb scale bytes of slot l.
__device__ __noinline__ void debug_flag_tile(unsigned* sched, long long n_rows, bool in_len, int raw, bool valid,
                                             const unsigned char* row_scales, int nsb) {
  unsigned bits = 0;
  if (in_len && (raw < -1 || (long long)raw >= n_rows)) bits |= 1u;
  if (valid && row_scales)
    for (int b = 0; b < nsb; ++b) {
      const int e = row_scales[b];
      if (e < kScaleMin || e > kScaleMax) bits |= 2u;
    }
  const unsigned long long m1 = __ballot(bits & 1u), m2 = __ballot(bits & 2u);
  if ((threadIdx.x & 63) == 0 && (m1 | m2)) atomicOr(sched + kDebugWord, (m1 ? 1u : 0u) | (m2 ? 2u : 0u));
}
#endif

// lane permutation within rows of 16 lanes (DPP control CTRL), all lanes written
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// The same for a permutation that reads only lanes of the row itself (quad_perm): no
// "old" value to materialize, so the compiler can fold the move into the instruction that
// uses it (v_fmac_f32_dpp and the like).
template <int CTRL>
__device__ __forceinline__ float dpp_perm_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// A zero the compiler cannot see through: lane-dependent address math derived from it
// is recomputed where it is used instead of being hoisted (and kept live) across loops.
// Lane pair (l, l ^ 32) exchanges through v_permlane32_swap (one VALU op, no LDS round
// trip): swapping a register with itself leaves lanes 0..31 of the first result and lanes
// 32..63 of the second holding their own value, the other lanes their partner's, so each
// lane sees both values of its pair in the two results.
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {  // the value of lane l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, true, false);
  return (threadIdx.x & 32) ? (uint32_t)r[0] : (uint32_t)r[1];
}
__device__ __forceinline__ float pair_max(float v) {  // max over the pair, in both lanes
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), true, false);
  return fmaxf(__uint_as_float((uint32_t)r[0]), __uint_as_float((uint32_t)r[1]));
}
__device__ __forceinline__ float xor32_f32(float v) {  // the value of lane l ^ 32
  return __uint_as_float(xor32_u32(__float_as_uint(v)));
}
// the same for rows of 16 lanes: v_permlane16_swap exchanges rows 0 <-> 1 and 2 <-> 3
__device__ __forceinline__ float xor16_max(float v) {  // max over lanes l and l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), true, false);
  return fmaxf(__uint_as_float((uint32_t)r[0]), __uint_as_float((uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {  // sum over the pair, in both lanes
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), true, false);
  return __uint_as_float((uint32_t)r[0]) + __uint_as_float((uint32_t)r[1]);
}

__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// NST k-steps (64 dims each) of the E4M3 QK^T contraction, s (+)= sum_j K_j (q_hi,j + q_lo,j):
// the scaled MFMAs run back to back (srcC = vdst of the previous one, which needs no
// wait states), step j taking byte j of the scale registers.  Written as asm so that
// the chain stays back to back with all K fragments of the block loaded before it.  The
// leading s_nop covers a VALU write of an operand just before the block.
template <int NST, bool FIRST>
__device__ __forceinline__ void qk_block(f32x16& s, const i32x8* A, const i32x8* qh, const i32x8* ql, uint32_t ka,
                                         uint32_t sh, uint32_t sl) {
  static_assert(NST == 1 || NST == 2 || NST == 4, "k-steps per block");
  if constexpr (NST == 4 && FIRST) {
    asm volatile("s_nop 4\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %5, 0, %13, %14 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %9, %0, %13, %15 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %6, %0, %13, %14 op_sel:[1,1,0] op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %10, %0, %13, %15 op_sel:[1,1,0] op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %3, %7, %0, %13, %14 op_sel_hi:[1,1,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %3, %11, %0, %13, %15 op_sel_hi:[1,1,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %4, %8, %0, %13, %14 op_sel:[1,1,0] op_sel_hi:[1,1,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %4, %12, %0, %13, %15 op_sel:[1,1,0] op_sel_hi:[1,1,0]"
        : "=&v"(s)
        : "v"(A[0]), "v"(A[1]), "v"(A[2]), "v"(A[3]), "v"(qh[0]), "v"(qh[1]), "v"(qh[2]), "v"(qh[3]), "v"(ql[0]), "v"(ql[1]), "v"(ql[2]), "v"(ql[3]), "v"(ka), "v"(sh), "v"(sl));
  } else if constexpr (NST == 4 && !FIRST) {
    asm volatile("s_nop 4\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %5, %0, %13, %14 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %9, %0, %13, %15 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %6, %0, %13, %14 op_sel:[1,1,0] op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %10, %0, %13, %15 op_sel:[1,1,0] op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %3, %7, %0, %13, %14 op_sel_hi:[1,1,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %3, %11, %0, %13, %15 op_sel_hi:[1,1,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %4, %8, %0, %13, %14 op_sel:[1,1,0] op_sel_hi:[1,1,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %4, %12, %0, %13, %15 op_sel:[1,1,0] op_sel_hi:[1,1,0]"
        : "+v"(s)
        : "v"(A[0]), "v"(A[1]), "v"(A[2]), "v"(A[3]), "v"(qh[0]), "v"(qh[1]), "v"(qh[2]), "v"(qh[3]), "v"(ql[0]), "v"(ql[1]), "v"(ql[2]), "v"(ql[3]), "v"(ka), "v"(sh), "v"(sl));
  } else if constexpr (NST == 2 && FIRST) {
    asm volatile("s_nop 4\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %3, 0, %7, %8 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %5, %0, %7, %9 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %4, %0, %7, %8 op_sel:[1,1,0] op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %6, %0, %7, %9 op_sel:[1,1,0] op_sel_hi:[0,0,0]"
        : "=&v"(s)
        : "v"(A[0]), "v"(A[1]), "v"(qh[0]), "v"(qh[1]), "v"(ql[0]), "v"(ql[1]), "v"(ka), "v"(sh), "v"(sl));
  } else if constexpr (NST == 2 && !FIRST) {
    asm volatile("s_nop 4\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %3, %0, %7, %8 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %5, %0, %7, %9 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %4, %0, %7, %8 op_sel:[1,1,0] op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %2, %6, %0, %7, %9 op_sel:[1,1,0] op_sel_hi:[0,0,0]"
        : "+v"(s)
        : "v"(A[0]), "v"(A[1]), "v"(qh[0]), "v"(qh[1]), "v"(ql[0]), "v"(ql[1]), "v"(ka), "v"(sh), "v"(sl));
  } else if constexpr (NST == 1 && FIRST) {
    asm volatile("s_nop 4\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %4, %5 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %3, %0, %4, %6 op_sel_hi:[0,0,0]"
        : "=&v"(s)
        : "v"(A[0]), "v"(qh[0]), "v"(ql[0]), "v"(ka), "v"(sh), "v"(sl));
  } else if constexpr (NST == 1 && !FIRST) {
    asm volatile("s_nop 4\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %4, %5 op_sel_hi:[0,0,0]\n\t"
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %3, %0, %4, %6 op_sel_hi:[0,0,0]"
        : "+v"(s)
        : "v"(A[0]), "v"(qh[0]), "v"(ql[0]), "v"(ka), "v"(sh), "v"(sl));
  }
}
// After the last QK step: 32 wait states before anything reads s (covers the
// MFMA-write -> VALU/LDS-read and srcC WAR hazards of a 16-pass MFMA).
__device__ __forceinline__ void qk_drain(f32x16& s) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s)); }

// Inverse RoPE + UE8M0/E4M3 quantization of heads [0, nheads) held in o_lds (f32, row
// stride OSTR), writing global heads head0 + hl of token tok.  One thread per (head,
// 32-dim block), heads fastest across lanes: the block amax is lane-local and the
// rotary partner dims (x +- rope_dim/2, same head) are read from the tile itself.
template <int D, int NT>
__device__ void epilogue(const float* o_lds, int OSTR, int nheads, int head0, int tok, const KArgs& a,
                         const float* cs, const float* sn) {
  constexpr int NBK = D / 32;
  const int R = a.rope_dim, o0 = D - R, half = R / 2;
  for (int u = threadIdx.x; u < nheads * NBK; u += NT) {
    const int hl = u % nheads, b = u / nheads;
    const float* row = o_lds + hl * OSTR;
    float v[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 q4 = *reinterpret_cast<const float4*>(row + 32 * b + 4 * j);
      v[4 * j] = q4.x; v[4 * j + 1] = q4.y; v[4 * j + 2] = q4.z; v[4 * j + 3] = q4.w;
    }
    if (32 * b + 32 > o0) {  // rotary dims in this block (chunks of 4 never straddle o0)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int x = 32 * b + 4 * j;
        if (x >= o0) {
          const int k = x - o0;
          const bool lo = k < half;
          const int kk = lo ? k : k - half;
          const float4 pr = *reinterpret_cast<const float4*>(row + (lo ? x + half : x - half));
          const float4 c4 = *reinterpret_cast<const float4*>(cs + kk);
          const float4 s4 = *reinterpret_cast<const float4*>(sn + kk);
          const float sg = lo ? 1.f : -1.f;
          v[4 * j] = v[4 * j] * c4.x + sg * pr.x * s4.x;
          v[4 * j + 1] = v[4 * j + 1] * c4.y + sg * pr.y * s4.y;
          v[4 * j + 2] = v[4 * j + 2] * c4.z + sg * pr.z * s4.z;
          v[4 * j + 3] = v[4 * j + 3] * c4.w + sg * pr.w * s4.w;
        }
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    const size_t g = ((size_t)tok * a.h_q + head0 + hl) * D + 32 * b;
    if (a.out_f32) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        reinterpret_cast<float4*>(a.out_f32 + g)[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    }
    const int e = ue8m0_exp(amax);
    const float sc = ue8m0_f32((uint32_t)e);  // codes = RNE(o / 2^(e-127))
    uint32_t wd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wd[j] = enc2(enc2(0u, v[4 * j], v[4 * j + 1], sc, false), v[4 * j + 2], v[4 * j + 3], sc, true);
    reinterpret_cast<uint4*>(a.out_fp8 + g)[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    reinterpret_cast<uint4*>(a.out_fp8 + g)[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    a.out_scales[((size_t)tok * a.h_q + head0 + hl) * NBK + b] = (uint8_t)e;
  }
}

// cos / sin of angle pos * theta^(-2i/R), i < R/2, computed in fp64
__device__ __forceinline__ void rope_table(int pos, const KArgs& a, float* cs, float* sn) {
  // angle pos * theta^(-2i/r) in fp64, reduced to [-pi, pi] in fp64 (Cody-Waite with a
  // two-part 2*pi: |n| < 2^13, so n * hi is exact in the fma), then sin / cos in fp32
  // of the reduced angle.  Entry i is computed by lane i / nw of wave i % nw.
  constexpr double kInv2Pi = 0.15915494309189535, k2PiHi = 6.283185307179586, k2PiLo = 2.4492935982947064e-16;
  const int half = a.rope_dim / 2, nw = blockDim.x / 64;
  for (int i = (threadIdx.x & 63) * nw + (threadIdx.x >> 6); i < half; i += blockDim.x) {
    const double ang = (double)pos * exp2(-(2.0 * i / (double)a.rope_dim) * a.log2_theta);
    const double n = rint(ang * kInv2Pi);
    const double r = fma(-n, k2PiLo, fma(-n, k2PiHi, ang));
    float s, c;
    sincosf((float)r, &s, &c);
    cs[i] = c;
    sn[i] = s;
  }
}

// q prologue: RMSNorm + RoPE of the 64 (padded) heads of token t into the LDS q tile
// (two E4M3 terms + UE8M0 scales for the E4M3 pool, bf16 for the bf16 pool).  One thread
// per (head, 32-dim block), blocks fastest across lanes: the loads are contiguous per
// head, the sum of squares is reduced over the head's D/32 adjacent lanes with DPP, and
// the block amax of each term is lane-local; each lane reads its block of norm_w from
// global memory.  RoPE with rope_dim 64 (and d a multiple of 64) pairs dims of two
// adjacent blocks, so one DPP lane swap gives every lane its partners; other widths run
// densely through the f32 staging area ystage ([HP][R + 4]): the lanes holding rotary
// dims stage them, every thread rotates four (dim, dim + r/2) pairs, and the lanes read
// their rotated dims back.  The q tile goes to OFF_Q.  Also fills the cos / sin table,
// and calls after_loads() (every thread, once) as soon as the q loads are in flight.
template <class C, class Hook>
__device__ void q_prologue(unsigned char* smem, int t, int pos, const KArgs& a, float* cs, float* sn,
                           float* ystage, Hook&& after_loads) {
  constexpr int D = C::kD, EB = C::kEB;
  constexpr int NBK = D / 32;                           // lanes per head
  constexpr int NU = HP * NBK;                          // units
  constexpr int NIT = (NU + NTHREADS - 1) / NTHREADS;   // units per thread
  static_assert((NU % NTHREADS == 0 || NU < NTHREADS) && NU % 64 == 0 && NBK <= 16, "prologue mapping");
  const bool act = (int)threadIdx.x < NU;  // whole waves idle when NU < NTHREADS
  const int R = a.rope_dim, o0 = D - R, half = R / 2, RS = R + 4;
  const int b = threadIdx.x % NBK;  // the same block in every unit of this thread
  uint4 qraw[NIT][4];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int h = (threadIdx.x + NTHREADS * it) / NBK;
    const uint4* src = reinterpret_cast<const uint4*>(a.q + ((size_t)t * a.h_q + h) * D + 32 * b);
#pragma unroll
    for (int j = 0; j < 4; ++j) qraw[it][j] = (act && h < a.h_q) ? src[j] : make_uint4(0u, 0u, 0u, 0u);
  }
  // block b of norm_w, straight from global memory (the lanes of one block read the same
  // 128 bytes)
  float wv[32];
  {
    const float4* wsrc = reinterpret_cast<const float4*>(a.norm_w + 32 * b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 w4 = wsrc[j];
      wv[4 * j] = w4.x; wv[4 * j + 1] = w4.y; wv[4 * j + 2] = w4.z; wv[4 * j + 3] = w4.w;
    }
  }
  after_loads();
  if (R > 0) rope_table(pos, a, cs, sn);  // overlaps the loads above

  const bool rotb = act && 32 * b + 32 > o0;  // this lane's block holds rotary dims
  float y[NIT][32];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t uu[4] = {qraw[it][j].x, qraw[it][j].y, qraw[it][j].z, qraw[it][j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[it][8 * j + 2 * k] = bf16_f32(uu[k] & 0xFFFFu);
        y[it][8 * j + 2 * k + 1] = bf16_f32(uu[k] >> 16);
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) ss += y[it][e] * y[it][e];
    // sum over the NBK lanes of this head (a row of 16 lanes or a quad): lane pairs
    // i^1, i^2 (quad_perm), then i <-> 7-i and i <-> 15-i (half / full row mirror), so
    // that every lane adds the same two partial sums and ends with the same value
    ss += dpp_f32<0xB1>(ss);
    ss += dpp_f32<0x4E>(ss);
    if constexpr (NBK == 16) {
      ss += dpp_f32<0x141>(ss);
      ss += dpp_f32<0x140>(ss);
    }
    // the softmax scale (in log2 units) rides on q: the scores come out ready for exp2
    const float inv = (a.sm_scale * 1.4426950408889634f) * __builtin_amdgcn_rsqf(ss / (float)D + a.rms_eps);
#pragma unroll
    for (int e = 0; e < 32; ++e) y[it][e] = y[it][e] * inv * wv[e];
  }

  if (R == 64 && o0 % 64 == 0) {
    // the pair (o0 + k, o0 + 32 + k) lies in blocks o0/32 (even) and o0/32 + 1: lanes i and
    // i ^ 1, so one DPP lane swap brings every lane its partner's value
    __syncthreads();  // cos / sin table visible
    const bool lo_lane = (b & 1) == 0;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (rotb) {  // (both lanes of a pair are rotary lanes: the swap reads active lanes only)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float4 c4 = *reinterpret_cast<const float4*>(cs + 4 * j);
          const float4 s4 = *reinterpret_cast<const float4*>(sn + 4 * j);
          const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, ssn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * j + i;
            // the partner times the sine (the lane swap folded into the multiply), then
            // y c - p s on the lower lane of the pair, y c + p s on the upper one
            const float ps = dpp_perm_f32<0xB1>(y[it][e]) * ssn[i];
            y[it][e] = __builtin_fmaf(y[it][e], cc[i], lo_lane ? -ps : ps);
          }
        }
      }
    }
  } else if (R > 0) {
    __syncthreads();  // cos / sin table visible
    // stage the rotary dims (chunks of 4 never straddle o0 or o0 + r/2)
    if (rotb) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int h = (threadIdx.x + NTHREADS * it) / NBK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int x = 32 * b + 4 * j;
          if (x >= o0)
            *reinterpret_cast<float4*>(ystage + h * RS + (x - o0)) =
                make_float4(y[it][4 * j], y[it][4 * j + 1], y[it][4 * j + 2], y[it][4 * j + 3]);
        }
      }
    }
    __syncthreads();  // staged rotary values visible
    // forward rotation of the pairs (k, k + r/2), four consecutive k per step
    const int q4 = half / 4;
    for (int u = threadIdx.x; u < HP * q4; u += NTHREADS) {
      const int h = u / q4, k = 4 * (u % q4);
      float* row = ystage + h * RS;
      const float4 lo = *reinterpret_cast<const float4*>(row + k);
      const float4 hi = *reinterpret_cast<const float4*>(row + k + half);
      const float4 c4 = *reinterpret_cast<const float4*>(cs + k);
      const float4 s4 = *reinterpret_cast<const float4*>(sn + k);
      *reinterpret_cast<float4*>(row + k) = make_float4(lo.x * c4.x - hi.x * s4.x, lo.y * c4.y - hi.y * s4.y,
                                                        lo.z * c4.z - hi.z * s4.z, lo.w * c4.w - hi.w * s4.w);
      *reinterpret_cast<float4*>(row + k + half) = make_float4(hi.x * c4.x + lo.x * s4.x, hi.y * c4.y + lo.y * s4.y,
                                                               hi.z * c4.z + lo.z * s4.z, hi.w * c4.w + lo.w * s4.w);
    }
    __syncthreads();  // rotated values visible
    if (rotb) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int h = (threadIdx.x + NTHREADS * it) / NBK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int x = 32 * b + 4 * j;
          if (x >= o0) {
            const float4 v = *reinterpret_cast<const float4*>(ystage + h * RS + (x - o0));
            y[it][4 * j] = v.x; y[it][4 * j + 1] = v.y; y[it][4 * j + 2] = v.z; y[it][4 * j + 3] = v.w;
          }
        }
      }
    }
    __syncthreads();  // staging reads done: the q tile below may overwrite it
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (!act) break;
    const int h = (threadIdx.x + NTHREADS * it) / NBK;
    if constexpr (EB == 1) {
      // two E4M3 terms, each with its own UE8M0 scale per 32 dims
      unsigned char* qf8 = smem + C::OFF_Q;
      unsigned char* qsc = smem + C::OFF_Q + C::OFF_QSC;
      int eq = 0;
#pragma unroll
      for (int term = 0; term < 2; ++term) {
        if (term == 0) {
          float amax = 0.f;
#pragma unroll
          for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(y[it][e]));
          eq = ue8m0_exp(amax);
        } else {
          // the residual of an RNE E4M3 code is at most 16 of its scale units (half an
          // ulp of the top binade): 2^-4 of the first scale holds it unsaturated
          eq = eq >= 4 ? eq - 4 : 0;
        }
        const float sc = ue8m0_f32((uint32_t)eq);
        uint32_t wd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          wd[j] = enc2(enc2(0u, y[it][4 * j], y[it][4 * j + 1], sc, false), y[it][4 * j + 2], y[it][4 * j + 3], sc,
                       true);
        uint4* dst = reinterpret_cast<uint4*>(qf8 + (term * HP + h) * C::QS8 + 32 * b);
        dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
        qsc[(term * HP + h) * C::NSB + b] = (unsigned char)eq;
        if (term == 0) {  // residual for the second term
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wd[j], sc, false);
            const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wd[j], sc, true);
            y[it][4 * j] -= d0[0];
            y[it][4 * j + 1] -= d0[1];
            y[it][4 * j + 2] -= d1[0];
            y[it][4 * j + 3] -= d1[1];
          }
        }
      }
    } else {
      uint4* dst = reinterpret_cast<uint4*>(smem + C::OFF_Q + (h * C::QS + 32 * b) * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pk[k] = bf16_rne(y[it][8 * j + 2 * k]) | (bf16_rne(y[it][8 * j + 2 * k + 1]) << 16);
        dst[j] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
  }
}

// The argument block of every step kernel, from the launch arguments.
inline KArgs make_kargs(const LaunchArgs& x) {
  KArgs k = {};
  k.q = x.q;
  k.pool = static_cast<const uint8_t*>(x.kv_pool);
  k.scales = x.kv_scales;
  k.indices = x.indices;
  k.topk_length = x.topk_length;
  k.positions = x.positions;
  k.norm_w = x.norm_w;
  k.out_fp8 = x.out_fp8;
  k.out_scales = x.out_scales;
  k.out_f32 = x.out_f32;
  k.sched = static_cast<unsigned*>(x.workspace);
  k.order = nullptr;
  k.ws = reinterpret_cast<float*>(static_cast<unsigned char*>(x.workspace) + kSchedBytes);
  k.s_q = x.s_q;
  k.h_q = x.h_q;
  k.rope_dim = x.rope_dim;
  k.topk = x.topk;
  k.num_splits = x.num_splits;
  const int ntiles = (x.topk + kTileRows - 1) / kTileRows;
  k.tiles_per_split = (ntiles + x.num_splits - 1) / x.num_splits;
  if (k.tiles_per_split < 1) k.tiles_per_split = 1;
  k.n_rows = x.n_rows;
  k.sm_scale = x.sm_scale;
  k.rms_eps = x.rms_eps;
  k.rope_theta = x.rope_theta;
  k.log2_theta = std::log2((double)x.rope_theta);
  k.cmp_pool = x.cmp_pool;
  k.cmp_scales = x.cmp_scales;
  k.n_cmp = x.n_cmp;
  k.swa_entries = x.swa_entries;
  return k;
}

}  // namespace
}  // namespace smla

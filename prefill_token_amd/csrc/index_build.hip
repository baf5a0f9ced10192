// Index-row builder: the step that writes the index rows the sparse-MLA step reads.
//
// For token t at position p, row t of `indices` holds
//   [0, window)                 the sliding-window rows of positions p - window + s ..
//                               p - 1 + s (s = 1 when the token's own row is in its
//                               window), each p' mod n_swa, or -1 for p' < 0;
//   [window, window + k)        cmp_base + c for the k = min(k_cmp, n_valid[t]) candidate
//                               columns c with the largest logits, ascending;
//   [window + k, topk)          -1, written here (the caller need not pre-fill the row);
// and topk_length[t] = window + k.
//   [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: combine_topk_swa_indices
//    builds each token's SWA + compressed-cache index row and must write its own -1
//    sentinels]
//   [vLLM #64364 "latency_specialized decode", Validation: the top-k rule -- torch.topk's
//    k-th value, selected columns ascending, ties toward the lowest column]
// Logits are bf16 and ordered as torch orders them: NaN above every number, -0 equal to
// +0.  Everything is integer work on 16-bit order keys, so the rows are exact.
//
// One 256-thread workgroup per token.  The order keys of the token's candidates go to
// LDS (8 per thread and step); a two-pass radix select (high byte, then low byte; one
// 256-bin histogram per 16 lanes with LDS atomics, then a suffix scan) finds the k-th key and how
// many of the columns equal to it to keep; then each thread takes a contiguous chunk of
// columns, and two block scans (shuffle scans within waves; of the tied columns, then of
// the kept columns) give every thread its place in the ascending output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kIbThreads = 256, kIbWaves = kIbThreads / 64;
// Radix histograms: one copy per 16 lanes (the high byte of a bf16 key holds the sign and
// exponent, so the keys of a wave crowd into a few bins; 16 copies cut the same-address
// atomics of an instruction fourfold), rows padded to 260 words so that one bin of the
// copies falls in different banks.
constexpr int kIbCopies = kIbThreads / 16, kIbBinStride = 260;

// bf16 bits -> 16-bit key whose unsigned order is the value order (NaN highest, -0 = +0)
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  if ((b & 0x7F80u) == 0x7F80u && (b & 0x007Fu) != 0u) return 0xFFFFu;  // NaN
  if (b == 0x8000u) b = 0u;                                            // -0 -> +0
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// Inclusive scan over a wave of 64 lanes with DPP moves: shifts by 1, 2, 4 and 8 within
// each row of 16 lanes, then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// then the total of rows 0-1 into rows 2-3 (row_bcast:31).  Lanes with no source add 0.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Inclusive scan of one value per thread over the workgroup: the wave scan, then the wave
// totals through LDS.  One barrier: the caller puts a barrier between this call's reads
// of wtot and the next call's writes.
template <int NWAVES>
__device__ __forceinline__ int block_scan_incl_1b(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_scan_incl(v);
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int j = 0; j < NWAVES; ++j) add += j < w ? wtot[j] : 0;
  return v + add;
}

// The same with a closing barrier, so calls may follow each other directly.
template <int NWAVES = kIbWaves>
__device__ __forceinline__ int block_scan_incl(int v, int* wtot) {
  v = block_scan_incl_1b<NWAVES>(v, wtot);
  __syncthreads();
  return v;
}

// Radix pass over the keys selected by (key >> shift_sel) == sel (all keys when shift_sel
// is 16): histograms of byte (key >> shift) & 255, one per 16 lanes, summed per bin, then
// the bin where the count of keys at or above it first reaches `need`.  Returns the bin;
// *above = keys in higher bins.
__device__ __forceinline__ int radix_pass(const uint16_t* keys, int nv, int shift, int shift_sel, int sel, int need,
                                          int (*hist)[kIbBinStride], int* wtot, int* res, int* above) {
  const int tid = threadIdx.x, cp = tid >> 4;
#pragma unroll
  for (int j = 0; j < kIbCopies; ++j) hist[j][tid] = 0;
  __syncthreads();
  for (int c8 = tid; 8 * c8 < nv; c8 += kIbThreads) {
    const uint4 k8 = reinterpret_cast<const uint4*>(keys)[c8];
    const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = (int)((kw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      if (8 * c8 + e < nv && (shift_sel >= 16 || (k >> shift_sel) == sel)) atomicAdd(&hist[cp][(k >> shift) & 255], 1);
    }
  }
  __syncthreads();
  // suffix sums: thread tid takes bin b = 255 - tid, so the inclusive scan is S(b), the
  // count at or above b
  const int b = 255 - tid;
  int hb = 0;
#pragma unroll
  for (int j = 0; j < kIbCopies; ++j) hb += hist[j][b];
  const int s_b = block_scan_incl(hb, wtot), s_next = s_b - hb;
  if (s_b >= need && s_next < need) {
    res[0] = b;
    res[1] = s_next;
  }
  __syncthreads();
  const int bin = res[0];
  *above = res[1];
  __syncthreads();
  return bin;
}

__global__ __launch_bounds__(kIbThreads) void build_index_kernel(IndexArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ib_smem[];
  __shared__ int hist[kIbCopies][kIbBinStride], wtot[kIbWaves], res[2];
  uint16_t* keys = reinterpret_cast<uint16_t*>(ib_smem);  // [n_cand rounded up to 8]
  const int t = blockIdx.x, tid = threadIdx.x;
  const int p = a.positions[t];
  int nv = a.n_valid ? a.n_valid[t] : a.n_cand;
  nv = nv < 0 ? 0 : (nv > a.n_cand ? a.n_cand : nv);
  const int k = a.k_cmp < nv ? a.k_cmp : nv;
  int32_t* row = a.indices + (size_t)t * a.topk;
  // sliding window, then the -1 tail
  for (int j = tid; j < a.window; j += kIbThreads) {
    const long long q = (long long)p - a.window + a.self_in_window + j;
    row[j] = q >= 0 ? (int32_t)(q % a.n_swa) : -1;
  }
  for (int j = a.window + k + tid; j < a.topk; j += kIbThreads) row[j] = -1;
  if (tid == 0) a.topk_length[t] = a.window + k;
  if (k == 0) return;
  int32_t* out = row + a.window;
  if (k == nv) {  // every candidate is kept
    for (int c = tid; c < nv; c += kIbThreads) out[c] = a.cmp_base + c;
    return;
  }
  // order keys into LDS, 8 per thread and step (16-byte loads when the row allows them)
  const uint16_t* lg = a.logits + (size_t)t * a.n_cand;
  const bool vec = ((reinterpret_cast<uintptr_t>(lg) & 15) == 0);
  for (int c8 = tid; 8 * c8 < nv; c8 += kIbThreads) {
    uint32_t kw[4];
    if (vec && 8 * c8 + 8 <= a.n_cand) {
      const uint4 r = reinterpret_cast<const uint4*>(lg)[c8];
      const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) kw[j] = order_key(rw[j] & 0xFFFFu) | (order_key(rw[j] >> 16) << 16);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 8 * c8 + 2 * j;
        const uint32_t lo = c < nv ? order_key(lg[c]) : 0u, hi = c + 1 < nv ? order_key(lg[c + 1]) : 0u;
        kw[j] = lo | (hi << 16);
      }
    }
    reinterpret_cast<uint4*>(keys)[c8] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
  }
  __syncthreads();
  int above1, above0;
  const int b1 = radix_pass(keys, nv, 8, 16, 0, k, hist, wtot, res, &above1);
  const int b0 = radix_pass(keys, nv, 0, 8, b1, k - above1, hist, wtot, res, &above0);
  const int kth = (b1 << 8) | b0;
  const int need = k - above1 - above0;  // columns equal to the k-th key to keep (>= 1)
  // contiguous chunks of columns per thread (multiples of 8), in order
  const int chunk = 8 * ((nv + 8 * kIbThreads - 1) / (8 * kIbThreads));
  const int c0 = tid * chunk, c1 = (c0 + chunk < nv) ? c0 + chunk : nv;
  int gt = 0, eq = 0;
  for (int c = c0; c < c1; c += 8) {
    const uint4 k8 = reinterpret_cast<const uint4*>(keys)[c >> 3];
    const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = (int)((kw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      const bool in = c + e < c1;
      gt += in && kk > kth;
      eq += in && kk == kth;
    }
  }
  const int eq_before = block_scan_incl(eq, wtot) - eq;
  int take_eq = need - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
  const int mine = gt + take_eq;
  int pos = block_scan_incl(mine, wtot) - mine;
  for (int c = c0; c < c1 && mine > 0; c += 8) {
    const uint4 k8 = reinterpret_cast<const uint4*>(keys)[c >> 3];
    const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = (int)((kw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      if (c + e < c1 && (kk > kth || (kk == kth && take_eq > 0))) {
        if (kk == kth) --take_eq;
        out[pos++] = a.cmp_base + c + e;
      }
    }
  }
}

// The same selection with the keys in registers, for up to 256 * KPT candidates.
//
// Keys: two 16-bit order keys per register, built from a bf16 pair with packed 16-bit
// integer arithmetic.  This key order is the value order torch uses: -inf is 0, -0 and +0
// are both 0x7F80, +inf is 0xFF00 and every NaN is 0xFF01.  A column at or past the token's
// valid count gets key 0, the key of -inf.  Such a column lies after every valid column,
// and ties go to the lowest columns, so it is never kept: the valid columns always hold at
// least k keys at or above the k-th.
__device__ __forceinline__ uint32_t order_keys2(uint32_t w) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t s = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, w) >> (short)15);  // 0xFFFF per negative half
  const uint32_t x = w ^ s;                                       // h, or 0x7FFF - |h| for a negative half
  const uint32_t c = (s & 0xFF81FF81u) | (~s & 0x7F807F80u);      // + 0x7F80, or - 0x7F (mod 2^16)
  u16x2 k = __builtin_bit_cast(u16x2, x) + __builtin_bit_cast(u16x2, c);
  k = __builtin_elementwise_min(k, (u16x2){0xFF01, 0xFF01});      // NaN (both signs land above 0xFF00)
  return __builtin_bit_cast(uint32_t, k);
}

// Radix histograms of the register path: one copy per lane of a half-wave (lane & 31), so
// the lanes of one LDS cycle never add to the same word; rows of 257 words put one bin of
// the copies in different banks.
constexpr int kRegCopies = 32, kRegStride = 257, kRegHistWords = kRegCopies * kRegStride;
static_assert(kRegHistWords % 4 == 0, "the copies are cleared as whole 16-byte units");

// After a radix pass has filled COPIES histogram copies: the bin where the count of keys at
// or above it first reaches `need` (thread tid < 256 sums bin 255 - tid over the copies, and
// a scan gives the suffix counts); *above = keys in higher bins.  Writes wtot and res; the
// caller's next write of either comes after another barrier.
template <int NT, int COPIES>
__device__ __forceinline__ int radix_select_bin(const uint32_t* hist, int need, int* wtot, int* res, int* above) {
  const int tid = threadIdx.x, b = 255 - tid;
  int hb = 0;
  if (tid < 256) {
#pragma unroll
    for (int c = 0; c < COPIES; ++c) hb += (int)hist[c * kRegStride + b];
  }
  const int s_b = block_scan_incl_1b<NT / 64>(hb, wtot), s_next = s_b - hb;
  if (tid < 256 && s_b >= need && s_next < need) {
    res[0] = b;
    res[1] = s_next;
  }
  __syncthreads();
  *above = res[1];
  return res[0];
}

// The keys of thread tid's units (unit j: columns 8 (tid + NT j) .. + 7, JU units in use)
// and the high-byte histograms (cleared here).  VEC: JU 16-byte loads, issued
// unconditionally (the address clamped to the last valid unit) before the clearing, so the
// counts of each unit can start as its load lands; else 2-byte loads, clamped to the row.
// Columns at or past nv read as -inf (key 0); units past JU hold key 0 and are not counted.
template <int KPT, int NT, int JU, bool VEC>
__device__ __forceinline__ void row_keys_high_hist(uint32_t (&kp)[KPT / 2], const uint16_t* lg, int nv, int nu,
                                                   uint32_t* hist) {
  constexpr int NU = KPT / 8;
  static_assert(JU >= 1 && JU <= NU, "units in use");
  constexpr uint32_t kNegInf2 = 0xFF80FF80u;
  const int tid = threadIdx.x;
  uint32_t rw[JU][4];
  if (VEC) {
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int u = tid + NT * j;
      const uint4 r = reinterpret_cast<const uint4*>(lg)[u < nu ? u : nu - 1];
      rw[j][0] = r.x;
      rw[j][1] = r.y;
      rw[j][2] = r.z;
      rw[j][3] = r.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int u = tid + NT * j;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * u + e;
        h[e] = lg[c < nv ? c : nv - 1];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) rw[j][q] = h[2 * q] | (h[2 * q + 1] << 16);
    }
  }
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int q = tid; q < kRegHistWords / 4; q += NT) h4[q] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  uint32_t* hc = hist + (tid & 31) * kRegStride;
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    if (j >= JU) {
#pragma unroll
      for (int q = 0; q < 4; ++q) kp[4 * j + q] = 0u;
      continue;
    }
    const int u = tid + NT * j;
    uint32_t x[4] = {rw[j][0], rw[j][1], rw[j][2], rw[j][3]};
    if (8 * u + 8 > nv) {  // the unit holding nv, or past it: columns at or past nv read as -inf
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * u + e >= nv) x[e >> 1] = (x[e >> 1] & (0xFFFF0000u >> (16 * (e & 1)))) | (0xFF80u << (16 * (e & 1)));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = order_keys2(x[q]);
      kp[4 * j + q] = w;
      atomicAdd(&hc[(w >> 8) & 255u], 1u);
      atomicAdd(&hc[w >> 24], 1u);
    }
  }
  __syncthreads();
}

template <int KPT, int NT, bool VEC>
__device__ __forceinline__ void row_keys_high_hist_ju(uint32_t (&kp)[KPT / 2], const uint16_t* lg, int nv, int nu,
                                                      int ju, uint32_t* hist) {
  switch (ju) {
    case 1: row_keys_high_hist<KPT, NT, 1, VEC>(kp, lg, nv, nu, hist); break;
    case 2: row_keys_high_hist<KPT, NT, (2 <= KPT / 8 ? 2 : 1), VEC>(kp, lg, nv, nu, hist); break;
    case 3: row_keys_high_hist<KPT, NT, (3 <= KPT / 8 ? 3 : 1), VEC>(kp, lg, nv, nu, hist); break;
    case 4: row_keys_high_hist<KPT, NT, (4 <= KPT / 8 ? 4 : 1), VEC>(kp, lg, nv, nu, hist); break;
    case 5: row_keys_high_hist<KPT, NT, (5 <= KPT / 8 ? 5 : 1), VEC>(kp, lg, nv, nu, hist); break;
    case 6: row_keys_high_hist<KPT, NT, (6 <= KPT / 8 ? 6 : 1), VEC>(kp, lg, nv, nu, hist); break;
    case 7: row_keys_high_hist<KPT, NT, (7 <= KPT / 8 ? 7 : 1), VEC>(kp, lg, nv, nu, hist); break;
    default: row_keys_high_hist<KPT, NT, KPT / 8, VEC>(kp, lg, nv, nu, hist); break;
  }
}

// NT threads per token, the token's row split in units of 8 columns.  For the two radix
// passes thread tid holds units tid, tid + NT, ..., so every load of the row is coalesced,
// a short row still spreads over every thread, and the high-byte histogram takes each
// unit's keys as its load lands.  Rows whose candidate count is a multiple of 8 and whose
// start is 16-byte aligned are read in 16-byte units; others column by column.  For the
// output the keys move through LDS so that each thread holds consecutive units; one scan
// of (columns above, columns equal) then gives every thread its place in the column-order
// row and its share of the ties.
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void build_index_reg(IndexArgs a) {
  constexpr int NU = KPT / 8, NW = NT / 64;
  static_assert(KPT % 8 == 0 && KPT <= 64, "a thread's columns are whole units and one 64-bit mask");
  static_assert(NT % 256 == 0 && KPT * NT <= 0xFFFF, "one thread per bin; the scanned totals fit 16 bits");
  static_assert(KPT * NT * 2 <= kRegHistWords * 4, "the keys fit the LDS area for the move");
  __shared__ __attribute__((aligned(16))) uint32_t hist[kRegHistWords];
  __shared__ int wtot[NW], res[2];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int p = a.positions[t];
  int nv = a.n_valid ? a.n_valid[t] : a.n_cand;
  nv = nv < 0 ? 0 : (nv > a.n_cand ? a.n_cand : nv);
  const int k = a.k_cmp < nv ? a.k_cmp : nv;
  int32_t* row = a.indices + (size_t)t * a.topk;
  for (int j = tid; j < a.window; j += NT) {
    const long long q = (long long)p - a.window + a.self_in_window + j;
    row[j] = q >= 0 ? (int32_t)(q % a.n_swa) : -1;
  }
  for (int j = a.window + k + tid; j < a.topk; j += NT) row[j] = -1;
  if (tid == 0) a.topk_length[t] = a.window + k;
  if (k == 0) return;
  int32_t* out = row + a.window;
  if (k == nv) {
    for (int c = tid; c < nv; c += NT) out[c] = a.cmp_base + c;
    return;
  }
  const uint16_t* lg = a.logits + (size_t)t * a.n_cand;
  const int nu = (nv + 7) >> 3, ju = (nu + NT - 1) / NT;  // units with valid columns; units per thread in use
  const bool vec = (a.n_cand & 7) == 0 && (reinterpret_cast<uintptr_t>(lg) & 15) == 0;
  uint32_t kp[KPT / 2];
  if (vec)
    row_keys_high_hist_ju<KPT, NT, true>(kp, lg, nv, nu, ju, hist);
  else
    row_keys_high_hist_ju<KPT, NT, false>(kp, lg, nv, nu, ju, hist);
  int above1, above0;
  const int b1 = radix_select_bin<NT, kRegCopies>(hist, k, wtot, res, &above1);
  // low byte of the keys in bin b1: they are few, so 8 copies (lane & 7)
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int q = tid; q < 8 * kRegStride / 4; q += NT) h4[q] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  {
    uint32_t* hc = hist + (tid & 7) * kRegStride;
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      if (j < ju) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = kp[4 * j + q];
          if (((w >> 8) & 255u) == (uint32_t)b1) atomicAdd(&hc[w & 255u], 1u);
          if ((w >> 24) == (uint32_t)b1) atomicAdd(&hc[(w >> 16) & 255u], 1u);
        }
      }
    }
  }
  __syncthreads();
  const int b0 = radix_select_bin<NT, 8>(hist, k - above1, wtot, res, &above0);
  const int kth = (b1 << 8) | b0;
  const int need = k - above1 - above0;  // columns equal to the k-th key to keep (>= 1)
  // The kept columns come out in column order: move the keys through LDS (free now) so
  // that thread tid holds the ju consecutive units tid ju .. tid ju + ju - 1.  Unit u sits in
  // slot u ^ ((u >> 3) & 7), which keeps both the stores and the loads free of bank conflicts.
  {
    uint4* st = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int u = tid + NT * j;
      if (j < ju) st[u ^ ((u >> 3) & 7)] = make_uint4(kp[4 * j], kp[4 * j + 1], kp[4 * j + 2], kp[4 * j + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int u = tid * ju + j;
      if (j < ju) {
        const uint4 x = st[u ^ ((u >> 3) & 7)];
        kp[4 * j] = x.x;
        kp[4 * j + 1] = x.y;
        kp[4 * j + 2] = x.z;
        kp[4 * j + 3] = x.w;
      }
    }
  }
  const int c0 = 8 * ju * tid;  // this thread's first column
  // bit i of gtm / gem: column c0 + i is above / at or above the k-th key (sign bits of
  // kth - key and kth - 1 - key shifted in from the top index down; indices past the
  // units in use are skipped first and so leave their bits 0)
  constexpr int NMW = (KPT + 31) / 32;
  uint32_t gtw[2] = {0u, 0u}, gew[2] = {0u, 0u};
#pragma unroll
  for (int q = 0; q < NMW; ++q) {
    uint32_t ag = 0u, ae = 0u;
#pragma unroll
    for (int i = (KPT - 32 * q < 32 ? KPT - 32 * q : 32) - 1; i >= 0; --i) {
      const int idx = 32 * q + i;
      if ((idx >> 3) < ju) {
        const int key = (int)((kp[idx >> 1] >> (16 * (idx & 1))) & 0xFFFFu);
        ag = __builtin_amdgcn_alignbit(ag, (uint32_t)(kth - key), 31);
        ae = __builtin_amdgcn_alignbit(ae, (uint32_t)(kth - 1 - key), 31);
      }
    }
    gtw[q] = ag;
    gew[q] = ae;
  }
  const uint64_t gtm = gtw[0] | ((uint64_t)gtw[1] << 32);
  uint64_t eqm = (gew[0] | ((uint64_t)gew[1] << 32)) & ~gtm;
  // one scan of (columns above, columns equal) packed in 16-bit halves (each total is at
  // most 8 NT): the threads before this one keep all their columns above the k-th key and
  // min(need, ties before) of the ties, lowest columns first
  const int gt = __popcll(gtm), eq = __popcll(eqm);
  const int packed = gt | (eq << 16);
  const int before = block_scan_incl_1b<NW>(packed, wtot) - packed;
  const int gt_before = before & 0xFFFF, eq_before = before >> 16;
  int take_eq = need - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
  for (int drop = eq - take_eq; drop > 0; --drop) eqm &= ~(1ull << (63 - __clzll(eqm)));  // keep the lowest
  uint64_t keep = gtm | eqm;
  int pos = gt_before + (need < eq_before ? need : eq_before);
  for (; keep && pos < k; keep &= keep - 1) out[pos++] = a.cmp_base + c0 + (__ffsll((unsigned long long)keep) - 1);
}

}  // namespace

hipError_t launch_build_index(const IndexArgs& a) {
  if (a.s_q <= 0) return hipSuccess;
  // up to 16384 candidates: the keys in registers
  if (a.n_cand <= 16 * 256) {
    hipLaunchKernelGGL((build_index_reg<16, 256>), dim3((unsigned)a.s_q), dim3(256), 0, a.stream, a);
    return hipGetLastError();
  }
  if (a.n_cand <= 64 * 256) {
    hipLaunchKernelGGL((build_index_reg<64, 256>), dim3((unsigned)a.s_q), dim3(256), 0, a.stream, a);
    return hipGetLastError();
  }
  const size_t lds = (size_t)((a.n_cand + 7) & ~7) * 2;  // up to 128 KB of order keys
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_index_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_index_kernel, dim3((unsigned)a.s_q), dim3(kIbThreads), lds, a.stream, a);
  return hipGetLastError();
}

}  // namespace smla

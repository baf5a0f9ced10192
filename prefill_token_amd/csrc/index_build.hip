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
// LDS (8 per thread and step); a two-pass radix select (high byte, then low byte; per-wave
// 256-bin histograms with LDS atomics, then a suffix scan) finds the k-th key and how
// many of the columns equal to it to keep; then each thread takes a contiguous chunk of
// columns, and two block scans (shuffle scans within waves; of the tied columns, then of
// the kept columns) give every thread its place in the ascending output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kIbThreads = 256, kIbWaves = kIbThreads / 64;

// bf16 bits -> 16-bit key whose unsigned order is the value order (NaN highest, -0 = +0)
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  if ((b & 0x7F80u) == 0x7F80u && (b & 0x007Fu) != 0u) return 0xFFFFu;  // NaN
  if (b == 0x8000u) b = 0u;                                            // -0 -> +0
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// Inclusive scan of one value per thread over the workgroup: a shuffle scan within each
// wave, then the wave totals through LDS (two barriers).
__device__ __forceinline__ int block_scan_incl(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int j = 0; j < kIbWaves; ++j) add += j < w ? wtot[j] : 0;
  __syncthreads();
  return v + add;
}

// Radix pass over the keys selected by (key >> shift_sel) == sel (all keys when shift_sel
// is 16): per-wave histograms of byte (key >> shift) & 255 (fewer colliding LDS atomics),
// summed per bin, then the bin where the count of keys at or above it first reaches
// `need`.  Returns the bin; *above = keys in higher bins.
__device__ __forceinline__ int radix_pass(const uint16_t* keys, int nv, int shift, int shift_sel, int sel, int need,
                                          int (*hist)[256], int* wtot, int* res, int* above) {
  const int tid = threadIdx.x, w = tid >> 6;
#pragma unroll
  for (int j = 0; j < kIbWaves; ++j) hist[j][tid] = 0;
  __syncthreads();
  for (int c8 = tid; 8 * c8 < nv; c8 += kIbThreads) {
    const uint4 k8 = reinterpret_cast<const uint4*>(keys)[c8];
    const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = (int)((kw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      if (8 * c8 + e < nv && (shift_sel >= 16 || (k >> shift_sel) == sel)) atomicAdd(&hist[w][(k >> shift) & 255], 1);
    }
  }
  __syncthreads();
  // suffix sums: thread tid takes bin b = 255 - tid, so the inclusive scan is S(b), the
  // count at or above b
  const int b = 255 - tid;
  int hb = 0;
#pragma unroll
  for (int j = 0; j < kIbWaves; ++j) hb += hist[j][b];
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
  __shared__ int hist[kIbWaves][256], wtot[kIbWaves], res[2];
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

}  // namespace

hipError_t launch_build_index(const IndexArgs& a) {
  if (a.s_q <= 0) return hipSuccess;
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

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
// LDS; a two-pass radix select (high byte, then low byte, 256-bin histograms with LDS
// atomics and a suffix scan) finds the k-th key and how many of the columns equal to it
// to keep; then each thread takes a contiguous chunk of columns, and two block scans
// (of the tied columns, then of the kept columns) give every thread its place in the
// ascending output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kIbThreads = 256;

// bf16 bits -> 16-bit key whose unsigned order is the value order (NaN highest, -0 = +0)
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  if ((b & 0x7F80u) == 0x7F80u && (b & 0x007Fu) != 0u) return 0xFFFFu;  // NaN
  if (b == 0x8000u) b = 0u;                                            // -0 -> +0
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// Inclusive block scan of one value per thread (Hillis-Steele in LDS); buf has 256 slots.
__device__ __forceinline__ int block_scan_incl(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kIbThreads; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

// Radix pass over the keys selected by (key >> shift_sel) == sel (all keys when shift_sel
// is 16): histogram of byte (key >> shift) & 255, then the bin where the count of keys
// at or above it first reaches `need`.  Returns the bin; *above = keys in higher bins.
__device__ __forceinline__ int radix_pass(const uint16_t* keys, int nv, int shift, int shift_sel, int sel, int need,
                                          int* hist, int* buf, int* res, int* above) {
  const int tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  for (int c = tid; c < nv; c += kIbThreads) {
    const int k = keys[c];
    if (shift_sel >= 16 || (k >> shift_sel) == sel) atomicAdd(&hist[(k >> shift) & 255], 1);
  }
  __syncthreads();
  // suffix sums: thread b holds S(b) = sum of bins >= b (scan over the reversed bins)
  const int s_incl = block_scan_incl(hist[255 - tid], buf);  // = S(255 - tid)
  const int b = 255 - tid;
  const int s_b = s_incl, s_next = s_incl - hist[b];       // S(b + 1)
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
  __shared__ int hist[256], buf[256], res[2];
  uint16_t* keys = reinterpret_cast<uint16_t*>(ib_smem);
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
  const uint16_t* lg = a.logits + (size_t)t * a.n_cand;
  for (int c = tid; c < nv; c += kIbThreads) keys[c] = (uint16_t)order_key(lg[c]);
  __syncthreads();
  int above1, above0;
  const int b1 = radix_pass(keys, nv, 8, 16, 0, k, hist, buf, res, &above1);
  const int b0 = radix_pass(keys, nv, 0, 8, b1, k - above1, hist, buf, res, &above0);
  const int kth = (b1 << 8) | b0;
  const int need = k - above1 - above0;  // columns equal to the k-th key to keep (>= 1)
  // contiguous chunks of columns per thread, in order
  const int chunk = (nv + kIbThreads - 1) / kIbThreads;
  const int c0 = tid * chunk, c1 = (c0 + chunk < nv) ? c0 + chunk : nv;
  int gt = 0, eq = 0;
  for (int c = c0; c < c1; ++c) {
    const int kk = keys[c];
    gt += kk > kth;
    eq += kk == kth;
  }
  const int eq_before = block_scan_incl(eq, buf) - eq;
  int take_eq = need - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
  const int mine = gt + take_eq;
  int pos = block_scan_incl(mine, buf) - mine;
  for (int c = c0; c < c1; ++c) {
    const int kk = keys[c];
    if (kk > kth || (kk == kth && take_eq > 0)) {
      if (kk == kth) --take_eq;
      out[pos++] = a.cmp_base + c;
    }
  }
}

}  // namespace

hipError_t launch_build_index(const IndexArgs& a) {
  if (a.s_q <= 0) return hipSuccess;
  const size_t lds = (size_t)a.n_cand * 2;  // up to 128 KB of order keys
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_index_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_index_kernel, dim3((unsigned)a.s_q), dim3(kIbThreads), lds, a.stream, a);
  return hipGetLastError();
}

}  // namespace smla

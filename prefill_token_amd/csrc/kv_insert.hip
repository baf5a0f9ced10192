// KV insert: the producer of the pool rows the sparse-MLA step gathers.
//
// For each new token i with position p = positions[i] >= 0, the 512-dim latent kv[i]
// (bf16) is RMS-normalised with norm_w, rotated (rotate-half RoPE on the last rope_dim
// dims at angle p * theta^(-2j/rope_dim)), cut into 32-element blocks, and stored as one
// pool row: 512 E4M3FN codes in kv_pool[p mod n_swa] and 16 UE8M0 exponents in
// kv_scales[p mod n_swa].  The block exponent is the smallest e in [10, 254] with
// 448 * 2^(e-127) >= the block's max |y|, and the codes are the round-to-nearest-even
// E4M3FN values of y * 2^(127-e).  The floor of 10 keeps every row inside the scale
// range the step dequantizes exactly (a larger exponent never saturates a code: blocks
// whose values all lie below 448 * 2^-117 only lose bits to E4M3 subnormals and zero).
//   [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: the fp8 SWA cache row of
//    512 E4M3 bytes plus UE8M0 scales (528 B), written by an insert kernel]
//   [vLLM #64364 "latency_specialized decode", Details, change table: the KV cache write
//    is folded into the kernel that normalises and quantizes q and kv]
//   [vLLM #56344, Test Plan: insert checked against a port of the reference quantizer]
//
// All arithmetic is fp64: the input is bf16 (exact in fp64), and every integer the step
// produces (codes, exponents) is decided from fp64 values, so it can be compared bit for
// bit with an fp64 reference.  The op moves about 1.6 KB per token and is bound by
// latency at decode sizes and by HBM at prefill sizes; fp64 VALU work per element is a
// few dozen instructions, far below what would matter at either bound.
//
// Layout: one wave64 per token.  Lane l holds dims 8l .. 8l+7 (one 16-byte load of bf16);
// a 32-element block is the four lanes 4b .. 4b+3; with rope_dim = r the rotary pairs
// (d - r + j, d - r/2 + j) sit r/16 lanes apart at the same slot of their lanes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kInsWaves = 4;  // tokens per workgroup

__device__ __forceinline__ double shfl_d(double v, int src) {
  return __shfl(v, src);
}

// Round-to-nearest-even of |v| * 2^(-shift) for the 53-bit significand m (implicit one
// included): the integer quotient with ties to even.  shift >= 1.
__device__ __forceinline__ uint64_t rne_shift(uint64_t m, int shift) {
  if (shift >= 64) return 0;  // m < 2^53 <= half of the divisor
  const uint64_t q = m >> shift, rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  return q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
}

// E4M3FN code of v (|v| <= 448 by the caller's scale), from the bits of the double:
// value = m * 2^(E - 52) with m the 53-bit significand.  Normal E4M3 numbers at binary
// exponent E >= -6 have the quantum 2^(E-3); below 2^-6 the quantum stays 2^-9
// (subnormals).  The sign bit is kept, so -0 and negative values that round to zero
// give 0x80.
__device__ __forceinline__ uint32_t e4m3_rne(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(b >> 63) << 7;
  const int ex = (int)((b >> 52) & 0x7FF);
  if (ex == 0) return sign;  // zero (fp64 subnormals are far below the E4M3 grid)
  const uint64_t m = (b & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int E = ex - 1023;
  uint32_t code;
  if (E < -6) {
    // n quanta of 2^-9: shift by 52 - E - 9; n <= 8, and n = 8 is the code of 2^-6
    code = (uint32_t)rne_shift(m, 43 - E);
  } else {
    uint32_t n = (uint32_t)rne_shift(m, 49);  // in [8, 16]
    int e = E;
    if (n == 16) {
      n = 8;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | (n - 8);
    if (code > 0x7E) code = 0x7E;
  }
  return sign | code;
}

// UE8M0 exponent of a block with max magnitude amax: the smallest e in [0, 254] with
// 448 * 2^(e-127) >= amax.  With amax = s * 2^E, s in [1, 2): 448 = 1.75 * 2^8, so
// e - 127 = E - 8 when s <= 1.75 and E - 7 otherwise (decided on the significand bits).
__device__ __forceinline__ int ue8m0_block_exp(double amax) {
  const uint64_t b = (uint64_t)__double_as_longlong(amax);
  const int ex = (int)((b >> 52) & 0x7FF);
  if (ex == 0) return 0;  // amax == 0
  const uint64_t frac = b & 0xFFFFFFFFFFFFFull;
  const int E = ex - 1023;
  const int s = (frac <= (3ull << 50)) ? E - 8 : E - 7;  // 0.75 * 2^52 = 3 * 2^50
  const int e = s + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

#pragma clang fp contract(off)
__global__ __launch_bounds__(64 * kInsWaves) void kv_insert_kernel(KvInsertArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * kInsWaves + (int)(threadIdx.x >> 6);
  if (tok >= a.n) return;  // whole waves leave together (tok is wave-uniform)
  const int pos = a.positions[tok];
  if (pos < 0) return;
  const int row = pos % a.n_swa;
  constexpr int D = 512;

  // x: dims 8 lane .. 8 lane + 7
  const uint4 raw = reinterpret_cast<const uint4*>(a.kv + (size_t)tok * D)[lane];
  const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
  double y[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    y[2 * m] = (double)__uint_as_float(u[m] << 16);
    y[2 * m + 1] = (double)__uint_as_float(u[m] & 0xFFFF0000u);
  }
  // RMSNorm: y = x / sqrt(mean(x^2) + eps) * w
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += y[k] * y[k];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const double inv = 1.0 / sqrt(ss / (double)D + (double)a.rms_eps);
  const float4 w0 = reinterpret_cast<const float4*>(a.norm_w)[2 * lane];
  const float4 w1 = reinterpret_cast<const float4*>(a.norm_w)[2 * lane + 1];
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = y[k] * inv * (double)wv[k];

  // RoPE on the last r dims: lane l (first half) pairs with lane l + r/16 (second half).
  const int r = a.rope_dim;
  if (r > 0) {
    const int half = r / 2, o0 = D - r, lstep = r / 16;
    const int first0 = o0 / 8, second0 = (o0 + half) / 8;
    // angle j = 0 .. half-1: its cosine and sine, one per lane over the whole wave
    // (lanes j < half: cos, half <= lanes < 2 half: sin; half <= 256, in rounds of 64)
    const bool in_first = lane >= first0 && lane < second0;
    const bool in_second = lane >= second0;
    const int partner = in_first ? lane + lstep : (in_second ? lane - lstep : lane);
    double px[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) px[k] = shfl_d(y[k], partner);
    const int j0 = in_first ? 8 * lane - o0 : 8 * lane - o0 - half;  // angle of slot 0
    for (int base = 0; base < half; base += 32) {
      // lane L computes angle base + (L & 31): cos for L < 32, sin for L >= 32
      const int jj = base + (lane & 31);
      double cs = 0.0;
      if (jj < half) {
        const double ifreq = pow((double)a.rope_theta, -(2.0 * jj) / (double)r);
        const double ang = (double)pos * ifreq;
        cs = lane < 32 ? cos(ang) : sin(ang);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = j0 + k;  // this slot's angle (for rotary lanes)
        const bool mine = (in_first || in_second) && j >= base && j < base + 32;
        const double c = shfl_d(cs, (j - base) & 31);
        const double s = shfl_d(cs, 32 + ((j - base) & 31));
        if (mine) {
          // first half: a c - b s; second half: b c + a s (a = first, b = second)
          y[k] = in_first ? (y[k] * c - px[k] * s) : (y[k] * c + px[k] * s);
        }
      }
    }
  }

  // block-32 exponent (4 lanes), codes, stores
  double amax = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmax(amax, fabs(y[k]));
  amax = fmax(amax, __shfl_xor(amax, 1));
  amax = fmax(amax, __shfl_xor(amax, 2));
  const int e0 = ue8m0_block_exp(amax);
  const int e = e0 < kScaleMin ? kScaleMin : e0;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t c = e4m3_rne(ldexp(y[k], 127 - e));
    if (k < 4)
      lo |= c << (8 * k);
    else
      hi |= c << (8 * (k - 4));
  }
  reinterpret_cast<uint2*>(a.kv_pool + (size_t)row * D)[lane] = make_uint2(lo, hi);
  if ((lane & 3) == 0) a.kv_scales[(size_t)row * (D / 32) + (lane >> 2)] = (uint8_t)e;
}

}  // namespace

hipError_t launch_kv_insert(const KvInsertArgs& a) {
  if (a.n <= 0) return hipSuccess;
  const int blocks = (a.n + kInsWaves - 1) / kInsWaves;
  hipLaunchKernelGGL(kv_insert_kernel, dim3(blocks), dim3(64 * kInsWaves), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace smla

// The consumer of the step's FP8 output: the per-group output projection (wo_a) computed
// straight from the E4M3 codes and UE8M0 block-32 scales of the attention output and of
// the weight, on gfx950's scaled FP8 MFMA (no dequantization of either operand).
//
//   y[t][g][o] = sum over h < hg, i < d of  x(t, g*hg + h, i) * w(g, o, h*d + i)
//
// with x(t, h, i) = e4m3(x_fp8[t][h][i]) * 2^(x_scales[t][h][i/32] - 127) and
// w(g, o, k) = e4m3(w_fp8[g][o][k]) * 2^(w_scales[g][o][k/32] - 127); y is bf16 (round to
// nearest even from the f32 accumulator).
// [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: the kernel's FP8 output is fed
//  straight into the wo_a einsum; the E4M3 + UE8M0 block-32 output format of the step.]
//
// One wave64 per (32-token tile, group, 128-output tile).  Lane (n = lane & 31, half
// hf = lane >> 5).  Per 64-wide k-step, v_mfma_scale_f32_32x32x64_f8f6f4 with A = 32
// weight rows (M = outputs) and B = 32 token rows (N = tokens): a lane holds bytes
// [64ks + 16hf, +16) and [64ks + 32 + 16hf, +16) of its row, and its scale byte is that of
// block 2ks + hf (the MFMA's K block hf is bytes 0..15 of both lane halves' first
// registers, i.e. row block 2ks, and block 1 the second registers, row block 2ks + 1).
// The rows are read straight from HBM into registers through range-checked buffer loads
// (tokens past s_q read as zeros): all of the token rows' fragments at once, then each
// 32-output weight block's fragments at once, so that a wave waits for a few rounds of
// loads instead of one per MFMA.  Accumulator register i of a lane holds output
// 8 (i >> 2) + 4 hf + (i & 3) of the tile for token n, so a lane stores four runs of 4
// consecutive bf16 outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int WO_D = 512;      // attention output dims per head
constexpr int WO_NSB = WO_D / 32;
constexpr int WO_OT = 128;     // outputs per wave
constexpr int WO_NB = WO_OT / 32;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wo_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x8 wo_frag(__amdgpu_buffer_rsrc_t rs, uint32_t row_off, int ks, int hf) {
  const auto lo = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off + 64u * ks + 16u * hf, 0, 0);
  const auto hi = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off + 64u * ks + 32u + 16u * hf, 0, 0);
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__global__ __launch_bounds__(64) void wo_a_kernel(WoArgs a) {
  const int lane = threadIdx.x, n = lane & 31, hf = lane >> 5;
  const int t0 = blockIdx.x * 32, g = blockIdx.y, o0 = blockIdx.z * WO_OT;
  const int H = a.h_q, hg = a.heads_per_group, dout = a.d_out;
  const int t = t0 + n;
  const uint32_t krow = (uint32_t)hg * WO_D;  // weight row length in bytes
  // x: rows (t, head) of 512 bytes; tokens >= s_q fall outside the resource and read zeros
  const __amdgpu_buffer_rsrc_t xr = wo_rsrc(a.x, (uint32_t)a.s_q * H * WO_D);
  const __amdgpu_buffer_rsrc_t xs = wo_rsrc(a.x_scales, (uint32_t)a.s_q * H * WO_NSB);
  const __amdgpu_buffer_rsrc_t wr = wo_rsrc(a.w, (uint32_t)a.n_groups * dout * krow);
  const __amdgpu_buffer_rsrc_t ws = wo_rsrc(a.w_scales, (uint32_t)a.n_groups * dout * (krow / 32));
  f32x16 acc[WO_NB];
#pragma unroll
  for (int b = 0; b < WO_NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  for (int hh = 0; hh < hg; ++hh) {
    // all of the token rows' fragments first (one round of loads), then per 32-output
    // block all of its weight fragments, then that block's 8 MFMAs
    const uint32_t xrow = ((uint32_t)t * H + (uint32_t)(g * hg + hh)) * WO_D;
    const auto xsc = __builtin_amdgcn_raw_buffer_load_b128(xs, xrow / 32, 0, 0);
    i32x8 bx[WO_D / 64];
#pragma unroll
    for (int ks = 0; ks < WO_D / 64; ++ks) bx[ks] = wo_frag(xr, xrow, ks, hf);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads together, ahead of their uses
#pragma unroll
    for (int b = 0; b < WO_NB; ++b) {
      const uint32_t wrow = (uint32_t)(g * dout + o0 + 32 * b + n) * krow + (uint32_t)hh * WO_D;
      const auto wsc = __builtin_amdgcn_raw_buffer_load_b128(ws, wrow / 32, 0, 0);
      i32x8 aw[WO_D / 64];
#pragma unroll
      for (int ks = 0; ks < WO_D / 64; ++ks) aw[ks] = wo_frag(wr, wrow, ks, hf);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < WO_D / 64; ++ks) {
        // scale byte of block 2ks + hf: word ks / 2, byte 2 (ks & 1) + hf
        const int sh = 8 * (2 * (ks & 1) + hf);
        const int sx = (int)((xsc[ks >> 1] >> sh) & 0xFFu);
        const int sw = (int)((wsc[ks >> 1] >> sh) & 0xFFu);
        acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aw[ks], bx[ks], acc[b], 0, 0, 0, sw, 0, sx);
      }
    }
  }
  if (t >= a.s_q) return;
  uint16_t* yrow = a.y + ((size_t)t * a.n_groups + g) * dout + o0;
#pragma unroll
  for (int b = 0; b < WO_NB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = 32 * b + 8 * q + 4 * hf;
      *reinterpret_cast<uint2*>(yrow + o) =
          make_uint2(pk_bf16(acc[b][4 * q], acc[b][4 * q + 1]), pk_bf16(acc[b][4 * q + 2], acc[b][4 * q + 3]));
    }
}

}  // namespace

hipError_t launch_wo_a(const WoArgs& a) {
  const dim3 grid((unsigned)((a.s_q + 31) / 32), (unsigned)a.n_groups, (unsigned)(a.d_out / WO_OT));
  hipLaunchKernelGGL(wo_a_kernel, grid, dim3(64), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace smla

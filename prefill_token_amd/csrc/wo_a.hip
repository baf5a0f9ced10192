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
// One 256-thread workgroup per (64-token tile, group, 128-output tile); wave w computes
// tokens 32 (w & 1) .. + 31 x outputs 64 (w >> 1) .. + 63.  Per head of the group, the K
// = 512 bytes of the rows go in two phases of 256: all threads load the phase's token and
// weight rows with row-contiguous 16-byte loads (16 threads per row piece; range-checked
// buffer loads, tokens past s_q read zeros) into LDS tiles whose 16-byte chunk c of row r
// sits at chunk c ^ (r & 15), then each wave reads its MFMA fragments from LDS.  Per
// 64-wide k-step, v_mfma_scale_f32_32x32x64_f8f6f4 with A = 32 weight rows (M = outputs)
// and B = 32 token rows (N = tokens): a lane (row n = lane & 31, half hf = lane >> 5)
// holds bytes [64ks + 16hf, +16) and [64ks + 32 + 16hf, +16) of its row, and its scale
// byte is that of block 2ks + hf (the MFMA's K block hf is bytes 0..15 of both lane
// halves' first registers, i.e. row block 2ks, and block 1 the second registers, row
// block 2ks + 1); the scales come straight from HBM into registers.  Accumulator register
// i of a lane holds output 8 (i >> 2) + 4 hf + (i & 3) of its 32-output block for token
// n, so a lane stores four runs of 4 consecutive bf16 outputs per block.
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

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// LDS tiles of one phase (256 bytes of K = 4 k-steps): rows of 256 bytes, 16-byte chunk c
// of row r stored at chunk c ^ (r & 15), so that the 32 rows a fragment read touches spread
// over the banks.
constexpr int WO_TT = 64;            // tokens per workgroup
constexpr int WO_PH = 256;           // K bytes per phase
constexpr int WO_XT = WO_TT * WO_PH; // 16 KB
constexpr int WO_WT = WO_OT * WO_PH; // 32 KB

__device__ __forceinline__ int wo_sw(int r, int c) { return 16 * (c ^ (r & 15)); }

__global__ __launch_bounds__(256) void wo_a_kernel(WoArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char xt[WO_XT];
  __shared__ __attribute__((aligned(16))) unsigned char wt[WO_WT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hf = lane >> 5;
  const int th = w & 1, oh = w >> 1;  // this wave: tokens 32 th .., outputs 64 oh ..
  const int t0 = blockIdx.x * WO_TT, g = blockIdx.y, o0 = blockIdx.z * WO_OT;
  const int H = a.h_q, hg = a.heads_per_group, dout = a.d_out;
  const uint32_t krow = (uint32_t)hg * WO_D;  // weight row length in bytes
  // tokens >= s_q fall outside the resources and read zeros
  const __amdgpu_buffer_rsrc_t xr = wo_rsrc(a.x, (uint32_t)a.s_q * H * WO_D);
  const __amdgpu_buffer_rsrc_t xs = wo_rsrc(a.x_scales, (uint32_t)a.s_q * H * WO_NSB);
  const __amdgpu_buffer_rsrc_t wr = wo_rsrc(a.w, (uint32_t)a.n_groups * dout * krow);
  const __amdgpu_buffer_rsrc_t ws = wo_rsrc(a.w_scales, (uint32_t)a.n_groups * dout * (krow / 32));
  f32x16 acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  // tile loads: thread tid moves chunk c = tid & 15 of rows (tid >> 4) + 16 k
  const int lc = tid & 15, lr = tid >> 4;
  for (int hh = 0; hh < hg; ++hh) {
    const int head = g * hg + hh;
    // this lane's block scales: its token row and its two weight rows (whole head)
    const int t = t0 + 32 * th + n;
    const auto xsc = __builtin_amdgcn_raw_buffer_load_b128(xs, ((uint32_t)t * H + head) * WO_NSB, 0, 0);
    uint32_t wsc[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint32_t o = (uint32_t)(g * dout + o0 + 64 * oh + 32 * b + n);
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(ws, o * (krow / 32) + (uint32_t)hh * WO_NSB, 0, 0);
      wsc[b][0] = v[0]; wsc[b][1] = v[1]; wsc[b][2] = v[2]; wsc[b][3] = v[3];
    }
#pragma unroll
    for (int ph = 0; ph < WO_D / WO_PH; ++ph) {
      // row-contiguous loads of the phase's tiles (16 threads per 256-byte row piece)
      uint4 xv[WO_TT / 16], wv[WO_OT / 16];
#pragma unroll
      for (int k = 0; k < WO_TT / 16; ++k) {
        const int r = lr + 16 * k;
        const uint32_t off = ((uint32_t)(t0 + r) * H + head) * WO_D + WO_PH * ph + 16 * lc;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        xv[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
      for (int k = 0; k < WO_OT / 16; ++k) {
        const int r = lr + 16 * k;
        const uint32_t off = (uint32_t)(g * dout + o0 + r) * krow + (uint32_t)hh * WO_D + WO_PH * ph + 16 * lc;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
        wv[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      __syncthreads();  // the previous phase's fragment reads are done
#pragma unroll
      for (int k = 0; k < WO_TT / 16; ++k)
        *reinterpret_cast<uint4*>(xt + (lr + 16 * k) * WO_PH + wo_sw(lr + 16 * k, lc)) = xv[k];
#pragma unroll
      for (int k = 0; k < WO_OT / 16; ++k)
        *reinterpret_cast<uint4*>(wt + (lr + 16 * k) * WO_PH + wo_sw(lr + 16 * k, lc)) = wv[k];
      __syncthreads();  // the tiles are complete
#pragma unroll
      for (int kq = 0; kq < WO_PH / 64; ++kq) {
        const int ks = 4 * ph + kq;  // k-step within the head
        const int xrw = 32 * th + n;
        const uint4 xlo = *reinterpret_cast<const uint4*>(xt + xrw * WO_PH + wo_sw(xrw, 4 * kq + hf));
        const uint4 xhi = *reinterpret_cast<const uint4*>(xt + xrw * WO_PH + wo_sw(xrw, 4 * kq + 2 + hf));
        const i32x8 bx = {(int)xlo.x, (int)xlo.y, (int)xlo.z, (int)xlo.w, (int)xhi.x, (int)xhi.y, (int)xhi.z, (int)xhi.w};
        // scale byte of block 2ks + hf: word ks / 2, byte 2 (ks & 1) + hf
        const int sh = 8 * (2 * (ks & 1) + hf);
        const int sx = (int)((xsc[ks >> 1] >> sh) & 0xFFu);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int wrw = 64 * oh + 32 * b + n;
          const uint4 wlo = *reinterpret_cast<const uint4*>(wt + wrw * WO_PH + wo_sw(wrw, 4 * kq + hf));
          const uint4 whi = *reinterpret_cast<const uint4*>(wt + wrw * WO_PH + wo_sw(wrw, 4 * kq + 2 + hf));
          const i32x8 aw = {(int)wlo.x, (int)wlo.y, (int)wlo.z, (int)wlo.w, (int)whi.x, (int)whi.y, (int)whi.z, (int)whi.w};
          const int sw = (int)((wsc[b][ks >> 1] >> sh) & 0xFFu);
          acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aw, bx, acc[b], 0, 0, 0, sw, 0, sx);
        }
      }
    }
  }
  const int t = t0 + 32 * th + n;
  if (t >= a.s_q) return;
  uint16_t* yrow = a.y + ((size_t)t * a.n_groups + g) * dout + o0 + 64 * oh;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = 32 * b + 8 * q + 4 * hf;
      *reinterpret_cast<uint2*>(yrow + o) =
          make_uint2(pk_bf16(acc[b][4 * q], acc[b][4 * q + 1]), pk_bf16(acc[b][4 * q + 2], acc[b][4 * q + 3]));
    }
}

}  // namespace

hipError_t launch_wo_a(const WoArgs& a) {
  const dim3 grid((unsigned)((a.s_q + WO_TT - 1) / WO_TT), (unsigned)a.n_groups, (unsigned)(a.d_out / WO_OT));
  hipLaunchKernelGGL(wo_a_kernel, grid, dim3(256), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace smla

// Measured ceilings for the roofline figures (libsmla_probe.so, used by bench.py; not part
// of the step's ABI): a pure MFMA loop per data type, so that achieved fractions can be
// read against what this device sustains as well as against the published peaks.
//
//   smla_probe_mfma(kind, iters, blocks, stream, out): `blocks` workgroups of 256 threads
//   (four wave64), each wave issuing `iters` rounds of 8 independent MFMA chains
//   (kind 0: v_mfma_f32_32x32x16_bf16, kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3
//   operands with unit UE8M0 scales); one float per workgroup is written to out[blocks]
//   so that nothing is dead.  Returns the flops one launch performs, or -1 on a bad
//   argument / launch failure.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void probe_bf16(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  s += __shfl_xor(s, 1);
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_fp8(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + ((lane + i) & 3);  // small E4M3 values
    b[i] = 0x30303030 + ((lane * 3 + i) & 3);
  }
  const int unit = 0x7F7F7F7F;  // UE8M0 127: scale 1
  f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, unit, 0, unit);
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  s += __shfl_xor(s, 1);
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

}  // namespace

extern "C" double smla_probe_mfma(int kind, int iters, int blocks, void* stream, float* out) {
  if (iters < 1 || blocks < 1 || !out || (kind != 0 && kind != 1)) return -1.0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(probe_bf16, dim3(blocks), dim3(256), 0, s, iters, out);
  else
    hipLaunchKernelGGL(probe_fp8, dim3(blocks), dim3(256), 0, s, iters, out);
  if (hipGetLastError() != hipSuccess) return -1.0;
  const double per_mfma = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  return per_mfma * kChains * (double)iters * 4.0 * (double)blocks;
}

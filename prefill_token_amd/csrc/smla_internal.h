// Internal launch interface between the C ABI layer and the gfx950 kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace smla {

struct LaunchArgs {
  const uint16_t* q;          // bf16 bits [s_q][h_q][d]
  const void* kv_pool;        // u8 E4M3 [n_rows][d] or bf16 bits [n_rows][d]
  const uint8_t* kv_scales;   // u8 [n_rows][d/32] (E4M3 pool) or null
  const int32_t* indices;     // [s_q][topk]
  const int32_t* topk_length; // [s_q]
  const int32_t* positions;   // [s_q]
  const float* norm_w;        // [d]
  uint8_t* out_fp8;           // [s_q][h_q][d]
  uint8_t* out_scales;        // [s_q][h_q][d/32]
  float* out_f32;             // [s_q][h_q][d] or null
  void* workspace;            // scheduler state (kSchedBytes), then the item order (num_splits = 1) or the partials
  int s_q, h_q, d, rope_dim, topk, kv_format, num_splits;
  int64_t n_rows;
  float sm_scale, rms_eps, rope_theta;
  hipStream_t stream;
  // two-pool (nvfp4_ds_mla) calls: the NVFP4 pool of the compressed rows (null otherwise);
  // kv_pool / kv_scales are then the E4M3 SWA pool
  const uint8_t* cmp_pool = nullptr;    // E2M1 pairs [n_cmp][d/2]
  const uint8_t* cmp_scales = nullptr;  // E4M3 [n_cmp][d/16]
  int64_t n_cmp = 0;
  int swa_entries = 0;                  // index entries [0, swa_entries) name SWA rows
  // optional events recorded on the stream: before the main kernel, between it and the
  // split combine (or after it when there is none), and after the last kernel
  hipEvent_t ev_main = nullptr, ev_split = nullptr, ev_end = nullptr;
};

// Largest rotary width the two-pool kernel stages (its q prologue's staging area).
constexpr int kNvMaxRope = 96;

// Rows of the index row processed per tile by one workgroup.
constexpr int kTileRows = 64;

// Bytes at the start of the workspace holding the work-item scheduler's two counters
// (zero before a call, left zero by it), then the debug build's error word.
constexpr size_t kSchedBytes = 256;
constexpr int kDebugWord = 2;  // u32 index of the error word (byte offset 8)

// UE8M0 pool scales the step dequantizes exactly: every E4M3 value times 2^(e-127) is a
// normal bf16 number for e in [10, 246].  The KV insert writes no exponent below 10.
constexpr int kScaleMin = 10, kScaleMax = 246;

// Workspace floats per (token, split): acc [64][d] + m [64] + l [64] (slots for the
// largest head count, whatever h_q is).
inline size_t partial_floats(int, int d) { return (size_t)64 * (size_t)(d + 2); }

// Enqueue the step; returns the HIP error of the first failed launch (hipSuccess if none).
hipError_t launch(const LaunchArgs& a);

// Device address of the allocation-free entry point's static scratch on the current device
// (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

// Compute units of the current device (256 if it cannot be queried).
int device_cus();

// KV insert (the pool-row producer): one token per wave64, d = 512.
struct KvInsertArgs {
  const uint16_t* kv;        // bf16 bits [n][512]
  const int32_t* positions;  // [n]; tokens with a negative position are skipped
  const float* norm_w;       // [512]
  uint8_t* kv_pool;          // u8 E4M3 [n_rows][512]; row p mod n_swa is written
  uint8_t* kv_scales;        // u8 UE8M0 [n_rows][16]
  int n, rope_dim, n_swa;
  float rms_eps, rope_theta;
  hipStream_t stream;
};

hipError_t launch_kv_insert(const KvInsertArgs& a);

// Index-row builder: one 256-thread workgroup per token.
struct IndexArgs {
  const int32_t* positions;  // [s_q]
  const uint16_t* logits;    // bf16 bits [s_q][n_cand]
  const int32_t* n_valid;    // [s_q] or null (all n_cand candidates valid)
  int32_t* indices;          // [s_q][topk]
  int32_t* topk_length;      // [s_q]
  int s_q, n_cand, topk, window, self_in_window, n_swa, cmp_base, k_cmp;
  hipStream_t stream;
};

hipError_t launch_build_index(const IndexArgs& a);

// The FP8 output consumer (wo_a): y[t][g][o] = sum_{h < hg, i < 512} x(t, g hg + h, i) w(g, o, 512 h + i).
struct WoArgs {
  const uint8_t* x;         // E4M3 [s_q][h_q][512]
  const uint8_t* x_scales;  // UE8M0 [s_q][h_q][16]
  const uint8_t* w;         // E4M3 [n_groups][d_out][heads_per_group * 512]
  const uint8_t* w_scales;  // UE8M0 [n_groups][d_out][heads_per_group * 16]
  uint16_t* y;              // bf16 bits [s_q][n_groups][d_out]
  int s_q, h_q, heads_per_group, n_groups, d_out;
  hipStream_t stream;
};

hipError_t launch_wo_a(const WoArgs& a);

}  // namespace smla

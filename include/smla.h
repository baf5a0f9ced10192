/*
 * smla.h -- C ABI of the fused sparse-MLA attention step for AMD Instinct MI355X (gfx950).
 *
 * The operation [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose, first
 * bullet: the fused norm + RoPE + sparse-attention + inverse-RoPE + FP8-cast kernel]:
 * for every query token t and head h,
 *
 *   1. x = q[t, h, :] (bf16); y = x / sqrt(mean(x^2) + eps) * norm_w   (per-head RMSNorm,
 *      [SGLang #39370 "[DSV4.1] Combine DSpark decode and prefill kernel optimizations",
 *      Summary: q_head_norm])
 *   2. rotate-half RoPE on the last rope_dim dims of y at angle positions[t] * theta^(-2i/rope_dim)
 *   3. J = { j < min(topk_length[t], topk) : indices[t, j] >= 0 }  -- entries at or beyond
 *      topk_length are never read, -1 marks an empty slot
 *      [vLLM #56344, Purpose, bug-fix bullet: reads capped at topk_length, -1 sentinels]
 *   4. v_j = dequant(kv_pool[indices[t, j]]) -- one latent row per entry, used as both K
 *      and V by every head (MLA), stored as 512 E4M3 bytes + one UE8M0 scale per 32
 *      elements [vLLM #56344, Purpose: fp8 528 B rows]
 *   5. o = sum_j softmax_j(sm_scale * <y, v_j>) v_j  (o = 0 when J is empty)
 *   6. inverse RoPE (rotation by the negated angle) on the last rope_dim dims of o
 *   7. per 32-element block: e = smallest integer in [0, 254] with 448 * 2^(e-127) >= max|o|,
 *      out_scales = e, out_fp8 = round-to-nearest-even E4M3FN(o * 2^(127-e))
 *      [SGLang #39370, commit note on the MXFP8 epilogue: UE8M0 block scales]
 *
 * Every decode or prefill token carries its own row of metadata (position, index row,
 * length), so one call covers a flattened batch of tokens
 * [vLLM #56344, Purpose, second bullet].
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (HIP global memory) to contiguous
 *     row-major arrays owned by the caller.  The library keeps no reference after
 *     the call returns, allocates nothing and never synchronizes the device.
 *   - q, kv_pool, norm_w, out_fp8, out_f32 and the workspace must be 16-byte aligned,
 *     kv_scales 4-byte aligned (SMLA_ERR_VALUE otherwise).
 *   - The work is enqueued on params->stream (a hipStream_t; NULL = the null stream)
 *     and completes asynchronously; the call may be captured in a HIP graph.
 *   - Errors are reported by return code, never by exception or abort; the
 *     thread-local message of the last failure is available from
 *     sparse_mla_last_error().  Argument checks run on the host before any HIP call,
 *     so a rejected call launches nothing.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 5

/* return codes */
#define SMLA_OK 0
#define SMLA_ERR_NULL 1  /* a required pointer is NULL */
#define SMLA_ERR_SHAPE 2 /* unsupported d / rope_dim / h_q / topk combination, or a
                            pool of 4 GiB or more */
#define SMLA_ERR_VALUE 3 /* bad scalar (s_q < 0, n_rows < 1, non-finite or non-positive
                            sm_scale / rms_eps / rope_theta, workspace too small,
                            bad kv_format, num_splits out of range) or a misaligned
                            array pointer */
#define SMLA_ERR_HIP 4   /* a HIP launch failed */

/* kv_pool formats */
#define SMLA_KV_E4M3_UE8M0 0 /* kv_pool u8 [n_rows][d] E4M3FN codes, kv_scales u8 [n_rows][d/32] UE8M0 */
#define SMLA_KV_BF16 1       /* kv_pool bf16 bits u16 [n_rows][d], kv_scales unused (may be NULL) */

typedef struct smla_params {
  int32_t s_q;      /* number of query tokens (0 = no-op) */
  int32_t h_q;      /* heads per token, 1..64 */
  int32_t d;        /* latent / head dim: 128 or 512 */
  int32_t rope_dim; /* rotary dims at the end of each head: 0..d, a multiple of 16 */
  int32_t topk;     /* row stride of `indices` (entries per token), 0..65536 */
  int32_t kv_format;
  int64_t n_rows;   /* rows in kv_pool (>= 1); every read index must lie in [-1, n_rows).
                       The pool is addressed with 32-bit byte offsets: n_rows * row bytes
                       must stay below 4 GiB - 16 (SMLA_ERR_SHAPE otherwise) */
  float sm_scale;   /* softmax scale, finite and > 0 (typically 1/sqrt(d)) */
  float rms_eps;    /* RMSNorm epsilon, finite and > 0 */
  float rope_theta; /* RoPE base, finite and > 0 */
  int32_t num_splits; /* 0 = automatic: tiles (64 index entries) per split are the
                         fewest that keep s_q x splits within one round of the device's
                         compute units, and at least 2 once s_q x tiles exceeds 64; then
                         as many splits as those tiles need (1 when no count keeps one
                         round).  Else split each token's entries over this many
                         workgroups (1..64) and combine */
  float* out_f32;   /* optional f32 [s_q][h_q][d]: o after inverse RoPE, before the FP8
                       cast (NULL = not written) */
  void* workspace;  /* device scratch of >= sparse_mla_workspace_size(params) bytes
                       (NULL only when that size is 0).  Its first 256 bytes hold the
                       work-item scheduler's counters: they must be zero before the
                       first call on this workspace, and every call leaves them zero
                       (zero-fill a new workspace once).  The rest (the item order of
                       an unsplit call, or the split partials) is clobbered.  Calls
                       sharing a workspace must not overlap. */
  size_t workspace_bytes;
  void* stream;     /* hipStream_t */
} smla_params;

/*
 * The fused step (steps 1-7 above) for params->s_q tokens.
 *
 *   q           bf16 [s_q][h_q][d]            (device, read)
 *   kv_pool     see kv_format                 (device, read)
 *   kv_scales   u8 [n_rows][d/32] or NULL     (device, read)
 *   indices     i32 [s_q][topk]               (device, read) -1 = empty slot; entries
 *                                             j >= topk_length[t] are ignored whatever
 *                                             they hold
 *   topk_length i32 [s_q]                     (device, read) values > topk are capped at
 *                                             topk, values <= 0 mean no entries
 *   positions   i32 [s_q]                     (device, read) RoPE position of each token
 *   norm_w      f32 [d]                       (device, read) RMSNorm weight
 *   out_fp8     u8 [s_q][h_q][d]              (device, written) E4M3FN codes
 *   out_scales  u8 [s_q][h_q][d/32]           (device, written) UE8M0 exponents
 *   params      host pointer, read during the call only
 *
 * Preconditions not checked on the device (the values are in device memory): read
 * indices lie in [-1, n_rows) (an id outside that range is read as an empty slot, never
 * dereferenced); kv_scales of read rows lie in [SMLA_KV_SCALE_MIN, SMLA_KV_SCALE_MAX] =
 * [10, 246], the range in which every dequantized E4M3 value is a normal bf16 number
 * (outside it, tiny values are rounded by the hardware conversion and huge ones
 * overflow).  sparse_mla_kv_insert writes rows in that range.  The debug build
 * (libsmla_debug.so, see sparse_mla_debug_checks) reports violations of both.
 *
 * Returns SMLA_OK, or SMLA_ERR_* with nothing launched (SMLA_ERR_HIP: a launch failed).
 */
int sparse_mla_fwd(const void* q, const void* kv_pool, const uint8_t* kv_scales,
                   const int32_t* indices, const int32_t* topk_length, const int32_t* positions,
                   const float* norm_w, uint8_t* out_fp8, uint8_t* out_scales,
                   const smla_params* params);

/*
 * The step over the two-pool nvfp4_ds_mla cache [vLLM #56344 "Deepseek V41 Attention
 * MegaKernel", Purpose: fp8 528 B SWA rows + fp4 288 B compressed rows, index segments of
 * their own; Performance: 1.38x the KV token capacity at 8k context].  Steps 1-7 above with
 * the rows of entry j of an index row taken from
 *   j <  swa_entries:  the SWA pool, E4M3 + UE8M0 as kv_format 0 (swa_pool u8 [n_rows][512],
 *                      swa_scales u8 [n_rows][16]; the same scale range as sparse_mla_fwd);
 *   j >= swa_entries:  the compressed pool, NVFP4: cmp_pool u8 [n_cmp_rows][256] holds the
 *                      E2M1 codes of a row, element 2i in the low nibble of byte i and 2i + 1
 *                      in the high nibble; cmp_scales u8 [n_cmp_rows][32] one E4M3 scale per
 *                      16 elements; value = e2m1(code) * e4m3(scale)  (OCP E2M1: sign, two
 *                      exponent bits with bias 1, one mantissa bit; no per-tensor scale).
 * An id that is negative or outside the pool its segment names is read as an empty slot
 * (never dereferenced).  Arithmetic: rows are dequantized
 * exactly to bf16, q' (after norm and RoPE, times sm_scale) is rounded to bf16, QK^T and
 * P.V accumulate in f32; the output codec is the same.
 *
 *   base          the shapes and scalars as for sparse_mla_fwd: d = 512, kv_format
 *                 SMLA_KV_E4M3_UE8M0 (the SWA pool), n_rows = SWA rows, rope_dim <= 96;
 *                 workspace of sparse_mla_workspace_size(&base) bytes (the same split rule)
 *   n_cmp_rows    rows of the compressed pool (>= 1; n_cmp_rows * 256 below 4 GiB)
 *   swa_entries   the segment boundary, a multiple of 64 in [0, 65536]
 * cmp_pool must be 16-byte aligned, cmp_scales 4-byte aligned; the rest as sparse_mla_fwd.
 * Returns SMLA_OK or SMLA_ERR_* with nothing launched.
 */
typedef struct smla_ds_params {
  smla_params base;
  int64_t n_cmp_rows;
  int32_t swa_entries;
  int32_t reserved; /* 0 */
} smla_ds_params;

int sparse_mla_fwd_ds_nvfp4(const void* q, const uint8_t* swa_pool, const uint8_t* swa_scales,
                            const uint8_t* cmp_pool, const uint8_t* cmp_scales, const int32_t* indices,
                            const int32_t* topk_length, const int32_t* positions, const float* norm_w,
                            uint8_t* out_fp8, uint8_t* out_scales, const smla_ds_params* params);

/*
 * Allocation-free variant of sparse_mla_fwd, for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, layouts, results and errors as sparse_mla_fwd, except
 * that params->workspace and workspace_bytes are ignored: the scratch (scheduler counters,
 * item order, split partials) is a static device array of SMLA_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends.  The call allocates nothing
 * and calls no allocating routine.
 *
 * The split count is sparse_mla_fwd's for the same params when that call's scratch fits the
 * array; with num_splits = 0 a split call too large for it runs unsplit (one split) instead
 * (sparse_mla_noalloc_num_splits returns the count used).  A call whose scratch cannot fit
 * (an explicit num_splits too large for the array, or more than about 8.9 M tokens) returns
 * SMLA_ERR_VALUE with nothing launched.  The array's scheduler counters are zero when the
 * library loads and every call leaves them zero.
 *
 * All calls on one GPU share its array: calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and must not be made; successive calls on one
 * stream are fine.  In the debug build the error word sits at byte SMLA_DEBUG_WORD_OFFSET
 * of the array, where the caller cannot read it.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (34u << 20)
int sparse_mla_fwd_noalloc(const void* q, const void* kv_pool, const uint8_t* kv_scales,
                           const int32_t* indices, const int32_t* topk_length, const int32_t* positions,
                           const float* norm_w, uint8_t* out_fp8, uint8_t* out_scales,
                           const smla_params* params);

/* Splits per token sparse_mla_fwd_noalloc uses for these parameters (>= 1), or 0 for
   parameters it would reject. */
int sparse_mla_noalloc_num_splits(const smla_params* params);

/*
 * Bytes of device workspace sparse_mla_fwd needs for these parameters: 256 bytes of
 * scheduler state, then either 4 * s_q bytes rounded up to 256 (the order in which an
 * unsplit call takes its tokens) or, when the call is split, the split partials (0 when
 * s_q = 0).
 * Depends on s_q, d, topk and num_splits, and with num_splits = 0 on the current
 * device's compute-unit count.  Returns 0 for parameters sparse_mla_fwd would reject.
 */
size_t sparse_mla_workspace_size(const smla_params* params);

/* The number of splits per token sparse_mla_fwd will use for these parameters (>= 1),
   or 0 for parameters it would reject. */
int sparse_mla_num_splits(const smla_params* params);

/*
 * KV insert: the producer of the pool rows sparse_mla_fwd gathers (the step before it).
 * For every new token i with p = positions[i] >= 0:
 *
 *   1. x = kv[i, :] (bf16); y = x / sqrt(mean(x^2) + rms_eps) * norm_w      (RMSNorm)
 *   2. rotate-half RoPE on the last rope_dim dims of y at angle p * rope_theta^(-2j/rope_dim)
 *   3. per 32-element block: e = smallest integer in [10, 254] with 448 * 2^(e-127) >= max|y|,
 *      kv_scales[p mod n_swa, block] = e,
 *      kv_pool[p mod n_swa, block elements] = round-to-nearest-even E4M3FN(y * 2^(127-e))
 *
 * [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: the fp8 SWA cache row, 512
 *  E4M3 bytes plus UE8M0 scales, written by an insert kernel; vLLM #64364
 *  "latency_specialized decode", Details, change table: the KV cache write folded into the
 *  norm + quantization kernel.]  Rows 0 .. n_swa-1 of the pool are the sliding-window ring;
 * a token's row is its position modulo n_swa.  Tokens with a negative position are
 * skipped (their rows are left as they are).  The arithmetic is fp64, so the codes and
 * exponents are those of an exact-arithmetic evaluation of steps 1-3 (up to the last-bit
 * rounding of the sum of squares and the cosine / sine).
 *
 *   kv          bf16 [n][512]            (device, read; 16-byte aligned)
 *   positions   i32 [n]                  (device, read)
 *   norm_w      f32 [512]                (device, read; 16-byte aligned)
 *   kv_pool     u8 [n_rows][512]         (device, rows p mod n_swa written; 16-byte aligned)
 *   kv_scales   u8 [n_rows][16]          (device, rows p mod n_swa written; 4-byte aligned)
 *   params      host pointer, read during the call only
 *
 * The exponent floor of 10 (SMLA_KV_SCALE_MIN) keeps every written row inside the scale
 * range sparse_mla_fwd decodes exactly; the top of that range (246) holds whenever every
 * |norm_w| is below 2^123 (|y| <= sqrt(512) max|norm_w| after the norm).
 *
 * Preconditions not checked on the device: the non-negative positions of one call fall
 * on distinct rows (distinct modulo n_swa); rows written by two tokens of one call hold
 * an unspecified mixture.  |norm_w| < 2^123.  Same conventions as sparse_mla_fwd otherwise (asynchronous on
 * params->stream, nothing allocated, errors by return code with nothing launched).
 */
typedef struct smla_kv_insert_params {
  int32_t n;        /* tokens to insert (0 = no-op) */
  int32_t d;        /* latent dim: 512 */
  int32_t rope_dim; /* rotary dims at the end of the row: 0..d, a multiple of 16 */
  int32_t n_swa;    /* sliding-window rows at the start of the pool: 1..n_rows */
  int64_t n_rows;   /* rows of kv_pool; n_rows * 512 must stay below 4 GiB */
  float rms_eps;    /* RMSNorm epsilon, finite and > 0 */
  float rope_theta; /* RoPE base, finite and > 0 */
  void* stream;     /* hipStream_t */
} smla_kv_insert_params;

int sparse_mla_kv_insert(const void* kv, const int32_t* positions, const float* norm_w, uint8_t* kv_pool,
                         uint8_t* kv_scales, const smla_kv_insert_params* params);

/*
 * Index-row builder: writes the index rows and lengths sparse_mla_fwd reads (the step
 * before it).  For token t at position p, row t of `indices` holds
 *
 *   [0, window)             the sliding-window rows of positions p - window + s .. p - 1 + s
 *                           (s = self_in_window), each p' mod n_swa, or -1 for p' < 0;
 *   [window, window + k)    cmp_base + c for the k = min(k_cmp, n_valid[t]) candidate columns
 *                           c < n_valid[t] with the largest logits, in ascending column order;
 *   [window + k, topk)      -1 (written by the call: the row needs no pre-fill);
 *
 * and topk_length[t] = window + k.  The top-k rule is torch.topk's: order by value, NaN
 * above every number, -0 equal to +0, ties toward the lowest column
 * [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: combine_topk_swa_indices
 *  must write its own -1 sentinels; vLLM #64364 "latency_specialized decode", Validation:
 *  the top-k kernel's specified output].  The rows are exact (integer work only).
 *
 *   positions    i32 [s_q]               (device, read)
 *   logits       bf16 [s_q][n_cand]      (device, read; 2-byte aligned) candidate scores
 *   n_valid      i32 [s_q] or NULL       (device, read) candidates of each token (clamped to
 *                                        [0, n_cand]); NULL = all n_cand
 *   indices      i32 [s_q][topk]         (device, written)
 *   topk_length  i32 [s_q]               (device, written)
 *   params       host pointer, read during the call only
 *
 * Same conventions as sparse_mla_fwd (asynchronous on params->stream, nothing allocated,
 * errors by return code with nothing launched).
 */
typedef struct smla_index_params {
  int32_t s_q;            /* tokens (0 = no-op) */
  int32_t n_cand;         /* candidate columns per token: 0..65536 */
  int32_t topk;           /* row stride of indices: window + k_cmp .. 65536 */
  int32_t window;         /* sliding-window entries: 0..n_swa */
  int32_t self_in_window; /* 1: the window ends at the token's own position; 0: just before it */
  int32_t n_swa;          /* sliding-window ring rows (>= 1) */
  int32_t cmp_base;       /* pool row of candidate column 0 (>= 0; cmp_base + n_cand < 2^31) */
  int32_t k_cmp;          /* compressed entries kept per token: 0..topk - window */
  void* stream;           /* hipStream_t */
} smla_index_params;

int sparse_mla_build_index(const int32_t* positions, const void* logits, const int32_t* n_valid, int32_t* indices,
                           int32_t* topk_length, const smla_index_params* params);

/*
 * The consumer of the step's FP8 output: the per-group output projection (wo_a), computed
 * from the E4M3 codes and UE8M0 block-32 scales of both operands on the scaled FP8 MFMA.
 * With x(t, h, i) = e4m3(x_fp8[t][h][i]) * 2^(x_scales[t][h][i/32] - 127) and
 * w(g, o, k) = e4m3(w_fp8[g][o][k]) * 2^(w_scales[g][o][k/32] - 127), hg = heads_per_group:
 *
 *   y[t][g][o] = bf16( sum over h < hg, i < 512 of x(t, g*hg + h, i) * w(g, o, 512*h + i) )
 *
 * accumulated in f32 and rounded to nearest even.  x and x_scales are the out_fp8 /
 * out_scales of sparse_mla_fwd as they are.
 * [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: the kernel's FP8 output is fed
 *  straight into the wo_a einsum.]  The pages do not give the projection's shape: the
 * output width d_out and the heads per group are parameters.
 *
 *   x_fp8      u8 [s_q][h_q][512]                       (device, read; 16-byte aligned)
 *   x_scales   u8 [s_q][h_q][16]                        (device, read; 16-byte aligned)
 *   w_fp8      u8 [h_q/hg][d_out][hg*512]               (device, read; 16-byte aligned)
 *   w_scales   u8 [h_q/hg][d_out][hg*16]                (device, read; 16-byte aligned)
 *   y          bf16 [s_q][h_q/hg][d_out]                (device, written; 8-byte aligned)
 *   params     host pointer, read during the call only
 *
 * Scales are expected in [10, 246] as for the pool (products and sums stay in f32 range).
 * Same conventions as sparse_mla_fwd (asynchronous on params->stream, nothing allocated,
 * errors by return code with nothing launched).
 */
typedef struct smla_wo_a_params {
  int32_t s_q;             /* tokens (0 = no-op) */
  int32_t h_q;             /* heads of x: 1..128, a multiple of heads_per_group */
  int32_t d;               /* dims per head: 512 */
  int32_t heads_per_group; /* heads contracted together: 1..h_q */
  int32_t d_out;           /* outputs per group: a positive multiple of 128, at most 4096 */
  void* stream;            /* hipStream_t */
} smla_wo_a_params;

int sparse_mla_wo_a(const uint8_t* x_fp8, const uint8_t* x_scales, const uint8_t* w_fp8, const uint8_t* w_scales,
                    void* y, const smla_wo_a_params* params);

/*
 * Debug build.  The library compiled with SMLA_DEBUG_CHECKS (libsmla_debug.so beside
 * libsmla.so; same entry points) checks sparse_mla_fwd's device-side preconditions while
 * it runs: an entry j < topk_length[t] outside [-1, n_rows) sets SMLA_DEBUG_BAD_INDEX, a
 * read row with a kv_scales byte outside [SMLA_KV_SCALE_MIN, SMLA_KV_SCALE_MAX] sets
 * SMLA_DEBUG_BAD_SCALE, in the u32 error word at byte SMLA_DEBUG_WORD_OFFSET of the
 * workspace (or-ed in; the library never clears it: zero it before the calls to check).
 * The call still completes normally (a bad id reads as an empty slot).  The production
 * library never touches the word.  [vLLM #56344 "Deepseek V41 Attention MegaKernel",
 * Purpose, bug-fix bullet: stale or unterminated index rows are the failure this reports.]
 * Returns 1 in the debug build, 0 in the production build.
 */
#define SMLA_DEBUG_WORD_OFFSET 8
#define SMLA_DEBUG_BAD_INDEX 1u
#define SMLA_DEBUG_BAD_SCALE 2u
#define SMLA_KV_SCALE_MIN 10
#define SMLA_KV_SCALE_MAX 246
int sparse_mla_debug_checks(void);

/* Thread-local, NUL-terminated message describing the last failed call on this thread
   ("" if none).  Valid until the next call on the same thread. */
const char* sparse_mla_last_error(void);

/* SMLA_ABI_VERSION of the loaded library. */
int sparse_mla_abi_version(void);

/* Per-kernel timing of the next step call (sparse_mla_fwd, sparse_mla_fwd_noalloc or
 * sparse_mla_fwd_ds_nvfp4) made on this thread: each non-NULL argument is a hipEvent_t the
 * caller created, recorded on that call's stream.  before_main: just before the main kernel
 * (after the item-order kernel, if any); after_main: just after it, i.e. before the split
 * combine when there is one; after_all: after the call's last kernel.  Every step call on
 * this thread consumes the armed events, whether it launches or fails its checks (then
 * nothing is recorded); calls with s_q = 0 record nothing.  For measurement tools: the
 * records become graph nodes when the call is captured.  Always returns SMLA_OK. */
int sparse_mla_profile_events(void* before_main, void* after_main, void* after_all);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */

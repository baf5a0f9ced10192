// C ABI of the fused sparse-MLA step, the KV insert and the index-row builder (declared in
// include/smla.h):
// argument checks on the host, split selection, workspace sizing and error reporting.  All checks run
// before any HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "smla.h"
#include "smla_internal.h"

namespace {

thread_local std::string g_last_error;
// events armed by sparse_mla_profile_events for this thread's next step call
thread_local void* g_prof_events[3] = {nullptr, nullptr, nullptr};

// the armed events, disarmed (every step call consumes them, launched or not)
void take_prof_events(smla::LaunchArgs& a) {
  a.ev_main = static_cast<hipEvent_t>(g_prof_events[0]);
  a.ev_split = static_cast<hipEvent_t>(g_prof_events[1]);
  a.ev_end = static_cast<hipEvent_t>(g_prof_events[2]);
  g_prof_events[0] = g_prof_events[1] = g_prof_events[2] = nullptr;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

// Shape/scalar checks shared by every entry point; returns SMLA_OK or an error code.
int check_params(const smla_params* p) {
  if (!p) return fail(SMLA_ERR_NULL, "params is NULL");
  if (p->s_q < 0) return fail(SMLA_ERR_VALUE, "s_q must be >= 0 (got %d)", p->s_q);
  if (p->n_rows < 1) return fail(SMLA_ERR_VALUE, "n_rows must be >= 1 (got %lld)", (long long)p->n_rows);
  if (p->kv_format != SMLA_KV_E4M3_UE8M0 && p->kv_format != SMLA_KV_BF16)
    return fail(SMLA_ERR_VALUE, "unknown kv_format %d", p->kv_format);
  if (!finite_pos(p->sm_scale)) return fail(SMLA_ERR_VALUE, "sm_scale must be finite and > 0");
  if (!finite_pos(p->rms_eps)) return fail(SMLA_ERR_VALUE, "rms_eps must be finite and > 0");
  if (!finite_pos(p->rope_theta)) return fail(SMLA_ERR_VALUE, "rope_theta must be finite and > 0");
  if (p->num_splits < 0 || p->num_splits > 64)
    return fail(SMLA_ERR_VALUE, "num_splits must be in [0, 64] (got %d)", p->num_splits);
  if (p->d != 128 && p->d != 512) return fail(SMLA_ERR_SHAPE, "d must be 128 or 512 (got %d)", p->d);
  if (p->d == 512 && p->kv_format == SMLA_KV_BF16)
    return fail(SMLA_ERR_SHAPE, "the bf16 pool is supported for d = 128 only");
  if (p->h_q < 1 || p->h_q > 64) return fail(SMLA_ERR_SHAPE, "h_q must be in [1, 64] (got %d)", p->h_q);
  if (p->rope_dim < 0 || p->rope_dim > p->d || p->rope_dim % 16 != 0)
    return fail(SMLA_ERR_SHAPE, "rope_dim must be a multiple of 16 in [0, d] (got %d)", p->rope_dim);
  if (p->topk < 0 || p->topk > 65536) return fail(SMLA_ERR_SHAPE, "topk must be in [0, 65536] (got %d)", p->topk);
  if ((long long)p->s_q * p->topk > 0x7FFFFFFFLL)
    return fail(SMLA_ERR_SHAPE, "s_q * topk must fit in int32");
  if (p->s_q > 0x7FFFFFFF / 64) return fail(SMLA_ERR_SHAPE, "s_q too large");
  // rows are gathered at 32-bit byte offsets into the pool (and its scales)
  const long long row_bytes = (long long)p->d * (p->kv_format == SMLA_KV_BF16 ? 2 : 1);
  if (p->n_rows > 0xFFFFFFF0LL / row_bytes)
    return fail(SMLA_ERR_SHAPE, "kv_pool must be smaller than 4 GiB (n_rows %lld x %lld bytes)",
                (long long)p->n_rows, row_bytes);
  return SMLA_OK;
}

int tiles_of(const smla_params* p) { return (p->topk + smla::kTileRows - 1) / smla::kTileRows; }

// Splits per token.  Tiles per split first: the fewest that keep the work items (token,
// split) within one round of the device's compute units (one persistent workgroup each),
// and at least 2 once the call has more than 64 tiles in all (then more, shorter splits
// cost more in partials and their combine than they save); then as many splits as those
// tiles need, so that no split is empty.  Measured on decode rows of 10 tiles: s_q = 1 and
// 4 run best at 10 splits, s_q = 16 and 32 at 5 (19.9 / 22.9 us against 21.6 / 26.0 us at
// 10 / 8), s_q = 64 at 4, s_q = 96 at 2; from 129 tokens on, unsplit.
int choose_splits(const smla_params* p) {
  const int tiles = tiles_of(p) > 0 ? tiles_of(p) : 1;
  int ns = p->num_splits;
  if (ns == 0) {
    const long long cus = smla::device_cus();
    const long long s_q = p->s_q > 0 ? p->s_q : 1;
    int tps = s_q * tiles > 64 ? 2 : 1;
    while (tps < tiles && s_q * ((tiles + tps - 1) / tps) > cus) ++tps;
    ns = (tiles + tps - 1) / tps;
    if (s_q * ns > cus) ns = 1;
  }
  if (ns > tiles) ns = tiles;
  if (ns < 1) ns = 1;
  return ns;
}

size_t workspace_bytes_for(const smla_params* p, int ns) {
  if (p->s_q <= 0) return 0;
  // one split: the item order (s_q int32, rounded up to 256 bytes); more: the partials
  const size_t rest = ns <= 1 ? ((size_t)p->s_q * 4 + 255) / 256 * 256
                              : (size_t)p->s_q * (size_t)ns * smla::partial_floats(p->h_q, p->d) * sizeof(float);
  return smla::kSchedBytes + rest;
}

// Split count of the allocation-free variant: the automatic (or given) count when its
// scratch fits the static array; with num_splits = 0 and a split call too large for it,
// one split (whose scratch is the scheduler state and the item order); 0 if nothing fits.
int noalloc_splits(const smla_params* p) {
  int ns = choose_splits(p);
  if (workspace_bytes_for(p, ns) <= (size_t)SMLA_NOALLOC_SCRATCH_BYTES) return ns;
  if (p->num_splits != 0) return 0;
  return workspace_bytes_for(p, 1) <= (size_t)SMLA_NOALLOC_SCRATCH_BYTES ? 1 : 0;
}

}  // namespace

extern "C" {

int sparse_mla_abi_version(void) { return SMLA_ABI_VERSION; }

int sparse_mla_profile_events(void* before_main, void* after_main, void* after_all) {
  g_prof_events[0] = before_main;
  g_prof_events[1] = after_main;
  g_prof_events[2] = after_all;
  return SMLA_OK;
}

int sparse_mla_debug_checks(void) {
#ifdef SMLA_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

const char* sparse_mla_last_error(void) { return g_last_error.c_str(); }

int sparse_mla_num_splits(const smla_params* p) {
  if (check_params(p) != SMLA_OK) return 0;
  return choose_splits(p);
}

size_t sparse_mla_workspace_size(const smla_params* p) {
  if (check_params(p) != SMLA_OK) return 0;
  return workspace_bytes_for(p, choose_splits(p));
}

}  // extern "C"

namespace {

// Argument checks of sparse_mla_fwd (and its allocation-free variant) that need the array
// pointers: SMLA_OK or an error code with the message set.
int check_fwd_arrays(const void* q, const void* kv_pool, const uint8_t* kv_scales, const int32_t* indices,
                     const int32_t* topk_length, const int32_t* positions, const float* norm_w,
                     const uint8_t* out_fp8, const uint8_t* out_scales, const smla_params* p) {
  if (!q || !kv_pool || !positions || !norm_w || !out_fp8 || !out_scales || !topk_length)
    return fail(SMLA_ERR_NULL, "a required array pointer is NULL");
  if (p->topk > 0 && !indices) return fail(SMLA_ERR_NULL, "indices is NULL");
  if (p->kv_format == SMLA_KV_E4M3_UE8M0 && !kv_scales)
    return fail(SMLA_ERR_NULL, "kv_scales is NULL for the E4M3 pool");
  // vector loads / stores of 16 bytes (4 for the scale rows)
  const struct {
    const void* ptr;
    uintptr_t align;
    const char* name;
  } al[] = {{q, 16, "q"}, {kv_pool, 16, "kv_pool"}, {kv_scales, 4, "kv_scales"}, {norm_w, 16, "norm_w"},
            {out_fp8, 16, "out_fp8"}, {p->out_f32, 16, "out_f32"}};
  for (const auto& x : al)
    if (reinterpret_cast<uintptr_t>(x.ptr) % x.align != 0)
      return fail(SMLA_ERR_VALUE, "%s must be %u-byte aligned", x.name, (unsigned)x.align);
  return SMLA_OK;
}

// Enqueue the step with the given scratch buffer and split count.
int launch_fwd(const void* q, const void* kv_pool, const uint8_t* kv_scales, const int32_t* indices,
               const int32_t* topk_length, const int32_t* positions, const float* norm_w, uint8_t* out_fp8,
               uint8_t* out_scales, const smla_params* p, void* workspace, int ns, const smla::LaunchArgs& ev) {
  smla::LaunchArgs a;
  a.ev_main = ev.ev_main;
  a.ev_split = ev.ev_split;
  a.ev_end = ev.ev_end;
  a.q = static_cast<const uint16_t*>(q);
  a.kv_pool = kv_pool;
  a.kv_scales = kv_scales;
  a.indices = indices;
  a.topk_length = topk_length;
  a.positions = positions;
  a.norm_w = norm_w;
  a.out_fp8 = out_fp8;
  a.out_scales = out_scales;
  a.out_f32 = p->out_f32;
  a.workspace = workspace;
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.d = p->d;
  a.rope_dim = p->rope_dim;
  a.topk = p->topk;
  a.kv_format = p->kv_format;
  a.num_splits = ns;
  a.n_rows = p->n_rows;
  a.sm_scale = p->sm_scale;
  a.rms_eps = p->rms_eps;
  a.rope_theta = p->rope_theta;
  a.stream = static_cast<hipStream_t>(p->stream);
  const hipError_t e = smla::launch(a);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

}  // namespace

extern "C" {

int sparse_mla_fwd(const void* q, const void* kv_pool, const uint8_t* kv_scales, const int32_t* indices,
                   const int32_t* topk_length, const int32_t* positions, const float* norm_w, uint8_t* out_fp8,
                   uint8_t* out_scales, const smla_params* p) {
  g_last_error.clear();
  smla::LaunchArgs ev;
  take_prof_events(ev);
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (p->s_q == 0) return SMLA_OK;
  rc = check_fwd_arrays(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, p);
  if (rc != SMLA_OK) return rc;
  if (reinterpret_cast<uintptr_t>(p->workspace) % 16 != 0) return fail(SMLA_ERR_VALUE, "workspace must be 16-byte aligned");
  const int ns = choose_splits(p);
  const size_t need = workspace_bytes_for(p, ns);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(SMLA_ERR_VALUE, "workspace of %zu bytes needed (got %zu)", need,
                p->workspace ? p->workspace_bytes : (size_t)0);
  return launch_fwd(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, p,
                    p->workspace, ns, ev);
}

int sparse_mla_fwd_noalloc(const void* q, const void* kv_pool, const uint8_t* kv_scales, const int32_t* indices,
                           const int32_t* topk_length, const int32_t* positions, const float* norm_w,
                           uint8_t* out_fp8, uint8_t* out_scales, const smla_params* p) {
  g_last_error.clear();
  smla::LaunchArgs ev;
  take_prof_events(ev);
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (p->s_q == 0) return SMLA_OK;
  rc = check_fwd_arrays(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, p);
  if (rc != SMLA_OK) return rc;
  const int ns = noalloc_splits(p);
  if (ns == 0)
    return fail(SMLA_ERR_VALUE, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                workspace_bytes_for(p, p->num_splits > 0 ? choose_splits(p) : 1),
                (size_t)SMLA_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  const hipError_t e = smla::noalloc_scratch(&scratch);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
  return launch_fwd(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, p,
                    scratch, ns, ev);
}

int sparse_mla_fwd_ds_nvfp4(const void* q, const uint8_t* swa_pool, const uint8_t* swa_scales,
                            const uint8_t* cmp_pool, const uint8_t* cmp_scales, const int32_t* indices,
                            const int32_t* topk_length, const int32_t* positions, const float* norm_w,
                            uint8_t* out_fp8, uint8_t* out_scales, const smla_ds_params* dp) {
  g_last_error.clear();
  smla::LaunchArgs a;
  take_prof_events(a);
  if (!dp) return fail(SMLA_ERR_NULL, "params is NULL");
  const smla_params* p = &dp->base;
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (p->d != 512 || p->kv_format != SMLA_KV_E4M3_UE8M0)
    return fail(SMLA_ERR_SHAPE, "the two-pool step needs d = 512 and an E4M3 + UE8M0 SWA pool");
  if (p->rope_dim > smla::kNvMaxRope)
    return fail(SMLA_ERR_SHAPE, "rope_dim must be at most %d for the two-pool step (got %d)", smla::kNvMaxRope,
                p->rope_dim);
  if (dp->n_cmp_rows < 1 || dp->n_cmp_rows > 0xFFFFFFF0LL / 256)
    return fail(SMLA_ERR_SHAPE, "n_cmp_rows must be in [1, 4 GiB / 256) (got %lld)", (long long)dp->n_cmp_rows);
  if (dp->swa_entries < 0 || dp->swa_entries > 65536 || dp->swa_entries % smla::kTileRows != 0)
    return fail(SMLA_ERR_SHAPE, "swa_entries must be a multiple of 64 in [0, 65536] (got %d)", dp->swa_entries);
  if (dp->reserved != 0) return fail(SMLA_ERR_VALUE, "reserved must be 0");
  if (p->s_q == 0) return SMLA_OK;
  rc = check_fwd_arrays(q, swa_pool, swa_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, p);
  if (rc != SMLA_OK) return rc;
  if (!cmp_pool || !cmp_scales) return fail(SMLA_ERR_NULL, "cmp_pool and cmp_scales are required");
  if (reinterpret_cast<uintptr_t>(cmp_pool) % 16 != 0 || reinterpret_cast<uintptr_t>(cmp_scales) % 4 != 0)
    return fail(SMLA_ERR_VALUE, "cmp_pool must be 16-byte and cmp_scales 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(p->workspace) % 16 != 0) return fail(SMLA_ERR_VALUE, "workspace must be 16-byte aligned");
  const int ns = choose_splits(p);
  const size_t need = workspace_bytes_for(p, ns);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(SMLA_ERR_VALUE, "workspace of %zu bytes needed (got %zu)", need,
                p->workspace ? p->workspace_bytes : (size_t)0);
  a.q = static_cast<const uint16_t*>(q);
  a.kv_pool = swa_pool;
  a.kv_scales = swa_scales;
  a.indices = indices;
  a.topk_length = topk_length;
  a.positions = positions;
  a.norm_w = norm_w;
  a.out_fp8 = out_fp8;
  a.out_scales = out_scales;
  a.out_f32 = p->out_f32;
  a.workspace = p->workspace;
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.d = p->d;
  a.rope_dim = p->rope_dim;
  a.topk = p->topk;
  a.kv_format = p->kv_format;
  a.num_splits = ns;
  a.n_rows = p->n_rows;
  a.sm_scale = p->sm_scale;
  a.rms_eps = p->rms_eps;
  a.rope_theta = p->rope_theta;
  a.stream = static_cast<hipStream_t>(p->stream);
  a.cmp_pool = cmp_pool;
  a.cmp_scales = cmp_scales;
  a.n_cmp = dp->n_cmp_rows;
  a.swa_entries = dp->swa_entries;
  const hipError_t e = smla::launch(a);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int sparse_mla_noalloc_num_splits(const smla_params* p) {
  if (check_params(p) != SMLA_OK) return 0;
  return noalloc_splits(p);
}

int sparse_mla_kv_insert(const void* kv, const int32_t* positions, const float* norm_w, uint8_t* kv_pool,
                         uint8_t* kv_scales, const smla_kv_insert_params* p) {
  g_last_error.clear();
  if (!p) return fail(SMLA_ERR_NULL, "params is NULL");
  if (p->n < 0) return fail(SMLA_ERR_VALUE, "n must be >= 0 (got %d)", p->n);
  if (p->d != 512) return fail(SMLA_ERR_SHAPE, "d must be 512 (got %d)", p->d);
  if (p->rope_dim < 0 || p->rope_dim > p->d || p->rope_dim % 16 != 0)
    return fail(SMLA_ERR_SHAPE, "rope_dim must be a multiple of 16 in [0, d] (got %d)", p->rope_dim);
  if (p->n_rows < 1 || p->n_rows > 0xFFFFFFF0LL / p->d)
    return fail(SMLA_ERR_SHAPE, "n_rows must be in [1, 4 GiB / 512) (got %lld)", (long long)p->n_rows);
  if (p->n_swa < 1 || p->n_swa > p->n_rows)
    return fail(SMLA_ERR_VALUE, "n_swa must be in [1, n_rows] (got %d)", p->n_swa);
  if (!finite_pos(p->rms_eps)) return fail(SMLA_ERR_VALUE, "rms_eps must be finite and > 0");
  if (!finite_pos(p->rope_theta)) return fail(SMLA_ERR_VALUE, "rope_theta must be finite and > 0");
  if (p->n == 0) return SMLA_OK;
  if (!kv || !positions || !norm_w || !kv_pool || !kv_scales)
    return fail(SMLA_ERR_NULL, "a required array pointer is NULL");
  const struct {
    const void* ptr;
    uintptr_t align;
    const char* name;
  } al[] = {{kv, 16, "kv"}, {norm_w, 16, "norm_w"}, {kv_pool, 16, "kv_pool"}, {kv_scales, 4, "kv_scales"}};
  for (const auto& x : al)
    if (reinterpret_cast<uintptr_t>(x.ptr) % x.align != 0)
      return fail(SMLA_ERR_VALUE, "%s must be %u-byte aligned", x.name, (unsigned)x.align);
  smla::KvInsertArgs a;
  a.kv = static_cast<const uint16_t*>(kv);
  a.positions = positions;
  a.norm_w = norm_w;
  a.kv_pool = kv_pool;
  a.kv_scales = kv_scales;
  a.n = p->n;
  a.rope_dim = p->rope_dim;
  a.n_swa = p->n_swa;
  a.rms_eps = p->rms_eps;
  a.rope_theta = p->rope_theta;
  a.stream = static_cast<hipStream_t>(p->stream);
  const hipError_t e = smla::launch_kv_insert(a);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int sparse_mla_build_index(const int32_t* positions, const void* logits, const int32_t* n_valid, int32_t* indices,
                           int32_t* topk_length, const smla_index_params* p) {
  g_last_error.clear();
  if (!p) return fail(SMLA_ERR_NULL, "params is NULL");
  if (p->s_q < 0) return fail(SMLA_ERR_VALUE, "s_q must be >= 0 (got %d)", p->s_q);
  if (p->n_cand < 0 || p->n_cand > 65536)
    return fail(SMLA_ERR_SHAPE, "n_cand must be in [0, 65536] (got %d)", p->n_cand);
  if (p->n_swa < 1) return fail(SMLA_ERR_VALUE, "n_swa must be >= 1 (got %d)", p->n_swa);
  if (p->window < 0 || p->window > p->n_swa)
    return fail(SMLA_ERR_SHAPE, "window must be in [0, n_swa] (got %d)", p->window);
  if (p->self_in_window != 0 && p->self_in_window != 1)
    return fail(SMLA_ERR_VALUE, "self_in_window must be 0 or 1 (got %d)", p->self_in_window);
  if (p->k_cmp < 0) return fail(SMLA_ERR_SHAPE, "k_cmp must be >= 0 (got %d)", p->k_cmp);
  if (p->topk > 65536 || (long long)p->window + p->k_cmp > p->topk)
    return fail(SMLA_ERR_SHAPE, "topk must be in [window + k_cmp, 65536] (got %d)", p->topk);
  if (p->cmp_base < 0 || (long long)p->cmp_base + p->n_cand > 0x7FFFFFFFLL)
    return fail(SMLA_ERR_VALUE, "cmp_base + n_cand must lie in [0, 2^31)");
  if ((long long)p->s_q * p->topk > 0x7FFFFFFFLL) return fail(SMLA_ERR_SHAPE, "s_q * topk must fit in int32");
  if (p->s_q == 0) return SMLA_OK;
  if (!positions || !indices || !topk_length || (p->n_cand > 0 && !logits))
    return fail(SMLA_ERR_NULL, "a required array pointer is NULL");
  if (reinterpret_cast<uintptr_t>(logits) % 2 != 0) return fail(SMLA_ERR_VALUE, "logits must be 2-byte aligned");
  smla::IndexArgs a;
  a.positions = positions;
  a.logits = static_cast<const uint16_t*>(logits);
  a.n_valid = n_valid;
  a.indices = indices;
  a.topk_length = topk_length;
  a.s_q = p->s_q;
  a.n_cand = p->n_cand;
  a.topk = p->topk;
  a.window = p->window;
  a.self_in_window = p->self_in_window;
  a.n_swa = p->n_swa;
  a.cmp_base = p->cmp_base;
  a.k_cmp = p->k_cmp;
  a.stream = static_cast<hipStream_t>(p->stream);
  const hipError_t e = smla::launch_build_index(a);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int sparse_mla_wo_a(const uint8_t* x_fp8, const uint8_t* x_scales, const uint8_t* w_fp8, const uint8_t* w_scales,
                    void* y, const smla_wo_a_params* p) {
  g_last_error.clear();
  if (!p) return fail(SMLA_ERR_NULL, "params is NULL");
  if (p->s_q < 0) return fail(SMLA_ERR_VALUE, "s_q must be >= 0 (got %d)", p->s_q);
  if (p->d != 512) return fail(SMLA_ERR_SHAPE, "d must be 512 (got %d)", p->d);
  if (p->h_q < 1 || p->h_q > 128) return fail(SMLA_ERR_SHAPE, "h_q must be in [1, 128] (got %d)", p->h_q);
  if (p->heads_per_group < 1 || p->heads_per_group > p->h_q || p->h_q % p->heads_per_group != 0)
    return fail(SMLA_ERR_SHAPE, "heads_per_group must divide h_q (got %d, h_q %d)", p->heads_per_group, p->h_q);
  if (p->d_out < 128 || p->d_out > 4096 || p->d_out % 128 != 0)
    return fail(SMLA_ERR_SHAPE, "d_out must be a multiple of 128 in [128, 4096] (got %d)", p->d_out);
  const long long n_groups = p->h_q / p->heads_per_group;
  if ((long long)p->s_q * p->h_q * 512 >= 0xFFFFFFFFLL)
    return fail(SMLA_ERR_SHAPE, "s_q * h_q * 512 must stay below 4 GiB");
  if (n_groups * p->d_out * p->heads_per_group * 512 >= 0xFFFFFFFFLL)
    return fail(SMLA_ERR_SHAPE, "the weight must stay below 4 GiB");
  if (p->s_q == 0) return SMLA_OK;
  if (!x_fp8 || !x_scales || !w_fp8 || !w_scales || !y) return fail(SMLA_ERR_NULL, "a required array pointer is NULL");
  const struct {
    const void* ptr;
    uintptr_t align;
    const char* name;
  } al[] = {{x_fp8, 16, "x_fp8"}, {x_scales, 16, "x_scales"}, {w_fp8, 16, "w_fp8"}, {w_scales, 16, "w_scales"},
            {y, 8, "y"}};
  for (const auto& x : al)
    if (reinterpret_cast<uintptr_t>(x.ptr) % x.align != 0)
      return fail(SMLA_ERR_VALUE, "%s must be %u-byte aligned", x.name, (unsigned)x.align);
  smla::WoArgs a;
  a.x = x_fp8;
  a.x_scales = x_scales;
  a.w = w_fp8;
  a.w_scales = w_scales;
  a.y = static_cast<uint16_t*>(y);
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.heads_per_group = p->heads_per_group;
  a.n_groups = (int)n_groups;
  a.d_out = p->d_out;
  a.stream = static_cast<hipStream_t>(p->stream);
  const hipError_t e = smla::launch_wo_a(a);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

}  // extern "C"

/*
 * sparse_mla_oracle.c -- plain fp64 CPU oracle of the fused sparse-MLA attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct reference the
 * GPU library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It shares
 * no code, header, table or constant with the GPU library: every step below is
 * written from the definition it cites.
 *
 * What it computes (per query token t, per head h), following the pages:
 *   [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose, first bullet]
 *     the fused step is: norm -> RoPE -> sparse attention -> inverse RoPE -> FP8 cast.
 *   [vLLM #56344, Purpose, bug-fix bullet]
 *     reads are capped at topk_length; entries beyond it are never dereferenced;
 *     -1 marks an empty slot.
 *   [vLLM #56344, Purpose, second bullet]
 *     every token carries its own metadata row (positions, SWA + compressed indices).
 *   [SGLang #39370 "[DSV4.1] Combine DSpark decode and prefill kernel optimizations",
 *    Summary] the query norm is per head ("q_head_norm").
 *   [vLLM #56344, Purpose] the KV cache row is 512 e4m3 bytes plus UE8M0 block
 *     scales (528 B), shared as K and V by every head (MLA latent).
 *   [SGLang #39370, commit note on the MXFP8 epilogue] UE8M0 block scales on the
 *     output.
 *
 * Readings taken where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - RMSNorm over the d dims of each head, eps inside the square root, one weight
 *     vector norm_w[d] shared by all heads.
 *   - RoPE is the rotate-half form on the last r dims: pairs (o0+i, o0+i+r/2),
 *     o0 = d - r, angle p * base^(-2i/r).  Inverse RoPE rotates by the negated
 *     angle at the same (query) position.  K rows are used as stored.
 *   - Softmax over the valid entries J of the row; duplicates count once per entry;
 *     an empty J gives o = 0.
 *   - Output scale: the smallest power of two S = 2^(e-127), e in [0, 254], with
 *     448 * S >= amax of the 32-element block; codes are round-to-nearest-even
 *     OCP E4M3FN of o / S (so they never saturate).
 *
 * Formats written from their public definitions:
 *   OCP 8-bit floating point specification, E4M3: bias 7, 3 mantissa bits,
 *   subnormals, max normal 448 (0x7E), NaN = S.1111.111, no infinities.
 *   bf16: the upper 16 bits of an IEEE-754 binary32.
 *
 * All arithmetic is double precision.  Parallel over tokens with OpenMP (the tokens
 * are independent; each token's arithmetic is the same serial loop either way).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)   /* bad sizes / scalars */
#define ORACLE_ERR_INDEX (-2) /* a valid-prefix index outside [-1, n_rows) */
#define ORACLE_ERR_NOMEM (-3)

#define KV_E4M3_UE8M0 0
#define KV_BF16 1

#define BLOCK 32

/* ---------------------------------------------------------------- decoders */

/* bf16 bit pattern -> exact double (bf16 is the top half of a binary32). */
double oracle_bf16_decode(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP E4M3FN code -> exact double.  NaN for S.1111.111. */
double oracle_e4m3_decode(uint8_t code) {
  int sign = (code >> 7) & 1;
  int ex = (code >> 3) & 15;
  int man = code & 7;
  double v;
  if (ex == 15 && man == 7) return NAN;
  if (ex == 0)
    v = ldexp((double)man, -9); /* subnormal: man/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

/*
 * OCP E2M1 (FP4) code (low 4 bits) -> exact double: sign bit 3, exponent bits 2-1 (bias 1),
 * mantissa bit 0; exponent 0 is subnormal (m * 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
double oracle_e2m1_decode(uint8_t code) {
  int sign = (code >> 3) & 1, ex = (code >> 1) & 3, man = code & 1;
  double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -v : v;
}

/* ---------------------------------------------------------------- encoders */

/*
 * Round-to-nearest-even onto the E4M3FN grid.  Requires |x| <= 448 (the caller's
 * scale guarantees it); larger magnitudes saturate to +-448 (0x7E / 0xFE), which the
 * path never produces.  The sign of x is kept, so a negative value that rounds to
 * zero gives 0x80.
 */
uint8_t oracle_e4m3_encode(double x) {
  uint8_t sign = (signbit(x) ? 0x80 : 0x00);
  double a = fabs(x);
  int k, E, code;
  double q, n;
  if (a == 0.0) return sign;
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  frexp(a, &k);        /* a = f * 2^k, f in [0.5, 1)  ->  floor(log2 a) = k - 1 */
  E = k - 1;
  if (E < -6) E = -6;  /* below the smallest normal the quantum stays 2^-9 */
  q = ldexp(1.0, E - 3);
  n = nearbyint(a / q); /* a / q is exact (power-of-two divisor); default mode is RNE */
  /* n in [0, 16]; n == 16 means the value rounded up to 2^(E+1). */
  if (E == -6 && n < 8) {
    code = (int)n; /* subnormal: mantissa n, exponent field 0 */
  } else if (n == 16.0) {
    code = ((E + 1 + 7) << 3);
  } else {
    code = ((E + 7) << 3) | ((int)n - 8);
  }
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

/*
 * UE8M0 exponent of a block: the smallest e in [0, 254] with 448 * 2^(e-127) >= amax.
 * 448 * 2^E is exact in double for every E used here, so the comparison decides the
 * exponent exactly (no log2 rounding).
 */
int oracle_ue8m0_exponent(double amax) {
  int E, k;
  if (!(amax > 0.0)) return 0; /* amax == 0 (or NaN): the clamp gives e = 0 */
  frexp(amax, &k);
  E = k - 1 - 9;               /* 448 * 2^E < amax here, since 448 < 2^9 */
  while (ldexp(448.0, E) < amax) E++;
  if (E + 127 < 0) return 0;
  if (E + 127 > 254) return 254;
  return E + 127;
}

/* Quantize n values (n a multiple of 32) in blocks of 32: scales[b] = e, codes = RNE(o / 2^(e-127)). */
void oracle_quantize_blocks(const double* o, int64_t n, uint8_t* codes, uint8_t* scales) {
  int64_t b, i;
  for (b = 0; b < n / BLOCK; ++b) {
    double amax = 0.0;
    int e;
    for (i = 0; i < BLOCK; ++i) {
      double a = fabs(o[b * BLOCK + i]);
      if (a > amax) amax = a;
    }
    e = oracle_ue8m0_exponent(amax);
    scales[b] = (uint8_t)e;
    for (i = 0; i < BLOCK; ++i) codes[b * BLOCK + i] = oracle_e4m3_encode(ldexp(o[b * BLOCK + i], 127 - e));
  }
}

/* ---------------------------------------------------------------- q path */

/* Per-head RMSNorm: y_i = x_i / sqrt(mean(x^2) + eps) * w_i. */
void oracle_rmsnorm(const double* x, const double* w, int d, double eps, double* y) {
  double ss = 0.0;
  int i;
  for (i = 0; i < d; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / d + eps);
  for (i = 0; i < d; ++i) y[i] = x[i] * inv * w[i];
}

/*
 * Rotate-half RoPE on the last r dims of y (in place) at position pos.  direction = +1
 * applies RoPE, direction = -1 applies its inverse (rotation by the negated angle).
 */
void oracle_rope(double* y, int d, int r, double pos, double base, int direction) {
  int o0 = d - r, half = r / 2, i;
  for (i = 0; i < half; ++i) {
    double inv_freq = pow(base, -(2.0 * i) / (double)r);
    double ang = (double)direction * pos * inv_freq;
    double c = cos(ang), s = sin(ang);
    double a = y[o0 + i], b = y[o0 + i + half];
    y[o0 + i] = a * c - b * s;
    y[o0 + i + half] = b * c + a * s;
  }
}

/* ---------------------------------------------------------------- the step */

#define KV_DS_NVFP4 2

/*
 * Where an index entry's row comes from.  kv_format 0 / 1: one pool (E4M3 + UE8M0, or
 * bf16).  KV_DS_NVFP4, the two-pool cache of the pages' nvfp4_ds_mla layout [vLLM #56344
 * "Deepseek V41 Attention MegaKernel", Purpose: fp8 528 B SWA rows + fp4 288 B compressed
 * rows]: entries j < swa_entries of an index row name rows of the E4M3 + UE8M0 pool (512
 * codes + 16 scales), entries j >= swa_entries name rows of the NVFP4 pool, 256 bytes of
 * E2M1 codes (element 2i in the low nibble of byte i, 2i + 1 in the high nibble) and 32
 * E4M3 scales, one per 16 elements: value = e2m1(code) * e4m3(scale).  (Reading: the
 * pages give the row sizes only; this is the OCP E2M1 / E4M3-scale-per-16 format that
 * fills 288 bytes, with no per-tensor scale.)
 */
typedef struct {
  int fmt, d, swa_entries;
  const void* pool;          /* fmt 0 / 1 / SWA: codes or bf16 bits */
  const uint8_t* scales;     /* fmt 0 / SWA: UE8M0 per 32 */
  const uint8_t* cmp_codes;  /* NVFP4 pool: E2M1 pairs [n_cmp][d/2] */
  const uint8_t* cmp_scales; /* NVFP4 pool: E4M3 per 16 [n_cmp][d/16] */
  int64_t n_rows, n_cmp;
} row_source;

/* Bounds of the ids entry j may hold: [-1, n) of the pool it names. */
static int64_t rows_of(const row_source* R, int j) {
  return (R->fmt == KV_DS_NVFP4 && j >= R->swa_entries) ? R->n_cmp : R->n_rows;
}

/* Decode row r named by entry j into v[d], exactly. */
static void decode_row(const row_source* R, int j, int32_t r, double* v) {
  int i, d = R->d;
  if (R->fmt == KV_BF16) {
    const uint16_t* bits = (const uint16_t*)R->pool;
    for (i = 0; i < d; ++i) v[i] = oracle_bf16_decode(bits[(int64_t)r * d + i]);
  } else if (R->fmt == KV_DS_NVFP4 && j >= R->swa_entries) {
    for (i = 0; i < d; ++i) {
      uint8_t byte = R->cmp_codes[(int64_t)r * (d / 2) + i / 2];
      uint8_t code = (i & 1) ? (byte >> 4) : (byte & 15);
      v[i] = oracle_e2m1_decode(code) * oracle_e4m3_decode(R->cmp_scales[(int64_t)r * (d / 16) + i / 16]);
    }
  } else {
    const uint8_t* codes = (const uint8_t*)R->pool;
    for (i = 0; i < d; ++i) {
      int e = R->scales[(int64_t)r * (d / BLOCK) + i / BLOCK];
      v[i] = oracle_e4m3_decode(codes[(int64_t)r * d + i]) * ldexp(1.0, e - 127);
    }
  }
}

static int step(const uint16_t* q, const row_source* R, const int32_t* indices, const int32_t* topk_length,
                const int32_t* positions, const double* norm_w, int s_q, int h, int d, int rope_dim, int topk,
                double sm_scale, double eps, double theta, double* out_f64, uint8_t* out_fp8,
                uint8_t* out_scales);

int oracle_sparse_mla(const uint16_t* q, const void* kv_pool, const uint8_t* kv_scales,
                      const int32_t* indices, const int32_t* topk_length, const int32_t* positions,
                      const double* norm_w, int s_q, int h, int d, int rope_dim, int topk,
                      int64_t n_rows, int kv_format, double sm_scale, double eps, double theta,
                      double* out_f64, uint8_t* out_fp8, uint8_t* out_scales) {
  row_source R;
  if (kv_format != KV_E4M3_UE8M0 && kv_format != KV_BF16) return ORACLE_ERR_ARG;
  if (kv_format == KV_E4M3_UE8M0 && kv_scales == NULL) return ORACLE_ERR_ARG;
  memset(&R, 0, sizeof R);
  R.fmt = kv_format;
  R.d = d;
  R.pool = kv_pool;
  R.scales = kv_scales;
  R.n_rows = n_rows;
  return step(q, &R, indices, topk_length, positions, norm_w, s_q, h, d, rope_dim, topk, sm_scale, eps, theta,
              out_f64, out_fp8, out_scales);
}

/*
 * The step over the two-pool nvfp4_ds_mla cache (see row_source): swa_codes / swa_scales
 * u8 [n_swa][d] / [n_swa][d/32], cmp_codes / cmp_scales u8 [n_cmp][d/2] / [n_cmp][d/16];
 * entries j < swa_entries of each index row are SWA rows, the rest compressed rows.  The
 * rest as oracle_sparse_mla.
 */
int oracle_sparse_mla_ds_nvfp4(const uint16_t* q, const uint8_t* swa_codes, const uint8_t* swa_scales,
                               const uint8_t* cmp_codes, const uint8_t* cmp_scales, const int32_t* indices,
                               const int32_t* topk_length, const int32_t* positions, const double* norm_w,
                               int s_q, int h, int d, int rope_dim, int topk, int swa_entries, int64_t n_swa,
                               int64_t n_cmp, double sm_scale, double eps, double theta, double* out_f64,
                               uint8_t* out_fp8, uint8_t* out_scales) {
  row_source R;
  if (!swa_codes || !swa_scales || !cmp_codes || !cmp_scales || d % 16 != 0 || swa_entries < 0 || n_cmp < 1)
    return ORACLE_ERR_ARG;
  memset(&R, 0, sizeof R);
  R.fmt = KV_DS_NVFP4;
  R.d = d;
  R.swa_entries = swa_entries;
  R.pool = swa_codes;
  R.scales = swa_scales;
  R.cmp_codes = cmp_codes;
  R.cmp_scales = cmp_scales;
  R.n_rows = n_swa;
  R.n_cmp = n_cmp;
  return step(q, &R, indices, topk_length, positions, norm_w, s_q, h, d, rope_dim, topk, sm_scale, eps, theta,
              out_f64, out_fp8, out_scales);
}

static int step(const uint16_t* q, const row_source* R, const int32_t* indices, const int32_t* topk_length,
                const int32_t* positions, const double* norm_w, int s_q, int h, int d, int rope_dim, int topk,
                double sm_scale, double eps, double theta, double* out_f64, uint8_t* out_fp8,
                uint8_t* out_scales) {
  int t;
  int status = ORACLE_OK;
  if (s_q < 0 || h < 1 || d < 1 || d % BLOCK != 0 || rope_dim < 0 || rope_dim > d || rope_dim % 2 != 0 ||
      topk < 0 || R->n_rows < 1)
    return ORACLE_ERR_ARG;

  /* validate the read prefix of every row first */
  for (t = 0; t < s_q; ++t) {
    int L = topk_length[t] < topk ? topk_length[t] : topk;
    int j;
    for (j = 0; j < L; ++j) {
      int32_t r = indices[(int64_t)t * topk + j];
      if (r < -1 || (int64_t)r >= rows_of(R, j)) return ORACLE_ERR_INDEX;
    }
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (t = 0; t < s_q; ++t) {
    int L = topk_length[t] < topk ? topk_length[t] : topk;
    int nv = 0, j, hh, i;
    double pos = (double)positions[t];
    /* rows of this token, decoded exactly: V[n][d] (K = V) */
    double* V = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * (size_t)d);
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!V || !x || !y || !s || !o) {
#pragma omp critical
      status = ORACLE_ERR_NOMEM;
      free(V); free(x); free(y); free(s); free(o);
      continue;
    }
    /* valid set J: entries j < L holding a row id >= 0, one term per entry */
    for (j = 0; j < L; ++j) {
      int32_t r = indices[(int64_t)t * topk + j];
      if (r < 0) continue;
      decode_row(R, j, r, V + (int64_t)nv * d);
      ++nv;
    }
    for (hh = 0; hh < h; ++hh) {
      int64_t base = ((int64_t)t * h + hh) * d;
      /* 1-3: decode q, per-head RMSNorm, RoPE at the token's position */
      for (i = 0; i < d; ++i) x[i] = oracle_bf16_decode(q[base + i]);
      oracle_rmsnorm(x, norm_w, d, eps, y);
      oracle_rope(y, d, rope_dim, pos, theta, +1);
      /* 4-6: softmax attention over the valid rows (exact two-pass softmax) */
      for (i = 0; i < d; ++i) o[i] = 0.0;
      if (nv > 0) {
        double m = -INFINITY, l = 0.0;
        for (j = 0; j < nv; ++j) {
          double acc = 0.0;
          for (i = 0; i < d; ++i) acc += y[i] * V[(int64_t)j * d + i];
          s[j] = sm_scale * acc;
          if (s[j] > m) m = s[j];
        }
        for (j = 0; j < nv; ++j) {
          double p = exp(s[j] - m);
          l += p;
          for (i = 0; i < d; ++i) o[i] += p * V[(int64_t)j * d + i];
        }
        for (i = 0; i < d; ++i) o[i] /= l;
      }
      /* 7: inverse RoPE at the same position */
      oracle_rope(o, d, rope_dim, pos, theta, -1);
      /* 8: UE8M0 + E4M3 */
      if (out_f64)
        for (i = 0; i < d; ++i) out_f64[base + i] = o[i];
      oracle_quantize_blocks(o, d, out_fp8 + base, out_scales + ((int64_t)t * h + hh) * (d / BLOCK));
    }
    free(V); free(x); free(y); free(s); free(o);
  }
  return status;
}

/* ---------------------------------------------------------------- KV insert */

/*
 * Exponent floor of the pool rows.  A pool row is consumed by the step, whose value
 * decoding e4m3(code) * 2^(e-127) stays a normal number in bf16 / f32 arithmetic only for
 * e >= 10 (the smallest E4M3 subnormal, 2^-9, times 2^-117 is 2^-126).  The producer
 * therefore never writes an exponent below 10: a block whose amax is below
 * 448 * 2^(10-127) is coded at e = 10, where its values round (RNE) onto the E4M3 grid at
 * that scale -- to subnormal codes or to zero -- and never saturate.  (Reading: the pages
 * fix the 528-byte row but not the producer's range; this is the range the row format is
 * consumed in.)
 */
#define POOL_EXP_MIN 10

static void quantize_pool_row(const double* y, int d, uint8_t* codes, uint8_t* scales) {
  int b, i;
  for (b = 0; b < d / BLOCK; ++b) {
    double amax = 0.0;
    int e;
    for (i = 0; i < BLOCK; ++i) {
      double a = fabs(y[b * BLOCK + i]);
      if (a > amax) amax = a;
    }
    e = oracle_ue8m0_exponent(amax);
    if (e < POOL_EXP_MIN) e = POOL_EXP_MIN;
    scales[b] = (uint8_t)e;
    for (i = 0; i < BLOCK; ++i) codes[b * BLOCK + i] = oracle_e4m3_encode(ldexp(y[b * BLOCK + i], 127 - e));
  }
}

/*
 * KV insert, the producer of the pool rows the step gathers
 *   [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: fp8 SWA cache rows of 512
 *    E4M3 bytes + UE8M0 scales written by an insert kernel]
 *   [vLLM #64364 "latency_specialized decode", Details, change table: the KV cache write
 *    happens in the kernel that normalises and quantizes q and kv]
 * Readings: the kv latent is RMS-normalised like a q head (same formula, its own weight),
 * its last r dims carry RoPE at the token's own position (the step's inverse RoPE on
 * the output only undoes a rotation the stored rows carry), and it is quantized with the
 * step's output codec with the exponent floored at POOL_EXP_MIN (above); the row is the position modulo the window size n_swa, and a
 * negative position means "no token".  Tokens are applied in order (a later token that
 * lands on the same row overwrites an earlier one).
 *   kv         bf16 bits [n][d]
 *   positions  i32 [n]
 *   norm_w     f64 [d]
 *   kv_pool    u8 [n_rows][d] (rows pos mod n_swa overwritten)
 *   kv_scales  u8 [n_rows][d/32]
 */
int oracle_kv_insert(const uint16_t* kv, const int32_t* positions, const double* norm_w, int n, int d,
                     int rope_dim, int n_swa, int64_t n_rows, double eps, double theta, uint8_t* kv_pool,
                     uint8_t* kv_scales) {
  int t, i;
  double *x, *y;
  if (n < 0 || d < 1 || d % BLOCK != 0 || rope_dim < 0 || rope_dim > d || rope_dim % 2 != 0 || n_swa < 1 ||
      (int64_t)n_swa > n_rows)
    return ORACLE_ERR_ARG;
  x = (double*)malloc(sizeof(double) * (size_t)d);
  y = (double*)malloc(sizeof(double) * (size_t)d);
  if (!x || !y) {
    free(x); free(y);
    return ORACLE_ERR_NOMEM;
  }
  for (t = 0; t < n; ++t) {
    int64_t row;
    if (positions[t] < 0) continue;
    row = positions[t] % n_swa;
    for (i = 0; i < d; ++i) x[i] = oracle_bf16_decode(kv[(int64_t)t * d + i]);
    oracle_rmsnorm(x, norm_w, d, eps, y);
    oracle_rope(y, d, rope_dim, (double)positions[t], theta, +1);
    quantize_pool_row(y, d, kv_pool + row * d, kv_scales + row * (d / BLOCK));
  }
  free(x); free(y);
  return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * CPU oracle for the dense fp16 GEMM  C[M,N] = A[M,K] . B[K,N].
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may call this; the GPU library never does, and this file
 * shares no code with it.
 *
 * What it computes is the definition, written out as the plain triple loop
 * over output row i, output column j and reduction index k that the tiling
 * tutorial ("Matrix multiplication and memory-access optimisation", section
 * 02, the straightforward implementation) and the TileLang tutorial (ch. 14,
 * rung 1, the defining triple loop) give:
 *
 *     C[i,j] = fp16_rne( sum_{k=0}^{K-1} A[i,k] * B[k,j] )
 *
 *   - Operands are read through element strides, as in the Triton article's
 *     section "shape gives meaning, stride gives addresses":
 *       A[i,k] = A[i*lda_m + k*lda_k],  B[k,j] = B[k*ldb_k + j*ldb_n],
 *       C[i,j] = C[i*ldc + j]  (the output's own row stride).
 *   - Every offset is formed in int64 before multiplying (same article,
 *     section "addresses and bounds in one short kernel": 65536*65536 must be
 *     2^32, not an int32 wrap to 0).
 *   - The sum runs over exactly k = 0..K-1 (no padding, no modulo), from +0.0,
 *     in ascending k, in binary64.  Products of two binary16 values have at
 *     most 22 significant bits, so each product is exact in binary64; the
 *     accumulated error is at most K * 2^-53 * sum|a*b|, far below half an
 *     fp16 ulp of the result for the workloads here.
 *   - One rounding to binary16 at the end, roundTiesToEven (the Triton
 *     article's precision paragraph: fp16 inputs, wider accumulation, a final
 *     conversion that may round or overflow; the rounding mode is IEEE 754's
 *     default, ties to even, and overflow gives +-inf).
 *
 * Build: gcc -O2 -ffp-contract=off (no -ffast-math).
 */
#include <pthread.h>
#include <stdint.h>
#include <string.h>

/* ---- IEEE 754 binary16 codec, written from the format definition --------
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-24
 *   exponent 1..30  : normal,    value = (1024 + fraction) * 2^(exponent-25)
 *   exponent 31     : fraction 0 -> infinity, otherwise NaN             */

double orc_f16_to_f64(uint16_t h) {
  uint64_t sign = (uint64_t)(h >> 15) << 63;
  uint32_t e = (h >> 10) & 0x1F;
  uint32_t f = h & 0x3FF;
  uint64_t bits;
  double out;
  if (e == 0) {
    out = (double)f * 0x1p-24; /* exact: f < 2^10 */
    return (h >> 15) ? -out : out;
  }
  if (e == 31) {
    bits = sign | (0x7FFull << 52) | ((uint64_t)f << 42) | (f ? (1ull << 51) : 0);
  } else {
    /* normal: 1.f * 2^(e-15): binary64 exponent field e - 15 + 1023 */
    bits = sign | ((uint64_t)(e - 15 + 1023) << 52) | ((uint64_t)f << 42);
  }
  memcpy(&out, &bits, sizeof out);
  return out;
}

/* Nearest binary16 to a binary64 value, ties to even, by integer rounding of
 * the binary64 significand at the binary16 quantum. */
uint16_t orc_f64_to_f16(double x) {
  uint64_t b;
  memcpy(&b, &x, sizeof b);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int ex = (int)((b >> 52) & 0x7FF);
  uint64_t frac = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return (uint16_t)(sign | (frac ? 0x7E00u : 0x7C00u));
  if (ex == 0) return sign; /* binary64 zero or subnormal: far below 2^-25 */
  int e = ex - 1023;                         /* x = sig * 2^(e-52) */
  uint64_t sig = (1ull << 52) | frac;
  int qe = (e < -14 ? -14 : e) - 10;         /* binary16 quantum exponent */
  int shift = qe - (e - 52);                 /* >= 42 */
  if (shift >= 64) return sign;              /* below a quarter quantum */
  uint64_t q = sig >> shift;
  uint64_t rem = sig & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  if (e < -14) {
    /* subnormal quantum 2^-24; q == 1024 is the smallest normal, whose
     * encoding 0x0400 is numerically the same as q. */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int E = e;
  if (q == 2048) { q = 1024; E += 1; }       /* carry into the next binade */
  if (E + 15 >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024));
}

/* ---- bfloat16 codec, written from the format definition -----------------
 * bfloat16: the upper 16 bits of an IEEE 754 binary32 -- 1 sign bit,
 * 8 exponent bits (bias 127), 7 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-133
 *   exponent 1..254 : normal,    value = (128 + fraction) * 2^(exponent-134)
 *   exponent 255    : fraction 0 -> infinity, otherwise NaN             */

double orc_bf16_to_f64(uint16_t h) {
  uint64_t sign = (uint64_t)(h >> 15) << 63;
  uint32_t e = (h >> 7) & 0xFF;
  uint32_t f = h & 0x7F;
  uint64_t bits;
  double out;
  if (e == 0) {
    out = (double)f * 0x1p-133; /* exact */
    return (h >> 15) ? -out : out;
  }
  if (e == 255) {
    bits = sign | (0x7FFull << 52) | ((uint64_t)f << 45) | (f ? (1ull << 51) : 0);
  } else {
    bits = sign | ((uint64_t)(e - 127 + 1023) << 52) | ((uint64_t)f << 45);
  }
  memcpy(&out, &bits, sizeof out);
  return out;
}

/* Nearest bfloat16 to a binary64 value, ties to even (one rounding, straight
 * from binary64), by integer rounding of the significand at the bfloat16
 * quantum. */
uint16_t orc_f64_to_bf16(double x) {
  uint64_t b;
  memcpy(&b, &x, sizeof b);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int ex = (int)((b >> 52) & 0x7FF);
  uint64_t frac = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return (uint16_t)(sign | (frac ? 0x7FC0u : 0x7F80u));
  if (ex == 0) return sign; /* binary64 zero or subnormal: far below 2^-134 */
  int e = ex - 1023;                         /* x = sig * 2^(e-52) */
  uint64_t sig = (1ull << 52) | frac;
  int qe = (e < -126 ? -126 : e) - 7;        /* bfloat16 quantum exponent */
  int shift = qe - (e - 52);                 /* >= 45 */
  if (shift >= 64) return sign;              /* below a quarter quantum */
  uint64_t q = sig >> shift;
  uint64_t rem = sig & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  if (e < -126) return (uint16_t)(sign | (uint16_t)q);   /* q == 128: smallest normal */
  int E = e;
  if (q == 256) { q = 128; E += 1; }
  if (E + 127 >= 255) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(q - 128));
}

/* ---- 8-bit floating-point formats (OCP FP8), decode only ----------------
 * Inputs arrive one byte per uint16_t element (the upper byte zero).
 * E4M3 ("FN" variant): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-9
 *   exponent 1..15  : normal,    value = (8 + fraction) * 2^(exponent-10)
 *   exponent 15 with fraction 7 is NaN; there are no infinities (max 448).
 * E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-16
 *   exponent 1..30  : normal,    value = (4 + fraction) * 2^(exponent-17)
 *   exponent 31     : fraction 0 -> infinity, otherwise NaN (max 57344). */

static double orc_nan(void) {
  uint64_t bits = 0x7FF8000000000000ull;
  double d;
  memcpy(&d, &bits, sizeof d);
  return d;
}

double orc_e4m3_to_f64(uint16_t v) {
  const int s = (v >> 7) & 1, e = (v >> 3) & 0xF, f = v & 7;
  double out;
  if (e == 15 && f == 7) return orc_nan();
  if (e == 0)
    out = (double)f * 0x1p-9;
  else
    out = (double)(8 + f) * (double)(1u << e) * 0x1p-10;   /* exact */
  return s ? -out : out;
}

double orc_e5m2_to_f64(uint16_t v) {
  const int s = (v >> 7) & 1, e = (v >> 2) & 0x1F, f = v & 3;
  double out;
  if (e == 31) {
    if (f) return orc_nan();
    out = 1.0 / 0.0;
  } else if (e == 0) {
    out = (double)f * 0x1p-16;
  } else {
    out = (double)(4 + f) * (double)(1u << e) * 0x1p-17;   /* exact */
  }
  return s ? -out : out;
}

typedef double (*orc_dec_fn)(uint16_t);
typedef uint16_t (*orc_enc_fn)(double);

/* One output element: the defining sum, ascending k, binary64. */
static double orc_dot(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                      int64_t ldb_k, int64_t ldb_n, int64_t i, int64_t j, int64_t K,
                      orc_dec_fn dec_a, orc_dec_fn dec_b) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k)
    s += dec_a(A[i * lda_m + k * lda_k]) * dec_b(B[k * ldb_k + j * ldb_n]);
  return s;
}

typedef struct {
  const uint16_t* A; int64_t lda_m, lda_k;
  const uint16_t* B; int64_t ldb_k, ldb_n;
  uint16_t* C; int64_t ldc;
  double* S;                 /* optional unrounded sums, [M][N] contiguous */
  int64_t M, N, K;
  const int64_t* pi;         /* point mode: output coordinates */
  const int64_t* pj;
  int64_t npts;
  orc_dec_fn dec;            /* element format of A: binary16, bfloat16, E4M3, E5M2 */
  orc_enc_fn enc;            /* output format: binary16 or bfloat16 */
  int nthreads, tid;
  orc_dec_fn dec_b;          /* element format of B (NULL: the same as A) */
} orc_job;

static void* orc_rows(void* p) {
  orc_job* j = (orc_job*)p;
  for (int64_t i = j->tid; i < j->M; i += j->nthreads)
    for (int64_t c = 0; c < j->N; ++c) {
      double s = orc_dot(j->A, j->lda_m, j->lda_k, j->B, j->ldb_k, j->ldb_n, i, c, j->K, j->dec,
                         j->dec_b ? j->dec_b : j->dec);
      j->C[i * j->ldc + c] = j->enc(s);
      if (j->S) j->S[i * j->N + c] = s;
    }
  return NULL;
}

static void* orc_points(void* p) {
  orc_job* j = (orc_job*)p;
  for (int64_t t = j->tid; t < j->npts; t += j->nthreads) {
    double s = orc_dot(j->A, j->lda_m, j->lda_k, j->B, j->ldb_k, j->ldb_n, j->pi[t], j->pj[t], j->K,
                       j->dec, j->dec_b ? j->dec_b : j->dec);
    j->C[t] = j->enc(s);
    if (j->S) j->S[t] = s;
  }
  return NULL;
}

static void orc_run(orc_job* proto, void* (*fn)(void*)) {
  int n = proto->nthreads < 1 ? 1 : (proto->nthreads > 512 ? 512 : proto->nthreads);
  pthread_t th[512];
  orc_job jobs[512];
  for (int t = 0; t < n; ++t) { jobs[t] = *proto; jobs[t].nthreads = n; jobs[t].tid = t; }
  int started = 0;
  for (int t = 1; t < n; ++t) {
    if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) break;
    started = t;
  }
  fn(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < n; ++t) fn(&jobs[t]);
}

/* Full product.  Threads take interleaved output rows; every element is the
 * same sequential sum whichever thread computes it.  S may be NULL.
 * Returns 0, or -1 for arguments outside the contract (sizes <= 0, NULL). */
int orc_gemm_f16(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                 int64_t ldb_k, int64_t ldb_n, uint16_t* C, int64_t ldc, double* S,
                 int64_t M, int64_t N, int64_t K, int nthreads) {
  if (!A || !B || !C || M <= 0 || N <= 0 || K <= 0) return -1;
  orc_job j = {A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, S, M, N, K, NULL, NULL, 0,
               orc_f16_to_f64, orc_f64_to_f16, nthreads, 0};
  orc_run(&j, orc_rows);
  return 0;
}

/* The same product for bfloat16 inputs and output (fp32 accumulation on the
 * GPU side; here the same binary64 sum and one rounding to bfloat16). */
int orc_gemm_bf16(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                  int64_t ldb_k, int64_t ldb_n, uint16_t* C, int64_t ldc, double* S,
                  int64_t M, int64_t N, int64_t K, int nthreads) {
  if (!A || !B || !C || M <= 0 || N <= 0 || K <= 0) return -1;
  orc_job j = {A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, S, M, N, K, NULL, NULL, 0,
               orc_bf16_to_f64, orc_f64_to_bf16, nthreads, 0};
  orc_run(&j, orc_rows);
  return 0;
}

/* Selected outputs: out[t] = C[pi[t], pj[t]] (and S[t] its unrounded sum). */
int orc_gemm_f16_points(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                        int64_t ldb_k, int64_t ldb_n, int64_t K, const int64_t* pi,
                        const int64_t* pj, int64_t npts, uint16_t* out, double* S,
                        int nthreads) {
  if (!A || !B || !out || !pi || !pj || K <= 0 || npts < 0) return -1;
  orc_job j = {A, lda_m, lda_k, B, ldb_k, ldb_n, out, 0, S, 0, 0, K, pi, pj, npts,
               orc_f16_to_f64, orc_f64_to_f16, nthreads, 0};
  orc_run(&j, orc_points);
  return 0;
}

int orc_gemm_bf16_points(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                         int64_t ldb_k, int64_t ldb_n, int64_t K, const int64_t* pi,
                         const int64_t* pj, int64_t npts, uint16_t* out, double* S,
                         int nthreads) {
  if (!A || !B || !out || !pi || !pj || K <= 0 || npts < 0) return -1;
  orc_job j = {A, lda_m, lda_k, B, ldb_k, ldb_n, out, 0, S, 0, 0, K, pi, pj, npts,
               orc_bf16_to_f64, orc_f64_to_bf16, nthreads, 0};
  orc_run(&j, orc_points);
  return 0;
}

/* FP8 inputs (fmt 0 = E4M3, 1 = E5M2, per operand; one byte per uint16_t
 * element), binary64 sum, one rounding to binary16. */
static orc_dec_fn orc_f8_dec(int fmt) {
  return fmt == 0 ? orc_e4m3_to_f64 : (fmt == 1 ? orc_e5m2_to_f64 : NULL);
}

int orc_gemm_f8(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                int64_t ldb_k, int64_t ldb_n, uint16_t* C, int64_t ldc, double* S,
                int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b, int nthreads) {
  if (!A || !B || !C || M <= 0 || N <= 0 || K <= 0) return -1;
  if (!orc_f8_dec(fmt_a) || !orc_f8_dec(fmt_b)) return -1;
  orc_job j = {A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, S, M, N, K, NULL, NULL, 0,
               orc_f8_dec(fmt_a), orc_f64_to_f16, nthreads, 0, orc_f8_dec(fmt_b)};
  orc_run(&j, orc_rows);
  return 0;
}

int orc_gemm_f8_points(const uint16_t* A, int64_t lda_m, int64_t lda_k, const uint16_t* B,
                       int64_t ldb_k, int64_t ldb_n, int64_t K, const int64_t* pi,
                       const int64_t* pj, int64_t npts, uint16_t* out, double* S, int fmt_a,
                       int fmt_b, int nthreads) {
  if (!A || !B || !out || !pi || !pj || K <= 0 || npts < 0) return -1;
  if (!orc_f8_dec(fmt_a) || !orc_f8_dec(fmt_b)) return -1;
  orc_job j = {A, lda_m, lda_k, B, ldb_k, ldb_n, out, 0, S, 0, 0, K, pi, pj, npts,
               orc_f8_dec(fmt_a), orc_f64_to_f16, nthreads, 0, orc_f8_dec(fmt_b)};
  orc_run(&j, orc_points);
  return 0;
}

void orc_e4m3_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t t = 0; t < n; ++t) out[t] = orc_e4m3_to_f64(in[t]);
}

void orc_e5m2_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t t = 0; t < n; ++t) out[t] = orc_e5m2_to_f64(in[t]);
}

/* Array forms of the codec, for the tests that sweep all 65536 patterns. */
void orc_f16_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t t = 0; t < n; ++t) out[t] = orc_f16_to_f64(in[t]);
}

void orc_f64_to_f16_array(const double* in, uint16_t* out, int64_t n) {
  for (int64_t t = 0; t < n; ++t) out[t] = orc_f64_to_f16(in[t]);
}

void orc_bf16_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t t = 0; t < n; ++t) out[t] = orc_bf16_to_f64(in[t]);
}

void orc_f64_to_bf16_array(const double* in, uint16_t* out, int64_t n) {
  for (int64_t t = 0; t < n; ++t) out[t] = orc_f64_to_bf16(in[t]);
}

/*
 * Seeded, counter-based input generator for fp16 matrices.
 *
 * This module holds no matrix-multiply arithmetic.  It only turns
 * (seed, tensor id, logical row, logical column) into an IEEE binary16 bit
 * pattern, so any element of A[M,K] or B[K,N] can be regenerated on its own,
 * whatever the storage layout (row-major, transposed view, strided slice).
 * Both the GPU tests and the CPU oracle read inputs made here.
 *
 * Hash: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014), applied as a chain
 *     h = sm(sm(sm(sm(seed) ^ tensor) ^ row) ^ col)
 * where sm(x) is one SplitMix64 step on state x.
 *
 * Value modes:
 *   SYNTH_UNIFORM: u = top 24 bits of h; x = (2u + 1 - 2^24) * 2^-24, an odd
 *                  multiple of 2^-24 inside (-1, 1), exact in binary32; the
 *                  element is x rounded to binary16 (ties to even).
 *   SYNTH_INT:     (h >> 40) % 9 - 4, an integer in [-4, 4] (exact in fp16).
 * With SYNTH_BF16 added to the mode the same value is rounded to bfloat16
 * (ties to even) instead of binary16.  With SYNTH_E4M3 or SYNTH_E5M2 it is
 * rounded (ties to even) to that OCP FP8 format and the destination holds
 * one byte per element.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_UNIFORM 0
#define SYNTH_INT 1
#define SYNTH_BF16 2
#define SYNTH_E4M3 4
#define SYNTH_E5M2 8

static inline uint64_t sm_step(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Round a finite double to binary16, ties to even, by scaling to the target
 * quantum and using the C library's round-to-nearest-even (nearbyint under
 * the default rounding mode). */
static uint16_t synth_to_half(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  int e2;
  frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1) */
  int ex = e2 - 1;          /* floor(log2 a) */
  if (ex < -14) ex = -14;   /* subnormal range shares the quantum 2^-24 */
  double q = ldexp(1.0, ex - 10);
  double m = nearbyint(a / q);
  double v = m * q;         /* exact */
  if (v >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
  frexp(v, &e2);
  int ev = e2 - 1;
  uint16_t mant = (uint16_t)(v / ldexp(1.0, ev - 10) - 1024.0);
  return (uint16_t)(sign | (uint16_t)((ev + 15) << 10) | mant);
}

/* Round a finite double to bfloat16 (8 exponent bits, 7 fraction bits),
 * ties to even, the same way: scale to the quantum, nearbyint, re-encode. */
static uint16_t synth_to_bf16(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (a == 0.0) return sign;
  const double big = ldexp(1.0, 128) * (1.0 - ldexp(1.0, -9));  /* rounds to 2^128 */
  if (a >= big) return (uint16_t)(sign | 0x7F80u);
  int e2;
  frexp(a, &e2);
  int ex = e2 - 1;
  if (ex < -126) ex = -126;
  double q = ldexp(1.0, ex - 7);
  double m = nearbyint(a / q);
  double v = m * q;
  if (v < ldexp(1.0, -126)) return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -133)));
  frexp(v, &e2);
  int ev = e2 - 1;
  if (ev + 127 >= 255) return (uint16_t)(sign | 0x7F80u);
  uint16_t mant = (uint16_t)(v / ldexp(1.0, ev - 7) - 128.0);
  return (uint16_t)(sign | (uint16_t)((ev + 127) << 7) | mant);
}

/* Round a finite double to an OCP FP8 format with `mbits` fraction bits,
 * exponent bias `bias`, ties to even: scale to the quantum, nearbyint,
 * re-encode.  E4M3 (mbits 3, bias 7) has no infinity and its largest finite
 * value is 448; a larger rounded magnitude gives its NaN (0x7F).  E5M2
 * (mbits 2, bias 15) overflows past 57344 to infinity (0x7C). */
static uint8_t synth_to_f8(double x, int mbits, int bias) {
  const int e4m3 = mbits == 3;
  uint8_t sign = signbit(x) ? 0x80u : 0u;
  double a = fabs(x);
  if (a == 0.0) return sign;
  const double maxv = e4m3 ? 448.0 : 57344.0;
  const int emin = 1 - bias;                 /* exponent of the smallest normal */
  int e2;
  frexp(a, &e2);
  int ex = e2 - 1;
  if (ex < emin) ex = emin;                  /* subnormals share the quantum */
  double q = ldexp(1.0, ex - mbits);
  if (ex > 20) return (uint8_t)(sign | (e4m3 ? 0x7Fu : 0x7Cu));
  double m = nearbyint(a / q);
  double v = m * q;
  if (v > maxv) return (uint8_t)(sign | (e4m3 ? 0x7Fu : 0x7Cu));
  if (v < ldexp(1.0, emin)) return (uint8_t)(sign | (uint8_t)(v / ldexp(1.0, emin - mbits)));
  frexp(v, &e2);
  int ev = e2 - 1;
  uint8_t mant = (uint8_t)(v / ldexp(1.0, ev - mbits) - (double)(1 << mbits));
  return (uint8_t)(sign | (uint8_t)((ev + bias) << mbits) | mant);
}

static inline double synth_draw(uint64_t h, int mode) {
  if ((mode & 1) == SYNTH_INT) return (double)((int)((h >> 40) % 9u) - 4);
  int64_t u = (int64_t)(h >> 40);
  return (double)(2 * u + 1 - (1ll << 24)) * 0x1p-24;
}

static inline uint16_t synth_value(uint64_t h, int mode) {
  const double x = synth_draw(h, mode);
  return (mode & SYNTH_BF16) ? synth_to_bf16(x) : synth_to_half(x);
}

typedef struct {
  uint16_t* dst;
  const int64_t* row_index; /* optional list of logical rows, NULL = row0.. */
  int64_t rows, cols, rs, cs, row0;
  uint64_t seed;
  uint64_t tensor;
  int mode, nthreads, tid;
} synth_job;

static void* synth_worker(void* p) {
  synth_job* j = (synth_job*)p;
  uint64_t base_t = sm_step(sm_step(j->seed) ^ j->tensor);
  for (int64_t r = j->tid; r < j->rows; r += j->nthreads) {
    int64_t lr = j->row_index ? j->row_index[r] : j->row0 + r;
    uint64_t base_r = sm_step(base_t ^ (uint64_t)lr);
    if (j->mode & (SYNTH_E4M3 | SYNTH_E5M2)) {
      const int e4 = (j->mode & SYNTH_E4M3) != 0;
      uint8_t* row8 = (uint8_t*)j->dst + r * j->rs;
      for (int64_t c = 0; c < j->cols; ++c)
        row8[c * j->cs] = synth_to_f8(synth_draw(sm_step(base_r ^ (uint64_t)c), j->mode),
                                      e4 ? 3 : 2, e4 ? 7 : 15);
      continue;
    }
    uint16_t* row = j->dst + r * j->rs;
    for (int64_t c = 0; c < j->cols; ++c)
      row[c * j->cs] = synth_value(sm_step(base_r ^ (uint64_t)c), j->mode);
  }
  return NULL;
}

/*
 * Fill dst[r*rs + c*cs] = element (logical row, logical col c) for r in
 * [0, rows), where the logical row is row_index[r] if row_index is not NULL,
 * else row0 + r.  Strides are in elements; dst holds uint16_t elements, or
 * bytes for the FP8 modes.  Returns 0, or -1 on bad args.
 */
int synth_fill(uint16_t* dst, int64_t rows, int64_t cols, int64_t rs, int64_t cs,
               int64_t row0, const int64_t* row_index, uint64_t seed, uint64_t tensor,
               int mode, int nthreads) {
  if (!dst || rows < 0 || cols < 0 || mode < 0 || mode > (SYNTH_INT | SYNTH_E5M2)) return -1;
  {
    const int fmts = (mode & SYNTH_BF16 ? 1 : 0) + (mode & SYNTH_E4M3 ? 1 : 0) + (mode & SYNTH_E5M2 ? 1 : 0);
    if (fmts > 1) return -1;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (rows < nthreads) nthreads = rows > 0 ? (int)rows : 1;
  pthread_t th[256];
  synth_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    synth_job j = {dst, row_index, rows, cols, rs, cs, row0, seed, tensor, mode, nthreads, t};
    jobs[t] = j;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, synth_worker, &jobs[t]) != 0) break;
    started = t;
  }
  synth_worker(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  /* Rows of threads that failed to start are done here. */
  for (int t = started + 1; t < nthreads; ++t) synth_worker(&jobs[t]);
  return 0;
}

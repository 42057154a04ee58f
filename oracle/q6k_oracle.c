/*
 * q6k_oracle.c -- plain, slow CPU oracle for the q6_K x int8 prefill GEMM
 *     Y[N x M] = X[N x K] . dequant(W_q6K[M x K])^T
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load this file.  The product library never links, loads or calls it, and it shares
 * no code, header, table or constant with the HIP kernels.
 *
 * Sources (titles of the pages of the optimisation log this follows):
 *   [r38]  "r38 — q6_K BT-style raw-byte mma kernel (LANDED)"
 *            sec. 2.1  the real q6_K layout: ql[128] low nibbles, qh[64] 2-bit high fields,
 *                      scales[16] int8 (one per 16 elements), f16 d; w = d * sc[sub] * (q - 32)
 *            sec. 2.2  rescale without a dmin term: sum += da * dsc, dsc = d * sc[16-sub-block]
 *            sec. 2.4  KSPLIT=2: each 32-k chunk is two 16-k halves with their own integer sums
 *            sec. 3.2  the per-element index map (ql/qh index and shift) and the dsc offsets 192/208
 *   [r41]  "r41 — q6_K B-expand widened to uint4 group loads (LANDED)", sec. 2: byte map of a block
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - activation scale: symmetric absmax per (token, 32-k chunk): da = amax / 127 in IEEE f32;
 *   - code: q = roundf(x / da) with one correctly rounded f32 division and round-half-away-
 *     from-zero, clamped to [-127, 127]; an all-zero chunk (da == 0) gives q = 0;
 *   - the f16 d is little-endian at bytes 208..209 and converted exactly (subnormals kept);
 *   - the output reference is the f64 sum of the per-sub-block terms da * (d * sc) * D, and the
 *     per-output tolerance scale T is the f64 sum of their magnitudes.
 *
 * Every function is plain loops; integer dots are accumulated in int64.  The functions over
 * many output rows (or tokens) take a thread count and hand each thread one contiguous range of
 * rows: rows are independent and each row's loops and arithmetic are the same whatever the range,
 * so the result is the same bit for bit for any thread count (threads <= 1: the calling thread
 * does everything).
 * Build: gcc -O2 -fPIC -shared -pthread (no -ffast-math: the f32 division and roundf must be IEEE).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <math.h>

#define QK 256          /* elements per super-block           [r38 sec. 2.1] */
#define BLOCK_BYTES 210 /* 128 ql + 64 qh + 16 sc + 2 d       [r38 sec. 2.1] */
#define OFF_QH 128
#define OFF_SC 192
#define OFF_D 208

/* Run fn(ctx, r0, r1) over rows [0, m) split into `threads` contiguous ranges, one per thread. */
typedef void (*q6o_rows_fn)(void* ctx, int64_t r0, int64_t r1);
struct q6o_rows_job {
  q6o_rows_fn fn;
  void* ctx;
  int64_t r0, r1;
};
static void* q6o_rows_thread(void* p) {
  struct q6o_rows_job* job = (struct q6o_rows_job*)p;
  job->fn(job->ctx, job->r0, job->r1);
  return NULL;
}
void q6o_parallel_rows(q6o_rows_fn fn, void* ctx, int64_t m, int threads) {
  if ((int64_t)threads > m) threads = (int)m;
  if (threads <= 1) {
    fn(ctx, 0, m);
    return;
  }
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  int* started = (int*)calloc((size_t)threads, sizeof(int));
  struct q6o_rows_job* job = (struct q6o_rows_job*)malloc(sizeof(*job) * (size_t)threads);
  for (int i = 0; i < threads; ++i) {
    job[i].fn = fn;
    job[i].ctx = ctx;
    job[i].r0 = m * i / threads;
    job[i].r1 = m * (i + 1) / threads;
    started[i] = pthread_create(&tid[i], NULL, q6o_rows_thread, &job[i]) == 0;
    if (!started[i]) q6o_rows_thread(&job[i]); /* no thread available: run the range here */
  }
  for (int i = 0; i < threads; ++i)
    if (started[i]) pthread_join(tid[i], NULL);
  free(tid);
  free(started);
  free(job);
}

/* IEEE 754 binary16 -> double, exact for every finite value including subnormals. */
double q6o_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 31;
  int man = h & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24);                  /* subnormal: man * 2^-24 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + man), ex - 25);     /* (1 + man/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

/* 6-bit code (0..63) of element e (0..255) of one raw block.
 * [r38 sec. 3.2]: the element splits into its 128-element half it = e / 128 and the offset
 * n = e % 128 inside that half.  The low 4 bits are nibble (n / 64) of ql[64*it + n % 64]; the
 * high 2 bits are field ((n / 32) % 4) of qh[32*it + n % 32]. */
int q6o_code(const uint8_t* blk, int e) {
  int it = e / 128;
  int n = e % 128;
  int lo = (blk[64 * it + n % 64] >> (4 * (n / 64))) & 15;
  int hi = (blk[OFF_QH + 32 * it + n % 32] >> (2 * ((n / 32) % 4))) & 3;
  return lo | (hi << 4);
}

/* Decode m rows of k/256 raw blocks each.
 *   wc[m][k]    centered value q - 32 in [-32, 31]             [r38 sec. 2.1]
 *   sc[m][k/16] signed sub-block scale (int8 at byte 192 + s)   [r38 sec. 3.2]
 *   d[m][k/256] super-block scale, f16 at byte 208              [r38 sec. 3.2]
 * Any output pointer may be NULL. */
void q6o_decode(const uint8_t* raw, int64_t m, int64_t k, int8_t* wc, int8_t* sc, double* d) {
  int64_t nsb = k / QK;
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t b = 0; b < nsb; ++b) {
      const uint8_t* blk = raw + (r * nsb + b) * BLOCK_BYTES;
      if (wc)
        for (int e = 0; e < QK; ++e) wc[r * k + b * QK + e] = (int8_t)(q6o_code(blk, e) - 32);
      if (sc)
        for (int s = 0; s < 16; ++s) sc[r * (k / 16) + b * 16 + s] = (int8_t)blk[OFF_SC + s];
      if (d) d[r * nsb + b] = q6o_f16_to_f64((uint16_t)(blk[OFF_D] | (blk[OFF_D + 1] << 8)));
    }
  }
}

/* Dequantized weights w[m][k] = d * sc * (q - 32) in f64 (exact).  [r38 sec. 2.1] */
void q6o_dequant(const uint8_t* raw, int64_t m, int64_t k, double* w) {
  int64_t nsb = k / QK;
  for (int64_t r = 0; r < m; ++r)
    for (int64_t b = 0; b < nsb; ++b) {
      const uint8_t* blk = raw + (r * nsb + b) * BLOCK_BYTES;
      double d = q6o_f16_to_f64((uint16_t)(blk[OFF_D] | (blk[OFF_D + 1] << 8)));
      for (int e = 0; e < QK; ++e) {
        int s = e / 16;
        double scale = d * (double)(int8_t)blk[OFF_SC + s];
        w[r * k + b * QK + e] = scale * (double)(q6o_code(blk, e) - 32);
      }
    }
}

/* Activation quantization per (token, 32-k chunk) with f32 scale da (reading above).
 *   xq[n][k] int8, da[n][k/32] f32. */
struct q6o_quantize_args {
  const float* x;
  int64_t k;
  int8_t* xq;
  float* da;
};
static void q6o_quantize_rows(void* p, int64_t t0, int64_t t1) {
  const struct q6o_quantize_args* a = (const struct q6o_quantize_args*)p;
  const float* x = a->x;
  int64_t k = a->k;
  int8_t* xq = a->xq;
  float* da = a->da;
  int64_t nc = k / 32;
  for (int64_t t = t0; t < t1; ++t)
    for (int64_t c = 0; c < nc; ++c) {
      const float* xc = x + t * k + c * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(xc[i]);
        if (a > amax) amax = a;
      }
      volatile float scale = amax / 127.0f;   /* one IEEE f32 division */
      da[t * nc + c] = scale;
      for (int i = 0; i < 32; ++i) {
        int q = 0;
        if (scale != 0.0f) {
          volatile float ratio = xc[i] / scale; /* one IEEE f32 division */
          float r = roundf(ratio);              /* half away from zero */
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          q = (int)r;
        }
        xq[t * k + c * 32 + i] = (int8_t)q;
      }
    }
}
void q6o_quantize(const float* x, int64_t n, int64_t k, int8_t* xq, float* da, int threads) {
  struct q6o_quantize_args a = {x, k, xq, da};
  q6o_parallel_rows(q6o_quantize_rows, &a, n, threads);
}

/* Decode one row of blocks into centered codes. */
static void decode_row(const uint8_t* row, int64_t k, int8_t* wc) {
  for (int64_t b = 0; b < k / QK; ++b)
    for (int e = 0; e < QK; ++e) wc[b * QK + e] = (int8_t)(q6o_code(row + b * BLOCK_BYTES, e) - 32);
}

/* Per-sub-block integer dots D[n][m][s] = sum_{k in sub-block s} xq[n][k] * wc[m][k]
 * (KSPLIT=2 halves, [r38 sec. 2.4]); exact, stored as int32 (|D| <= 16*127*32). */
struct q6o_dots_args {
  const int8_t* xq;
  const uint8_t* raw;
  int64_t n, m, k;
  int32_t* dots;
};
static void q6o_subdots_rows(void* p, int64_t j0, int64_t j1) {
  const struct q6o_dots_args* a = (const struct q6o_dots_args*)p;
  const int8_t* xq = a->xq;
  int64_t n = a->n, m = a->m, k = a->k;
  int32_t* dots = a->dots;
  int64_t ns = k / 16;
  int64_t row_bytes = (k / QK) * BLOCK_BYTES;
  int8_t* wc = (int8_t*)malloc((size_t)k);
  for (int64_t j = j0; j < j1; ++j) {
    decode_row(a->raw + j * row_bytes, k, wc);
    for (int64_t t = 0; t < n; ++t)
      for (int64_t s = 0; s < ns; ++s) {
        int64_t acc = 0;
        for (int i = 0; i < 16; ++i) acc += (int64_t)xq[t * k + s * 16 + i] * (int64_t)wc[s * 16 + i];
        dots[(t * m + j) * ns + s] = (int32_t)acc;
      }
  }
  free(wc);
}
void q6o_subdots(const int8_t* xq, const uint8_t* raw, int64_t n, int64_t m, int64_t k,
                 int32_t* dots, int threads) {
  struct q6o_dots_args a = {xq, raw, n, m, k, dots};
  q6o_parallel_rows(q6o_subdots_rows, &a, m, threads);
}

/* SwiGLU product feeding ffn_down, in f64: h = up * silu(gate), silu(g) = g / (1 + exp(-g)), for
 * `count` elements.  The pages quantize this product right after it is produced (the fused
 * producers of "r53 — q6_K bundle: W_exp pre-expansion plane + cp.async B staging (LANDED)",
 * sec. 1); the quantization itself is q6o_quantize. */
void q6o_swiglu(const float* gate, const float* up, int64_t count, double* h) {
  for (int64_t i = 0; i < count; ++i) {
    double g = (double)gate[i];
    h[i] = (double)up[i] * (g / (1.0 + exp(-g)));
  }
}

/* Per-chunk integer numerators with the sub-block scales applied:
 *   E[n][m][c] = sum over the 32 elements i of chunk c of xq[n][i] * sc[m][i/16] * (q[m][i] - 32)
 * (int64 accumulation, stored as int32: |E| <= 32 * 127 * 4096 < 2^24).  [r38 sec. 2.1] gives
 * one f16 d per 256-element super-block and one int8 sc per 16 elements, so the chunk's share of
 * y is da[n][c] * d[m][c/8] * E[n][m][c], which equals the two per-half terms of sec. 2.2 summed
 * in exact arithmetic.  Written from the definition: decode each element, multiply by its own
 * scale, sum over the chunk. */
static void q6o_chunkdots_rows(void* p, int64_t j0, int64_t j1) {
  const struct q6o_dots_args* a = (const struct q6o_dots_args*)p;
  const int8_t* xq = a->xq;
  int64_t n = a->n, m = a->m, k = a->k;
  int32_t* dots = a->dots;
  int64_t nc = k / 32;
  int64_t row_bytes = (k / QK) * BLOCK_BYTES;
  int32_t* ws = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  for (int64_t j = j0; j < j1; ++j) {
    const uint8_t* row = a->raw + j * row_bytes;
    for (int64_t i = 0; i < k; ++i) {
      const uint8_t* blk = row + (i / QK) * BLOCK_BYTES;
      int sc = (int8_t)blk[OFF_SC + (i % QK) / 16];
      ws[i] = sc * (q6o_code(blk, (int)(i % QK)) - 32);
    }
    for (int64_t t = 0; t < n; ++t)
      for (int64_t c = 0; c < nc; ++c) {
        int64_t acc = 0;
        for (int i = 0; i < 32; ++i) acc += (int64_t)xq[t * k + c * 32 + i] * (int64_t)ws[c * 32 + i];
        dots[(t * m + j) * nc + c] = (int32_t)acc;
      }
  }
  free(ws);
}
void q6o_chunkdots(const int8_t* xq, const uint8_t* raw, int64_t n, int64_t m, int64_t k,
                   int32_t* dots, int threads) {
  struct q6o_dots_args a = {xq, raw, n, m, k, dots};
  q6o_parallel_rows(q6o_chunkdots_rows, &a, m, threads);
}

/* Reference output: y[n][m] = sum_s da[n][s/2] * (d[m][s/16] * sc[m][s]) * D[n][m][s] in f64,
 * and t[n][m] = sum_s |that term|, the tolerance scale ([r38 sec. 2.2]: one rescale per
 * 16-element half, no dmin term).  t may be NULL. */
struct q6o_gemm_args {
  const int8_t* xq;
  const float* da;
  int64_t n;
  const uint8_t* raw;
  int64_t m, k;
  double *y, *t;
};
static void q6o_gemm_rows(void* p, int64_t j0, int64_t j1) {
  const struct q6o_gemm_args* a = (const struct q6o_gemm_args*)p;
  const int8_t* xq = a->xq;
  const float* da = a->da;
  int64_t n = a->n, m = a->m, k = a->k;
  double *y = a->y, *t = a->t;
  int64_t nsb = k / QK, ns = k / 16, nc = k / 32;
  int64_t row_bytes = nsb * BLOCK_BYTES;
  int8_t* wc = (int8_t*)malloc((size_t)k);
  double* dsc = (double*)malloc(sizeof(double) * (size_t)ns);
  for (int64_t j = j0; j < j1; ++j) {
    const uint8_t* row = a->raw + j * row_bytes;
    decode_row(row, k, wc);
    for (int64_t s = 0; s < ns; ++s) {
      const uint8_t* blk = row + (s / 16) * BLOCK_BYTES;
      double d = q6o_f16_to_f64((uint16_t)(blk[OFF_D] | (blk[OFF_D + 1] << 8)));
      dsc[s] = d * (double)(int8_t)blk[OFF_SC + s % 16];
    }
    for (int64_t tk = 0; tk < n; ++tk) {
      double sum = 0.0, mag = 0.0;
      for (int64_t s = 0; s < ns; ++s) {
        int64_t acc = 0;
        for (int i = 0; i < 16; ++i) acc += (int64_t)xq[tk * k + s * 16 + i] * (int64_t)wc[s * 16 + i];
        double term = (double)da[tk * nc + s / 2] * dsc[s] * (double)acc;
        sum += term;
        mag += fabs(term);
      }
      y[tk * m + j] = sum;
      if (t) t[tk * m + j] = mag;
    }
  }
  free(wc);
  free(dsc);
}
void q6o_gemm(const int8_t* xq, const float* da, int64_t n, const uint8_t* raw, int64_t m,
              int64_t k, double* y, double* t, int threads) {
  struct q6o_gemm_args a = {xq, da, n, raw, m, k, y, t};
  q6o_parallel_rows(q6o_gemm_rows, &a, m, threads);
}

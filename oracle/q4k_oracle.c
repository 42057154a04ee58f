/*
 * q4k_oracle.c -- plain, slow CPU oracle for the q4_K x int8 prefill GEMM
 *     Y[N x M] = X[N x K] . dequant(W_q4K[M x K])^T
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load this file.  The product library never links, loads or calls it, and it shares
 * no code, header, table or constant with the HIP kernels.
 *
 * Source: "r18: Load-time B pre-expansion — staging becomes a bulk copy (W_exp's debut,
 * REVERTED)", sec. 1 (a q4_K super-block is 144 bytes: a 16-byte header and 128 bytes of packed
 * 4-bit codes, 8 sub-blocks of 32), sec. 2 (the codes are raw nibbles 0..15 in element order; each
 * 32-element chunk carries the pair d*sc and -dmin*m), sec. 3.2 (d and dmin are the f16 words at
 * bytes 0 and 2, sc and m come from 6-bit fields of the 12 header bytes at 4), and "r38 — q6_K
 * BT-style raw-byte mma kernel (LANDED)", sec. 2.2 (q4_K's rescale has two terms, d and dmin,
 * and needs the activations' per-chunk sum).
 *
 * Readings where the pages are silent (each also listed in the design notes): the pages follow
 * the GGUF/ggml block conventions but do not print the q4_K bit packing, which is taken from that
 * published format:
 *   - the 12 scale bytes hold eight 6-bit (sc, m) pairs: for sub-block j < 4, sc = s[j] & 63 and
 *     m = s[j+4] & 63; for j >= 4, sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4 and
 *     m = (s[j+4] >> 4) | (s[j] >> 6) << 4;
 *   - code byte qs[32g + l] (g = 0..3, l = 0..31) holds element 64g + l in its low nibble and
 *     element 64g + 32 + l in its high nibble;
 *   - w = d * sc * q - dmin * m for an element of sub-block j with code q.
 * The activations are quantized exactly as for q6_K (q6o_quantize); S is the sum of a chunk's
 * 32 int8 codes, so the chunk's contribution is da * (d*sc*D - dmin*m*S) with D = sum xq * q.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>

#define Q4_QK 256
#define Q4_BLOCK 144
#define Q4_OFF_SCALES 4
#define Q4_OFF_QS 16

double q6o_f16_to_f64(uint16_t h); /* exact binary16 decode, in q6k_oracle.c */
/* rows [0, m) in contiguous ranges over `threads` threads, in q6k_oracle.c */
typedef void (*q6o_rows_fn)(void* ctx, int64_t r0, int64_t r1);
void q6o_parallel_rows(q6o_rows_fn fn, void* ctx, int64_t m, int threads);

/* The 6-bit scale and min of sub-block j (0..7) from the 12 scale bytes s. */
void q4o_scale_min(const uint8_t* s, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = s[j] & 63;
    *m = s[j + 4] & 63;
  } else {
    *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

/* 4-bit code (0..15) of element e (0..255) of one 144-byte block. */
int q4o_code(const uint8_t* blk, int e) {
  int g = e / 64, r = e % 64;
  uint8_t byte = blk[Q4_OFF_QS + 32 * g + (r % 32)];
  return r < 32 ? (byte & 15) : (byte >> 4);
}

/* codes [m][k] (0..15), sc and mn [m][k/32], d and dmin [m][k/256] of raw blocks, row j's
 * super-block b at byte (j*(k/256) + b)*144. */
void q4o_decode(const uint8_t* raw, int64_t m, int64_t k, uint8_t* codes, uint8_t* sc,
                uint8_t* mn, double* d, double* dmin) {
  int64_t nsb = k / Q4_QK;
  for (int64_t j = 0; j < m; ++j)
    for (int64_t b = 0; b < nsb; ++b) {
      const uint8_t* blk = raw + (j * nsb + b) * Q4_BLOCK;
      d[j * nsb + b] = q6o_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
      dmin[j * nsb + b] = q6o_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
      for (int s = 0; s < 8; ++s) {
        int a, mm;
        q4o_scale_min(blk + Q4_OFF_SCALES, s, &a, &mm);
        sc[j * (k / 32) + b * 8 + s] = (uint8_t)a;
        mn[j * (k / 32) + b * 8 + s] = (uint8_t)mm;
      }
      for (int e = 0; e < Q4_QK; ++e) codes[j * k + b * Q4_QK + e] = (uint8_t)q4o_code(blk, e);
    }
}

/* Dequantized weights w[m][k] = d*sc*q - dmin*m in f64. */
void q4o_dequant(const uint8_t* raw, int64_t m, int64_t k, double* w) {
  int64_t nsb = k / Q4_QK;
  for (int64_t j = 0; j < m; ++j)
    for (int64_t b = 0; b < nsb; ++b) {
      const uint8_t* blk = raw + (j * nsb + b) * Q4_BLOCK;
      double d = q6o_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
      double dmin = q6o_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
      for (int e = 0; e < Q4_QK; ++e) {
        int a, mm;
        q4o_scale_min(blk + Q4_OFF_SCALES, e / 32, &a, &mm);
        w[j * k + b * Q4_QK + e] = d * a * q4o_code(blk, e) - dmin * mm;
      }
    }
}

/* Per-chunk integer dots D[n][m][k/32] = sum over the chunk of xq * q (exact, |D| <= 32*127*15). */
struct q4o_dots_args {
  const int8_t* xq;
  const uint8_t* raw;
  int64_t n, m, k;
  int32_t* dots;
};
static void q4o_chunkdots_rows(void* p, int64_t j0, int64_t j1) {
  const struct q4o_dots_args* a = (const struct q4o_dots_args*)p;
  const int8_t* xq = a->xq;
  const uint8_t* raw = a->raw;
  int64_t n = a->n, m = a->m, k = a->k;
  int32_t* dots = a->dots;
  int64_t nc = k / 32, nsb = k / Q4_QK;
  uint8_t* q = (uint8_t*)malloc((size_t)k);
  for (int64_t j = j0; j < j1; ++j) {
    for (int64_t i = 0; i < k; ++i) q[i] = (uint8_t)q4o_code(raw + (j * nsb + i / Q4_QK) * Q4_BLOCK, (int)(i % Q4_QK));
    for (int64_t t = 0; t < n; ++t)
      for (int64_t c = 0; c < nc; ++c) {
        int64_t acc = 0;
        for (int i = 0; i < 32; ++i) acc += (int64_t)xq[t * k + c * 32 + i] * (int64_t)q[c * 32 + i];
        dots[(t * m + j) * nc + c] = (int32_t)acc;
      }
  }
  free(q);
}
void q4o_chunkdots(const int8_t* xq, const uint8_t* raw, int64_t n, int64_t m, int64_t k,
                   int32_t* dots, int threads) {
  struct q4o_dots_args a = {xq, raw, n, m, k, dots};
  q6o_parallel_rows(q4o_chunkdots_rows, &a, m, threads);
}

/* Per-chunk activation sums S[n][k/32] = sum of the chunk's 32 int8 codes. */
void q4o_chunksums(const int8_t* xq, int64_t n, int64_t k, int32_t* sums) {
  int64_t nc = k / 32;
  for (int64_t t = 0; t < n; ++t)
    for (int64_t c = 0; c < nc; ++c) {
      int32_t s = 0;
      for (int i = 0; i < 32; ++i) s += xq[t * k + c * 32 + i];
      sums[t * nc + c] = s;
    }
}

/* Reference output: y[n][m] = sum over chunks c of da*(d*sc)*D - da*(dmin*m)*S in f64, and
 * t[n][m] = the sum of the magnitudes of those two terms over all chunks (tolerance scale).
 * t may be NULL. */
struct q4o_gemm_args {
  const int8_t* xq;
  const float* da;
  int64_t n;
  const uint8_t* raw;
  int64_t m, k;
  double *y, *t;
};
static void q4o_gemm_rows(void* p, int64_t j0, int64_t j1) {
  const struct q4o_gemm_args* g = (const struct q4o_gemm_args*)p;
  const int8_t* xq = g->xq;
  const float* da = g->da;
  const uint8_t* raw = g->raw;
  int64_t n = g->n, m = g->m, k = g->k;
  double *y = g->y, *t = g->t;
  int64_t nc = k / 32, nsb = k / Q4_QK;
  uint8_t* q = (uint8_t*)malloc((size_t)k);
  double* dsc = (double*)malloc(sizeof(double) * (size_t)nc);
  double* dmm = (double*)malloc(sizeof(double) * (size_t)nc);
  for (int64_t j = j0; j < j1; ++j) {
    for (int64_t c = 0; c < nc; ++c) {
      const uint8_t* blk = raw + (j * nsb + c / 8) * Q4_BLOCK;
      int a, mm;
      q4o_scale_min(blk + Q4_OFF_SCALES, (int)(c % 8), &a, &mm);
      dsc[c] = q6o_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8))) * a;
      dmm[c] = q6o_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8))) * mm;
    }
    for (int64_t i = 0; i < k; ++i) q[i] = (uint8_t)q4o_code(raw + (j * nsb + i / Q4_QK) * Q4_BLOCK, (int)(i % Q4_QK));
    for (int64_t tt = 0; tt < n; ++tt) {
      double sum = 0.0, mag = 0.0;
      for (int64_t c = 0; c < nc; ++c) {
        int64_t dd = 0, ss = 0;
        for (int i = 0; i < 32; ++i) {
          dd += (int64_t)xq[tt * k + c * 32 + i] * (int64_t)q[c * 32 + i];
          ss += xq[tt * k + c * 32 + i];
        }
        double a = (double)da[tt * nc + c];
        double t1 = a * dsc[c] * (double)dd;
        double t2 = -a * dmm[c] * (double)ss;
        sum += t1 + t2;
        mag += fabs(t1) + fabs(t2);
      }
      y[tt * m + j] = sum;
      if (t) t[tt * m + j] = mag;
    }
  }
  free(q);
  free(dsc);
  free(dmm);
}
void q4o_gemm(const int8_t* xq, const float* da, int64_t n, const uint8_t* raw, int64_t m,
              int64_t k, double* y, double* t, int threads) {
  struct q4o_gemm_args g = {xq, da, n, raw, m, k, y, t};
  q6o_parallel_rows(q4o_gemm_rows, &g, m, threads);
}

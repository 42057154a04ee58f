/*
 * q4k.h -- C ABI of the q4_K variant in libq6k.so: the q4_K x int8 prefill GEMM on MI355X
 *
 *     Y[N x M] = X[N x K] . dequant(W_q4K[M x K])^T
 *
 * Pages (titles of the optimisation log this follows):
 *   "r18: Load-time B pre-expansion — staging becomes a bulk copy (W_exp's debut, REVERTED)"
 *       sec. 1    a q4_K super-block: 256 weights in 144 bytes, a 16-byte header (f16 d at 0,
 *                 f16 dmin at 2, twelve bytes of 6-bit scale/min pairs at 4) and 128 bytes of
 *                 4-bit codes; eight sub-blocks of 32
 *       sec. 2    the load-time EB plane (codes as one byte each, 0..15) and SB plane (the pair
 *                 d*sc, -dmin*m per 32-element chunk and row)
 *   "r38 — q6_K BT-style raw-byte mma kernel (LANDED)", sec. 2.2: q4_K's rescale has two terms
 *       and needs the activations' per-chunk sum next to their scale
 * The bit packing the pages do not print is the GGUF K-quant one: for sub-block j < 4,
 * sc = s[j] & 63, m = s[j+4] & 63; for j >= 4, sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
 * m = (s[j+4] >> 4) | (s[j] >> 6) << 4 (s = the 12 scale bytes); code byte 16 + 32g + l holds
 * element 64g + l in its low nibble and 64g + 32 + l in its high nibble; w = d*sc*q - dmin*m.
 *
 * Conventions, status codes and the tiled activation layout (xq, da) are those of q6k.h: the
 * activations are quantized by q4k_quantize_act, which also writes das = da * S per (token,
 * chunk), S the sum of the chunk's 32 codes, in the tiled order of da; or by q6k_quantize_act (or
 * q6k_swiglu_quantize_act) followed by q4k_act_sums, which adds das to existing xq and da.  Every pointer is a device pointer owned by the caller; calls are
 * asynchronous on `stream`; arguments are checked on the host and nothing is launched on error.
 *
 * Prepared weights (q4k_expand_weights), rows padded to MP = m rounded up to 128:
 *   codes : byte ((R*nchunk + c)*64 + l)*16 + b holds the code (0..15) of row 32R + p at
 *           k = 32c + 16*(b/8) + 8g + b%8 (l = p + 32g: the lane order of xq)
 *   pairs : at byte offset MP*k, float2 ((R*(k/256) + s)*8 + cc)*32 + p = (d*sc, -dmin*m) of row
 *           32R + p, chunk 8s + cc
 * 1.25 bytes per weight; padding rows hold zeros.
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#include "q6k.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of the prepared weights of an m x k q4_K matrix; 0 if invalid. */
size_t q4k_weight_bytes(int64_t m, int64_t k);

/* Load-time preparation.  Input: raw q4_K blocks, row j's super-block b at byte (j*(k/256)+b)*144,
 * 16-byte aligned.  Output: the codes and pairs above, w_out_bytes >= q4k_weight_bytes(m, k). */
q6k_status q4k_expand_weights(const void* w_raw, int64_t m, int64_t k, void* w_out,
                              size_t w_out_bytes, void* stream);

/* The q4_K prepass in one pass over x: q6k_quantize_act's xq and da (same arguments and rules)
 * and das = da * S, S the sum of each (token, chunk)'s 32 codes, with the size and order of da;
 * das 16-byte aligned, das_bytes >= da's size (Q6K_ESIZE otherwise).  The per-chunk sum travels
 * with the scale as in "r38 — q6_K BT-style raw-byte mma kernel (LANDED)", sec. 2.2 (q4_K's
 * rescale needs it).  xq, da and das equal those of q6k_quantize_act followed by q4k_act_sums,
 * bit for bit. */
q6k_status q4k_quantize_act(const float* x, int64_t n, int64_t k, int64_t ldx, void* xq,
                            size_t xq_bytes, float* da, size_t da_bytes, float* das,
                            size_t das_bytes, void* stream);

/* das = da * S for the tiled activations of q6k_quantize_act (same n, k); das has the size and
 * order of da (q6k_act_bytes). */
q6k_status q4k_act_sums(const void* xq, const float* da, int64_t n, int64_t k, float* das,
                        size_t das_bytes, void* stream);

/* The GEMM: y[t][j] = sum over chunks c of da*(d*sc)*D - (dmin*m)*das, D the exact int32 dot of
 * the int8 activations with the 4-bit codes over the chunk.  y f32 [n][ldy], ldy >= m, 4-byte
 * aligned, y_bytes >= 4*((n-1)*ldy + m); xq, da, das, w 16-byte aligned and at least the sizes
 * above (Q6K_ESIZE otherwise); k < 2^26.  The work split, the workspace and its rules are
 * q6k_gemm's (output tiles of a partial last round are split along k, their pieces stored into
 * workspace slabs and added in piece order by a second kernel on the same stream), so y is the
 * same bit for bit from run to run. */
q6k_status q4k_gemm(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                    const float* das, size_t das_bytes, int64_t n, const void* w, size_t w_bytes,
                    int64_t m, int64_t k, float* y, size_t y_bytes, int64_t ldy, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes that q4k_gemm needs for this n, m, k on the current device (3 workgroup slots
 * per compute unit: at most 24 MiB on a 256-CU device); 0 when no tile is split or the problem
 * is empty.  Errors as q6k_gemm_workspace. */
q6k_status q4k_gemm_workspace(int64_t n, int64_t m, int64_t k, size_t* bytes);

/* Test-only export of the same kernel source, with the grid and work split of q4k_gemm: the int32
 * chunk dots D of tokens [tok0, tok0 + ntok) x rows [row0, row0 + nrow) to dots
 * int32 [ntok][nrow][k/32] (window and size rules of q6k_gemm_subdots). */
q6k_status q4k_gemm_dots(const void* xq, size_t xq_bytes, int64_t n, const void* w,
                         size_t w_bytes, int64_t m, int64_t k, int64_t tok0, int64_t ntok,
                         int64_t row0, int64_t nrow, int32_t* dots, size_t dots_bytes,
                         void* stream);

/* Liveness counter: q4k_gemm and q4k_gemm_dots launches since load. */
uint64_t q4k_launches(void);

#ifdef __cplusplus
}
#endif
#endif /* Q4K_H */

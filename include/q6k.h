/*
 * q6k.h -- C ABI of libq6k.so: the q6_K x int8 prefill GEMM on MI355X (gfx950)
 *
 *     Y[N x M] = X[N x K] . dequant(W_q6K[M x K])^T
 *
 * Method (page titles of the optimisation log it follows):
 *   "r38 — q6_K BT-style raw-byte mma kernel (LANDED)"
 *       sec. 2.1  q6_K super-block: 256 weights in 210 B -- ql[128] low nibbles at 0, qh[64] 2-bit
 *                 high fields at 128, int8 scales[16] at 192 (one per 16 weights), f16 d at 208;
 *                 w = d * sc[sub-block] * (q - 32)
 *       sec. 2.2  rescale without a dmin term: acc += da * dsc, dsc = d * sc
 *       sec. 2.3  expanded B: weights staged as centered int8 (-32..31)
 *       sec. 2.4  KSPLIT=2: every 32-k chunk is two 16-k halves with their own integer dot and
 *                 their own d*sc rescale, applied as two independent f32 additions
 *   "r41 — q6_K B-expand widened to uint4 group loads (LANDED)": B expanded from wide loads
 *   "r53 — q6_K bundle: W_exp pre-expansion plane + cp.async B staging (LANDED)": optional load-time plane of
 *       centered int8 weights (extra memory, no expand work in the GEMM)
 *   "r42 — q6_K stage-wide dsc scale reads (REVERTED)", sec. 3.2 (W_dsc arm): d*sc precomputed as f32
 * Layout 2 applies the same weights (w = d * sc * (q - 32), "r38 ..." sec. 2.1) with the int8 sc
 * folded into the integer dot, so each 32-k chunk carries one f32 rescale da * d instead of two.
 *
 * Conventions for every entry point
 *   - Every buffer pointer is a DEVICE pointer owned by the caller; the library never allocates,
 *     frees or retains memory (apart from q6k_gemm_noalloc's static scratch array, which is
 *     part of the loaded code object).  `stream` is a hipStream_t (NULL = the null stream).
 *   - Calls are asynchronous on `stream` and never synchronize.  Arguments are checked on the
 *     host before anything is launched; on any error nothing is launched and the output buffers
 *     are untouched.  A fault inside a kernel surfaces at the caller's next synchronization.
 *   - There is no fallback path: an unsupported request returns an error code.
 *   - n == 0 or m == 0 is an empty problem: the call returns Q6K_OK and launches nothing.
 *   - k must be a positive multiple of 256 (whole super-blocks).
 *   - Buffers read with 16-byte accesses (x, xq, da, w) must be 16-byte aligned; y and dots
 *     need 4-byte alignment; raw q6_K weights need 2-byte alignment (a 210-byte block is only
 *     2-byte aligned, so a row of blocks cannot promise more).
 *   - The tiled activations, the prepared weights and every output buffer come with their size
 *     in bytes, checked against what the call reads or writes (Q6K_ESIZE if too small); a caller
 *     that passes a size larger than the allocation defeats the check.  Row-major inputs (x,
 *     gate, up, raw weights) are sized by n, k and their leading dimension alone.
 *
 * Tiled layouts (produced and consumed only by this library; the byte order is documented so
 * callers and tests can rebuild the plain [row][k] views):
 *   token tiles  : NP = n rounded up to 128; tile T holds tokens 32T .. 32T+31
 *   row tiles    : MP = m rounded up to 128; tile R holds weight rows 32R .. 32R+31
 *   chunk c      : k range 32c .. 32c+31, nchunk = k/32; half h = 0 (k 0..15) / 1 (k 16..31)
 *   lane l       : 0..63, position p = l % 32, group g = l / 32
 *   xq  (int8)   : byte ((T*nchunk + c)*64 + l)*16 + b  holds  Xq[32T + p][32c + 16*(b/8) + 8g + b%8]
 *   da  (f32)    : float (T*nchunk + c)*32 + 16g + 4q + r  holds  da[32T + 8q + 4g + r][c]
 *   layout 1 (Q6K_LAYOUT_EXPANDED):
 *     codes int8 : byte ((R*nchunk + c)*64 + l)*16 + b  holds  q - 32 of row 32R + p at
 *                  k = 32c + 16*(b/8) + 8g + b%8
 *     scales f32 : at byte offset MP*k, float ((R*nchunk + c)*32 + p)*2 + h = d*sc[2c + h] of row
 *                  32R + p (sub-block index counted along the whole row)
 *   layout 0 (Q6K_LAYOUT_PACKED), 6 bits per weight plus layout 1's scale plane:
 *     codes      : 12 bytes at ((R*nchunk + c)*64 + l)*12 for row 32R + p, three little-endian
 *                  words X, Y, Z; with a_e (e = 0..7) the 6-bit codes at k = 32c + 8g + e and
 *                  b_e those at k = 32c + 16 + 8g + e, byte t (t = 0..3) of
 *                    X = a_t << 2     | (b_{t+4} & 3)
 *                    Y = a_{t+4} << 2 | ((b_{t+4} >> 2) & 3)
 *                    Z = b_t << 2     | (b_{t+4} >> 4)
 *                  (the GEMM turns a byte s into (s & 0xFC) ^ 0x80 = 4 * (q - 32))
 *     scales f32 : at byte offset MP*k*3/4, as layout 1's: float ((R*nchunk + c)*32 + p)*2 + h
 *                  = d*sc[2c + h] of row 32R + p
 *   layout 2 (Q6K_LAYOUT_FOLDED), the int8 sub-block scale applied to the codes ahead of time:
 *     v = sc[k/16] * (q - 32) (in [-4064, 4096]) of row 32R + p at k = 32c + 16*(b/8) + 8g + b%8
 *     is stored as two int8 digits, lo = ((v + 32) mod 64) - 32 and hi = (v - lo) / 64:
 *     codes      : byte ((R*nchunk + c)*2 + h)*1024 + l*16 + b  holds lo (h = 0) or hi (h = 1)
 *     scales     : at byte offset MP*k*2, float (R*(k/256) + s)*32 + p = d of row 32R + p,
 *                  super-block s (the f16 d converted exactly)
 *   Padding tokens / rows hold zeros.
 */
#ifndef Q6K_H
#define Q6K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  Q6K_OK = 0,
  Q6K_EINVAL = -1, /* null pointer, negative size, unknown layout, ld too small */
  Q6K_ESHAPE = -2, /* k not a positive multiple of 256 */
  Q6K_EALIGN = -3, /* a pointer or leading dimension breaks the 16-byte alignment rule */
  Q6K_ESIZE = -4,  /* a buffer is smaller than the call reads or writes, or sizes overflow */
  Q6K_EHIP = -5,   /* the HIP runtime rejected a launch */
  Q6K_ESCRATCH = -6 /* q6k_gemm_noalloc: the problem needs more than its static scratch holds */
} q6k_status;

enum { Q6K_LAYOUT_PACKED = 0, Q6K_LAYOUT_EXPANDED = 1, Q6K_LAYOUT_FOLDED = 2 };

/* Sizes in bytes of the tiled activation buffers for n tokens of k values: returns the size
 * of xq and stores the size of da in *da_bytes (may be NULL).  Returns 0 for invalid n/k. */
size_t q6k_act_bytes(int64_t n, int64_t k, size_t* da_bytes);

/* Activation quantize-transpose prepass ("r38 — q6_K BT-style raw-byte mma kernel", sec. 2.2 and
 * 3.2: int8 activations with one scale per token and 32-k chunk, laid out ahead of the GEMM).
 * For every token t < n and chunk c: amax = max |x|, da = amax / 127 (IEEE f32 division),
 * q = roundf(x / da) (IEEE f32 division, half away from zero) clamped to [-127, 127]; an
 * all-zero chunk gives da = 0 and q = 0.
 *   x       : f32 [n][ldx] row-major, ldx >= k, ldx % 4 == 0, 16-byte aligned
 *   xq, da  : tiled outputs (see above) of at least the sizes q6k_act_bytes returns
 * Padding tokens are written as zeros.  Inf/NaN inputs are outside the contract. */
q6k_status q6k_quantize_act(const float* x, int64_t n, int64_t k, int64_t ldx, void* xq,
                            size_t xq_bytes, float* da, size_t da_bytes, void* stream);

/* Fused producer for ffn_down: quantizes h = up * silu(gate), silu(g) = g / (1 + e^-g), exactly as
 * q6k_quantize_act quantizes x, without writing h ("r53 — q6_K bundle: W_exp pre-expansion
 * plane + cp.async B staging (LANDED)", sec. 1: the SwiGLU product's producers fused).  h is
 * formed in f32 with expf (a few ulp); the codes and da are those q6k_quantize_act gives for that
 * f32 h.
 *   gate, up: f32 [n][ld] row-major, ld >= k, ld % 4 == 0, both 16-byte aligned
 *   xq, da  : tiled outputs as for q6k_quantize_act */
q6k_status q6k_swiglu_quantize_act(const float* gate, const float* up, int64_t n, int64_t k,
                                   int64_t ld, void* xq, size_t xq_bytes, float* da,
                                   size_t da_bytes, void* stream);

/* Test-only export of the producer's f32 h = up * silu(gate): h [n][ldh] row-major, ldh >= k;
 * 4-byte aligned pointers; n * k below 2^38. */
q6k_status q6k_swiglu_f32(const float* gate, const float* up, int64_t n, int64_t k, int64_t ld,
                          float* h, int64_t ldh, void* stream);

/* Size in bytes of the weight buffer of an m x k q6_K matrix in `layout`; 0 if invalid. */
size_t q6k_weight_bytes(int64_t m, int64_t k, int layout);

/* Load-time weight preparation.  Input: raw q6_K blocks, row j's super-block b at byte
 * (j*(k/256) + b)*210 (byte map of "r38 ..." sec. 2.1; 2-byte aligned: Q6K_EALIGN otherwise).  Output: layout 0 (6-bit
 * codes regrouped for wide loads plus the f32 d*sc plane; expanded to centered int8 inside the
 * GEMM, "r41 ..." sec. 2), layout 1 (centered int8 plane plus f32 d*sc plane, "r53 ..." sec.
 * 2.3 and the W_dsc plane of "r42 ..." sec. 3.2) or layout 2 (two int8 digit planes of
 * sc * (q - 32) plus one f32 d per super-block).  Padding rows are written as zeros. */
q6k_status q6k_expand_weights(const void* w_raw, int64_t m, int64_t k, int layout, void* w_out,
                              size_t w_out_bytes, void* stream);

/* The GEMM: y[t][j] = sum over 16-k sub-blocks s of da[t][s/2] * (d*sc)[j][s] * D[t][j][s],
 * D the exact int32 dot of the int8 activations with the centered weights over sub-block s
 * ("r38 ..." sec. 2.2, 2.4).  Layouts 0 and 1 accumulate each 32-k chunk as two independent f32
 * additions, one per 16-k half.  Layout 2 forms the chunk's exact integer
 * E = sc[2c]*D[2c] + sc[2c+1]*D[2c+1] and adds da * E once per chunk, then applies d once per
 * super-block; the result differs from layouts 0/1 only in f32 rounding.
 * Work split (every layout): output tiles of 64 tokens x 128 rows are dealt out in rounds of one
 * per workgroup slot of the GPU; when the last round would leave slots idle, its tiles are split
 * along k into pieces of whole super-blocks.  Each piece stores its partial sums into a 32 KiB
 * slab of the workspace, and a second kernel, enqueued right after the GEMM on the same stream,
 * adds each split tile's slabs in piece order into y.  On layout 2, when whole rounds precede
 * the split tiles, their pieces are graded (piece i of P weighs P - i) and handed out in the
 * order the workgroups start, largest first, through a 4-byte claim counter in the workspace
 * after the slabs (the launch sets it to 0 as it starts and the second kernel again after it),
 * so that the workgroups that start last take the smallest pieces.  A piece's k-range and slab
 * depend only on (tile, piece), and the order of every addition is fixed, so y is the same bit
 * for bit from run to run (and in a captured graph's replays).  The workspace is scratch: its
 * contents are not needed before the call and mean nothing after it; two calls in flight at
 * once (on different streams) need workspaces of their own, and two that write the same y
 * concurrently race.
 *   xq, da  : outputs of q6k_quantize_act for the same n, k; xq_bytes, da_bytes at least what
 *             q6k_act_bytes returns (the kernels read whole padded tiles)
 *   w       : output of q6k_expand_weights for the same m, k and `layout`; w_bytes at least
 *             q6k_weight_bytes(m, k, layout)
 *   y       : f32 [n][ldy] row-major, ldy >= m, 4-byte aligned, y_bytes >= 4*((n-1)*ldy + m);
 *             only y[0..n)[0..m) is written
 *   workspace, workspace_bytes : device memory owned by the caller, 16-byte aligned, at least
 *             the bytes q6k_gemm_workspace returns for this n, m, k, layout on the current
 *             device (NULL and 0 when that is 0); Q6K_EINVAL if NULL when needed, Q6K_EALIGN if
 *             misaligned, Q6K_ESIZE if too small
 * Layout 2 also needs k < 2^25, layouts 0 and 1 k < 2^26 (Q6K_ESIZE otherwise). */
q6k_status q6k_gemm(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                    int64_t n, const void* w, size_t w_bytes, int layout, int64_t m, int64_t k,
                    float* y, size_t y_bytes, int64_t ldy, void* workspace,
                    size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): q6k_gemm with its split-k workspace taken
 * from a static device array of the library instead of a caller buffer.  Same arguments (minus
 * the workspace), kernels, work split and results (bit for bit) as q6k_gemm.  The array holds
 * 24 MiB + 256 bytes (768 slabs of 32 KiB: 3 workgroup slots per compute unit on a 256-CU
 * device, the most any layout needs there, and the claim counter); a problem that needs more
 * returns Q6K_ESCRATCH and launches nothing.
 * Each GPU holds its own copy, from the first call on it until the process ends; the call
 * itself allocates and frees nothing.  Every call on one GPU uses that GPU's one array (no part
 * of it needs clearing: a call reads only what it wrote), so calls that overlap on one GPU (on
 * different streams, or from several threads) race; calls on one stream are ordered. */
q6k_status q6k_gemm_noalloc(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                            int64_t n, const void* w, size_t w_bytes, int layout, int64_t m,
                            int64_t k, float* y, size_t y_bytes, int64_t ldy, void* stream);

/* Workspace bytes that q6k_gemm needs for this n, m, k and layout on the device current on the
 * calling thread (the work split depends on its compute-unit count): 32 KiB per piece of a
 * split tile, at most 32 KiB x the workgroup slots of the device (2 per compute unit on layout
 * 2, 3 on layouts 0 and 1: 16 and 24 MiB on a 256-CU device), plus 256 bytes for the claim
 * counter when layout 2 hands its pieces out in start order; 0 when no tile is split or the
 * problem is empty.  Shape errors as q6k_gemm; Q6K_EHIP if the device cannot be queried;
 * *bytes is 0 on any error. */
q6k_status q6k_gemm_workspace(int64_t n, int64_t m, int64_t k, int layout, size_t* bytes);

/* Test-only export of the same kernel source, launched with the same grid and work split as
 * q6k_gemm for this n, m, k and layout: instead of y, stores the int32 sub-block dots D[t][j][s]
 * (the two KSPLIT halves of every chunk) of the window of tokens t in [tok0, tok0 + ntok) and
 * rows j in [row0, row0 + nrow) to dots, int32 [ntok][nrow][k/16] (dots_bytes at least
 * 4 * ntok * nrow * k/16).  The window must lie inside the n x m problem (Q6K_EINVAL otherwise);
 * an empty window launches nothing.  Layouts 0 and 1 only (layout 2 never forms them:
 * Q6K_EINVAL). */
q6k_status q6k_gemm_subdots(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                            int64_t n, const void* w, size_t w_bytes, int layout, int64_t m,
                            int64_t k, int64_t tok0, int64_t ntok, int64_t row0, int64_t nrow,
                            int32_t* dots, size_t dots_bytes, void* stream);

/* Test-only export of the layout-2 kernel, with the window rules of q6k_gemm_subdots: stores the
 * per-chunk integer numerators E[t][j][c] = sc[j][2c]*D[t][j][2c] + sc[j][2c+1]*D[t][j][2c+1]
 * (|E| < 2^24), as the kernel reconstructs them from its two digit products, to dots
 * int32 [ntok][nrow][k/32].  Layout 2 only (Q6K_EINVAL otherwise). */
q6k_status q6k_gemm_chunkdots(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                              int64_t n, const void* w, size_t w_bytes, int layout, int64_t m,
                              int64_t k, int64_t tok0, int64_t ntok, int64_t row0, int64_t nrow,
                              int32_t* dots, size_t dots_bytes, void* stream);

/* Human-readable text of a status code (static storage). */
const char* q6k_strerror(int status);

/* Liveness counters: number of GEMM launches (q6k_gemm and the test exports) per layout since
 * load; out[L] = layout L for L = 0, 1, 2.  Fast-path liveness check in the spirit of
 * "r53 ..." sec. 3.3 (a path that silently never runs is invisible to parity tests). */
void q6k_stats(uint64_t out[3]);

#ifdef __cplusplus
}
#endif
#endif /* Q6K_H */

/*
 * q6k_ceilings.h -- C ABI of libq6k_ceilings.so: microbenchmarks of the gfx950 units that bound
 * the q6_K x int8 prefill GEMM (measurement code beside the product library; nothing in
 * libq6k.so depends on it).
 *
 * The GEMM of "r38 — q6_K BT-style raw-byte mma kernel (LANDED)" spends, per output and 32-k
 * chunk, one int8 matrix product over the chunk (sec. 2.4: two 16-k halves) and an f32 rescale per
 * half (sec. 2.2).  These probes measure the rates the GEMM is priced against: the int8 MFMA forms
 * (K = 16, 32, 64) and an f16 one, vector-ALU instruction issue at a chosen number of waves per
 * SIMD, the GEMMs' per-tile operation without memory traffic, and HBM streaming.
 *
 * Conventions are those of q6k.h (status codes, device pointers, asynchronous on `stream`).
 * Probe output: for each of the q6c_probe_waves(W) waves, four uint64 -- shader-clock cycles
 * between the wave's first and last instruction (s_memtime), wall-clock ticks over the same span
 * (s_memrealtime, q6c_wall_clock_khz() per millisecond), the wave's hardware id register, and a
 * value that depends on every result.  out_bytes must hold 32 bytes per wave.
 * W (waves per SIMD) is 1..8: each workgroup (4 waves, one per SIMD) reserves 160 KiB / W of LDS,
 * so a CU holds at most W of them, and the grid has W workgroups per CU.
 */
#ifndef Q6K_CEILINGS_H
#define Q6K_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#include "q6k.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  Q6C_MFMA_I8_32x32x16 = 0,  /* v_mfma_i32_32x32x16_i8: 32768 int8 ops per wave instruction */
  Q6C_MFMA_I8_32x32x32 = 1,  /* v_mfma_i32_32x32x32_i8: 65536 */
  Q6C_MFMA_I8_16x16x64 = 2,  /* v_mfma_i32_16x16x64_i8: 32768 */
  Q6C_MFMA_F16_32x32x16 = 3  /* v_mfma_f32_32x32x16_f16: 32768 flops */
};
enum {
  Q6C_VALU_FMA_F32 = 0,      /* v_fma_f32 d, a, b, c (three register operands) */
  Q6C_VALU_FMAC_F32 = 1,     /* v_fmac_f32 d, a, b (two-operand encoding) */
  Q6C_VALU_ADD_F32 = 2,
  Q6C_VALU_MUL_F32 = 3,
  Q6C_VALU_CVT_F32_I32 = 4,
  Q6C_VALU_ADD_U32 = 5
};
enum {
  Q6C_TILEOP_FOLDED = 0,     /* per tile and chunk: 2 x 32x32x32 int8 MFMA + 48 VALU (fold, rescale) */
  Q6C_TILEOP_HALVES = 1,     /* per tile and chunk: 2 x 32x32x16 int8 MFMA + 64 VALU (two halves) */
  Q6C_TILEOP_FOLDED_PIPE = 2, /* FOLDED with each tile's MFMAs issued half a step ahead of its fold */
  Q6C_TILEOP_ZERO_C = 3,      /* FOLDED's instruction mix, MFMA accumulator input an inline zero */
  Q6C_TILEOP_F16 = 4          /* per tile and chunk: 4 x 32x32x16 f16 MFMA on the digit planes as
                                 f16 integers, chained from zero (E exact in f32) + 16 VALU (da) */
};
enum { Q6C_STREAM_READ = 0, Q6C_STREAM_COPY = 1, Q6C_STREAM_READ_NT = 2 };
enum {
  Q6C_OVERLAP_ROLES = 0,     /* 12 waves per CU: waves 0-3 MFMA only, waves 4-11 VALU only */
  Q6C_OVERLAP_SAME_WAVE = 1  /* 4 waves per CU: each alternates 1 MFMA and 8 independent VALU */
};

/* Waves one probe launch runs with W waves per SIMD (-1 without a device). */
int q6c_probe_waves(int waves_per_simd);

/* Rate of the wall clock that s_memrealtime counts, in kHz (-1 without a device). */
int q6c_wall_clock_khz(void);

/* `iters` rounds of 4 independent MFMAs of `kind` per wave. */
int q6c_mfma(int kind, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
             void* stream);

/* `iters` rounds of 64 VALU instructions of `kind` per wave (8 independent chains of 8). */
int q6c_valu(int kind, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
             void* stream);

/* `iters` rounds of the tile operation of `kind` on two 32x32 output tiles per wave. */
int q6c_tileop(int kind, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
               void* stream);

/* Whether MFMA execution and VALU issue overlap on one SIMD (one workgroup per CU; the output
 * holds 4 uint64 per wave as above, 12 waves per CU for ROLES and 4 for SAME_WAVE): ROLES runs
 * iters_mfma rounds of 4 v_mfma_i32_32x32x32_i8 on waves 0-3 and iters_valu rounds of 64
 * v_add_f32 on waves 4-11 (two per SIMD); SAME_WAVE runs iters_mfma rounds of
 * 4 x (1 MFMA + 8 v_add_f32). */
int q6c_overlap(int kind, int iters_mfma, int iters_valu, uint64_t* out, size_t out_bytes,
                void* stream);

/* HBM stream over `bytes` (multiple of 16, 16-byte aligned): READ xors src into one word per
 * thread of 8 workgroups per CU (dst_bytes >= 4 * 256 * 8 * CUs), READ_NT does the same with
 * nontemporal loads (the prepass reads its input so), COPY copies src to dst. */
int q6c_stream(int mode, const void* src, void* dst, size_t bytes, size_t dst_bytes,
               void* stream);

#ifdef __cplusplus
}
#endif
#endif /* Q6K_CEILINGS_H */

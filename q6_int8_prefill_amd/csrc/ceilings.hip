// ceilings.hip -- microbenchmarks of the gfx950 units the q6_K x int8 GEMM leans on, built into
// libq6k_ceilings.so (C ABI in include/q6k_ceilings.h) and run by `bench.py --ceilings`.  They
// measure what the hardware sustains, so that the GEMM's roofline figures can be set against
// measured ceilings rather than assumed ones:
//   - matrix cores: back-to-back independent MFMAs of one kind (the int8 forms with K = 16, 32 and
//     64, and the f16 form of the same output shape for comparison);
//   - vector ALU: chains of independent f32 / integer instructions with register operands, at a
//     chosen number of waves per SIMD (is an instruction issued every 4 cycles, or faster when
//     several waves have work?);
//   - the GEMMs' tile operation without memory traffic: per 32x32 output tile and 32-k chunk, the
//     folded layout's two K=32 MFMAs and 48 VALU instructions, or the two-halves layouts' two
//     K=16 MFMAs and 64 VALU instructions;
//   - HBM: a streaming read and a streaming copy with 16-byte accesses.
// Every probe wave records its shader-clock cycles (s_memtime) and constant-rate wall ticks
// (s_memrealtime) between its first and last instruction, so the host gets cycles per
// instruction and the clock the chip actually ran at during the probe.
//
// Occupancy: a workgroup is 4 waves (one per SIMD of a CU) and asks for 160 KiB / W of LDS, so at
// most W workgroups share a CU; with 256 * W workgroups on a 256-CU device every SIMD runs W
// waves.  The MFMA and tile probes are built for at most 256 registers per wave, as the GEMM
// kernels are, so their MFMA results land in ordinary vector registers as in the kernels (with
// more registers allowed, the compiler puts them in accumulation registers and adds a copy per
// result).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q6k_ceilings.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kLdsPerCu = 160 * 1024;

struct WaveTimes {
  uint64_t c0, w0;
};

__device__ __forceinline__ WaveTimes start_times() {
  WaveTimes t;
  t.c0 = __builtin_amdgcn_s_memtime();
  t.w0 = __builtin_amdgcn_s_memrealtime();
  return t;
}

// out[4 * wave_id + 0..3] = cycles, wall ticks, hardware id (XCC/SE/CU/SIMD bits), a value that
// depends on every result (so that no computation can be dropped)
__device__ __forceinline__ void finish(const WaveTimes& t, uint64_t* out, uint32_t sink) {
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
  const int lane = threadIdx.x & 63;
  const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const uint32_t hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));  // HW_ID, all 32 bits
  uint32_t x = sink;
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) {
    out[4 * wave + 0] = c1 - t.c0;
    out[4 * wave + 1] = w1 - t.w0;
    out[4 * wave + 2] = hw;
    out[4 * wave + 3] = x;
  }
}

// ---------------------------------------------------------------------------------------------
// MFMA issue rate: 4 independent accumulators per wave, `iters` rounds of 4 MFMAs.
// ---------------------------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_kernel(int iters, uint64_t* out) {
  extern __shared__ uint8_t lds_reserve[];  // occupancy control only
  const WaveTimes t = start_times();
  const int lane = threadIdx.x & 63;
  uint32_t sink = 0;
  if (KIND == Q6C_MFMA_I8_32x32x16 || KIND == Q6C_MFMA_I8_32x32x32 || KIND == Q6C_MFMA_I8_16x16x64) {
    v4i a = {lane, lane * 3, lane ^ 5, 7}, b = {lane + 1, 2, lane * 5, lane};
    if (KIND == Q6C_MFMA_I8_16x16x64) {
      v4i c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
      for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c3, 0, 0, 0);
      }
      for (int r = 0; r < 4; ++r) sink ^= c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    } else {
      v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int i = 0; i < iters; ++i) {
        if (KIND == Q6C_MFMA_I8_32x32x16) {
          const long al = ((long)a.y << 32) | (unsigned)a.x, bl = ((long)b.y << 32) | (unsigned)b.x;
          c0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(al, bl, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(al, bl, c1, 0, 0, 0);
          c2 = __builtin_amdgcn_mfma_i32_32x32x16_i8(al, bl, c2, 0, 0, 0);
          c3 = __builtin_amdgcn_mfma_i32_32x32x16_i8(al, bl, c3, 0, 0, 0);
        } else {
          c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
          c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
          c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
        }
      }
      for (int r = 0; r < 16; ++r) sink ^= c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    }
  } else {
    v8h a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(lane * 0.01f + i);
      b[i] = (_Float16)(i * 0.5f - lane * 0.001f);
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    for (int r = 0; r < 16; ++r) sink ^= __float_as_uint(c0[r] + c1[r] + c2[r] + c3[r]);
  }
  finish(t, out, sink);
}

// ---------------------------------------------------------------------------------------------
// VALU issue rate: 8 independent chains per lane, 8 instructions per chain per round (64 per
// round), every operand a register.  The instruction forms are written out so the compiler cannot
// change them.
// ---------------------------------------------------------------------------------------------
#define Q6C_CHAINS(OP)                                                                             \
  asm volatile(OP OP OP OP OP OP OP OP                                                             \
               : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7) \
               : "v"(s1), "v"(s2))

template <int KIND>
__global__ __launch_bounds__(256) void valu_kernel(int iters, uint64_t* out) {
  extern __shared__ uint8_t lds_reserve[];
  const WaveTimes t = start_times();
  const int lane = threadIdx.x & 63;
  float r0 = lane, r1 = lane + 1, r2 = lane + 2, r3 = lane + 3, r4 = lane + 4, r5 = lane + 5,
        r6 = lane + 6, r7 = lane + 7;
  float s1 = 1.0000001f, s2 = -0.5f;
  for (int i = 0; i < iters; ++i) {
    if (KIND == Q6C_VALU_FMA_F32) {
      Q6C_CHAINS(
          "v_fma_f32 %0, %0, %8, %9\n\tv_fma_f32 %1, %1, %8, %9\n\tv_fma_f32 %2, %2, %8, %9\n\t"
          "v_fma_f32 %3, %3, %8, %9\n\tv_fma_f32 %4, %4, %8, %9\n\tv_fma_f32 %5, %5, %8, %9\n\t"
          "v_fma_f32 %6, %6, %8, %9\n\tv_fma_f32 %7, %7, %8, %9\n\t");
    } else if (KIND == Q6C_VALU_FMAC_F32) {
      Q6C_CHAINS(
          "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %2, %8, %9\n\t"
          "v_fmac_f32 %3, %8, %9\n\tv_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\t"
          "v_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9\n\t");
    } else if (KIND == Q6C_VALU_ADD_F32) {
      Q6C_CHAINS(
          "v_add_f32 %0, %0, %9\n\tv_add_f32 %1, %1, %9\n\tv_add_f32 %2, %2, %9\n\t"
          "v_add_f32 %3, %3, %9\n\tv_add_f32 %4, %4, %9\n\tv_add_f32 %5, %5, %9\n\t"
          "v_add_f32 %6, %6, %9\n\tv_add_f32 %7, %7, %9\n\t");
    } else if (KIND == Q6C_VALU_MUL_F32) {
      Q6C_CHAINS(
          "v_mul_f32 %0, %0, %8\n\tv_mul_f32 %1, %1, %8\n\tv_mul_f32 %2, %2, %8\n\t"
          "v_mul_f32 %3, %3, %8\n\tv_mul_f32 %4, %4, %8\n\tv_mul_f32 %5, %5, %8\n\t"
          "v_mul_f32 %6, %6, %8\n\tv_mul_f32 %7, %7, %8\n\t");
    } else if (KIND == Q6C_VALU_CVT_F32_I32) {
      Q6C_CHAINS(
          "v_cvt_f32_i32 %0, %0\n\tv_cvt_f32_i32 %1, %1\n\tv_cvt_f32_i32 %2, %2\n\t"
          "v_cvt_f32_i32 %3, %3\n\tv_cvt_f32_i32 %4, %4\n\tv_cvt_f32_i32 %5, %5\n\t"
          "v_cvt_f32_i32 %6, %6\n\tv_cvt_f32_i32 %7, %7\n\t");
    } else {  // Q6C_VALU_ADD_U32
      Q6C_CHAINS(
          "v_add_u32 %0, %0, %9\n\tv_add_u32 %1, %1, %9\n\tv_add_u32 %2, %2, %9\n\t"
          "v_add_u32 %3, %3, %9\n\tv_add_u32 %4, %4, %9\n\tv_add_u32 %5, %5, %9\n\t"
          "v_add_u32 %6, %6, %9\n\tv_add_u32 %7, %7, %9\n\t");
    }
  }
  const float v = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7;
  finish(t, out, __float_as_uint(v));
}
#undef Q6C_CHAINS

// ---------------------------------------------------------------------------------------------
// The GEMMs' tile operation with no memory traffic: two 32x32 output tiles per wave (as in the
// kernels), per round and tile the MFMAs of one 32-k chunk and the rescale of its 16 outputs per
// lane, in the kernels' forms.
// ---------------------------------------------------------------------------------------------
constexpr int kBiasI = 0x4B400000;      // 1.5 * 2^23
constexpr int kBiasHiI = 0x4E400000;    // 1.5 * 2^29
constexpr float kBiasF = 12582912.0f;

template <int KIND>
__global__ __launch_bounds__(256, 2) void tileop_kernel(int iters, uint64_t* out) {
  extern __shared__ uint8_t lds_reserve[];
  const WaveTimes t = start_times();
  const int lane = threadIdx.x & 63;
  v4i a = {lane, lane * 3, lane ^ 5, 7}, b0 = {lane + 1, 2, lane * 5, lane}, b1 = b0 ^ 0x01010101;
  float acc[2][16], sb[2][16];
  for (int u = 0; u < 2; ++u)
    for (int r = 0; r < 16; ++r) acc[u][r] = sb[u][r] = 0.0f;
  float da0 = 1.0f + lane * 1e-3f, da1 = 0.5f + lane * 1e-3f;
  if (KIND == Q6C_TILEOP_FOLDED_PIPE) {
    // the folded tile operation with each tile's MFMAs issued one half-step ahead of its fold:
    // while the wave folds one tile, the matrix core works on the other tile's products
    v16i bias_lo, bias_hi;
    for (int r = 0; r < 16; ++r) {
      bias_lo[r] = kBiasI;
      bias_hi[r] = kBiasHiI;
    }
    float kk = -65.0f * kBiasF;
    asm("" : "+v"(kk));
    v16i fh0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, bias_hi, 0, 0, 0);
    v16i fl0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1, b0, bias_lo, 0, 0, 0);
    for (int i = 0; i < iters; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      v16i fh1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, bias_hi, 0, 0, 0);
      v16i fl1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1, b1, bias_lo, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __int_as_float(fh0[r]) + kk;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] += __int_as_float(fl0[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[0][r] = __builtin_fmaf(e[r], da0, sb[0][r]);
      }
      __builtin_amdgcn_sched_barrier(0);
      fh0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, bias_hi, 0, 0, 0);
      fl0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1, b0, bias_lo, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __int_as_float(fh1[r]) + kk;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] += __int_as_float(fl1[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[1][r] = __builtin_fmaf(e[r], da1, sb[1][r]);
      }
      asm volatile("" : "+v"(da0), "+v"(da1));
    }
    for (int r = 0; r < 16; ++r) sb[0][r] += __int_as_float(fh0[r] ^ fl0[r]);
  } else if (KIND == Q6C_TILEOP_ZERO_C) {
    // the folded tile operation's instruction mix with the MFMAs' accumulator input an inline
    // zero instead of bias registers (results not meaningful: probes the cost of reading C)
    float kk = -65.0f * kBiasF;
    asm("" : "+v"(kk));
    const v16i zero = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4i x = u ? b1 : b0;
        v16i fh = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, x, zero, 0, 0, 0);
        v16i fl = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1, x, zero, 0, 0, 0);
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __int_as_float(fh[r]) + kk;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] += __int_as_float(fl[r]);
        const float dav = u ? da1 : da0;
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[u][r] = __builtin_fmaf(e[r], dav, sb[u][r]);
      }
      asm volatile("" : "+v"(da0), "+v"(da1));
    }
  } else if (KIND == Q6C_TILEOP_F16) {
    // the folded operation on f16 MFMAs: the activation codes and the two digit planes (lo and
    // 64*hi) as f16 integers, two K=16 halves each, four v_mfma_f32_32x32x16_f16 per tile and
    // chunk chained from an inline zero (every partial sum an integer below 2^24, so E is exact
    // in f32 with no fold), then one fma with da per output
    v8h fa0, fa1, fl, fh;
    for (int i = 0; i < 8; ++i) {
      fa0[i] = (_Float16)(float)((lane * 7 + i * 13) % 255 - 127);
      fa1[i] = (_Float16)(float)((lane * 11 + i * 5) % 255 - 127);
      fl[i] = (_Float16)(float)((lane * 3 + i * 17) % 64 - 32);
      fh[i] = (_Float16)(float)(64 * ((lane * 5 + i * 3) % 33 - 16));
    }
    const v16f zero = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v8h bl = u ? fh : fl, bh = u ? fl : fh;
        v16f e = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa0, bl, zero, 0, 0, 0);
        e = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa1, bl, e, 0, 0, 0);
        e = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa0, bh, e, 0, 0, 0);
        e = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa1, bh, e, 0, 0, 0);
        const float dav = u ? da1 : da0;
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[u][r] = __builtin_fmaf(e[r], dav, sb[u][r]);
      }
      asm volatile("" : "+v"(da0), "+v"(da1));
    }
  } else if (KIND == Q6C_TILEOP_FOLDED) {
    v16i bias_lo, bias_hi;
    for (int r = 0; r < 16; ++r) {
      bias_lo[r] = kBiasI;
      bias_hi[r] = kBiasHiI;
    }
    float kk = -65.0f * kBiasF;
    asm("" : "+v"(kk));
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4i x = u ? b1 : b0;
        v16i fh = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, x, bias_hi, 0, 0, 0);
        v16i fl = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1, x, bias_lo, 0, 0, 0);
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __int_as_float(fh[r]) + kk;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] += __int_as_float(fl[r]);
        const float dav = u ? da1 : da0;
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[u][r] = __builtin_fmaf(e[r], dav, sb[u][r]);
      }
      asm volatile("" : "+v"(da0), "+v"(da1));  // keep the rounds apart
    }
  } else {
    v16i bias;
    for (int r = 0; r < 16; ++r) bias[r] = kBiasI;
    float s0 = 0.25f + lane * 1e-4f, s1 = 0.125f - lane * 1e-4f;
    const float nb0 = -kBiasF * s0, nb1 = -kBiasF * s1;
    float dav[16];
    for (int r = 0; r < 16; ++r) dav[r] = 1.0f + (lane + r) * 1e-3f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4i x = u ? b1 : b0;
        const long alo = ((long)a.y << 32) | (unsigned)a.x, ahi = ((long)a.w << 32) | (unsigned)a.z;
        const long blo = ((long)x.y << 32) | (unsigned)x.x, bhi = ((long)x.w << 32) | (unsigned)x.z;
        const v16i lo_d = __builtin_amdgcn_mfma_i32_32x32x16_i8(alo, blo, bias, 0, 0, 0);
        const v16i hi_d = __builtin_amdgcn_mfma_i32_32x32x16_i8(ahi, bhi, bias, 0, 0, 0);
        float tt[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tt[r] = __builtin_fmaf(__int_as_float(lo_d[r]), s0, nb0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = __builtin_fmaf(tt[r], dav[r], acc[u][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) tt[r] = __builtin_fmaf(__int_as_float(hi_d[r]), s1, nb1);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = __builtin_fmaf(tt[r], dav[r], acc[u][r]);
      }
      asm volatile("" : "+v"(s0), "+v"(s1));
    }
  }
  float v = 0.0f;
  for (int u = 0; u < 2; ++u)
    for (int r = 0; r < 16; ++r) v += acc[u][r] + sb[u][r];
  finish(t, out, __float_as_uint(v));
}

// ---------------------------------------------------------------------------------------------
// Can the vector ALU issue while the matrix core of the same SIMD runs an MFMA?
//   ROLES: a workgroup of 12 waves on one CU (waves w, w + 4 and w + 8 share SIMD w % 4);
//          waves 0-3 run only MFMAs (v_mfma_i32_32x32x32_i8, 4 independent accumulators), waves
//          4-11 only VALU (64 v_add_f32 per round, 8 independent chains), two per SIMD so that
//          the SIMD can issue VALU from two waves at once; each role's iteration count is chosen
//          by the host so that the two would take about as long alone.  If the SIMD overlaps
//          them, each wave's span stays near its time alone; if not, both stretch.
//   SAME_WAVE: one wave per SIMD alternating one MFMA and 8 independent v_add_f32 (none of them
//          reading the MFMA's result): overlap gives about max(MFMA, 8 VALU) cycles per round,
//          none gives the sum.
// ---------------------------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(768, 1) void overlap_kernel(int iters_mfma, int iters_valu,
                                                         uint64_t* out) {
  extern __shared__ uint8_t lds_reserve[];
  const WaveTimes t = start_times();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v4i a = {lane, lane * 3, lane ^ 5, 7}, b = {lane + 1, 2, lane * 5, lane};
  uint32_t sink = 0;
  float r0 = lane, r1 = lane + 1, r2 = lane + 2, r3 = lane + 3, r4 = lane + 4, r5 = lane + 5,
        r6 = lane + 6, r7 = lane + 7;
  const float s2 = -0.5f;
  if (KIND == Q6C_OVERLAP_ROLES) {
    if (wave < 4) {
      v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int i = 0; i < iters_mfma; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
      }
      for (int r = 0; r < 16; ++r) sink ^= c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    } else {
#define Q6C_ADD8                                                                           \
  "v_add_f32 %0, %0, %8\n\tv_add_f32 %1, %1, %8\n\tv_add_f32 %2, %2, %8\n\t"            \
  "v_add_f32 %3, %3, %8\n\tv_add_f32 %4, %4, %8\n\tv_add_f32 %5, %5, %8\n\t"            \
  "v_add_f32 %6, %6, %8\n\tv_add_f32 %7, %7, %8\n\t"
      for (int i = 0; i < iters_valu; ++i) {
        asm volatile(Q6C_ADD8 Q6C_ADD8 Q6C_ADD8 Q6C_ADD8 Q6C_ADD8 Q6C_ADD8 Q6C_ADD8 Q6C_ADD8
                     : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6),
                       "+v"(r7)
                     : "v"(s2));
      }
#undef Q6C_ADD8
    }
  } else {
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters_mfma; ++i) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the MFMA and the VALU block in this order
      asm volatile(
          "v_add_f32 %0, %0, %8\n\tv_add_f32 %1, %1, %8\n\tv_add_f32 %2, %2, %8\n\t"
          "v_add_f32 %3, %3, %8\n\tv_add_f32 %4, %4, %8\n\tv_add_f32 %5, %5, %8\n\t"
          "v_add_f32 %6, %6, %8\n\tv_add_f32 %7, %7, %8"
          : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7)
          : "v"(s2));
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the MFMA and the VALU block in this order
      asm volatile(
          "v_add_f32 %0, %0, %8\n\tv_add_f32 %1, %1, %8\n\tv_add_f32 %2, %2, %8\n\t"
          "v_add_f32 %3, %3, %8\n\tv_add_f32 %4, %4, %8\n\tv_add_f32 %5, %5, %8\n\t"
          "v_add_f32 %6, %6, %8\n\tv_add_f32 %7, %7, %8"
          : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7)
          : "v"(s2));
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the MFMA and the VALU block in this order
      asm volatile(
          "v_add_f32 %0, %0, %8\n\tv_add_f32 %1, %1, %8\n\tv_add_f32 %2, %2, %8\n\t"
          "v_add_f32 %3, %3, %8\n\tv_add_f32 %4, %4, %8\n\tv_add_f32 %5, %5, %8\n\t"
          "v_add_f32 %6, %6, %8\n\tv_add_f32 %7, %7, %8"
          : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7)
          : "v"(s2));
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the MFMA and the VALU block in this order
      asm volatile(
          "v_add_f32 %0, %0, %8\n\tv_add_f32 %1, %1, %8\n\tv_add_f32 %2, %2, %8\n\t"
          "v_add_f32 %3, %3, %8\n\tv_add_f32 %4, %4, %8\n\tv_add_f32 %5, %5, %8\n\t"
          "v_add_f32 %6, %6, %8\n\tv_add_f32 %7, %7, %8"
          : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7)
          : "v"(s2));
    }
    for (int r = 0; r < 16; ++r) sink ^= c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  }
  sink ^= __float_as_uint(r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7);
  finish(t, out, sink);
}

// ---------------------------------------------------------------------------------------------
// HBM streams: grid-stride 16-byte accesses, 4 in flight per lane.
// ---------------------------------------------------------------------------------------------
typedef unsigned stream_v4u __attribute__((ext_vector_type(4)));

// 16 bytes at src + i, with a plain or a nontemporal load
template <bool NT>
__device__ __forceinline__ stream_v4u stream_load(const uint4* src, int64_t i) {
  const stream_v4u* p = reinterpret_cast<const stream_v4u*>(src + i);
  return NT ? __builtin_nontemporal_load(p) : *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const stream_v4u a = stream_load<NT>(src, i), b = stream_load<NT>(src, i + stride),
                     c = stream_load<NT>(src, i + 2 * stride), d = stream_load<NT>(src, i + 3 * stride);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const stream_v4u a = stream_load<NT>(src, i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, int64_t n16,
                                                   uint4* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int device_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return v;
}

template <typename K>
int launch_probe(K kernel, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
                 void* stream) {
  if (iters <= 0 || waves_per_simd < 1 || waves_per_simd > 8 || !out) return Q6K_EINVAL;
  const int cus = device_cus();
  if (cus <= 0) return Q6K_EHIP;
  const int64_t blocks = (int64_t)cus * waves_per_simd;
  if (out_bytes < (size_t)blocks * 4 * 4 * sizeof(uint64_t)) return Q6K_ESIZE;
  const size_t lds = (size_t)(kLdsPerCu / waves_per_simd) & ~(size_t)1023;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return Q6K_EHIP;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), lds,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? Q6K_OK : Q6K_EHIP;
}

}  // namespace

extern "C" {

int q6c_probe_waves(int waves_per_simd) {
  const int cus = device_cus();
  return cus <= 0 ? -1 : cus * waves_per_simd * 4;
}

int q6c_wall_clock_khz(void) {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return v;
}

int q6c_mfma(int kind, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
             void* stream) {
  switch (kind) {
    case Q6C_MFMA_I8_32x32x16:
      return launch_probe(mfma_kernel<Q6C_MFMA_I8_32x32x16>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_MFMA_I8_32x32x32:
      return launch_probe(mfma_kernel<Q6C_MFMA_I8_32x32x32>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_MFMA_I8_16x16x64:
      return launch_probe(mfma_kernel<Q6C_MFMA_I8_16x16x64>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_MFMA_F16_32x32x16:
      return launch_probe(mfma_kernel<Q6C_MFMA_F16_32x32x16>, iters, waves_per_simd, out, out_bytes, stream);
    default:
      return Q6K_EINVAL;
  }
}

int q6c_valu(int kind, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
             void* stream) {
  switch (kind) {
    case Q6C_VALU_FMA_F32:
      return launch_probe(valu_kernel<Q6C_VALU_FMA_F32>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_VALU_FMAC_F32:
      return launch_probe(valu_kernel<Q6C_VALU_FMAC_F32>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_VALU_ADD_F32:
      return launch_probe(valu_kernel<Q6C_VALU_ADD_F32>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_VALU_MUL_F32:
      return launch_probe(valu_kernel<Q6C_VALU_MUL_F32>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_VALU_CVT_F32_I32:
      return launch_probe(valu_kernel<Q6C_VALU_CVT_F32_I32>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_VALU_ADD_U32:
      return launch_probe(valu_kernel<Q6C_VALU_ADD_U32>, iters, waves_per_simd, out, out_bytes, stream);
    default:
      return Q6K_EINVAL;
  }
}

int q6c_tileop(int kind, int iters, int waves_per_simd, uint64_t* out, size_t out_bytes,
               void* stream) {
  switch (kind) {
    case Q6C_TILEOP_FOLDED:
      return launch_probe(tileop_kernel<Q6C_TILEOP_FOLDED>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_TILEOP_HALVES:
      return launch_probe(tileop_kernel<Q6C_TILEOP_HALVES>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_TILEOP_ZERO_C:
      return launch_probe(tileop_kernel<Q6C_TILEOP_ZERO_C>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_TILEOP_FOLDED_PIPE:
      return launch_probe(tileop_kernel<Q6C_TILEOP_FOLDED_PIPE>, iters, waves_per_simd, out, out_bytes, stream);
    case Q6C_TILEOP_F16:
      return launch_probe(tileop_kernel<Q6C_TILEOP_F16>, iters, waves_per_simd, out, out_bytes, stream);
    default:
      return Q6K_EINVAL;
  }
}

int q6c_overlap(int kind, int iters_mfma, int iters_valu, uint64_t* out, size_t out_bytes,
                void* stream) {
  if (iters_mfma < 0 || iters_valu < 0 || !out) return Q6K_EINVAL;
  if (kind != Q6C_OVERLAP_ROLES && kind != Q6C_OVERLAP_SAME_WAVE) return Q6K_EINVAL;
  const int cus = device_cus();
  if (cus <= 0) return Q6K_EHIP;
  // one workgroup per CU: 12 waves (three per SIMD) for ROLES, 4 waves (one per SIMD) otherwise
  const int threads = kind == Q6C_OVERLAP_ROLES ? 768 : 256;
  if (out_bytes < (size_t)cus * (threads / 64) * 4 * sizeof(uint64_t)) return Q6K_ESIZE;
  const size_t lds = (size_t)kLdsPerCu;
  auto kernel = kind == Q6C_OVERLAP_ROLES ? overlap_kernel<Q6C_OVERLAP_ROLES>
                                          : overlap_kernel<Q6C_OVERLAP_SAME_WAVE>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return Q6K_EHIP;
  hipLaunchKernelGGL(kernel, dim3((unsigned)cus), dim3(threads), lds,
                     static_cast<hipStream_t>(stream), iters_mfma, iters_valu, out);
  return hipGetLastError() == hipSuccess ? Q6K_OK : Q6K_EHIP;
}

int q6c_stream(int mode, const void* src, void* dst, size_t bytes, size_t dst_bytes,
               void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16) return Q6K_EINVAL;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return Q6K_EALIGN;
  const int cus = device_cus();
  if (cus <= 0) return Q6K_EHIP;
  const int64_t blocks = (int64_t)cus * 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == Q6C_STREAM_READ || mode == Q6C_STREAM_READ_NT) {
    if (dst_bytes < (size_t)blocks * 256 * 4) return Q6K_ESIZE;
    if (mode == Q6C_STREAM_READ)
      hipLaunchKernelGGL(read_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                         static_cast<const uint4*>(src), (int64_t)(bytes / 16),
                         static_cast<uint32_t*>(dst));
    else
      hipLaunchKernelGGL(read_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                         static_cast<const uint4*>(src), (int64_t)(bytes / 16),
                         static_cast<uint32_t*>(dst));
  } else if (mode == Q6C_STREAM_COPY) {
    if (dst_bytes < bytes) return Q6K_ESIZE;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4*>(src), (int64_t)(bytes / 16),
                       static_cast<uint4*>(dst));
  } else {
    return Q6K_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? Q6K_OK : Q6K_EHIP;
}

}  // extern "C"

// q6k.hip -- HIP kernels for gfx950 and the C ABI of libq6k.so (declared in include/q6k.h).
//
// Kernels
//   quantize_act_kernel : activation quantize-transpose prepass (HBM-bound)
//   expand_kernel<L>    : load-time weight preparation, layout 0 (packed 6-bit) or 1 (int8 plane)
//   gemm_kernel<L, D>   : q6_K x int8 GEMM on v_mfma_i32_32x32x16_i8 (the int8 MFMA whose
//                         K is 16, so the two 16-k halves of a chunk stay separate integers);
//                         D = true is the test-only sub-block dot export of the same source
//   folded_kernel<D>    : the same GEMM on layout 2, where the int8 sub-block scale is applied
//                         inside the integer dot (two int8 digit planes of sc * (q - 32)) and
//                         each chunk needs one f32 rescale instead of two; D = true exports the
//                         per-chunk integer numerators
//
// The method follows "r38 — q6_K BT-style raw-byte mma kernel (LANDED)" (sec. 2.1 layout,
// sec. 2.2 rescale without dmin, sec. 2.4 KSPLIT=2), "r41 — q6_K B-expand widened to uint4
// group loads (LANDED)" (expand from wide loads) and "r53 — q6_K bundle: W_exp pre-expansion
// plane + cp.async B staging (LANDED)" (optional pre-expanded plane).  The tiling is this library's own.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "q4k.h"
#include "q6k.h"
#ifdef Q6K_TIMELINE
#include "q6k_timeline.h"
#endif

namespace {

constexpr int kTile = 32;        // MFMA tile edge: 32 tokens x 32 weight rows
constexpr int kWgTok = 128;      // token padding of the tiled activation buffers
constexpr int kWgRow = 128;      // row padding of the prepared weight buffers (4 row tiles)
constexpr int kFragBytes = 16;   // per lane per chunk: 8 bytes for half 0, 8 for half 1
constexpr int kPackBytes = 12;   // layout 0: per lane per chunk, 16 codes of 6 bits
constexpr int kBiasI = 0x4B400000;      // bit pattern of 1.5 * 2^23
constexpr float kBiasF = 12582912.0f;   // 1.5 * 2^23

std::atomic<uint64_t> g_launches[3];
std::atomic<uint64_t> g_q4k_launches;

typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) | ((uint32_t)(c & 255) << 16) |
         ((uint32_t)(d & 255) << 24);
}

// ---------------------------------------------------------------------------------------------
// Prepass.  Block = 4 waves = one token tile (32 tokens) x 8 chunks (256 k values).  Wave w walks
// tokens 8w .. 8w+7 of the tile; per token its 64 lanes read the 1 KiB of those 256 values with
// one coalesced 16-byte load each (lane l holds k 4l .. 4l+3 of the window, chunk l / 8).  The 8
// lanes of a chunk exchange their maxima through DPP moves (da = amax / 127, IEEE f32), each quantizes its four
// values (q = roundf(x / da) on the correctly rounded f32 quotient, clamped to +-127; see
// quant_code for how the division is avoided without changing any result) and puts them, as
// one 4-byte word, at their place of the tiled layout in LDS; the block then writes its eight
// 1 KiB code blocks and 1 KiB of scales with coalesced 16-byte stores.
// With SWIGLU the input value is produced on the fly from two rows, h = up * silu(gate), so that
// the f32 product feeding ffn_down is quantized without ever being written ("r53 — q6_K bundle:
// W_exp pre-expansion plane + cp.async B staging (LANDED)", sec. 1: fused producers).
// ---------------------------------------------------------------------------------------------

// up * silu(gate), silu(g) = g / (1 + e^-g), in f32 (expf within a few ulp; e^-g overflows to
// infinity for very negative g and gives a signed zero).  The test export computes h with this
// same function.
__device__ __forceinline__ float swiglu_f32(float g, float u) { return u * (g / (1.0f + expf(-g))); }

// A lane's neighbour value through a DPP move (no LDS traffic); CTRL is the DPP control code.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, true));
}

// q = roundf(x / s) with the correctly rounded f32 quotient (ties away from zero), clamped to
// [-127, 127], without a full division in the common case.  r = rcp(s) is within 1 ulp of 1/s,
// so y = x * r is within 2 ulps of the quotient (< 2^-15 absolute for |x / s| <= 127.5); when y
// is farther than 2^-12 from a half-integer, the rounded quotient and y round to the same
// integer and neither is a tie, so rint(y) is the result.  Near a half-integer, or when s lies
// outside [2^-100, 2^100] (subnormal or huge scales, whose reciprocal may lose precision), the
// exact division decides.  A NaN x gives a NaN q on both paths.
__device__ __forceinline__ int quant_code(float x, float s, float r, bool fast) {
  const float y = x * r;
  const float yr = __builtin_rintf(y);
  float q;
  if (fast && !(fabsf(y - yr) > 0.5f - 0x1p-12f))
    q = yr;
  else
    q = roundf(x / s);
  return (int)fminf(fmaxf(q, -127.0f), 127.0f);
}

// SUMS: also write das = da * S per (token, chunk), S the sum of the chunk's 32 codes, in the order
// of da (the per-chunk activation sum the q4_K rescale needs next to da).
// 16 bytes of a tensor read exactly once: a nontemporal load (streams at ~6.0 TB/s on MI355X
// against ~5.4 for a plain load in a 2 GiB read probe).
__device__ __forceinline__ float4 load_stream(const float* p) {
  const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}

template <bool SWIGLU, bool SUMS>
__global__ __launch_bounds__(256) void quantize_act_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ up,
                                                           int64_t n, int64_t ldx, int64_t nchunk,
                                                           uint8_t* __restrict__ xq,
                                                           float* __restrict__ da,
                                                           float* __restrict__ das, int64_t t0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // workgroup order: the 8-chunk block of k varies fastest, so workgroups running together read
  // consecutive kilobytes of the same rows (sequential DRAM streams) rather than 1 KiB pieces of
  // rows 44 KB apart
  const int64_t T = t0 + blockIdx.y, kb = blockIdx.x;
  const int64_t c = kb * 8 + (lane >> 3);  // this lane's chunk
  const int kk = 4 * (lane & 7);                             // its first k inside the chunk
  const bool live_c = c < nchunk;
  // place of the lane's 4 codes in the chunk's 1 KiB block: slot p + 32*g, byte 8*h + kk % 8
  const int g = (kk >> 3) & 1, h = kk >> 4;
  __shared__ __attribute__((aligned(16))) uint8_t codes[8 * 1024];
  __shared__ __attribute__((aligned(16))) float scales[8 * 32];
  __shared__ __attribute__((aligned(16))) float sums[SUMS ? 8 * 32 : 4];
  // all loads first (eight rows, with SWIGLU sixteen, in flight per wave), then the arithmetic.
  // The loads are unconditional, from the row and chunk clamped into the input, and lanes outside
  // it take zeros afterwards: a load under a branch would make the compiler wait for it.
  float4 v[8], u[8];
  const int64_t cl = live_c ? c : nchunk - 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t tok = T * kTile + 8 * wave + j;
    const int64_t off = (tok < n ? tok : n - 1) * ldx + cl * 32 + kk;
    v[j] = load_stream(x + off);
    if (SWIGLU) u[j] = load_stream(up + off);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t tok = T * kTile + 8 * wave + j;
    if (SWIGLU) {
      v[j].x = swiglu_f32(v[j].x, u[j].x);
      v[j].y = swiglu_f32(v[j].y, u[j].y);
      v[j].z = swiglu_f32(v[j].z, u[j].z);
      v[j].w = swiglu_f32(v[j].w, u[j].w);
    }
    if (!(tok < n && live_c)) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = 8 * wave + j;
    float amax = fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
    amax = fmaxf(amax, dpp_f32<0xB1>(amax));   // lane ^ 1 (quad_perm 1,0,3,2)
    amax = fmaxf(amax, dpp_f32<0x4E>(amax));   // lane ^ 2 (quad_perm 2,3,0,1)
    amax = fmaxf(amax, dpp_f32<0x141>(amax));  // the other quad of the 8 (row_half_mirror)
    const float scale = amax / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (scale != 0.0f) {
      const float r = __builtin_amdgcn_rcpf(scale);
      const bool fast = scale >= 0x1p-100f && scale <= 0x1p100f;
      q0 = quant_code(v[j].x, scale, r, fast);
      q1 = quant_code(v[j].y, scale, r, fast);
      q2 = quant_code(v[j].z, scale, r, fast);
      q3 = quant_code(v[j].w, scale, r, fast);
    }
    // stage the tile's codes and scales in LDS in their global order
    *reinterpret_cast<uint32_t*>(codes + (lane >> 3) * 1024 + (p + 32 * g) * kFragBytes + 8 * h +
                                 (kk & 7)) = pack4(q0, q1, q2, q3);
    // token p = 8*qq + 4*gg + r  ->  float slot 16*gg + 4*qq + r
    const int slot = (lane >> 3) * 32 + 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
    if ((lane & 7) == 0) scales[slot] = scale;
    if (SUMS) {
      // the chunk's 32 codes are 4 per lane in 8 lanes: the same three exchanges as amax
      int sum = q0 + q1 + q2 + q3;
      sum += __builtin_amdgcn_mov_dpp(sum, 0xB1, 0xF, 0xF, true);
      sum += __builtin_amdgcn_mov_dpp(sum, 0x4E, 0xF, 0xF, true);
      sum += __builtin_amdgcn_mov_dpp(sum, 0x141, 0xF, 0xF, true);
      if ((lane & 7) == 0) sums[slot] = scale * (float)sum;
    }
  }
  __syncthreads();
  // coalesced stores: thread t writes 32 bytes of chunk t / 32's 1 KiB block; threads 0..63 the
  // 8 x 32 scales
  const int t = threadIdx.x;
  const int64_t ct = kb * 8 + (t >> 5);
  if (ct < nchunk) {
    const uint4* srcq = reinterpret_cast<const uint4*>(codes + t * 32);
    uint4* dstq = reinterpret_cast<uint4*>(xq + (T * nchunk + ct) * 64 * kFragBytes + (t & 31) * 32);
    dstq[0] = srcq[0];
    dstq[1] = srcq[1];
  }
  if (t < 64) {
    const int64_t cd = kb * 8 + (t >> 3);
    if (cd < nchunk)
      reinterpret_cast<float4*>(da + (T * nchunk + cd) * 32)[t & 7] =
          reinterpret_cast<const float4*>(scales)[t];
  } else if (SUMS && t < 128) {
    const int64_t cd = kb * 8 + ((t - 64) >> 3);
    if (cd < nchunk)
      reinterpret_cast<float4*>(das + (T * nchunk + cd) * 32)[t & 7] =
          reinterpret_cast<const float4*>(sums)[t - 64];
  }
}

// Test export: h = up * silu(gate) with the producer's own function, row-major [n][ldh].
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ gate,
                                                     const float* __restrict__ up, int64_t n,
                                                     int64_t k, int64_t ld, float* __restrict__ h,
                                                     int64_t ldh) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * k) return;
  const int64_t t = i / k, e = i % k;
  h[t * ldh + e] = swiglu_f32(gate[t * ld + e], up[t * ld + e]);
}

// ---------------------------------------------------------------------------------------------
// Weight preparation.  Block = one row tile (32 rows) x one super-block (8 chunks); the 32 raw
// 210-byte blocks are first copied to LDS with 2-byte loads (a raw block is 2-byte aligned),
// then thread (p, cc) decodes chunk cc of row 32R + p.
// Code of element e of a block ("r38 ..." sec. 3.2): half it = e / 128, offset nn = e % 128;
// low 4 bits = nibble nn / 64 of ql[64 it + nn % 64]; high 2 bits = field (nn / 32) % 4 of
// qh[32 it + nn % 32].  For chunk cc (elements 32cc + i): it = cc / 4, the ql byte is
// 64 it + 32 (cc % 2) + i with nibble (cc % 4) / 2, the qh byte is 32 it + i with field cc % 4.
// ---------------------------------------------------------------------------------------------
constexpr int kRawBlock = 210;
constexpr int kLdsRow = 212;  // 4-byte aligned LDS row pitch for one raw block

template <int LAYOUT>
__global__ __launch_bounds__(256) void expand_kernel(const uint8_t* __restrict__ raw, int64_t m,
                                                     int64_t nsb, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  __shared__ uint16_t blk16[kTile * kLdsRow / 2];
  const int64_t R = blockIdx.x;
  const int64_t sb = blockIdx.y;
  const int64_t nchunk = nsb * 8;
  for (int idx = threadIdx.x; idx < kTile * (kRawBlock / 2); idx += 256) {
    const int j = idx / (kRawBlock / 2), w = idx % (kRawBlock / 2);
    const int64_t row = R * kTile + j;
    uint16_t val = 0;
    if (row < m) {
      const uint8_t* b = raw + (row * nsb + sb) * kRawBlock;
      val = reinterpret_cast<const uint16_t*>(b)[w];
    }
    blk16[j * (kLdsRow / 2) + w] = val;
  }
  __syncthreads();
  const int p = threadIdx.x & 31;
  const int cc = threadIdx.x >> 5;
  const int64_t c = sb * 8 + cc;
  const uint8_t* blk = reinterpret_cast<const uint8_t*>(blk16) + p * kLdsRow;
  const int it = cc >> 2;
  const int qlb = 64 * it + 32 * (cc & 1);
  const int qls = 4 * ((cc & 3) >> 1);
  const int qhb = 128 + 32 * it;
  const int qhs = 2 * (cc & 3);
  int code[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    code[i] = ((blk[qlb + i] >> qls) & 15) | (((blk[qhb + i] >> qhs) & 3) << 4);
  const int8_t sc0 = (int8_t)blk[192 + 2 * (cc & 7)];
  const int8_t sc1 = (int8_t)blk[192 + 2 * (cc & 7) + 1];
  const uint16_t dbits = (uint16_t)(blk[208] | (blk[209] << 8));
  const int64_t tc = R * nchunk + c;  // (row tile, chunk) index
  if (LAYOUT == Q6K_LAYOUT_FOLDED) {
    // v = sc * (q - 32) in [-4064, 4096] = 64 * hi + lo with lo in [-32, 31], hi in [-63, 64]
    const bool live = R * kTile + p < m;
    int lo[32], hi[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int v = live ? (i < 16 ? sc0 : sc1) * (code[i] - 32) : 0;
      lo[i] = ((v + 32) & 63) - 32;
      hi[i] = (v - lo[i]) / 64;  // exact: v - lo is a multiple of 64
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int* cv = h ? hi : lo;
      uint4 s0, s1;
      s0.x = pack4(cv[0], cv[1], cv[2], cv[3]);
      s0.y = pack4(cv[4], cv[5], cv[6], cv[7]);
      s0.z = pack4(cv[16], cv[17], cv[18], cv[19]);
      s0.w = pack4(cv[20], cv[21], cv[22], cv[23]);
      s1.x = pack4(cv[8], cv[9], cv[10], cv[11]);
      s1.y = pack4(cv[12], cv[13], cv[14], cv[15]);
      s1.z = pack4(cv[24], cv[25], cv[26], cv[27]);
      s1.w = pack4(cv[28], cv[29], cv[30], cv[31]);
      uint4* dst = reinterpret_cast<uint4*>(codes + (tc * 2 + h) * 64 * kFragBytes);
      dst[p] = s0;
      dst[p + 32] = s1;
    }
    if (cc == 0)
      reinterpret_cast<float*>(scales)[(R * nsb + sb) * 32 + p] =
          live ? __half2float(__ushort_as_half(dbits)) : 0.0f;
  } else if (LAYOUT == Q6K_LAYOUT_EXPANDED) {
    const bool live = R * kTile + p < m;  // padding rows are stored as zeros
    int cv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) cv[i] = live ? code[i] - 32 : 0;
    uint4 s0, s1;
    s0.x = pack4(cv[0], cv[1], cv[2], cv[3]);
    s0.y = pack4(cv[4], cv[5], cv[6], cv[7]);
    s0.z = pack4(cv[16], cv[17], cv[18], cv[19]);
    s0.w = pack4(cv[20], cv[21], cv[22], cv[23]);
    s1.x = pack4(cv[8], cv[9], cv[10], cv[11]);
    s1.y = pack4(cv[12], cv[13], cv[14], cv[15]);
    s1.z = pack4(cv[24], cv[25], cv[26], cv[27]);
    s1.w = pack4(cv[28], cv[29], cv[30], cv[31]);
    uint4* dst = reinterpret_cast<uint4*>(codes + tc * 64 * kFragBytes);
    dst[p] = s0;
    dst[p + 32] = s1;
    const float d = __half2float(__ushort_as_half(dbits));
    float2 s;
    s.x = d * (float)sc0;  // exact: an 11-bit significand times an 8-bit integer
    s.y = d * (float)sc1;
    if (R * kTile + p >= m) s.x = s.y = 0.0f;
    reinterpret_cast<float2*>(scales)[tc * 32 + p] = s;
  } else {
    // lane p (g = 0) takes k 8g + e = e and 16 + e; lane p + 32 (g = 1) takes 8 + e and 24 + e.
    // Three words X, Y, Z hold the codes a_0..3, a_4..7, b_0..3 as q << 2 (bits 2-7 of each
    // byte); bits 0-1 of byte t of X, Y, Z hold bits 0-1, 2-3, 4-5 of b_{4+t}.
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int* a = code + 8 * g;       // half 0 codes a_0..a_7
      const int* b = code + 16 + 8 * g;  // half 1 codes b_0..b_7
      uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int f = b[t + 4];
        w0 |= (uint32_t)((a[t] << 2) | (f & 3)) << (8 * t);
        w1 |= (uint32_t)((a[t + 4] << 2) | ((f >> 2) & 3)) << (8 * t);
        w2 |= (uint32_t)((b[t] << 2) | (f >> 4)) << (8 * t);
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (tc * 64 + p + 32 * g) * kPackBytes);
      dst[0] = w0;
      dst[1] = w1;
      dst[2] = w2;
    }
    // the (d*sc0, d*sc1) plane of layout 1
    const float d = __half2float(__ushort_as_half(dbits));
    float2 sp;
    sp.x = d * (float)sc0;  // exact: an 11-bit significand times an 8-bit integer
    sp.y = d * (float)sc1;
    if (R * kTile + p >= m) sp.x = sp.y = 0.0f;
    reinterpret_cast<float2*>(scales)[tc * 32 + p] = sp;
  }
}

// Layout 0 in-register expand of one lane's 16 codes into the two 8-byte MFMA fragments, as
// centered int8 times 4: a byte s = (q << 2) | x (q the 6-bit code, x two bits stored for the
// fourth word) becomes (s & 0xFC) ^ 0x80 = 4q - 128 = 4 (q - 32) in [-128, 124] -- one SWAR
// operation per word, no carries -- and the fourth word's bytes are gathered from the x bits of
// the other three and then treated alike.  The MFMA then yields 4 D exactly (|4 D| < 2^22, so the
// float bias trick still holds); the rescale uses d*sc itself, so the accumulators hold 4 y and
// the store multiplies by 1/4 (exact: a power of two).
__device__ __forceinline__ uint32_t center4x4(uint32_t s) { return (s & 0xFCFCFCFCu) ^ 0x80808080u; }

// Bits 0-1 of byte t of x, y, z become bits 2-3, 4-5, 6-7 of byte t (4 b_{4+t}), centered like
// the others.  Each shift drags a neighbouring byte's bits into the positions it does not keep;
// the two bit-field inserts and the final mask take only the wanted ones.
__device__ __forceinline__ uint32_t fourth4x4(uint32_t x, uint32_t y, uint32_t z) {
  const uint32_t a = x << 2, b = y << 4, c = z << 6;
  const uint32_t ab = (a & 0x0C0C0C0Cu) | (b & ~0x0C0C0C0Cu);
  const uint32_t abc = (ab & 0x3C3C3C3Cu) | (c & ~0x3C3C3C3Cu);
  return (abc & 0xFCFCFCFCu) ^ 0x80808080u;
}

// ---------------------------------------------------------------------------------------------
// Work split shared by the GEMM kernels.  Every GEMM workgroup computes one 64-token x 128-row
// output tile (gx x gy tiles).  The tiles are dealt out in rounds of one per workgroup slot of
// the GPU (workgroups per CU x CUs); when the last round would leave slots idle, its tiles are
// split along k into `pieces` pieces of whole super-blocks that run side by side.  Workgroups
// 0 .. n_full-1 take whole tiles and store them into y; workgroup n_full + i takes piece
// i % pieces of split tile i / pieces (or, on layout 2 behind whole rounds, the piece it claims
// as it starts: tile_work) and stores its partial sums into that piece's slab of the caller's
// workspace (one 64 x 128 f32 tile per piece), and split_reduce_kernel, launched next on the same
// stream, adds each tile's slabs in piece order into y.  The sum's order is fixed, so every output
// is the same bit for bit from run to run.
// ---------------------------------------------------------------------------------------------
// XCD-aware tile order: workgroup t of the dispatch order runs on XCD (t + c) % 8, c fixed within a
// launch (the dispatcher's round robin carries on from the previous launch), so the workgroups
// with one value j of t % 8 share an XCD and its L2; when the grid splits evenly, they take one
// (gx/4) x (gy/2) rectangle of the output tiles (token pairs fastest inside it), so each
// activation tile is fetched into 2 of the 8 L2s and each weight tile into 4.  On ffn_down at N=3314 this fetches 23 % fewer bytes across the
// fabric than (gx/2) x (gy/4) rectangles (0.92 against 1.20 GB per launch) and runs 1-2 % faster;
// a plain row-major order runs about 1 % slower than either.
__device__ __forceinline__ void tile_of(uint32_t t, uint32_t gx, uint32_t gy, uint32_t* bx,
                                        uint32_t* by) {
  if (gx % 4 == 0 && gy % 2 == 0) {
    const uint32_t xcd = t % 8, local = t / 8, rw = gx / 4, rh = gy / 2;
    *bx = (xcd % 4) * rw + local % rw;
    *by = (xcd / 4) * rh + local / rw;
  } else {
    *bx = t % gx;
    *by = t / gx;
  }
}

struct TileWork {
  uint32_t bx, by;  // token-tile pair and row-tile quad of the output tile
  int64_t s0, s1;   // super-blocks [s0, s1) of k
  bool split;       // a piece of a split tile: store into workspace slab `slab`
  uint32_t slab;    // pid - n_full for a piece
};

// Workgroup timeline, compiled in only by the instrumented build of this file (Q6K_TIMELINE
// defined, libq6k_timeline.so): the first thread of GEMM workgroup b writes record b of the
// last launch, eight words: start and end on the 100 MHz constant clock, start and end shader
// cycles, the XCD (high word) and HW_ID register (low word), the tile (bx, by), its k range of
// super-blocks (s0, s1) and whether it is a split-k piece.  The product build has no trace of it.
#ifdef Q6K_TIMELINE
constexpr int kTimelineWgs = 16384;
__device__ uint64_t q6k_timeline_rec[kTimelineWgs * 8];
struct WgStamp {
  uint64_t t, c;
};
__device__ __forceinline__ WgStamp wg_stamp() {
  return WgStamp{__builtin_amdgcn_s_memrealtime(), __builtin_amdgcn_s_memtime()};
}
__device__ __forceinline__ void wg_record(const WgStamp& s, const TileWork& tw) {
  if (threadIdx.x != 0 || blockIdx.x >= (uint32_t)kTimelineWgs) return;
  uint32_t xcc, hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime(), c1 = __builtin_amdgcn_s_memtime();
  uint64_t* o = q6k_timeline_rec + 8 * (uint64_t)blockIdx.x;
  o[0] = s.t;
  o[1] = t1;
  o[2] = s.c;
  o[3] = c1;
  o[4] = ((uint64_t)xcc << 32) | hw;
  o[5] = (uint64_t)tw.bx | ((uint64_t)tw.by << 32);
  o[6] = (uint64_t)tw.s0 | ((uint64_t)tw.s1 << 32);
  o[7] = tw.split ? 1 : 0;
}
#else
struct WgStamp {};
__device__ __forceinline__ WgStamp wg_stamp() { return WgStamp{}; }
__device__ __forceinline__ void wg_record(const WgStamp&, const TileWork&) {}
#endif

constexpr int kSlabTok = 64;                     // tokens of an output tile (every GEMM)
constexpr int64_t kSlabFloats = kSlabTok * 128;  // one output tile, f32 [64][128]

// Where a workgroup's output tile goes: y itself, or the piece's workspace slab, addressed with
// the tile's own (token, row) offsets, so that the store of output (tok, row) is
// p[(tok - tok0) * ld + (row - row0)].
struct OutDst {
  float* p;
  int64_t ld, tok0, row0;
};

__device__ __forceinline__ OutDst out_dst(const TileWork& tw, float* y, int64_t ldy, float* ws) {
  OutDst o;
  if (tw.split) {
    o.p = ws + (int64_t)tw.slab * kSlabFloats;
    o.ld = 128;
    o.tok0 = (int64_t)tw.bx * kSlabTok;
    o.row0 = (int64_t)tw.by * 128;
  } else {
    o.p = y;
    o.ld = ldy;
    o.tok0 = 0;
    o.row0 = 0;
  }
  return o;
}

// Where the test exports store their integer dots: tokens [tok0, tok0 + ntok) x rows
// [row0, row0 + nrow) of the full problem, as int32 [ntok][nrow][per], per = dots per row and
// token (k/16 or k/32).  The window lies inside the problem; the kernel still computes every tile.
struct DotsOut {
  int32_t* p;
  int64_t tok0, ntok, row0, nrow;
};

// One lane's dots slots along the 16 registers of a 32x32 tile: register r holds index
// first + dt(r), dt(r) = 8*(r/4) + r%4, of the varying dimension (tokens when VARY_TOK, else rows);
// the lane's other index is fixed.  The offsets pass through an empty statement at every chunk,
// so the compiler forms the 16 slot addresses (and their bounds tests) where they are stored
// instead of holding them all live across the chunk loop.
struct DotsRun {
  int64_t off;     // window offset of register 0's slot, chunk term included
  int64_t vary;    // varying index of register 0 inside the window (may lie outside it)
  int64_t stride;  // window offset between consecutive values of the varying index
  int64_t limit;   // window extent along the varying index
  bool fixed_ok;   // the fixed index lies inside the window
};

template <bool VARY_TOK>
__device__ __forceinline__ DotsRun dots_run(const DotsOut& w, int64_t tok, int64_t row,
                                            int64_t per, int64_t cterm) {
  DotsRun d;
  const int64_t ti = tok - w.tok0, ri = row - w.row0;
  d.off = (ti * w.nrow + ri) * per + cterm;
  d.vary = VARY_TOK ? ti : ri;
  d.stride = VARY_TOK ? w.nrow * per : per;
  d.limit = VARY_TOK ? w.ntok : w.nrow;
  d.fixed_ok = VARY_TOK ? (uint64_t)ri < (uint64_t)w.nrow : (uint64_t)ti < (uint64_t)w.ntok;
  asm volatile("" : "+v"(d.off), "+v"(d.vary));
  return d;
}

// Register r's slot, or nullptr outside the window.
__device__ __forceinline__ int32_t* dots_slot(const DotsOut& w, const DotsRun& d, int r) {
  const int dt = 8 * (r >> 2) + (r & 3);
  if (!d.fixed_ok || (uint64_t)(d.vary + dt) >= (uint64_t)d.limit) return nullptr;
  return w.p + d.off + dt * d.stride;
}

// The result is uniform across the workgroup; the divisions in it run on the vector ALU, so each
// field goes through readfirstlane to tell the compiler (and keep everything derived from it in
// scalar registers).
// Super-block bound j of a split tile's pieces.  grade 0: equal pieces.  grade G >= 1: piece i
// weighs P - i + G - 1, so piece 0 is the largest and the sizes fall off linearly; the host
// checks that every piece keeps at least one super-block.
__host__ __device__ inline int64_t tail_bound(int64_t nsb, uint32_t P, uint32_t grade,
                                              uint32_t j) {
  if (grade == 0) return nsb * j / P;
  const int64_t g = (int64_t)grade - 1;
  const int64_t wj = (int64_t)j * (P + g) - (int64_t)j * (j - 1) / 2;
  const int64_t wp = (int64_t)P * (P + g) - (int64_t)P * (P - 1) / 2;
  return nsb * wj / wp;
}

// `pieces` carries the piece count P in its low 16 bits and the grade in the next 8.  With a
// grade and a workspace, the tail is claimed: the split tiles' workgroups start as slots free up
// behind the whole rounds, at different times on different XCDs and CUs, and each takes the next
// claim c of the launch at its start (one fetch-and-add on the claim word that follows the slabs
// in the workspace) -- piece c / nsplit (the largest pieces first) of split tile c % nsplit -- so
// the workgroups that start last get the smallest pieces and the launch's last ends draw
// together.  A piece's k-range and slab depend only on (tile, piece), never on which workgroup
// ran it, so the reduction's sums are the same bit for bit.  The claim word starts each launch at
// 0: workgroup 0, a whole tile (the host claims only behind a whole round, so every split tile's
// workgroup is dispatched after a workgroup of the first round has run a whole tile), stores 0
// as it starts, and split_reduce_kernel, next on the stream, stores 0 again after the launch.
template <bool XCD_ORDER>
__device__ __forceinline__ TileWork tile_work(uint32_t pid, uint32_t gx, uint32_t gy,
                                              uint32_t n_full, uint32_t pieces, int64_t nsb,
                                              float* ws) {
  __shared__ uint32_t claim_lds;
  TileWork w;
  const uint32_t P = pieces & 0xFFFF, grade = (pieces >> 16) & 0xFF;
  const bool claimed = grade && ws;
  w.split = pid >= n_full;
  uint32_t tile = pid, piece = 0;
  const uint32_t nsplit = gx * gy - n_full;
  uint32_t* claim = claimed ? reinterpret_cast<uint32_t*>(ws + (int64_t)nsplit * P * kSlabFloats)
                            : nullptr;
  if (claimed && pid == 0 && threadIdx.x == 0)
    __hip_atomic_store(claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (w.split) {
    uint32_t c = pid - n_full;
    if (claimed) {
      if (threadIdx.x == 0)
        claim_lds = __hip_atomic_fetch_add(claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) %
                    (nsplit * P);
      __syncthreads();
      c = claim_lds;
      tile = n_full + c % nsplit;
      piece = c / nsplit;
    } else {
      tile = n_full + c / P;
      piece = c % P;
    }
  }
  if (XCD_ORDER) {
    tile_of(tile, gx, gy, &w.bx, &w.by);
  } else {
    w.bx = tile % gx;
    w.by = tile / gx;
  }
  w.s0 = w.split ? tail_bound(nsb, P, grade, piece) : 0;
  w.s1 = w.split ? tail_bound(nsb, P, grade, piece + 1) : nsb;
  w.bx = __builtin_amdgcn_readfirstlane(w.bx);
  w.by = __builtin_amdgcn_readfirstlane(w.by);
  w.s0 = __builtin_amdgcn_readfirstlane((int)w.s0);
  w.s1 = __builtin_amdgcn_readfirstlane((int)w.s1);
  w.split = __builtin_amdgcn_readfirstlane((int)w.split) != 0;
  w.slab = __builtin_amdgcn_readfirstlane(w.split ? (tile - n_full) * P + piece : 0u);
  return w;
}

// y over the tiles that a GEMM split along k (tiles n_full .. gx*gy-1 of the GEMM's tile order,
// XCD-aware or plain): the sum of the tile's `pieces` workspace slabs, added in piece order.  A
// workgroup covers kReduceTok tokens of a tile, a thread 4 consecutive rows of one token; its
// pieces are loaded four at a time (the loads in flight together) and added one after another,
// so the order of the additions is fixed.  vec: y is 16-byte aligned and ldy % 4 == 0.
constexpr int kReduceTok = 8;  // tokens per reducing workgroup (256 threads x 4 rows)
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ y, int64_t ldy,
                                                           int64_t n, int64_t m, uint32_t gx,
                                                           uint32_t gy, uint32_t n_full,
                                                           uint32_t pieces, int xcd_order,
                                                           int vec, uint32_t* claim) {
  // the GEMM before it on the stream has handed out all its claims: leave the word at 0
  if (claim && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr uint32_t parts = kSlabTok / kReduceTok;
  const uint32_t t = n_full + blockIdx.x / parts, part = blockIdx.x % parts;
  uint32_t bx, by;
  if (xcd_order) {
    tile_of(t, gx, gy, &bx, &by);
  } else {
    bx = t % gx;
    by = t / gx;
  }
  const int tl = part * kReduceTok + (threadIdx.x >> 5), rl = 4 * (threadIdx.x & 31);
  const int64_t tok = (int64_t)bx * kSlabTok + tl, r = (int64_t)by * 128 + rl;
  if (tok >= n || r >= m) return;
  const float4* src = reinterpret_cast<const float4*>(
      ws + (int64_t)(t - n_full) * pieces * kSlabFloats + tl * 128 + rl);
  constexpr int64_t kStride = kSlabFloats / 4;  // float4s from one piece's slab to the next
  float4 v = src[0];
  uint32_t pc = 1;
  for (; pc + 4 <= pieces; pc += 4) {
    const float4 a = src[pc * kStride], b = src[(pc + 1) * kStride], c = src[(pc + 2) * kStride],
                 d = src[(pc + 3) * kStride];
    v.x = v.x + a.x + b.x + c.x + d.x;
    v.y = v.y + a.y + b.y + c.y + d.y;
    v.z = v.z + a.z + b.z + c.z + d.z;
    v.w = v.w + a.w + b.w + c.w + d.w;
  }
  for (; pc < pieces; ++pc) {
    const float4 a = src[pc * kStride];
    v.x += a.x;
    v.y += a.y;
    v.z += a.z;
    v.w += a.w;
  }
  float* dst = y + tok * ldy + r;
  if (vec && r + 3 < m) {
    *reinterpret_cast<float4*>(dst) = v;
  } else {
    dst[0] = v.x;
    if (r + 1 < m) dst[1] = v.y;
    if (r + 2 < m) dst[2] = v.z;
    if (r + 3 < m) dst[3] = v.w;
  }
}

// ---------------------------------------------------------------------------------------------
// GEMM on layouts 0 and 1.  Workgroup = 4 waves = one output tile of 64 tokens (token tiles 2*bx,
// 2*bx+1) x 128 weight rows (row tiles 4*by .. 4*by+3), over the k-range tile_work gives it.
// Wave w computes token tile w%2 against row tiles 2*(w/2) and 2*(w/2)+1: two 32x32 output
// tiles, 32 f32 accumulators per lane.
//
// Staging: a ring of kRing LDS slots, one 32-k chunk of the workgroup's operands per slot.  Each
// wave fills its share of a slot with gfx950 direct-to-LDS loads through buffer resources
// (buffer_load_dwordx4 ... lds, 16 bytes per lane, no registers): row tile w's weight codes and
// (d*sc0, d*sc1) pairs, and, for waves 0 and 1, token tile w's activations and da.  Loads run kRing-1 chunks
// ahead of the compute.  Step c (chunk c, slot c % kRing) of a wave, entered with chunk c complete
// in LDS for every wave and this wave's A and B fragments of chunk c on their way to registers:
//   1. wait for the fragments, start the LDS reads of chunk c's da and scale pairs, start the
//      four MFMAs (the reads land behind them);
//   2. issue the loads of chunk c+kRing-1 into chunk c-1's slot, which every wave finished
//      reading before the meeting of step c-1;
//   3. wait for this wave's own loads of chunk c+1 (kRing-2 newer chunks may stay in flight) and
//      for the da and scale reads;
//   4. layout 0: start the LDS reads of this wave's packed codes of chunk c+1; rescale tile 0 of
//      chunk c (the reads land meanwhile); expand row tile w of chunk c+1 into B fragments of
//      4 x the centered int8 codes in its slot;
//   5. meet: every wave's share of chunk c+1 is in its slot (loads landed, layout 0 expanded),
//      and every wave is done with chunk c's da and scales;
//   6. start the LDS reads of chunk c+1's fragments, then rescale tile 1 of chunk c (the reads
//      land meanwhile).
// The chunk loop is unrolled over the ring, so every slot address is a per-lane base register
// plus an immediate offset (no address arithmetic per chunk).  LDS reads and writes are inline
// assembly with explicit waits: the compiler would otherwise wait for every outstanding
// direct-to-LDS load before each LDS access, which would serialize the ring.
//
// Per chunk and output tile: two v_mfma_i32_32x32x16_i8 (halves 0 and 1), each started from the
// bit pattern of 1.5*2^23 so that the int32 result D (4 D on layout 0) is read as the float
// 1.5*2^23 + D exactly (|4 D| <= 4*16*127*32 < 2^22).  The rescale of each half is then
//     t = fma(F, dsc, -1.5*2^23*dsc)  (= D*dsc rounded once; the bias product is exact)
//     acc = fma(t, da, acc)
// i.e. the two independent += of the method, four VALU fma per output per chunk.
//
// Output layout of the MFMA: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4 (a token)
// and column l%32 (a weight row).
// ---------------------------------------------------------------------------------------------
#ifndef Q6K_GEMM01_XCD_ORDER
#define Q6K_GEMM01_XCD_ORDER 0
#endif
#ifndef Q6K_WG_PER_CU
#define Q6K_WG_PER_CU 3
#endif
constexpr int kWgTokTiles = 2;   // token tiles per workgroup
constexpr int kSlotA = 0;        // 2 token tiles x 1 KiB of A fragments
constexpr int kSlotD = 2048;     // 2 token tiles x 32 da f32
constexpr int kSlotB = 2304;     // 4 row tiles x 1 KiB of centered int8 B fragments
constexpr int kSlotS = 6400;     // 4 row tiles x 32 rows x (dsc0, dsc1) f32
constexpr int kSlotRawB = 7424;  // layout 0: 4 row tiles x 768 B of packed 6-bit codes

template <int LAYOUT>
struct SlotSize {
  static constexpr int value = LAYOUT == Q6K_LAYOUT_EXPANDED ? 7424 : 10496;
};
// LDS slots per workgroup (loads run kRing-1 chunks ahead), sized so that Q6K_WG_PER_CU
// workgroups fit in the 160 KiB of LDS of a CU.
template <int LAYOUT>
struct RingSize {
  static constexpr int fit = 160 * 1024 / (Q6K_WG_PER_CU * SlotSize<LAYOUT>::value);
  static constexpr int value = fit > 6 ? 6 : fit;
  static_assert(value >= 3, "the ring needs at least 3 slots");
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)(p);
}

// Direct-to-LDS load of 16 bytes per lane through a buffer resource: the wave's LDS base goes in
// M0, the lane offset is a constant register and the chunk offset a scalar, so no per-load
// address arithmetic runs on the vector ALU.  Lanes past the resource's size read zeros.
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                       uint8_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds_wave_base), 16, voff, soff, 0, 0);
}

// Buffer resource over `bytes` bytes at p (raw, no stride; 32-bit range, checked on the host).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Buffer resources of one workgroup's operands: this wave's row tile (codes and scales) and, for
// waves 0 and 1, token tile `wave` (activations and da).  (Spreading the activation loads over
// all four waves, half a tile each, measured 2-3 % slower.)
struct GemmSrc {
  __amdgpu_buffer_rsrc_t a, d, b, s;
};

// Issue this wave's loads of chunk c (already clamped to a valid chunk) into `slot`.
template <int LAYOUT>
__device__ __forceinline__ void issue_chunk(uint8_t* slot, const GemmSrc& src, uint32_t c, int wave,
                                            int lane) {
  const uint32_t l16 = lane * 16;
  if (LAYOUT == Q6K_LAYOUT_EXPANDED)
    bdma16(src.b, l16, c * 1024, slot + kSlotB + wave * 1024);
  else if (lane < 48)
    bdma16(src.b, l16, c * 768, slot + kSlotRawB + wave * 768);
  if (lane < 16) bdma16(src.s, l16, c * 256, slot + kSlotS + wave * 256);
  if (wave < kWgTokTiles) {
    bdma16(src.a, l16, c * 1024, slot + kSlotA + wave * 1024);
    if (lane < 8) bdma16(src.d, l16, c * 128, slot + kSlotD + wave * 128);
  }
}

// s_waitcnt vmcnt(chunks * loads of this wave per chunk)
template <int CHUNKS>
__device__ __forceinline__ void wait_chunks(bool loads_a) {
  if (loads_a)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CHUNKS * 4) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CHUNKS * 2) : "memory");
}

// Per-lane LDS addresses of a workgroup's operands in ring slot 0; slot j adds j * slot size,
// which the LDS instructions take as an immediate offset (no per-chunk address arithmetic).
struct GemmLanes {
  uint32_t aa, dd, bb, ss;         // reads: A fragment, da, B fragments, scales
  uint32_t raw, bdst;              // layout 0 expand: packed codes in, B fragments out (row
                                   // tile `wave`)
};

// Layout 0: this lane's packed codes of row tile `wave` in the slot at byte offset OFF.  No wait:
// the caller waits (with the registers as operands) after other work.
struct RawCodes {
  uint32_t x, y, z;
};
template <int OFF>
__device__ __forceinline__ void expand_read(const GemmLanes& L, RawCodes& r) {
  asm volatile(
      "ds_read_b32 %0, %3 offset:%4\n\t"
      "ds_read_b32 %1, %3 offset:%5\n\t"
      "ds_read_b32 %2, %3 offset:%6"
      : "=&v"(r.x), "=&v"(r.y), "=&v"(r.z)
      : "v"(L.raw), "n"(OFF), "n"(OFF + 4), "n"(OFF + 8)
      : "memory");
}

// Layout 0: write row tile `wave` of the slot at OFF as B fragments of 4 x the centered int8
// codes.  (Its (d*sc0, d*sc1) pairs arrive by direct-to-LDS load, as on layout 1.)
template <int OFF>
__device__ __forceinline__ void expand_write(const GemmLanes& L, const RawCodes& r) {
  v4u b;
  b.x = center4x4(r.x);
  b.y = center4x4(r.y);
  b.z = center4x4(r.z);
  b.w = fourth4x4(r.x, r.y, r.z);
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(L.bdst), "v"(b), "n"(OFF) : "memory");
}

// The MFMAs of one 32x32 output tile for one chunk (halves 0 and 1).
__device__ __forceinline__ void tile_mfma(v16i& lo_d, v16i& hi_d, const v16i& bias, long alo,
                                          long ahi, v4u b) {
  const long blo = (long)(((uint64_t)b.y << 32) | b.x);
  const long bhi = (long)(((uint64_t)b.w << 32) | b.z);
  lo_d = __builtin_amdgcn_mfma_i32_32x32x16_i8(alo, blo, bias, 0, 0, 0);
  hi_d = __builtin_amdgcn_mfma_i32_32x32x16_i8(ahi, bhi, bias, 0, 0, 0);
}

// Rescale of one 32x32 output tile for one chunk, or (SUBDOTS) the store of its sub-block dots.
// s = (dsc0, dsc1, nb0, nb1).  SHIFT: log2 of the factor the staged B operand carries (2 for
// layout 0, whose fragments hold 4 x the centered codes; its dots come out as 4 D and are
// exported as D).
template <bool SUBDOTS, int SHIFT>
__device__ __forceinline__ void tile_rescale(float (&acc)[16], const v16i& lo_d, const v16i& hi_d,
                                             v4f s, const float (&dav)[16], int lane, uint32_t c,
                                             int64_t T, int64_t R, int64_t nchunk,
                                             const DotsOut& dots) {
  if (SUBDOTS) {
    const int p = lane & 31, g = lane >> 5;
    const DotsRun d = dots_run<true>(dots, T * kTile + 4 * g, R * kTile + p, 2 * nchunk, 2 * c);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int32_t* o = dots_slot(dots, d, r);
      if (o) {
        o[0] = (lo_d[r] - kBiasI) >> SHIFT;
        o[1] = (hi_d[r] - kBiasI) >> SHIFT;
      }
    }
  } else {
    // four phases of 16 independent fma: no VALU instruction depends on the one before it
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = __builtin_fmaf(__int_as_float(lo_d[r]), s.x, s.z);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(t[r], dav[r], acc[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = __builtin_fmaf(__int_as_float(hi_d[r]), s.y, s.w);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(t[r], dav[r], acc[r]);
  }
}

// An empty statement that reads and rewrites one tile's 16 accumulators: the rescale that
// produces them stays ahead of it (the compiler would otherwise sink whole steps' rescales to the
// end of the unrolled loop and keep every step's MFMA results live at once).
__device__ __forceinline__ void pin_acc(float (&a)[16]) {
  asm volatile(""
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                 "+v"(a[6]), "+v"(a[7]), "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]),
                 "+v"(a[12]), "+v"(a[13]), "+v"(a[14]), "+v"(a[15]));
}

// What one wave of gemm_kernel carries from chunk to chunk.
struct GemmCtx {
  uint8_t* smem;
  GemmSrc src;
  GemmLanes lanes;
  uint32_t c1;  // the piece's chunk end
  int64_t nchunk, T, R0;
  DotsOut dots;
  int wave, lane, tt, rp;
  bool loads_a;
};

// This wave's MFMA operands of one chunk: its token tile's A fragment and the B fragments of its
// two row tiles, read from LDS one step ahead of their MFMAs.
struct GemmFrags {
  v4u a, b0, b1;
};

template <int OFF>
__device__ __forceinline__ void read_frags(const GemmLanes& L, GemmFrags& f) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7"
      : "=&v"(f.a), "=&v"(f.b0), "=&v"(f.b1)
      : "v"(L.aa), "v"(L.bb), "n"(OFF), "n"(OFF), "n"(OFF + 1024)
      : "memory");
}

// Step c (chunk c in ring slot J; chunk c0 + i lives in slot i % KRING), as described above.
// Every slot offset is a compile-time constant.  On entry chunk c is complete in LDS for every
// wave and its fragments are on their way into f; on exit the same holds for chunk c + 1.
template <int LAYOUT, bool SUBDOTS, int KRING, int J>
__device__ __forceinline__ void gemm_step(const GemmCtx& k, uint32_t c, float (&acc)[2][16],
                                          v16i& bias, GemmFrags& f) {
  constexpr int kSlot = SlotSize<LAYOUT>::value;
  constexpr int kCur = J * kSlot;
  constexpr int kNext = ((J + 1) % KRING) * kSlot;
  constexpr int kIssue = ((J + KRING - 1) % KRING) * kSlot;
  constexpr bool kPacked = LAYOUT == Q6K_LAYOUT_PACKED;
  // keep the steps apart: the scheduler would otherwise sink one step's rescale below the next
  // step's reads and lengthen every live range
  __builtin_amdgcn_sched_barrier(0);
  // the MFMA bias stays in its 16 VGPRs (instead of being rebuilt from scalars every step)
  asm volatile("" : "+v"(bias));
  // 1. the fragments of chunk c have landed; read its da and scale pairs (they land behind the
  // MFMAs)
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.a), "+v"(f.b0), "+v"(f.b1)::"memory");
  v4f d0, d1, d2, d3;
  v2f t0, t1;
  asm volatile(
      "ds_read_b64 %0, %6 offset:%8\n\t"
      "ds_read_b128 %2, %7 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%9\n\t"
      "ds_read_b128 %4, %7 offset:%10\n\t"
      "ds_read_b128 %5, %7 offset:%11\n\t"
      "ds_read_b64 %1, %6 offset:%12"
      : "=&v"(t0), "=&v"(t1), "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(k.lanes.ss), "v"(k.lanes.dd), "n"(kCur), "n"(kCur + 16), "n"(kCur + 32),
        "n"(kCur + 48), "n"(kCur + 256)
      : "memory");
  // (the reads stay ahead of the MFMAs, so their registers are never the fragments' registers,
  // which an MFMA may still be reading when a read lands)
  __builtin_amdgcn_sched_barrier(0);
  // 2. the MFMAs of both tiles
  const long alo = (long)(((uint64_t)f.a.y << 32) | f.a.x);
  const long ahi = (long)(((uint64_t)f.a.w << 32) | f.a.z);
  v16i lo0, hi0, lo1, hi1;
  tile_mfma(lo0, hi0, bias, alo, ahi, f.b0);
  tile_mfma(lo1, hi1, bias, alo, ahi, f.b1);
  // 3. chunk c+KRING-1 into chunk c-1's slot: every wave has passed a meeting since its last
  // read of that slot
  const uint32_t ci = c + KRING - 1;
  issue_chunk<LAYOUT>(k.smem + kIssue, k.src, ci < k.c1 ? ci : k.c1 - 1, k.wave, k.lane);
  // 4. this wave's loads of chunk c+1 have landed
  wait_chunks<KRING - 2>(k.loads_a);
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t0), "+v"(t1), "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3)::"memory");
  // (d*sc0, d*sc1) and their bias products (exact, see above)
  const v4f s0 = v4f{t0.x, t0.y, -kBiasF * t0.x, -kBiasF * t0.y};
  const v4f s1 = v4f{t1.x, t1.y, -kBiasF * t1.x, -kBiasF * t1.y};
  const float dav[16] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w,
                         d2.x, d2.y, d2.z, d2.w, d3.x, d3.y, d3.z, d3.w};
  // 5. layout 0: the LDS reads of this wave's packed codes of chunk c+1, landing behind tile 0's
  // rescale; then their expand into the slot
  RawCodes raw;
  if (kPacked) expand_read<kNext>(k.lanes, raw);
  constexpr int kShift = kPacked ? 2 : 0;
  tile_rescale<SUBDOTS, kShift>(acc[0], lo0, hi0, s0, dav, k.lane, c, k.T, k.R0 + 2 * k.rp,
                                k.nchunk, k.dots);
  if (!SUBDOTS) pin_acc(acc[0]);
  if (kPacked) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z));
    expand_write<kNext>(k.lanes, raw);
  }
  // 6. chunk c+1 complete in LDS for every wave (loads landed, layout 0's expand written)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // 7. its fragments, landing behind tile 1's rescale
  read_frags<kNext>(k.lanes, f);
  __builtin_amdgcn_sched_barrier(0);  // the reads go out before any of tile 1's rescale
  tile_rescale<SUBDOTS, kShift>(acc[1], lo1, hi1, s1, dav, k.lane, c, k.T, k.R0 + 2 * k.rp + 1,
                                k.nchunk, k.dots);
  if (!SUBDOTS) pin_acc(acc[1]);
}

// Chunks cb .. cb+KRING-1 (slots 0 .. KRING-1), stopping at the piece's end (a piece has a
// multiple of 8 chunks, so a ring of 4 never stops early).
template <int LAYOUT, bool SUBDOTS, int KRING, int J>
struct GemmSteps {
  __device__ __forceinline__ static void run(const GemmCtx& k, uint32_t cb, float (&acc)[2][16],
                                             v16i& bias, GemmFrags& f) {
    if (8 % KRING != 0 && cb + J >= k.c1) return;
    gemm_step<LAYOUT, SUBDOTS, KRING, J>(k, cb + J, acc, bias, f);
    GemmSteps<LAYOUT, SUBDOTS, KRING, J + 1>::run(k, cb, acc, bias, f);
  }
};
template <int LAYOUT, bool SUBDOTS, int KRING>
struct GemmSteps<LAYOUT, SUBDOTS, KRING, KRING> {
  __device__ __forceinline__ static void run(const GemmCtx&, uint32_t, float (&)[2][16], v16i&,
                                             GemmFrags&) {}
};

template <int LAYOUT, bool SUBDOTS>
__global__ __launch_bounds__(256, Q6K_WG_PER_CU) void gemm_kernel(const uint8_t* __restrict__ xq,
                                                      const float* __restrict__ da,
                                                      const uint8_t* __restrict__ wcodes,
                                                      const uint8_t* __restrict__ wscales,
                                                      int64_t n, int64_t m, int64_t nchunk,
                                                      float* __restrict__ y, int64_t ldy,
                                                      float* __restrict__ ws, DotsOut dots,
                                                      uint32_t gx, uint32_t gy, uint32_t n_full,
                                                      uint32_t pieces) {
  constexpr int kSlot = SlotSize<LAYOUT>::value;
  constexpr int kRing = RingSize<LAYOUT>::value;
  constexpr bool kPacked = LAYOUT == Q6K_LAYOUT_PACKED;
  static_assert(Q6K_WG_PER_CU * kRing * kSlot <= 160 * 1024, "LDS budget");
  static_assert(kRing * kSlot + 1024 < 65536, "slot offsets fit the LDS immediate offset");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kSlot];
  const WgStamp stamp = wg_stamp();
  GemmCtx k;
  k.smem = smem;
  k.lane = threadIdx.x & 63;
  k.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  k.loads_a = k.wave < kWgTokTiles;
  k.tt = k.wave & 1;                                    // token tile of this wave in the workgroup
  k.rp = k.wave >> 1;                                   // row-tile pair of this wave
  const TileWork tw = tile_work<Q6K_GEMM01_XCD_ORDER != 0>(blockIdx.x, gx, gy, n_full, pieces,
                                                           nchunk / 8, ws);
  const uint32_t c0 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * tw.s0));  // chunks [c0, c1)
  k.c1 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * tw.s1));
  k.nchunk = nchunk;
  k.T = (int64_t)tw.bx * kWgTokTiles + k.tt;
  k.R0 = (int64_t)tw.by * 4;                            // the workgroup's first row tile
  k.dots = dots;
  const int lane = k.lane, wave = k.wave;
  const int64_t Ta = (int64_t)tw.bx * kWgTokTiles + (k.loads_a ? wave : 0);

  k.src.a = make_rsrc(xq + Ta * nchunk * 1024, nchunk * 1024);
  k.src.d = make_rsrc(reinterpret_cast<const uint8_t*>(da) + Ta * nchunk * 128, nchunk * 128);
  if (LAYOUT == Q6K_LAYOUT_EXPANDED) {
    k.src.b = make_rsrc(wcodes + (k.R0 + wave) * nchunk * 1024, nchunk * 1024);
    k.src.s = make_rsrc(wscales + (k.R0 + wave) * nchunk * 256, nchunk * 256);
  } else {
    k.src.b = make_rsrc(wcodes + (k.R0 + wave) * nchunk * 768, nchunk * 768);
    k.src.s = make_rsrc(wscales + (k.R0 + wave) * nchunk * 256, nchunk * 256);
  }
  const int p = lane & 31, g = lane >> 5;
  k.lanes.aa = lds_addr(smem + kSlotA + k.tt * 1024 + lane * 16);
  k.lanes.dd = lds_addr(smem + kSlotD + k.tt * 128 + g * 64);
  k.lanes.bb = lds_addr(smem + kSlotB + k.rp * 2048 + lane * 16);
  k.lanes.ss = lds_addr(smem + kSlotS + k.rp * 512 + p * 8);
  k.lanes.raw = lds_addr(smem + kSlotRawB + wave * 768 + lane * 12);
  k.lanes.bdst = lds_addr(smem + kSlotB + wave * 1024 + lane * 16);

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasI;
  float acc[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.0f;

  // Prologue: chunks c0 .. c0+kRing-2 in flight in slots 0 .. kRing-2; this wave's share of chunk
  // c0 landed (and, layout 0, expanded), the meeting makes it every wave's, then chunk c0's
  // fragments are read.
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j)
    issue_chunk<LAYOUT>(smem + j * kSlot, k.src, c0 + j < k.c1 ? c0 + j : k.c1 - 1, wave, lane);
  wait_chunks<kRing - 2>(k.loads_a);
  if (kPacked) {
    RawCodes raw;
    expand_read<0>(k.lanes, raw);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z));
    expand_write<0>(k.lanes, raw);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  GemmFrags f;
  read_frags<0>(k.lanes, f);

  for (uint32_t cb = c0; cb < k.c1; cb += kRing)
    GemmSteps<LAYOUT, SUBDOTS, kRing, 0>::run(k, cb, acc, bias, f);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // drain the trailing loads

  if (SUBDOTS) return;
  // layout 0's accumulators hold 4 y (its B fragments are 4 x the centered codes)
  const float out_scale = kPacked ? 0.25f : 1.0f;
  const int64_t T = k.T;
  const OutDst o = out_dst(tw, y, ldy, ws);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t mcol = (k.R0 + 2 * k.rp + u) * kTile + p;
    if (mcol >= m) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t tok = T * kTile + 8 * (r >> 2) + 4 * g + (r & 3);
      // a lane's 16 values are one row of 16 tokens; an instruction covers 32 consecutive rows
      // of 2 tokens
      if (tok < n) o.p[(tok - o.tok0) * o.ld + (mcol - o.row0)] = acc[u][r] * out_scale;
    }
  }
  wg_record(stamp, tw);
}

// ---------------------------------------------------------------------------------------------
// GEMM on layout 2 (folded scales).  q6_K has one f16 d per 256-element super-block and one int8
// sc per 16 elements, so a 32-k chunk contributes da * d * E to y with the exact integer
//     E = sum_k xq[k] * v[k],   v = sc[k/16] * (q[k] - 32)  in [-4064, 4096].
// v does not fit an int8 MFMA operand; it is stored as two int8 digit planes v = 64*hi + lo
// (lo in [-32, 31], hi in [-63, 64]).  Per chunk and 32x32 tile: two v_mfma_i32_32x32x32_i8 (low
// and high digits, full 32-k chunk each) whose int32 accumulators start from float bit patterns,
// so that each result reads exactly as a float without a conversion (|E_lo| <= 32*127*32 and
// |E_hi| <= 32*127*64 are both below 2^22, so the sum never leaves the starting binade):
//     low digits from 1.5*2^23 (ulp 1):   F_lo = 1.5*2^23 + E_lo
//     high digits from 1.5*2^29 (ulp 64): F_hi = 1.5*2^29 + 64*E_hi
// Then
//     u  = F_hi - (1.5*2^29 + 1.5*2^23)   = 64*E_hi - 1.5*2^23   (a multiple of 64 below 2^25:
//                                                               exact)
//     e  = u + F_lo                       = E                    (|E| < 2^24: exact)
//     sb = fma(e, da, sb)
// three VALU operations per output per chunk, all exact up to the single rounding of the last,
// and all three short (two-operand) encodings with register operands only, which issue faster
// than a multiply-add with a literal 64.  After the 8th chunk of a super-block,
// acc = fma(sb, d, acc) and sb restarts at 0.
//
// Orientation: the weights are the MFMA's A operand and the activations its B operand, so lane l,
// register r of a tile holds weight row 8*(r/4) + 4*(l/32) + r%4 and token l%32: each lane needs a
// single da per token tile and chunk.  Workgroup = 4 waves = 64 tokens (token tiles 2*bx, 2*bx+1)
// x 128 weight rows (row tiles 4*by .. 4*by+3); wave w computes row tile 4*by + w against both
// token tiles.
// ---------------------------------------------------------------------------------------------
constexpr int kBiasHiI = 0x4E400000;       // bit pattern of 1.5 * 2^29 (ulp 64)
constexpr float kFoldK = -65.0f * kBiasF;  // -(1.5*2^29 + 1.5*2^23), exact: 195 * 2^22


// e = 64*E_hi + E_lo from the two biased digit products (exact, see above), in two phases of 16
// independent operations (no VALU instruction depends on the one before it).
// kk holds kFoldK in a register (VOP2 adds take no literal), set once per kernel.
__device__ __forceinline__ void fold_digits(float (&e)[16], const v16i& fh, const v16i& fl,
                                            float kk) {
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __int_as_float(fh[r]) + kk;
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] += __int_as_float(fl[r]);
}

// ---------------------------------------------------------------------------------------------
// folded_kernel<DOTS>: how the operands reach the MFMAs, with few synchronisations per chunk:
//   - the digit planes of a wave's row tile are private to that wave, so each wave loads them
//     straight into registers (a 4-entry register ring, 3 chunks ahead) instead of through LDS;
//   - only the activations and their da, shared by the 4 waves, go through LDS: one ring slot
//     holds a whole super-block (2 token tiles x 8 chunks x 1 KiB + 2 x 1 KiB of da), the ring
//     has 4 slots and runs 3 super-blocks ahead, so the workgroup meets at a barrier once per
//     super-block instead of once per chunk;
//   - per chunk, tile 0's MFMAs and rescale, then tile 1's: one tile's MFMA results are live at a
//     time (the other wave on the SIMD issues VALU work while this one waits for its MFMAs);
//   - 2 workgroups per CU (up to 256 VGPRs per wave).
// Work split: tile_work (rounds of one tile per workgroup slot, a partial last round split along
// k into pieces that add into y).
// ---------------------------------------------------------------------------------------------
// Waves per workgroup.  The kernel is written for 4 (64 tokens x 128 rows, 2 workgroups per CU)
// or 8 (128 x 128, 1 per CU, two waves reading each row tile's planes); 8 measured 1 % faster on
// ffn_down and 2-4 % slower on attn_v N=512, so 4 it is.
constexpr int kFWaves = 4;
static_assert(kFWaves == 4 || kFWaves == 8, "4 or 8 waves");
constexpr int kFoldedWgPerCu = 8 / kFWaves;
constexpr int kFTok = kFWaves / 2;         // token tiles per workgroup (2 per wave row)
constexpr int kFSlotDa = kFTok * 8192;     // after kFTok tiles x 8 chunks x 1 KiB of activations
constexpr int kFSlot = kFTok * 9216;
constexpr int kFRing = 4;
constexpr int kFAhead = 3;  // super-blocks whose activations are in flight
static_assert(kFoldedWgPerCu * kFRing * kFSlot <= 160 * 1024, "LDS budget");
static_assert(kFAhead < kFRing, "ring slot reuse");

struct FoldCtx {
  __amdgpu_buffer_rsrc_t a, da, b, w;  // both token tiles, their da, row tile planes, row tile d
  uint8_t* smem;
  uint32_t l16, dvoff;      // lane * 16; byte offset of this lane's d values in a super-block
  int wave, lane;
  int64_t nchunk, c_begin;  // this piece's first chunk
  uint32_t c_end, s_end;    // and its chunk and super-block ends
  int64_t n, m, tok0, row0;
  DotsOut dots;
};

struct FoldState {
  float acc[2][16], sb[2][16];
  v4i x0, x1;        // activations of the current chunk, token tiles 0 and 1
  float da0, da1;    // their da (this lane's token)
  v4i blo[4], bhi[4];  // digit planes of chunk c in entry c % 4
  float d[16];       // d of this lane's 16 rows, for the super-block being finished
  float kk;          // kFoldK, kept in a register
};


// Digit planes of chunk c (clamped to the piece's last chunk, so every load stays in range).
__device__ __forceinline__ void fold_load_planes(const FoldCtx& k, int64_t c, v4i& lo, v4i& hi) {
  const uint32_t cc = min((uint32_t)c, k.c_end - 1);
  lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(k.b, k.l16, cc * 2048, 0));
  hi = __builtin_bit_cast(v4i,
                          __builtin_amdgcn_raw_buffer_load_b128(k.b, k.l16 + 1024, cc * 2048, 0));
}

// d of super-block s for this lane's rows 8q + 4g + i (q, i = 0..3).
// The lane offset passes through an empty statement that reads the accumulators just updated
// with the previous d, so the loads cannot be hoisted above that update and the new values can
// take the old ones' registers (no copies at the loop's back edge).
__device__ __forceinline__ void fold_load_d(const FoldCtx& k, int64_t s, float (&d)[16],
                                            const float (&a0)[16], const float (&a1)[16]) {
  const uint32_t so = (uint32_t)s * 128;
  uint32_t voff = k.dvoff;
  asm volatile(""
               : "+v"(voff)
               : "v"(a0[0]), "v"(a0[1]), "v"(a0[2]), "v"(a0[3]), "v"(a0[4]), "v"(a0[5]),
                 "v"(a0[6]), "v"(a0[7]), "v"(a0[8]), "v"(a0[9]), "v"(a0[10]), "v"(a0[11]),
                 "v"(a0[12]), "v"(a0[13]), "v"(a0[14]), "v"(a0[15]), "v"(a1[0]), "v"(a1[1]),
                 "v"(a1[2]), "v"(a1[3]), "v"(a1[4]), "v"(a1[5]), "v"(a1[6]), "v"(a1[7]),
                 "v"(a1[8]), "v"(a1[9]), "v"(a1[10]), "v"(a1[11]), "v"(a1[12]), "v"(a1[13]),
                 "v"(a1[14]), "v"(a1[15]));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4f v =
        __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(k.w, voff + 32 * q, so, 0));
    d[4 * q] = v.x;
    d[4 * q + 1] = v.y;
    d[4 * q + 2] = v.z;
    d[4 * q + 3] = v.w;
  }
}

// This wave's share of super-block s's activations and da, direct to LDS slot s % 4: four 1 KiB
// chunk tiles of token tile wave/2 and the da of token tile wave % kFTok (the other waves write
// the same da bytes again).  Nothing is loaded past the piece's last super-block.
__device__ __forceinline__ void fold_dma(const FoldCtx& k, int64_t s) {
  if ((uint32_t)s >= k.s_end) return;
  uint8_t* slot = k.smem + (s % kFRing) * kFSlot;
  const int u = k.wave >> 1, j0 = 4 * (k.wave & 1), ud = k.wave % kFTok;
  const uint32_t abase = (uint32_t)((u * k.nchunk + 8 * s + j0) * 1024);
#pragma unroll
  for (int i = 0; i < 4; ++i) bdma16(k.a, k.l16, abase + i * 1024, slot + u * 8192 + (j0 + i) * 1024);
  bdma16(k.da, k.l16, (uint32_t)((ud * k.nchunk + 8 * s) * 128), slot + kFSlotDa + ud * 1024);
}

// LDS reads of one chunk's activations and da (immediate offsets within the slot).  The previous
// values are inputs, so the new ones land in other registers than those the MFMAs just issued
// are reading.
template <int OFFX, int OFFD>
__device__ __forceinline__ void fold_read(uint32_t xb, uint32_t dab, FoldState& st) {
  v4i x0, x1;
  float d0, d1;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%6\n\t"
      "ds_read_b128 %1, %4 offset:%7\n\t"
      "ds_read_b32 %2, %5 offset:%8\n\t"
      "ds_read_b32 %3, %5 offset:%9"
      : "=&v"(x0), "=&v"(x1), "=&v"(d0), "=&v"(d1)
      : "v"(xb), "v"(dab), "n"(OFFX), "n"(OFFX + 8192), "n"(OFFD), "n"(OFFD + 1024),
        "v"(st.x0), "v"(st.x1)
      : "memory");
  st.x0 = x0;
  st.x1 = x1;
  st.da0 = d0;
  st.da1 = d1;
}

// sb (+)= e * da, or the store of e for the test export.
template <bool DOTS, bool FIRST>
__device__ __forceinline__ void fold_rescale(float (&sb)[16], const float (&e)[16], float dav,
                                           const FoldCtx& k, int64_t c, int u) {
  if (DOTS) {
    const int g = k.lane >> 5;
    const DotsRun d = dots_run<false>(k.dots, k.tok0 + kTile * u, k.row0 + 4 * g, k.nchunk, c);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int32_t* o = dots_slot(k.dots, d, r);
      if (o) *o = (int32_t)e[r];
    }
  } else if (FIRST) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sb[r] = e[r] * dav;
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) sb[r] = __builtin_fmaf(e[r], dav, sb[r]);
  }
}

// Chunk c = 8s + J.  xb/dab: this lane's LDS addresses in super-block s's slot; xn/dn: in slot
// s + 1 (read by the last step).  Tile 0's MFMAs, its rescale, then tile 1's MFMAs and rescale:
// one tile's MFMA results are live at a time, and the other wave on the SIMD keeps the VALU busy
// while this one waits for its MFMAs.
template <bool DOTS, int J>
__device__ __forceinline__ void fold_step(const FoldCtx& k, int64_t s, uint32_t xb, uint32_t dab,
                                        uint32_t xn, uint32_t dn, FoldState& st,
                                        const v16i& bias_lo, const v16i& bias_hi) {
  const int64_t c = 8 * s + J;
  asm volatile("" : "+v"(st.kk));
  if (J == 0) {
    // both tiles have finished super-block s - 1: apply its d, then fetch super-block s's
    if (!DOTS) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[u][r] = __builtin_fmaf(st.sb[u][r], st.d[r], st.acc[u][r]);
    }
    fold_load_d(k, s, st.d, st.acc[0], st.acc[1]);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(st.x0), "+v"(st.x1), "+v"(st.da0), "+v"(st.da1));
  const v4i lo = st.blo[J % 4], hi = st.bhi[J % 4];
  const v4i x1 = st.x1;
  const float da0 = st.da0, da1 = st.da1;
  v16i fh = __builtin_amdgcn_mfma_i32_32x32x32_i8(hi, st.x0, bias_hi, 0, 0, 0);
  v16i fl = __builtin_amdgcn_mfma_i32_32x32x32_i8(lo, st.x0, bias_lo, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  fold_load_planes(k, c + 3, st.blo[(J + 3) % 4], st.bhi[(J + 3) % 4]);
  if (J == 0) fold_dma(k, s + kFAhead);
  if (J == 7) {
    // super-block s + 1's slot: this wave's share of it has landed, and after the barrier every
    // wave's has.  vmcnt(N) waits until at most the N most recently issued vector memory loads
    // of this wave are outstanding (loads complete in issue order for this count), so it
    // suffices that at least 8 loads were issued after the last load of super-block s + 1's
    // slot and before this wait.  That holds whatever order the compiler picks inside a step:
    // the slot's loads were issued in step 0 of super-block s - 2, and this statement and the
    // same one of super-blocks s - 2 and s - 1 are volatile and clobber memory, so no load can
    // cross them; the 16 digit-plane loads of super-block s - 1 (two per step, every step,
    // clamped to the piece but never skipped) therefore sit between the slot's loads and this
    // wait.  (The slots of a piece's first three super-blocks were loaded in the prologue, which
    // waits for all of its loads.)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    fold_read<0, 0>(xn, dn, st);
  } else {
    fold_read<(J + 1) * 1024, (J + 1) * 128>(xb, dab, st);
  }
  asm volatile("" : "+v"(fh), "+v"(fl));
  {
    float e[16];
    fold_digits(e, fh, fl, st.kk);
    fold_rescale<DOTS, J == 0>(st.sb[0], e, da0, k, c, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  fh = __builtin_amdgcn_mfma_i32_32x32x32_i8(hi, x1, bias_hi, 0, 0, 0);
  fl = __builtin_amdgcn_mfma_i32_32x32x32_i8(lo, x1, bias_lo, 0, 0, 0);
  asm volatile("" : "+v"(fh), "+v"(fl));
  {
    float e[16];
    fold_digits(e, fh, fl, st.kk);
    fold_rescale<DOTS, J == 0>(st.sb[1], e, da1, k, c, 1);
  }
}

template <bool DOTS>
__global__ __launch_bounds__(64 * kFWaves, kFoldedWgPerCu) void folded_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ da,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wd, int64_t n, int64_t m,
    int64_t nchunk, float* __restrict__ y, int64_t ldy, int vec_store, float* __restrict__ ws,
    DotsOut dots, uint32_t gx, uint32_t gy, uint32_t n_full, uint32_t pieces) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kFRing * kFSlot];
  const WgStamp stamp = wg_stamp();
  const TileWork tw = tile_work<true>(blockIdx.x, gx, gy, n_full, pieces, nchunk / 8, ws);
  const bool split = tw.split;
  const uint32_t bx = tw.bx, by = tw.by;
  const int64_t nsb = nchunk / 8;
  const int64_t s0 = tw.s0, s1 = tw.s1;

  FoldCtx k;
  k.smem = smem;
  k.lane = threadIdx.x & 63;
  k.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = k.lane & 31, g = k.lane >> 5;
  const int rw = k.wave & 3, tp = k.wave >> 2;  // the wave's row tile and token-tile pair
  const int64_t T0 = (int64_t)bx * kFTok, R = (int64_t)by * 4 + rw;
  k.a = make_rsrc(xq + T0 * nchunk * 1024, kFTok * nchunk * 1024);
  k.da = make_rsrc(reinterpret_cast<const uint8_t*>(da) + T0 * nchunk * 128,
                   kFTok * nchunk * 128);
  k.b = make_rsrc(wcodes + R * nchunk * 2048, nchunk * 2048);
  k.w = make_rsrc(wd + R * nsb * 128, nsb * 128);
  k.l16 = k.lane * 16;
  k.dvoff = 16 * g;
  k.nchunk = nchunk;
  k.c_begin = 8 * s0;
  k.c_end = (uint32_t)(8 * s1);
  k.s_end = (uint32_t)s1;
  k.n = n;
  k.m = m;
  k.tok0 = (T0 + 2 * tp) * kTile + p;
  k.row0 = R * kTile;
  k.dots = dots;
  // this lane's LDS addresses in slot 0: its 16 activation bytes, its token's da
  // (da of token p sits at position 16*((p/4)%2) + 4*(p/8) + p%4 of a chunk's 32 floats)
  const uint32_t xb0 = lds_addr(smem) + 2 * tp * 8192 + k.l16;
  const uint32_t db0 = lds_addr(smem) + kFSlotDa + 2 * tp * 1024 +
                       4 * (16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3));

  v16i bias_lo, bias_hi;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    bias_lo[r] = kBiasI;
    bias_hi[r] = kBiasHiI;
  }
  FoldState st;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[u][r] = st.sb[u][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) st.d[r] = 0.0f;
  st.kk = kFoldK;

  // prologue: super-blocks s0 .. s0+2 of activations, chunks c0 .. c0+2 of digit planes; wait
  // for all of them, meet, read chunk c0's operands
#pragma unroll
  for (int i = 0; i < kFAhead; ++i) fold_dma(k, s0 + i);
  fold_load_planes(k, 8 * s0 + 0, st.blo[0], st.bhi[0]);
  fold_load_planes(k, 8 * s0 + 1, st.blo[1], st.bhi[1]);
  fold_load_planes(k, 8 * s0 + 2, st.blo[2], st.bhi[2]);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  st.x0 = st.x1 = v4i{0, 0, 0, 0};
  const uint32_t slot0 = (uint32_t)(s0 % kFRing) * kFSlot;
  fold_read<0, 0>(xb0 + slot0, db0 + slot0, st);

  const uint32_t sb0 = __builtin_amdgcn_readfirstlane((uint32_t)s0),
                 sb1 = __builtin_amdgcn_readfirstlane((uint32_t)s1);
  for (uint32_t s = sb0; s < sb1; ++s) {
    const uint32_t cur = (uint32_t)(s % kFRing) * kFSlot;
    const uint32_t nxt = (uint32_t)((s + 1) % kFRing) * kFSlot;
    const uint32_t xb = xb0 + cur, dab = db0 + cur, xn = xb0 + nxt, dn = db0 + nxt;
    fold_step<DOTS, 0>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 1>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 2>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 3>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 4>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 5>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 6>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
    fold_step<DOTS, 7>(k, s, xb, dab, xn, dn, st, bias_lo, bias_hi);
  }
  // the last super-block's d
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // drain the trailing loads
  if (DOTS) return;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[u][r] = __builtin_fmaf(st.sb[u][r], st.d[r], st.acc[u][r]);

  // The workgroup's (32 kFTok)-token x 128-row output tile goes through LDS (the ring is free once
  // every wave has passed the first barrier), so that each store instruction below
  // covers consecutive rows of one token instead of 64 scattered 4-row pieces.
  constexpr int kOutLd = 132;  // floats per token in LDS: 128 rows + 4 of padding
  static_assert(kTile * kFTok * kOutLd * 4 <= kFRing * kFSlot, "output tile fits the ring");
  float* out = reinterpret_cast<float*>(smem);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(out + (kTile * (2 * tp + u) + p) * kOutLd + kTile * rw + 8 * q + 4 * g) =
          make_float4(st.acc[u][4 * q], st.acc[u][4 * q + 1], st.acc[u][4 * q + 2],
                      st.acc[u][4 * q + 3]);
  __syncthreads();
  const int64_t tok_base = T0 * kTile, row_base = (int64_t)by * kWgRow;
  // a piece's slab is 16-byte aligned with rows of 128 floats: always the vector path
  const OutDst o = out_dst(tw, y, ldy, ws);
  if (split || vec_store) {
    // two tokens per instruction, 4 rows per lane: 2 x 512 contiguous bytes
    const int half = k.lane >> 5, r4 = 4 * (k.lane & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 16 * k.wave + 2 * i + half;
      const int64_t tok = tok_base + t, row = row_base + r4;
      if (tok >= n || row >= m) continue;
      const float4 v = *reinterpret_cast<const float4*>(out + t * kOutLd + r4);
      float* dst = o.p + (tok - o.tok0) * o.ld + (row - o.row0);
      if (row + 3 < m) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        dst[0] = v.x;
        if (row + 1 < m) dst[1] = v.y;
        if (row + 2 < m) dst[2] = v.z;
      }
    }
  } else {
    // one token per instruction, one row per lane: 256 contiguous bytes
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int t = 16 * k.wave + i;
      const int64_t tok = tok_base + t;
      if (tok >= n) break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t row = row_base + 64 * h + k.lane;
        if (row >= m) continue;
        y[tok * ldy + row] = out[t * kOutLd + 64 * h + k.lane];
      }
    }
  }
  wg_record(stamp, tw);
}


// =============================================================================================
// q4_K variant ("r18: Load-time B pre-expansion — staging becomes a bulk copy (W_exp's debut,
// REVERTED)"): 144-byte super-blocks of 256 weights, f16 d and dmin, eight 6-bit (sc, m) pairs,
// 4-bit codes; w = d*sc*q - dmin*m per 32-element chunk.  A chunk contributes
//     da * (d*sc) * D - da * (dmin*m) * S,   D = sum xq*q (exact int),   S = sum xq
// so the activations carry da and da*S (the pages' per-token d|ssum pair, "r38 — q6_K BT-style
// raw-byte mma kernel (LANDED)", sec. 2.2), and the weights are prepared at load time as the
// pages' EB plane (codes as int8 0..15, here in MFMA lane order) and SB plane ((d*sc, -dmin*m)
// f32 pairs per row and chunk).
// =============================================================================================
constexpr int kQ4Block = 144;

// Prepass with sums: the q6_K prepass plus das = da * S per (token, chunk), S the sum of the
// chunk's 32 codes (exact in int), rounded once to f32; stored in the tiled order of da.
__global__ __launch_bounds__(256) void q4k_act_sums_kernel(const uint8_t* __restrict__ xq,
                                                           const float* __restrict__ da,
                                                           int64_t ntile, int64_t nchunk,
                                                           float* __restrict__ das) {
  // one thread per (token tile, chunk, token): sums the token's two 16-byte lane slots
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= ntile * nchunk * 32) return;
  const int64_t tc = i / 32;
  const int p = (int)(i % 32);
  const uint8_t* blk = xq + tc * 64 * kFragBytes;
  int sum = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 v = reinterpret_cast<const uint4*>(blk)[p + 32 * h];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += (int8_t)((w[b] >> (8 * e)) & 255);
  }
  const int slot = 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
  das[tc * 32 + slot] = da[tc * 32 + slot] * (float)sum;
}

// Load-time planes.  Block = one row tile (32 rows) x one super-block; the 32 raw blocks are
// staged in LDS (16-byte rows), then thread (p, cc) decodes chunk cc (sub-block cc) of row 32R+p:
// its 32 codes into lane slots p and p+32 of the (R, c) 1 KiB block (the activation lane order),
// and (d*sc, -dmin*m) into the SB plane at [R][super-block][cc][p].
// Codes: byte 16 + 32g + l of a block holds element 64g + l (low nibble) and 64g + 32 + l (high
// nibble); for sub-block j < 4, sc = s[j] & 63, m = s[j+4] & 63, for j >= 4,
// sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4, m = (s[j+4] >> 4) | (s[j] >> 6) << 4, s the 12 bytes
// at offset 4 (the GGUF K-quant packing the pages follow).
__global__ __launch_bounds__(256) void q4k_expand_kernel(const uint8_t* __restrict__ raw,
                                                         int64_t m, int64_t nsb,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ sbp) {
  __shared__ __attribute__((aligned(16))) uint8_t blk[kTile * kQ4Block];
  const int64_t R = blockIdx.x, sb = blockIdx.y, nchunk = nsb * 8;
  for (int idx = threadIdx.x; idx < kTile * kQ4Block / 16; idx += 256) {
    const int j = idx / (kQ4Block / 16), w = idx % (kQ4Block / 16);
    const int64_t row = R * kTile + j;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < m) v = reinterpret_cast<const uint4*>(raw + (row * nsb + sb) * kQ4Block)[w];
    reinterpret_cast<uint4*>(blk + j * kQ4Block)[w] = v;
  }
  __syncthreads();
  const int p = threadIdx.x & 31, cc = threadIdx.x >> 5;
  const uint8_t* b = blk + p * kQ4Block;
  const int g = cc >> 1, hi = cc & 1;
  int q[32];
#pragma unroll
  for (int l = 0; l < 32; ++l) {
    const int byte = b[16 + 32 * g + l];
    q[l] = hi ? (byte >> 4) : (byte & 15);
  }
  const uint8_t* s = b + 4;
  int sc, mn;
  if (cc < 4) {
    sc = s[cc] & 63;
    mn = s[cc + 4] & 63;
  } else {
    sc = (s[cc + 4] & 15) | ((s[cc - 4] >> 6) << 4);
    mn = (s[cc + 4] >> 4) | ((s[cc] >> 6) << 4);
  }
  const float d = __half2float(__ushort_as_half((unsigned short)(b[0] | (b[1] << 8))));
  const float dmin = __half2float(__ushort_as_half((unsigned short)(b[2] | (b[3] << 8))));
  const int64_t c = sb * 8 + cc;
  uint4 s0, s1;  // lane p: k 0..7 and 16..23; lane p + 32: k 8..15 and 24..31
  s0.x = pack4(q[0], q[1], q[2], q[3]);
  s0.y = pack4(q[4], q[5], q[6], q[7]);
  s0.z = pack4(q[16], q[17], q[18], q[19]);
  s0.w = pack4(q[20], q[21], q[22], q[23]);
  s1.x = pack4(q[8], q[9], q[10], q[11]);
  s1.y = pack4(q[12], q[13], q[14], q[15]);
  s1.z = pack4(q[24], q[25], q[26], q[27]);
  s1.w = pack4(q[28], q[29], q[30], q[31]);
  uint4* dst = reinterpret_cast<uint4*>(codes + (R * nchunk + c) * 64 * kFragBytes);
  dst[p] = s0;
  dst[p + 32] = s1;
  float2 pr;
  pr.x = d * (float)sc;  // exact: an 11-bit significand times a 6-bit integer
  pr.y = -(dmin * (float)mn);
  if (R * kTile + p >= m) pr.x = pr.y = 0.0f;  // padding rows (their codes are zero too)
  reinterpret_cast<float2*>(sbp)[((R * nsb + sb) * 8 + cc) * 32 + p] = pr;
}

// GEMM.  Workgroup = 4 waves = 64 tokens (token tiles 2*bx, 2*bx+1) x 128 weight rows (row tiles
// 4*by .. 4*by+3); wave w computes token tile w%2 against row tiles 2*(w/2) and 2*(w/2)+1 (rows
// of the MFMA = tokens, columns = weight rows, so each lane owns one weight row and 16 tokens).
// Per chunk and tile one v_mfma_i32_32x32x32_i8 (the whole 32-element sub-block has one scale),
// started from the bit pattern of 1.5*2^23 (|D| <= 32*127*15 < 2^22), then
//     t   = fma(F, d*sc, -1.5*2^23*d*sc)     (= D*d*sc rounded once)
//     acc = fma(t, da, acc)
//     acc = fma(-dmin*m, da*S, acc)
// three VALU per output.  Staging: a 4-slot ring of direct-to-LDS buffer loads (activation tiles
// by waves 0 and 1, each wave its row tile's codes), and, once per super-block into a buffer of
// that super-block's parity, da and da*S of the token tiles and the SB pairs of the row tiles.
constexpr int kQ4SlotA = 0;       // 2 token tiles x 1 KiB
constexpr int kQ4SlotB = 2048;    // 4 row tiles x 1 KiB
constexpr int kQ4Slot = 6144;
constexpr int kQ4Ring = 4;
constexpr int kQ4SbDa = 0;        // per parity: 2 token tiles x 1 KiB of da
constexpr int kQ4SbDas = 2048;    //             2 token tiles x 1 KiB of da*S
constexpr int kQ4SbSb = 4096;     //             4 row tiles x 2 KiB of (d*sc, -dmin*m)
constexpr int kQ4SbBytes = 12288;
#ifndef Q4K_WG_PER_CU
#define Q4K_WG_PER_CU 3
#endif
static_assert(Q4K_WG_PER_CU * (kQ4Ring * kQ4Slot + 2 * kQ4SbBytes) <= 160 * 1024, "LDS budget");

struct Q4Src {
  __amdgpu_buffer_rsrc_t a, da, das, b, sb;
};

// Loads of chunk ci (ci % 8 == CI8) into `slot`; chunks past the end repeat the last one so each
// wave issues at least 1 load per chunk (2 for waves 0 and 1).  At a super-block's first chunk the
// per-super-block planes follow (extra loads, only for real chunks): they go to the buffers of the
// super-block's parity, last read for super-block s - 2 (at the start of step 8s - 9, before that
// step's meeting); they are issued in step 8s - 3 and land before the meeting of step 8s - 1.
template <int CI8>
__device__ __forceinline__ void q4_issue(uint8_t* slot, uint8_t* sbuf, const Q4Src& src,
                                         uint32_t ci, uint32_t c_end, int wave, int lane) {
  const bool live = ci < c_end;
  const uint32_t cl = live ? ci : c_end - 1;
  const uint32_t l16 = lane * 16;
  bdma16(src.b, l16, cl * 1024, slot + kQ4SlotB + wave * 1024);
  if (wave < kWgTokTiles) bdma16(src.a, l16, cl * 1024, slot + kQ4SlotA + wave * 1024);
  if (CI8 == 0 && live) {
    uint8_t* par = sbuf + ((ci >> 3) & 1) * kQ4SbBytes;
    const uint32_t s = ci >> 3;
    bdma16(src.sb, l16, s * 2048, par + kQ4SbSb + wave * 2048);
    bdma16(src.sb, l16 + 1024, s * 2048, par + kQ4SbSb + wave * 2048 + 1024);
    if (wave < kWgTokTiles) {
      bdma16(src.da, l16, s * 1024, par + kQ4SbDa + wave * 1024);
      bdma16(src.das, l16, s * 1024, par + kQ4SbDas + wave * 1024);
    }
  }
}

template <int CHUNKS>
__device__ __forceinline__ void q4_wait(bool loads_a) {
  if (loads_a)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CHUNKS * 2) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CHUNKS * 1) : "memory");
}

struct Q4Ctx {
  uint8_t* smem;
  uint8_t* sbuf;
  Q4Src src;
  uint32_t c_end;  // the piece's chunk end
  int64_t nchunk, n, m, tok_base, col;
  DotsOut dots;
  uint32_t aa, bb, dd, ss;  // per-lane LDS addresses: A in slot 0, B in slot 0, da and SB (parity 0)
  int wave, lane;
  bool loads_a;
};

// An empty volatile statement that "modifies" a tile's accumulators: the instruction selector
// cannot move the next step's loads and MFMAs above the rescale that produced them.
__device__ __forceinline__ void q4_order(float (&v)[16]) {
  asm volatile(""
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                 "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15]));
}

// The rescale of output tile u for chunk c (or, DOTS, the store of its chunk dots).
template <bool DOTS>
__device__ __forceinline__ void q4_tile(const Q4Ctx& k, uint32_t c, int u, const v16i& f, v2f pr,
                                        const float (&dav)[16], const float (&dsv)[16],
                                        float (&acc)[16]) {
  if (DOTS) {
    const int g = k.lane >> 5;
    const DotsRun d = dots_run<true>(k.dots, k.tok_base + 4 * g, k.col + u * kTile, k.nchunk, c);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int32_t* o = dots_slot(k.dots, d, r);
      if (o) *o = f[r] - kBiasI;
    }
  } else {
    const float nb = -kBiasF * pr.x;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = __builtin_fmaf(__int_as_float(f[r]), pr.x, nb);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(t[r], dav[r], acc[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(pr.y, dsv[r], acc[r]);
  }
  q4_order(acc);  // keep the steps in program order (bounded register lifetimes)
}

// This wave's MFMA operands of one chunk (A fragment, B fragments of its two row tiles), read from
// LDS one step ahead of their MFMAs.
struct Q4Frags {
  v4i a, b0, b1;
};

template <int OFF>
__device__ __forceinline__ void q4_read_frags(const Q4Ctx& k, Q4Frags& f) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7"
      : "=&v"(f.a), "=&v"(f.b0), "=&v"(f.b1)
      : "v"(k.aa), "v"(k.bb), "n"(OFF + kQ4SlotA), "n"(OFF + kQ4SlotB),
        "n"(OFF + kQ4SlotB + 1024)
      : "memory");
}

// Step CC of super-block s (chunk c = 8s + CC in ring slot CC % kQ4Ring), entered with chunk c
// complete in LDS for every wave and its fragments on their way into f:
//   1. wait for the fragments, start the LDS reads of the chunk's (d*sc, -dmin*m) pairs, da and
//      da*S, start both MFMAs (the reads land behind them);
//   2. issue the loads of chunk c+3 into chunk c-1's slot (every wave finished reading it before
//      the meeting of step c-1), wait for this wave's own loads of chunk c+1 and for the reads;
//   3. tile 0's rescale; meet (chunk c+1 complete for every wave, every wave done with chunk c's
//      scales); start the reads of chunk c+1's fragments; tile 1's rescale (they land meanwhile).
template <bool DOTS, int CC>
__device__ __forceinline__ void q4_step(const Q4Ctx& k, uint32_t s, uint32_t par, v16i& bias,
                                        float (&acc)[2][16], Q4Frags& f) {
  const uint32_t c = 8 * s + CC;
  constexpr int kN = ((CC + 1) % kQ4Ring) * kQ4Slot;  // slot of chunk c + 1
  // the MFMA bias stays in its 16 VGPRs (instead of being rebuilt from scalars every step)
  asm volatile("" : "+v"(bias));
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.a), "+v"(f.b0), "+v"(f.b1)::"memory");
  v4f d0, d1, d2, d3, s0, s1, s2, s3;
  v2f p0, p1;
  const uint32_t ddp = k.dd + par, ssp = k.ss + par;
  asm volatile(
      "ds_read_b64 %0, %11 offset:%12\n\t"
      "ds_read_b64 %1, %11 offset:%13\n\t"
      "ds_read_b128 %2, %10 offset:%14\n\t"
      "ds_read_b128 %3, %10 offset:%15\n\t"
      "ds_read_b128 %4, %10 offset:%16\n\t"
      "ds_read_b128 %5, %10 offset:%17\n\t"
      "ds_read_b128 %6, %10 offset:%18\n\t"
      "ds_read_b128 %7, %10 offset:%19\n\t"
      "ds_read_b128 %8, %10 offset:%20\n\t"
      "ds_read_b128 %9, %10 offset:%21"
      : "=&v"(p0), "=&v"(p1), "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3), "=&v"(s0), "=&v"(s1),
        "=&v"(s2), "=&v"(s3)
      : "v"(ddp), "v"(ssp), "n"(CC * 256), "n"(CC * 256 + 2048), "n"(CC * 128),
        "n"(CC * 128 + 16), "n"(CC * 128 + 32), "n"(CC * 128 + 48),
        "n"(kQ4SbDas + CC * 128), "n"(kQ4SbDas + CC * 128 + 16),
        "n"(kQ4SbDas + CC * 128 + 32), "n"(kQ4SbDas + CC * 128 + 48)
      : "memory");
  // (the reads stay ahead of the MFMAs, so their registers are never the fragments' registers,
  // which an MFMA may still be reading when a read lands)
  __builtin_amdgcn_sched_barrier(0);
  const v16i f0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a, f.b0, bias, 0, 0, 0);
  const v16i f1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a, f.b1, bias, 0, 0, 0);
  q4_issue<(CC + kQ4Ring - 1) % 8>(k.smem + ((CC + kQ4Ring - 1) % kQ4Ring) * kQ4Slot, k.sbuf,
                                   k.src, c + kQ4Ring - 1, k.c_end, k.wave, k.lane);
  q4_wait<kQ4Ring - 2>(k.loads_a);
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(p0), "+v"(p1), "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3), "+v"(s0), "+v"(s1),
                 "+v"(s2), "+v"(s3)::"memory");
  const float dav[16] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w,
                         d2.x, d2.y, d2.z, d2.w, d3.x, d3.y, d3.z, d3.w};
  const float dsv[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                         s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};
  q4_tile<DOTS>(k, c, 0, f0, p0, dav, dsv, acc[0]);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  q4_read_frags<kN>(k, f);
  __builtin_amdgcn_sched_barrier(0);  // the reads go out before any of tile 1's rescale
  q4_tile<DOTS>(k, c, 1, f1, p1, dav, dsv, acc[1]);
}

template <bool DOTS>
__global__ __launch_bounds__(256, Q4K_WG_PER_CU) void q4k_gemm_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ da, const float* __restrict__ das,
    const uint8_t* __restrict__ wcodes, const float* __restrict__ wsb, int64_t n, int64_t m,
    int64_t nchunk, float* __restrict__ y, int64_t ldy, float* __restrict__ ws, DotsOut dots,
    uint32_t gx, uint32_t gy, uint32_t n_full, uint32_t pieces) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kQ4Ring * kQ4Slot + 2 * kQ4SbBytes];
  const WgStamp stamp = wg_stamp();
  Q4Ctx k;
  k.smem = smem;
  k.sbuf = smem + kQ4Ring * kQ4Slot;
  k.lane = threadIdx.x & 63;
  k.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  k.loads_a = k.wave < kWgTokTiles;
  const int tt = k.wave & 1, rp = k.wave >> 1;
  const int64_t nsb = nchunk / 8;
  const TileWork tw = tile_work<true>(blockIdx.x, gx, gy, n_full, pieces, nsb, ws);
  const int64_t T = (int64_t)tw.bx * kWgTokTiles + tt;
  const int64_t R0 = (int64_t)tw.by * 4;
  const int64_t Ta = (int64_t)tw.bx * kWgTokTiles + (k.loads_a ? k.wave : 0);
  k.src.a = make_rsrc(xq + Ta * nchunk * 1024, nchunk * 1024);
  k.src.da = make_rsrc(reinterpret_cast<const uint8_t*>(da) + Ta * nchunk * 128, nchunk * 128);
  k.src.das = make_rsrc(reinterpret_cast<const uint8_t*>(das) + Ta * nchunk * 128, nchunk * 128);
  k.src.b = make_rsrc(wcodes + (R0 + k.wave) * nchunk * 1024, nchunk * 1024);
  k.src.sb = make_rsrc(reinterpret_cast<const uint8_t*>(wsb) + (R0 + k.wave) * nsb * 2048,
                       nsb * 2048);
  k.nchunk = nchunk;
  k.c_end = __builtin_amdgcn_readfirstlane((uint32_t)(8 * tw.s1));
  k.n = n;
  k.m = m;
  k.dots = dots;
  const int p = k.lane & 31, g = k.lane >> 5;
  k.tok_base = T * kTile;
  k.col = (R0 + 2 * rp) * kTile + p;
  k.aa = lds_addr(smem) + tt * 1024 + k.lane * 16;
  k.bb = lds_addr(smem) + 2 * rp * 1024 + k.lane * 16;
  k.dd = lds_addr(k.sbuf) + kQ4SbDa + tt * 1024 + g * 64;
  k.ss = lds_addr(k.sbuf) + kQ4SbSb + 2 * rp * 2048 + p * 8;

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasI;
  float acc[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.0f;

  const uint32_t c0 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * tw.s0));
  q4_issue<0>(smem + 0 * kQ4Slot, k.sbuf, k.src, c0 + 0, k.c_end, k.wave, k.lane);
  q4_issue<1>(smem + 1 * kQ4Slot, k.sbuf, k.src, c0 + 1, k.c_end, k.wave, k.lane);
  q4_issue<2>(smem + 2 * kQ4Slot, k.sbuf, k.src, c0 + 2, k.c_end, k.wave, k.lane);
  q4_wait<kQ4Ring - 2>(k.loads_a);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  Q4Frags f;
  q4_read_frags<0>(k, f);

  for (uint32_t s = c0 / 8; s < k.c_end / 8; ++s) {
    const uint32_t par = (s & 1) * kQ4SbBytes;
    q4_step<DOTS, 0>(k, s, par, bias, acc, f);
    q4_step<DOTS, 1>(k, s, par, bias, acc, f);
    q4_step<DOTS, 2>(k, s, par, bias, acc, f);
    q4_step<DOTS, 3>(k, s, par, bias, acc, f);
    q4_step<DOTS, 4>(k, s, par, bias, acc, f);
    q4_step<DOTS, 5>(k, s, par, bias, acc, f);
    q4_step<DOTS, 6>(k, s, par, bias, acc, f);
    q4_step<DOTS, 7>(k, s, par, bias, acc, f);
  }
  // drain the trailing (unused) loads and fragment reads
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  if (DOTS) return;
  const OutDst o = out_dst(tw, y, ldy, ws);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t mcol = k.col + u * kTile;
    if (mcol >= m) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t tok = T * kTile + 8 * (r >> 2) + 4 * g + (r & 3);
      if (tok < n) o.p[(tok - o.tok0) * o.ld + (mcol - o.row0)] = acc[u][r];
    }
  }
  wg_record(stamp, tw);
}

// ---------------------------------------------------------------------------------------------
// Host-side helpers
// ---------------------------------------------------------------------------------------------
inline int64_t round_up(int64_t v, int64_t q) { return (v + q - 1) / q * q; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
constexpr int64_t kMaxDim = (int64_t)1 << 40;

bool act_sizes(int64_t n, int64_t k, size_t* xq_bytes, size_t* da_bytes) {
  if (n < 0 || k <= 0 || k % 256 || n > kMaxDim || k > kMaxDim) return false;
  const int64_t np = round_up(n, kWgTok);
  if (np != 0 && k > (int64_t)(SIZE_MAX / 8) / np) return false;
  *xq_bytes = (size_t)np * (size_t)k;
  *da_bytes = (size_t)np * (size_t)(k / 32) * sizeof(float);
  return true;
}

bool valid_layout(int layout) {
  return layout == Q6K_LAYOUT_PACKED || layout == Q6K_LAYOUT_EXPANDED || layout == Q6K_LAYOUT_FOLDED;
}

bool weight_sizes(int64_t m, int64_t k, int layout, size_t* codes, size_t* scales) {
  if (m < 0 || k <= 0 || k % 256 || m > kMaxDim || k > kMaxDim) return false;
  if (!valid_layout(layout)) return false;
  const int64_t mp = round_up(m, kWgRow);
  if (mp != 0 && k > (int64_t)(SIZE_MAX / 8) / mp) return false;
  if (layout == Q6K_LAYOUT_FOLDED) {
    *codes = (size_t)mp * (size_t)k * 2;
    *scales = (size_t)mp * (size_t)(k / 256) * sizeof(float);
  } else if (layout == Q6K_LAYOUT_EXPANDED) {
    *codes = (size_t)mp * (size_t)k;
    *scales = (size_t)mp * (size_t)(k / 16) * sizeof(float);
  } else {
    *codes = (size_t)mp * (size_t)k / 4 * 3;
    *scales = (size_t)mp * (size_t)(k / 16) * sizeof(float);
  }
  return true;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev < 0 || dev >= 64) return -1;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Work split of a GEMM launch (see tile_work): n_full whole tiles, then the remaining tiles in
// `pieces` pieces each; nblocks workgroups in all.
struct SplitPlan {
  int64_t n_full, pieces, nblocks;
  uint32_t grade;  // tail_bound's grade of the split tiles' pieces (0: equal, static order)
};

// tail_bound's grade of a claimed tail (tile_work): piece i of P weighs P - i.  On ffn_down the
// layout-2 GEMM ran 1.6 % faster with it than with equal pieces in the static order (468.5
// against 476.3 us, three alternating same-box runs each; weights P - i + 1: 471.4); the GEMMs of
// layouts 0/1 and q4_K gained nothing (within +-0.3 %) and keep the static order.
constexpr uint32_t kTailGrade = 1;

q6k_status plan_split(int64_t gx, int64_t gy, int wg_per_cu, int64_t nsb, bool claim,
                      SplitPlan* sp) {
  const int cus = device_cus();
  if (cus <= 0) return Q6K_EHIP;
  const int64_t ntiles = gx * gy, slots = (int64_t)wg_per_cu * cus;
  const int64_t rem = ntiles % slots;
  int64_t pieces = rem ? std::min<int64_t>(slots / rem, nsb) : 1;
  // A split saves each split tile nsb - ceil(nsb / pieces) super-blocks of time and costs the
  // reducing kernel, 5-7 us or the time of 2-3 super-blocks: below 3 saved it does not pay (64 x
  // 256 x 512, two super-blocks: layout 2 9.1 us unsplit against 13.4 us in two pieces).
  if (pieces >= 2 && nsb - (nsb + pieces - 1) / pieces < 3) pieces = 1;
  if (pieces < 2) pieces = 1;
  sp->n_full = pieces > 1 ? ntiles - rem : ntiles;
  sp->pieces = pieces;
  sp->nblocks = sp->n_full + (ntiles - sp->n_full) * pieces;
  // Behind at least one whole round the split tiles' workgroups start staggered: claim their
  // pieces, largest first, if every graded piece keeps a super-block.
  sp->grade = 0;
  if (claim && pieces > 1 && sp->n_full >= slots && pieces <= 0xFFFF) {
    const uint32_t g = kTailGrade;
    bool ok = true;
    for (uint32_t j = 0; j < (uint32_t)pieces; ++j)
      ok = ok && tail_bound(nsb, (uint32_t)pieces, g, j + 1) >
                     tail_bound(nsb, (uint32_t)pieces, g, j);
    if (ok) sp->grade = g;
  }
  return sp->nblocks > INT32_MAX ? Q6K_ESIZE : Q6K_OK;
}

static_assert(kTile * kFTok == kSlabTok && kTile * kWgTokTiles == kSlabTok,
              "every GEMM's output tile is one workspace slab");
static_assert(kSlabTok % kReduceTok == 0 && kReduceTok * 128 == 256 * 4,
              "reducing workgroups cover whole tiles, 4 rows per thread");

// Workspace bytes of a plan: one slab per piece of a split tile, then (claimed tail) the 4-byte
// claim word, in a 256-byte block of its own.
constexpr size_t kClaimBytes = 256;
inline size_t plan_workspace_bytes(const SplitPlan& sp) {
  return (size_t)(sp.nblocks - sp.n_full) * (size_t)kSlabFloats * sizeof(float) +
         (sp.grade ? kClaimBytes : 0);
}

// The claim word of a plan's workspace (after the slabs), or null.
inline uint32_t* plan_claim_word(const SplitPlan& sp, float* ws) {
  if (!sp.grade || !ws) return nullptr;
  return reinterpret_cast<uint32_t*>(ws + (sp.nblocks - sp.n_full) * kSlabFloats);
}

// The pieces argument of the GEMM kernels: piece count and grade.
inline uint32_t pieces_arg(const SplitPlan& sp) {
  return (uint32_t)sp.pieces | (sp.grade << 16);
}

// The workspace of a launch that needs `need` bytes: 16-byte aligned, at least that large.
q6k_status check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return Q6K_OK;
  if (!ws) return Q6K_EINVAL;
  if (((uintptr_t)ws & 15) != 0) return Q6K_EALIGN;
  return ws_bytes < need ? Q6K_ESIZE : Q6K_OK;
}

// After the GEMM on the same stream: y over the split tiles from their slabs (nothing if the plan
// splits none).
void reduce_split_tiles(const SplitPlan& sp, int64_t gx, int64_t gy, bool xcd_order,
                        const float* ws, float* y, int64_t ldy, int64_t n, int64_t m,
                        hipStream_t s) {
  const int64_t nsplit = gx * gy - sp.n_full;
  if (nsplit > 0)
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)(nsplit * (kSlabTok / kReduceTok))),
                       dim3(256), 0, s, ws, y, ldy, n, m, (uint32_t)gx, (uint32_t)gy,
                       (uint32_t)sp.n_full, (uint32_t)sp.pieces, xcd_order ? 1 : 0,
                       aligned16(y) && ldy % 4 == 0 ? 1 : 0,
                       plan_claim_word(sp, const_cast<float*>(ws)));
}

q6k_status launch_status() {
  return hipGetLastError() == hipSuccess ? Q6K_OK : Q6K_EHIP;
}

enum { kOutY = 0, kOutSubdots = 1, kOutChunkdots = 2 };

// The f32 output [n][ldy] (only [0, n) x [0, m) written): ldy >= m, and the buffer holds the
// last row's first m values.
q6k_status check_y(const float* y, size_t y_bytes, int64_t n, int64_t m, int64_t ldy) {
  if (!y) return Q6K_EINVAL;
  if (ldy < m) return Q6K_EINVAL;
  if (ldy > kMaxDim) return Q6K_ESIZE;
  if (((uintptr_t)y & 3) != 0) return Q6K_EALIGN;
  if ((uint64_t)(n - 1) > (SIZE_MAX / 4 - (uint64_t)m) / (uint64_t)ldy) return Q6K_ESIZE;
  if (y_bytes / 4 < (uint64_t)(n - 1) * (uint64_t)ldy + (uint64_t)m) return Q6K_ESIZE;
  return Q6K_OK;
}

// A test export's window of tokens x rows inside the n x m problem, and its int32 buffer of
// ntok * nrow * per values.
q6k_status check_window(const DotsOut& w, size_t dots_bytes, int64_t n, int64_t m, int64_t per) {
  if (w.tok0 < 0 || w.ntok < 0 || w.row0 < 0 || w.nrow < 0) return Q6K_EINVAL;
  if (w.tok0 > n || w.ntok > n - w.tok0 || w.row0 > m || w.nrow > m - w.row0) return Q6K_EINVAL;
  if (w.ntok == 0 || w.nrow == 0) return Q6K_OK;
  if (!w.p) return Q6K_EINVAL;
  if (((uintptr_t)w.p & 3) != 0) return Q6K_EALIGN;
  if ((uint64_t)w.ntok > SIZE_MAX / 4 / (uint64_t)w.nrow / (uint64_t)per) return Q6K_ESIZE;
  if (dots_bytes / 4 < (uint64_t)w.ntok * (uint64_t)w.nrow * (uint64_t)per) return Q6K_ESIZE;
  return Q6K_OK;
}

// The shape rules of a q6_K GEMM (any output).
q6k_status gemm_shape(int64_t n, int64_t m, int64_t k, int layout) {
  if (n < 0 || m < 0) return Q6K_EINVAL;
  if (!valid_layout(layout)) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  if (n > kMaxDim || m > kMaxDim || k > kMaxDim) return Q6K_ESIZE;
  // layout 2 addresses a row tile's digit planes (k/32 * 2048 bytes) through one 32-bit buffer
  // range
  if (layout == Q6K_LAYOUT_FOLDED && k / 32 * 2048 > INT32_MAX) return Q6K_ESIZE;
  // layouts 0 and 1 address a tile's activations or codes (k/32 * 1024 bytes) likewise
  if (layout != Q6K_LAYOUT_FOLDED && k / 32 * 1024 > INT32_MAX) return Q6K_ESIZE;
  return Q6K_OK;
}

// Output tiles (gx x gy of kSlabTok tokens x 128 rows) and work split of a non-empty q6_K GEMM
// on the current device.
q6k_status gemm_plan(int64_t n, int64_t m, int64_t k, int layout, int64_t* gx, int64_t* gy,
                     SplitPlan* sp) {
  *gx = round_up(n, kWgTok) / kSlabTok;
  *gy = round_up(m, kWgRow) / kWgRow;
  if (*gy > INT32_MAX || *gx > INT32_MAX) return Q6K_ESIZE;
  const int wg_per_cu = layout == Q6K_LAYOUT_FOLDED ? kFoldedWgPerCu : Q6K_WG_PER_CU;
  return plan_split(*gx, *gy, wg_per_cu, k / 256, layout == Q6K_LAYOUT_FOLDED, sp);
}

template <int OUT>
q6k_status gemm_common(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                       int64_t n, const void* w, size_t w_bytes, int layout, int64_t m, int64_t k,
                       float* y, size_t y_bytes, int64_t ldy, void* wsp, size_t ws_bytes,
                       DotsOut dots, size_t dots_bytes, void* stream) {
  const q6k_status shape = gemm_shape(n, m, k, layout);
  if (shape != Q6K_OK) return shape;
  if (OUT == kOutSubdots && layout == Q6K_LAYOUT_FOLDED) return Q6K_EINVAL;
  if (OUT == kOutChunkdots && layout != Q6K_LAYOUT_FOLDED) return Q6K_EINVAL;
  if (n == 0 || m == 0) return Q6K_OK;
  if (!xq || !da || !w) return Q6K_EINVAL;
  if (!aligned16(xq) || !aligned16(da) || !aligned16(w)) return Q6K_EALIGN;
  size_t need_x, need_d, codes_bytes, scales_bytes;
  if (!act_sizes(n, k, &need_x, &need_d)) return Q6K_ESIZE;
  if (!weight_sizes(m, k, layout, &codes_bytes, &scales_bytes)) return Q6K_ESIZE;
  if (xq_bytes < need_x || da_bytes < need_d || w_bytes < codes_bytes + scales_bytes)
    return Q6K_ESIZE;
  if (OUT != kOutY) {
    const q6k_status ws = check_window(dots, dots_bytes, n, m, OUT == kOutSubdots ? k / 16 : k / 32);
    if (ws != Q6K_OK) return ws;
    if (dots.ntok == 0 || dots.nrow == 0) return Q6K_OK;
  } else {
    const q6k_status ys = check_y(y, y_bytes, n, m, ldy);
    if (ys != Q6K_OK) return ys;
  }
  int64_t gx, gy;
  SplitPlan sp;
  const q6k_status plan = gemm_plan(n, m, k, layout, &gx, &gy, &sp);
  if (plan != Q6K_OK) return plan;
  // the test exports store no y and so no slabs
  float* slabs = nullptr;
  if (OUT == kOutY) {
    const q6k_status wst = check_workspace(wsp, ws_bytes, plan_workspace_bytes(sp));
    if (wst != Q6K_OK) return wst;
    slabs = static_cast<float*>(wsp);
  }
  const int64_t nchunk = k / 32;
  const uint8_t* wc = static_cast<const uint8_t*>(w);
  const uint8_t* wsc = wc + codes_bytes;
  const uint8_t* a = static_cast<const uint8_t*>(xq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  constexpr bool kDots = OUT != kOutY;
  const dim3 grid((unsigned)sp.nblocks),
      block(layout == Q6K_LAYOUT_FOLDED ? 64 * kFWaves : 256);
  const uint32_t gx32 = (uint32_t)gx, gy32 = (uint32_t)gy, nf = (uint32_t)sp.n_full,
                 pc = pieces_arg(sp);
  if (layout == Q6K_LAYOUT_FOLDED) {
    const int vec_store = OUT == kOutY && aligned16(y) && ldy % 4 == 0;
    hipLaunchKernelGGL((folded_kernel<kDots>), grid, block, 0, s, a, da, wc, wsc, n, m, nchunk,
                       y, ldy, vec_store, slabs, dots, gx32, gy32, nf, pc);
  } else if (layout == Q6K_LAYOUT_EXPANDED) {
    hipLaunchKernelGGL((gemm_kernel<Q6K_LAYOUT_EXPANDED, kDots>), grid, block, 0, s, a, da, wc,
                       wsc, n, m, nchunk, y, ldy, slabs, dots, gx32, gy32, nf, pc);
  } else {
    hipLaunchKernelGGL((gemm_kernel<Q6K_LAYOUT_PACKED, kDots>), grid, block, 0, s, a, da, wc,
                       wsc, n, m, nchunk, y, ldy, slabs, dots, gx32, gy32, nf, pc);
  }
  if (OUT == kOutY)
    reduce_split_tiles(sp, gx, gy, layout == Q6K_LAYOUT_FOLDED || Q6K_GEMM01_XCD_ORDER, slabs, y,
                       ldy, n, m, s);
  const q6k_status st = launch_status();
  if (st == Q6K_OK) g_launches[layout].fetch_add(1, std::memory_order_relaxed);
  return st;
}

template <bool SWIGLU, bool SUMS>
q6k_status quantize_common(const float* x, const float* up, int64_t n, int64_t k, int64_t ldx,
                           void* xq, size_t xq_bytes, float* da, size_t da_bytes, float* das,
                           size_t das_bytes, void* stream) {
  if (n < 0) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  size_t need_x, need_d;
  if (!act_sizes(n, k, &need_x, &need_d)) return Q6K_ESIZE;
  if (n == 0) return Q6K_OK;
  if (!x || !xq || !da || (SUMS && !das)) return Q6K_EINVAL;
  if (ldx < k) return Q6K_EINVAL;
  if (!aligned16(x) || ldx % 4 || !aligned16(xq) || !aligned16(da) || (SUMS && !aligned16(das)))
    return Q6K_EALIGN;
  if (xq_bytes < need_x || da_bytes < need_d || (SUMS && das_bytes < need_d)) return Q6K_ESIZE;
  const int64_t np = round_up(n, kWgTok);
  const int64_t nchunk = k / 32;
  const int64_t ntt = np / kTile, nkb = (nchunk + 7) / 8;
  if (nkb > INT32_MAX) return Q6K_ESIZE;
  // grid x = 8-chunk blocks of k, y = token tiles (at most 65535 per launch)
  for (int64_t t0 = 0; t0 < ntt; t0 += 65535)
    hipLaunchKernelGGL((quantize_act_kernel<SWIGLU, SUMS>),
                       dim3((unsigned)nkb, (unsigned)std::min<int64_t>(65535, ntt - t0)),
                       dim3(256), 0, static_cast<hipStream_t>(stream), x, up, n, ldx, nchunk,
                       static_cast<uint8_t*>(xq), da, das, t0);
  return launch_status();
}

// The shape rules of a q4_K GEMM (any output).
q6k_status q4k_gemm_shape(int64_t n, int64_t m, int64_t k) {
  if (n < 0 || m < 0) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  if (n > kMaxDim || m > kMaxDim || k > kMaxDim) return Q6K_ESIZE;
  if (k / 32 * 1024 > INT32_MAX) return Q6K_ESIZE;  // one 32-bit buffer range per tile
  return Q6K_OK;
}

// Output tiles and work split of a non-empty q4_K GEMM on the current device.
q6k_status q4k_gemm_plan(int64_t n, int64_t m, int64_t k, int64_t* gx, int64_t* gy,
                         SplitPlan* sp) {
  *gx = round_up(n, kWgTok) / kSlabTok;
  *gy = round_up(m, kWgRow) / kWgRow;
  if (*gy > 65535 || *gx > INT32_MAX) return Q6K_ESIZE;
  return plan_split(*gx, *gy, Q4K_WG_PER_CU, k / 256, false, sp);
}

template <bool DOTS>
q6k_status q4k_gemm_common(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                           const float* das, size_t das_bytes, int64_t n, const void* w,
                           size_t w_bytes, int64_t m, int64_t k, float* y, size_t y_bytes,
                           int64_t ldy, void* wsp, size_t ws_bytes, DotsOut dots,
                           size_t dots_bytes, void* stream) {
  const q6k_status shape = q4k_gemm_shape(n, m, k);
  if (shape != Q6K_OK) return shape;
  if (n == 0 || m == 0) return Q6K_OK;
  if (!xq || !w || (!DOTS && (!da || !das))) return Q6K_EINVAL;
  if (!aligned16(xq) || !aligned16(w) || (!DOTS && (!aligned16(da) || !aligned16(das))))
    return Q6K_EALIGN;
  size_t need_x, need_d;
  if (!act_sizes(n, k, &need_x, &need_d)) return Q6K_ESIZE;
  const size_t need_w = q4k_weight_bytes(m, k);
  if (need_w == 0) return Q6K_ESIZE;
  if (xq_bytes < need_x || w_bytes < need_w) return Q6K_ESIZE;
  if (!DOTS && (da_bytes < need_d || das_bytes < need_d)) return Q6K_ESIZE;
  if (DOTS) {
    const q6k_status ws = check_window(dots, dots_bytes, n, m, k / 32);
    if (ws != Q6K_OK) return ws;
    if (dots.ntok == 0 || dots.nrow == 0) return Q6K_OK;
  } else {
    const q6k_status ys = check_y(y, y_bytes, n, m, ldy);
    if (ys != Q6K_OK) return ys;
  }
  int64_t gx, gy;
  SplitPlan sp;
  const q6k_status plan = q4k_gemm_plan(n, m, k, &gx, &gy, &sp);
  if (plan != Q6K_OK) return plan;
  float* slabs = nullptr;
  if (!DOTS) {
    const q6k_status wst = check_workspace(wsp, ws_bytes, plan_workspace_bytes(sp));
    if (wst != Q6K_OK) return wst;
    slabs = static_cast<float*>(wsp);
  }
  const int64_t mp = round_up(m, kWgRow);
  const int64_t nchunk = k / 32;
  const uint8_t* wc = static_cast<const uint8_t*>(w);
  const float* ws = reinterpret_cast<const float*>(wc + (size_t)mp * (size_t)k);
  // the test export reads no scales: point them at the codes, which are never dereferenced as such
  const float* dap = DOTS ? reinterpret_cast<const float*>(xq) : da;
  const float* dasp = DOTS ? reinterpret_cast<const float*>(xq) : das;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL((q4k_gemm_kernel<DOTS>), dim3((unsigned)sp.nblocks), dim3(256), 0, s,
                     static_cast<const uint8_t*>(xq), dap, dasp, wc, ws, n, m, nchunk, y, ldy,
                     slabs, dots, (uint32_t)gx, (uint32_t)gy, (uint32_t)sp.n_full,
                     pieces_arg(sp));
  if (!DOTS) reduce_split_tiles(sp, gx, gy, true, slabs, y, ldy, n, m, s);
  const q6k_status st = launch_status();
  if (st == Q6K_OK) g_q4k_launches.fetch_add(1, std::memory_order_relaxed);
  return st;
}

// The workspace of q6k_gemm_noalloc: split-k slabs in static device memory, one copy per GPU the
// library runs on, held until the process ends.  kScratchSlabs = 3 workgroup slots per CU x 256
// CUs, the most any q6_K layout splits into on such a device (24 MiB).  Host code never uses the
// array's name as an address: each device's address comes from hipGetSymbolAddress, taken on the
// first call on that device with the device current, and kept in scratch_addr.
constexpr int64_t kScratchSlabs = 768;
constexpr size_t kScratchBytes = (size_t)kScratchSlabs * kSlabFloats * sizeof(float) + kClaimBytes;
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// The current device's address of `scratch`.
q6k_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q6K_EHIP;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q6K_EHIP;
      scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return Q6K_OK;
}

}  // namespace

extern "C" {

size_t q4k_weight_bytes(int64_t m, int64_t k) {
  if (m < 0 || k <= 0 || k % 256 || m > kMaxDim || k > kMaxDim) return 0;
  const int64_t mp = round_up(m, kWgRow);
  if (mp != 0 && k > (int64_t)(SIZE_MAX / 16) / mp) return 0;
  return (size_t)mp * (size_t)k + (size_t)mp * (size_t)(k / 32) * 8;
}

q6k_status q4k_expand_weights(const void* w_raw, int64_t m, int64_t k, void* w_out,
                              size_t w_out_bytes, void* stream) {
  if (m < 0) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  const size_t need = q4k_weight_bytes(m, k);
  if (need == 0 && m > 0) return Q6K_ESIZE;
  if (m == 0) return Q6K_OK;
  if (!w_raw || !w_out) return Q6K_EINVAL;
  if (!aligned16(w_raw) || !aligned16(w_out)) return Q6K_EALIGN;
  if (w_out_bytes < need) return Q6K_ESIZE;
  const int64_t mp = round_up(m, kWgRow);
  const int64_t nsb = k / 256;
  if (mp / kTile > INT32_MAX || nsb > 65535) return Q6K_ESIZE;
  uint8_t* codes = static_cast<uint8_t*>(w_out);
  hipLaunchKernelGGL(q4k_expand_kernel, dim3((unsigned)(mp / kTile), (unsigned)nsb), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(w_raw), m, nsb,
                     codes, reinterpret_cast<float*>(codes + (size_t)mp * (size_t)k));
  return launch_status();
}

q6k_status q4k_quantize_act(const float* x, int64_t n, int64_t k, int64_t ldx, void* xq,
                            size_t xq_bytes, float* da, size_t da_bytes, float* das,
                            size_t das_bytes, void* stream) {
  return quantize_common<false, true>(x, nullptr, n, k, ldx, xq, xq_bytes, da, da_bytes, das,
                                      das_bytes, stream);
}

q6k_status q4k_act_sums(const void* xq, const float* da, int64_t n, int64_t k, float* das,
                        size_t das_bytes, void* stream) {
  if (n < 0) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  size_t need_x, need_d;
  if (!act_sizes(n, k, &need_x, &need_d)) return Q6K_ESIZE;
  if (n == 0) return Q6K_OK;
  if (!xq || !da || !das) return Q6K_EINVAL;
  if (!aligned16(xq) || !aligned16(da) || !aligned16(das)) return Q6K_EALIGN;
  if (das_bytes < need_d) return Q6K_ESIZE;
  const int64_t ntile = round_up(n, kWgTok) / kTile, nchunk = k / 32;
  const int64_t blocks = (ntile * nchunk * 32 + 255) / 256;
  if (blocks > INT32_MAX) return Q6K_ESIZE;
  hipLaunchKernelGGL(q4k_act_sums_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(xq), da, ntile,
                     nchunk, das);
  return launch_status();
}

q6k_status q4k_gemm_workspace(int64_t n, int64_t m, int64_t k, size_t* bytes) {
  if (!bytes) return Q6K_EINVAL;
  *bytes = 0;
  const q6k_status shape = q4k_gemm_shape(n, m, k);
  if (shape != Q6K_OK || n == 0 || m == 0) return shape;
  int64_t gx, gy;
  SplitPlan sp;
  const q6k_status plan = q4k_gemm_plan(n, m, k, &gx, &gy, &sp);
  if (plan == Q6K_OK) *bytes = plan_workspace_bytes(sp);
  return plan;
}

q6k_status q4k_gemm(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                    const float* das, size_t das_bytes, int64_t n, const void* w, size_t w_bytes,
                    int64_t m, int64_t k, float* y, size_t y_bytes, int64_t ldy, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return q4k_gemm_common<false>(xq, xq_bytes, da, da_bytes, das, das_bytes, n, w, w_bytes, m, k,
                                y, y_bytes, ldy, workspace, workspace_bytes,
                                DotsOut{nullptr, 0, 0, 0, 0}, 0, stream);
}

q6k_status q4k_gemm_dots(const void* xq, size_t xq_bytes, int64_t n, const void* w,
                         size_t w_bytes, int64_t m, int64_t k, int64_t tok0, int64_t ntok,
                         int64_t row0, int64_t nrow, int32_t* dots, size_t dots_bytes,
                         void* stream) {
  return q4k_gemm_common<true>(xq, xq_bytes, nullptr, 0, nullptr, 0, n, w, w_bytes, m, k, nullptr,
                               0, 0, nullptr, 0, DotsOut{dots, tok0, ntok, row0, nrow}, dots_bytes,
                               stream);
}

uint64_t q4k_launches(void) { return g_q4k_launches.load(std::memory_order_relaxed); }


size_t q6k_act_bytes(int64_t n, int64_t k, size_t* da_bytes) {
  size_t xb = 0, db = 0;
  if (!act_sizes(n, k, &xb, &db)) {
    if (da_bytes) *da_bytes = 0;
    return 0;
  }
  if (da_bytes) *da_bytes = db;
  return xb;
}

q6k_status q6k_quantize_act(const float* x, int64_t n, int64_t k, int64_t ldx, void* xq,
                            size_t xq_bytes, float* da, size_t da_bytes, void* stream) {
  return quantize_common<false, false>(x, nullptr, n, k, ldx, xq, xq_bytes, da, da_bytes, nullptr,
                                      0, stream);
}

q6k_status q6k_swiglu_quantize_act(const float* gate, const float* up, int64_t n, int64_t k,
                                   int64_t ld, void* xq, size_t xq_bytes, float* da,
                                   size_t da_bytes, void* stream) {
  if (n > 0 && !up) return Q6K_EINVAL;
  if (n > 0 && up && !aligned16(up)) return Q6K_EALIGN;
  return quantize_common<true, false>(gate, up, n, k, ld, xq, xq_bytes, da, da_bytes, nullptr, 0,
                                     stream);
}

q6k_status q6k_swiglu_f32(const float* gate, const float* up, int64_t n, int64_t k, int64_t ld,
                          float* h, int64_t ldh, void* stream) {
  if (n < 0 || k < 0) return Q6K_EINVAL;
  if (n == 0 || k == 0) return Q6K_OK;
  if (!gate || !up || !h) return Q6K_EINVAL;
  if (ld < k || ldh < k) return Q6K_EINVAL;
  if (((uintptr_t)gate | (uintptr_t)up | (uintptr_t)h) & 3) return Q6K_EALIGN;
  if (n > kMaxDim || k > kMaxDim || k > ((int64_t)1 << 38) / n) return Q6K_ESIZE;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n * k + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), gate, up, n, k, ld, h, ldh);
  return launch_status();
}

size_t q6k_weight_bytes(int64_t m, int64_t k, int layout) {
  size_t c, s;
  if (!weight_sizes(m, k, layout, &c, &s)) return 0;
  return c + s;
}

q6k_status q6k_expand_weights(const void* w_raw, int64_t m, int64_t k, int layout, void* w_out,
                              size_t w_out_bytes, void* stream) {
  if (m < 0) return Q6K_EINVAL;
  if (!valid_layout(layout)) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  size_t cb, sb;
  if (!weight_sizes(m, k, layout, &cb, &sb)) return Q6K_ESIZE;
  if (m == 0) return Q6K_OK;
  if (!w_raw || !w_out) return Q6K_EINVAL;
  if (((uintptr_t)w_raw & 1) || !aligned16(w_out)) return Q6K_EALIGN;
  if (w_out_bytes < cb + sb) return Q6K_ESIZE;
  const int64_t mp = round_up(m, kWgRow);
  const int64_t nsb = k / 256;
  if (mp / kTile > INT32_MAX || nsb > 65535) return Q6K_ESIZE;
  uint8_t* codes = static_cast<uint8_t*>(w_out);
  dim3 grid((unsigned)(mp / kTile), (unsigned)nsb), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (layout == Q6K_LAYOUT_FOLDED)
    hipLaunchKernelGGL(expand_kernel<Q6K_LAYOUT_FOLDED>, grid, block, 0, s,
                       static_cast<const uint8_t*>(w_raw), m, nsb, codes, codes + cb);
  else if (layout == Q6K_LAYOUT_EXPANDED)
    hipLaunchKernelGGL(expand_kernel<Q6K_LAYOUT_EXPANDED>, grid, block, 0, s,
                       static_cast<const uint8_t*>(w_raw), m, nsb, codes, codes + cb);
  else
    hipLaunchKernelGGL(expand_kernel<Q6K_LAYOUT_PACKED>, grid, block, 0, s,
                       static_cast<const uint8_t*>(w_raw), m, nsb, codes, codes + cb);
  return launch_status();
}

q6k_status q6k_gemm_workspace(int64_t n, int64_t m, int64_t k, int layout, size_t* bytes) {
  if (!bytes) return Q6K_EINVAL;
  *bytes = 0;
  const q6k_status shape = gemm_shape(n, m, k, layout);
  if (shape != Q6K_OK || n == 0 || m == 0) return shape;
  int64_t gx, gy;
  SplitPlan sp;
  const q6k_status plan = gemm_plan(n, m, k, layout, &gx, &gy, &sp);
  if (plan == Q6K_OK) *bytes = plan_workspace_bytes(sp);
  return plan;
}

q6k_status q6k_gemm(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                    int64_t n, const void* w, size_t w_bytes, int layout, int64_t m, int64_t k,
                    float* y, size_t y_bytes, int64_t ldy, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return gemm_common<kOutY>(xq, xq_bytes, da, da_bytes, n, w, w_bytes, layout, m, k, y, y_bytes,
                            ldy, workspace, workspace_bytes, DotsOut{nullptr, 0, 0, 0, 0}, 0,
                            stream);
}

q6k_status q6k_gemm_noalloc(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                            int64_t n, const void* w, size_t w_bytes, int layout, int64_t m,
                            int64_t k, float* y, size_t y_bytes, int64_t ldy, void* stream) {
  const q6k_status shape = gemm_shape(n, m, k, layout);
  if (shape != Q6K_OK || n == 0 || m == 0) return shape;
  size_t need = 0;
  const q6k_status ws = q6k_gemm_workspace(n, m, k, layout, &need);
  if (ws != Q6K_OK) return ws;
  if (need > kScratchBytes) return Q6K_ESCRATCH;
  void* p = nullptr;
  if (need > 0) {
    const q6k_status sp = scratch_ptr(&p);
    if (sp != Q6K_OK) return sp;
  }
  return gemm_common<kOutY>(xq, xq_bytes, da, da_bytes, n, w, w_bytes, layout, m, k, y, y_bytes,
                            ldy, p, need, DotsOut{nullptr, 0, 0, 0, 0}, 0, stream);
}

q6k_status q6k_gemm_subdots(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                            int64_t n, const void* w, size_t w_bytes, int layout, int64_t m,
                            int64_t k, int64_t tok0, int64_t ntok, int64_t row0, int64_t nrow,
                            int32_t* dots, size_t dots_bytes, void* stream) {
  return gemm_common<kOutSubdots>(xq, xq_bytes, da, da_bytes, n, w, w_bytes, layout, m, k,
                                  nullptr, 0, 0, nullptr, 0, DotsOut{dots, tok0, ntok, row0, nrow},
                                  dots_bytes, stream);
}

q6k_status q6k_gemm_chunkdots(const void* xq, size_t xq_bytes, const float* da, size_t da_bytes,
                              int64_t n, const void* w, size_t w_bytes, int layout, int64_t m,
                              int64_t k, int64_t tok0, int64_t ntok, int64_t row0, int64_t nrow,
                              int32_t* dots, size_t dots_bytes, void* stream) {
  return gemm_common<kOutChunkdots>(xq, xq_bytes, da, da_bytes, n, w, w_bytes, layout, m, k,
                                    nullptr, 0, 0, nullptr, 0,
                                    DotsOut{dots, tok0, ntok, row0, nrow}, dots_bytes, stream);
}

const char* q6k_strerror(int status) {
  switch (status) {
    case Q6K_OK: return "ok";
    case Q6K_EINVAL: return "invalid argument (null pointer, negative size, unknown layout or leading dimension too small)";
    case Q6K_ESHAPE: return "k must be a positive multiple of 256 (whole q6_K super-blocks)";
    case Q6K_EALIGN: return "pointer or leading dimension not 16-byte aligned";
    case Q6K_ESIZE: return "buffer smaller than required, or problem too large";
    case Q6K_EHIP: return "HIP runtime rejected a kernel launch";
    case Q6K_ESCRATCH: return "problem needs more split-k scratch than q6k_gemm_noalloc's static array holds";
    default: return "unknown status";
  }
}

void q6k_stats(uint64_t out[3]) {
  if (!out) return;
  for (int i = 0; i < 3; ++i) out[i] = g_launches[i].load(std::memory_order_relaxed);
}

#ifdef Q6K_TIMELINE
int64_t q6k_timeline_capacity(void) { return kTimelineWgs; }

q6k_status q6k_timeline_clear(void* stream) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(q6k_timeline_rec)) != hipSuccess) return Q6K_EHIP;
  return hipMemsetAsync(p, 0, sizeof(q6k_timeline_rec), (hipStream_t)stream) == hipSuccess
             ? Q6K_OK
             : Q6K_EHIP;
}

q6k_status q6k_timeline_read(uint64_t* records, int64_t max_wgs) {
  if (!records || max_wgs < 0) return Q6K_EINVAL;
  const int64_t n = std::min<int64_t>(max_wgs, kTimelineWgs);
  if (n == 0) return Q6K_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(q6k_timeline_rec)) != hipSuccess) return Q6K_EHIP;
  return hipMemcpy(records, p, (size_t)n * 8 * sizeof(uint64_t), hipMemcpyDeviceToHost) ==
                 hipSuccess
             ? Q6K_OK
             : Q6K_EHIP;
}
#endif

}  // extern "C"

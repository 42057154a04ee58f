// q6k.hip -- HIP kernels for gfx950 and the C ABI of libq6k.so (declared in include/q6k.h).
//
// Kernels
//   quantize_act_kernel : activation quantize-transpose prepass (HBM-bound)
//   expand_kernel<L>    : load-time weight preparation, layout 0 (packed 6-bit) or 1 (int8 plane)
//   gemm_kernel<L, D>   : q6_K x int8 GEMM on v_mfma_i32_32x32x16_i8 (the int8 MFMA whose
//                         K is 16, so the two 16-k halves of a chunk stay separate integers);
//                         D = true is the test-only sub-block dot export of the same source
//
// The method follows "r38 q6_K BT-style raw-byte mma kernel (LANDED)" (sec. 2.1 layout,
// sec. 2.2 rescale without dmin, sec. 2.4 KSPLIT=2), "r41 q6_K B-expand widened to uint4 group
// loads (LANDED)" (expand from wide loads) and "r53 W_exp pre-expansion plane + cp.async B
// staging (LANDED)" (optional pre-expanded plane).  The tiling is this library's own.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "q6k.h"

namespace {

constexpr int kTile = 32;        // MFMA tile edge: 32 tokens x 32 weight rows
constexpr int kWgTok = 128;      // tokens per GEMM workgroup (4 token tiles)
constexpr int kWgRow = 128;      // weight rows per GEMM workgroup (4 row tiles)
constexpr int kFragBytes = 16;   // per lane per chunk: 8 bytes for half 0, 8 for half 1
constexpr int kPackBytes = 12;   // layout 0: per lane per chunk, 16 codes of 6 bits
constexpr int kBiasI = 0x4B400000;      // bit pattern of 1.5 * 2^23
constexpr float kBiasF = 12582912.0f;   // 1.5 * 2^23

std::atomic<uint64_t> g_launches[2];

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) | ((uint32_t)(c & 255) << 16) |
         ((uint32_t)(d & 255) << 24);
}

// ---------------------------------------------------------------------------------------------
// Prepass.  Block = 32 tokens (one token tile) x 8 chunks; thread (p, cc) owns token 32T + p and
// chunk 8*blockIdx.y + cc.  Each thread reads its 128 contiguous input bytes, computes
// da = amax / 127 and q = roundf(x / da) with correctly rounded f32 divisions, and writes the two
// 16-byte lane slots of that token (lane p and lane p + 32) plus its da.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_act_kernel(const float* __restrict__ x, int64_t n,
                                                           int64_t ldx, int64_t nchunk,
                                                           uint8_t* __restrict__ xq,
                                                           float* __restrict__ da) {
  const int p = threadIdx.x & 31;
  const int64_t c = (int64_t)blockIdx.y * 8 + (threadIdx.x >> 5);
  const int64_t T = blockIdx.x;
  if (c >= nchunk) return;
  const int64_t tok = T * kTile + p;
  float v[32];
  if (tok < n) {
    const float4* src = reinterpret_cast<const float4*>(x + tok * ldx + c * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = src[i];
      v[4 * i + 0] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float scale = amax / 127.0f;
  int q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float r = 0.0f;
    if (scale != 0.0f) r = fminf(fmaxf(roundf(v[i] / scale), -127.0f), 127.0f);
    q[i] = (int)r;
  }
  // lane p   : k 0..7  (half 0) and k 16..23 (half 1)
  // lane p+32: k 8..15 (half 0) and k 24..31 (half 1)
  uint4 s0, s1;
  s0.x = pack4(q[0], q[1], q[2], q[3]);
  s0.y = pack4(q[4], q[5], q[6], q[7]);
  s0.z = pack4(q[16], q[17], q[18], q[19]);
  s0.w = pack4(q[20], q[21], q[22], q[23]);
  s1.x = pack4(q[8], q[9], q[10], q[11]);
  s1.y = pack4(q[12], q[13], q[14], q[15]);
  s1.z = pack4(q[24], q[25], q[26], q[27]);
  s1.w = pack4(q[28], q[29], q[30], q[31]);
  uint4* dst = reinterpret_cast<uint4*>(xq + (T * nchunk + c) * 64 * kFragBytes);
  dst[p] = s0;
  dst[p + 32] = s1;
  // token p = 8*qq + 4*g + r  ->  float slot 16*g + 4*qq + r
  da[(T * nchunk + c) * 32 + 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3)] = scale;
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
  if (LAYOUT == Q6K_LAYOUT_EXPANDED) {
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
    // lane p (g = 0) takes k 8g + e = e and 16 + e; lane p + 32 (g = 1) takes 8 + e and 24 + e
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int* a = code + 8 * g;       // half 0 codes a_0..a_7
      const int* b = code + 16 + 8 * g;  // half 1 codes b_0..b_7
      uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w0 |= (uint32_t)((a[t] & 15) | ((a[t + 4] & 15) << 4)) << (8 * t);
        w1 |= (uint32_t)((b[t] & 15) | ((b[t + 4] & 15) << 4)) << (8 * t);
        w2 |= (uint32_t)((a[t] >> 4) | ((a[t + 4] >> 4) << 2) | ((b[t] >> 4) << 4) |
                         ((b[t + 4] >> 4) << 6))
              << (8 * t);
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (tc * 64 + p + 32 * g) * kPackBytes);
      dst[0] = w0;
      dst[1] = w1;
      dst[2] = w2;
    }
    uint32_t s = (uint32_t)(uint8_t)sc0 | ((uint32_t)(uint8_t)sc1 << 8) | ((uint32_t)dbits << 16);
    if (R * kTile + p >= m) s = 0;
    reinterpret_cast<uint32_t*>(scales)[tc * 32 + p] = s;
  }
}

// Layout 0 in-register expand of one lane's 16 codes into the two 8-byte MFMA fragments of
// centered int8.  Per byte: q = nibble | field << 4 (0..63); q - 32 = (q + 0x60) ^ 0x80, which
// neither carries nor borrows across bytes for q <= 63.
__device__ __forceinline__ uint32_t center4(uint32_t nib, uint32_t fld) {
  const uint32_t q = (nib & 0x0F0F0F0Fu) | ((fld & 0x03030303u) << 4);
  return (q + 0x60606060u) ^ 0x80808080u;
}

// ---------------------------------------------------------------------------------------------
// GEMM.  Workgroup = 4 waves = 128 tokens x 128 weight rows; wave (wt, wr) owns token tiles
// 4*bx + 2*wt + {0,1} and row tiles 4*by + 2*wr + {0,1}: four 32x32 output tiles, 64 f32
// accumulators per lane.  Operands come straight from the tiled global buffers (one 16-byte
// load per lane per tile and chunk for int8 operands).
//
// Per chunk and output tile: two v_mfma_i32_32x32x16_i8 (halves 0 and 1), each started from the
// bit pattern of 1.5*2^23 so that the int32 result D is read as the float 1.5*2^23 + D exactly
// (|D| <= 16*127*32 < 2^22).  The rescale of each half is then
//     t = fma(F, dsc, -1.5*2^23*dsc)  (= D*dsc rounded once; the bias product is exact)
//     acc = fma(t, da, acc)
// i.e. the two independent += of the method, four VALU fma per output per chunk.
//
// Output layout of the MFMA: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4 (a token)
// and column l%32 (a weight row).
// ---------------------------------------------------------------------------------------------
template <int LAYOUT, bool SUBDOTS>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint8_t* __restrict__ xq,
                                                      const float* __restrict__ da,
                                                      const uint8_t* __restrict__ wcodes,
                                                      const uint8_t* __restrict__ wscales,
                                                      int64_t n, int64_t m, int64_t nchunk,
                                                      float* __restrict__ y, int64_t ldy,
                                                      int32_t* __restrict__ dots) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = lane & 31;
  const int g = lane >> 5;
  const int64_t T0 = (int64_t)blockIdx.x * 4 + 2 * (wave & 1);
  const int64_t R0 = (int64_t)blockIdx.y * 4 + 2 * (wave >> 1);

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasI;

  float acc[2][2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

  for (int64_t c = 0; c < nchunk; ++c) {
    uint4 a[2];
    float dav[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t tc = (T0 + t) * nchunk + c;
      a[t] = reinterpret_cast<const uint4*>(xq + tc * 64 * kFragBytes)[lane];
      const float4* dp = reinterpret_cast<const float4*>(da + tc * 32 + 16 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = dp[q];
        dav[t][4 * q + 0] = f.x;
        dav[t][4 * q + 1] = f.y;
        dav[t][4 * q + 2] = f.z;
        dav[t][4 * q + 3] = f.w;
      }
    }
    uint4 b[2];
    float dsc0[2], dsc1[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t rc = (R0 + u) * nchunk + c;
      if (LAYOUT == Q6K_LAYOUT_EXPANDED) {
        b[u] = reinterpret_cast<const uint4*>(wcodes + rc * 64 * kFragBytes)[lane];
        const float2 s = reinterpret_cast<const float2*>(wscales)[rc * 32 + p];
        dsc0[u] = s.x;
        dsc1[u] = s.y;
      } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(wcodes + (rc * 64 + lane) * kPackBytes);
        const uint32_t n0 = src[0], n1 = src[1], h = src[2];
        b[u].x = center4(n0, h);
        b[u].y = center4(n0 >> 4, h >> 2);
        b[u].z = center4(n1, h >> 4);
        b[u].w = center4(n1 >> 4, h >> 6);
        const uint32_t s = reinterpret_cast<const uint32_t*>(wscales)[rc * 32 + p];
        const float d = __half2float(__ushort_as_half((unsigned short)(s >> 16)));
        dsc0[u] = d * (float)(int8_t)(s & 255);
        dsc1[u] = d * (float)(int8_t)((s >> 8) & 255);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float nb0 = -kBiasF * dsc0[u];
      const float nb1 = -kBiasF * dsc1[u];
      const long blo = (long)(((uint64_t)b[u].y << 32) | b[u].x);
      const long bhi = (long)(((uint64_t)b[u].w << 32) | b[u].z);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const long alo = (long)(((uint64_t)a[t].y << 32) | a[t].x);
        const long ahi = (long)(((uint64_t)a[t].w << 32) | a[t].z);
        const v16i dlo = __builtin_amdgcn_mfma_i32_32x32x16_i8(alo, blo, bias, 0, 0, 0);
        const v16i dhi = __builtin_amdgcn_mfma_i32_32x32x16_i8(ahi, bhi, bias, 0, 0, 0);
        if (SUBDOTS) {
          const int64_t mcol = (R0 + u) * kTile + p;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t tok = (T0 + t) * kTile + 8 * (r >> 2) + 4 * g + (r & 3);
            if (tok < n && mcol < m) {
              int32_t* o = dots + (tok * m + mcol) * (2 * nchunk) + 2 * c;
              o[0] = dlo[r] - kBiasI;
              o[1] = dhi[r] - kBiasI;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float lo = __builtin_fmaf(__int_as_float(dlo[r]), dsc0[u], nb0);
            acc[t][u][r] = __builtin_fmaf(lo, dav[t][r], acc[t][u][r]);
            const float hi = __builtin_fmaf(__int_as_float(dhi[r]), dsc1[u], nb1);
            acc[t][u][r] = __builtin_fmaf(hi, dav[t][r], acc[t][u][r]);
          }
        }
      }
    }
  }
  if (SUBDOTS) return;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t mcol = (R0 + u) * kTile + p;
      if (mcol >= m) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t tok = (T0 + t) * kTile + 8 * (r >> 2) + 4 * g + (r & 3);
        if (tok < n) y[tok * ldy + mcol] = acc[t][u][r];
      }
    }
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

bool weight_sizes(int64_t m, int64_t k, int layout, size_t* codes, size_t* scales) {
  if (m < 0 || k <= 0 || k % 256 || m > kMaxDim || k > kMaxDim) return false;
  if (layout != Q6K_LAYOUT_PACKED && layout != Q6K_LAYOUT_EXPANDED) return false;
  const int64_t mp = round_up(m, kWgRow);
  if (mp != 0 && k > (int64_t)(SIZE_MAX / 8) / mp) return false;
  if (layout == Q6K_LAYOUT_EXPANDED) {
    *codes = (size_t)mp * (size_t)k;
    *scales = (size_t)mp * (size_t)(k / 16) * sizeof(float);
  } else {
    *codes = (size_t)mp * (size_t)k / 4 * 3;
    *scales = (size_t)mp * (size_t)(k / 32) * 4;
  }
  return true;
}

q6k_status launch_status() {
  return hipGetLastError() == hipSuccess ? Q6K_OK : Q6K_EHIP;
}

template <bool SUBDOTS>
q6k_status gemm_common(const void* xq, const float* da, int64_t n, const void* w, int layout,
                       int64_t m, int64_t k, float* y, int64_t ldy, int32_t* dots, void* stream) {
  if (n < 0 || m < 0) return Q6K_EINVAL;
  if (layout != Q6K_LAYOUT_PACKED && layout != Q6K_LAYOUT_EXPANDED) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  if (n > kMaxDim || m > kMaxDim || k > kMaxDim) return Q6K_ESIZE;
  if (n == 0 || m == 0) return Q6K_OK;
  if (!xq || !da || !w) return Q6K_EINVAL;
  if (!aligned16(xq) || !aligned16(da) || !aligned16(w)) return Q6K_EALIGN;
  if (SUBDOTS) {
    if (!dots) return Q6K_EINVAL;
    if (((uintptr_t)dots & 3) != 0) return Q6K_EALIGN;
  } else {
    if (!y) return Q6K_EINVAL;
    if (ldy < m) return Q6K_EINVAL;
    if (((uintptr_t)y & 3) != 0) return Q6K_EALIGN;
  }
  const int64_t np = round_up(n, kWgTok), mp = round_up(m, kWgRow);
  const int64_t gx = np / kWgTok, gy = mp / kWgRow;
  if (gy > 65535 || gx > INT32_MAX) return Q6K_ESIZE;
  const int64_t nchunk = k / 32;
  size_t codes_bytes, scales_bytes;
  weight_sizes(m, k, layout, &codes_bytes, &scales_bytes);
  const uint8_t* wc = static_cast<const uint8_t*>(w);
  const uint8_t* ws = wc + codes_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)gx, (unsigned)gy), block(256);
  if (layout == Q6K_LAYOUT_EXPANDED)
    hipLaunchKernelGGL((gemm_kernel<Q6K_LAYOUT_EXPANDED, SUBDOTS>), grid, block, 0, s,
                       static_cast<const uint8_t*>(xq), da, wc, ws, n, m, nchunk, y, ldy, dots);
  else
    hipLaunchKernelGGL((gemm_kernel<Q6K_LAYOUT_PACKED, SUBDOTS>), grid, block, 0, s,
                       static_cast<const uint8_t*>(xq), da, wc, ws, n, m, nchunk, y, ldy, dots);
  const q6k_status st = launch_status();
  if (st == Q6K_OK) g_launches[layout].fetch_add(1, std::memory_order_relaxed);
  return st;
}

}  // namespace

extern "C" {

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
  if (n < 0) return Q6K_EINVAL;
  if (k <= 0 || k % 256) return Q6K_ESHAPE;
  size_t need_x, need_d;
  if (!act_sizes(n, k, &need_x, &need_d)) return Q6K_ESIZE;
  if (n == 0) return Q6K_OK;
  if (!x || !xq || !da) return Q6K_EINVAL;
  if (ldx < k) return Q6K_EINVAL;
  if (!aligned16(x) || ldx % 4 || !aligned16(xq) || !aligned16(da)) return Q6K_EALIGN;
  if (xq_bytes < need_x || da_bytes < need_d) return Q6K_ESIZE;
  const int64_t np = round_up(n, kWgTok);
  const int64_t nchunk = k / 32;
  const int64_t gx = np / kTile, gy = (nchunk + 7) / 8;
  if (gx > INT32_MAX || gy > 65535) return Q6K_ESIZE;
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0,
                     static_cast<hipStream_t>(stream), x, n, ldx, nchunk,
                     static_cast<uint8_t*>(xq), da);
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
  if (layout != Q6K_LAYOUT_PACKED && layout != Q6K_LAYOUT_EXPANDED) return Q6K_EINVAL;
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
  if (layout == Q6K_LAYOUT_EXPANDED)
    hipLaunchKernelGGL(expand_kernel<Q6K_LAYOUT_EXPANDED>, grid, block, 0, s,
                       static_cast<const uint8_t*>(w_raw), m, nsb, codes, codes + cb);
  else
    hipLaunchKernelGGL(expand_kernel<Q6K_LAYOUT_PACKED>, grid, block, 0, s,
                       static_cast<const uint8_t*>(w_raw), m, nsb, codes, codes + cb);
  return launch_status();
}

q6k_status q6k_gemm(const void* xq, const float* da, int64_t n, const void* w, int layout,
                    int64_t m, int64_t k, float* y, int64_t ldy, void* stream) {
  return gemm_common<false>(xq, da, n, w, layout, m, k, y, ldy, nullptr, stream);
}

q6k_status q6k_gemm_subdots(const void* xq, const float* da, int64_t n, const void* w, int layout,
                            int64_t m, int64_t k, int32_t* dots, void* stream) {
  return gemm_common<true>(xq, da, n, w, layout, m, k, nullptr, 0, dots, stream);
}

const char* q6k_strerror(int status) {
  switch (status) {
    case Q6K_OK: return "ok";
    case Q6K_EINVAL: return "invalid argument (null pointer, negative size, unknown layout or leading dimension too small)";
    case Q6K_ESHAPE: return "k must be a positive multiple of 256 (whole q6_K super-blocks)";
    case Q6K_EALIGN: return "pointer or leading dimension not 16-byte aligned";
    case Q6K_ESIZE: return "buffer smaller than required, or problem too large";
    case Q6K_EHIP: return "HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}

void q6k_stats(uint64_t out[2]) {
  if (!out) return;
  out[0] = g_launches[0].load(std::memory_order_relaxed);
  out[1] = g_launches[1].load(std::memory_order_relaxed);
}

}  // extern "C"

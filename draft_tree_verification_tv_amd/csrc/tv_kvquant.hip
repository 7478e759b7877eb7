// Quantised key/value caches: the quantisers (FP8 E4M3 rows; 4-bit E2M1 blocks).
//
// The pages reach long contexts in small memory through a quantised KV cache (Lucebox-Hub
// review, aichain-blog.pages.dev, "2. DFlash"); the format here is self-defined: OCP E4M3
// codes (bias 7, largest finite 448, subnormals at exponent 0) with one power-of-two
// scale 2^e per (token, KV head) row, e the smallest exponent with max|x| <= 448 * 2^e.
// Every step is exact except the intended rounding: x * 2^-e (ldexp), then
// round-to-nearest-even onto the E4M3 grid by the hardware conversion. Dequantised values code * 2^e are exact in bfloat16, which is what the
// FP8 attention path feeds to its MFMAs.
#include <cmath>

#include "tv_internal.h"

namespace tv {

namespace {

// E4M3 codes of four values with |y| <= 448, packed little-endian: the hardware
// conversion (OCP E4M3, round to nearest even), then the sign bit cleared on zero codes
// (a negative value that rounds to zero is coded +0). Byte trick: for a 7-bit magnitude
// m, bit 7 of (m + 0x7F) | m is set iff m != 0, and no carry crosses a byte.
__device__ __forceinline__ uint32_t e4m3_pack4(float y0, float y1, float y2, float y3) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  const uint32_t mag = w & 0x7F7F7F7Fu;
  const uint32_t nz = ((mag + 0x7F7F7F7Fu) | mag) & 0x80808080u;
  return w & (nz | 0x7F7F7F7Fu);
}

// 16 lanes per (token, head) row of 128 values, 8 per lane (one 16-byte load, one 8-byte
// store); 16 rows per 256-thread block.
__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ src, int64_t st, int64_t sh,
                                                          int T, int H, uint8_t* __restrict__ codes, int64_t cst,
                                                          int64_t csh, int32_t* __restrict__ exps) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= (int64_t)T * H) return;  // whole 16-lane groups leave together
  const int64_t t = row / H;
  const int h = (int)(row % H);
  const u32x4 w = *reinterpret_cast<const u32x4*>(src + t * st + (int64_t)h * sh + 8 * sub);
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_lo(w[j]);
    x[2 * j + 1] = bf16_hi(w[j]);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int e = 0;
  if (amax > 0.f) {
    int k;
    const float m = frexpf(amax, &k);  // amax = m * 2^k, m in [0.5, 1); 448 = 0.875 * 2^9
    e = m <= 0.875f ? k - 9 : k - 8;
  }
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = ldexpf(x[j], -e);  // exact: a power-of-two scaling
  const uint32_t lo = e4m3_pack4(y[0], y[1], y[2], y[3]);
  const uint32_t hi = e4m3_pack4(y[4], y[5], y[6], y[7]);
  *reinterpret_cast<uint2*>(codes + t * cst + (int64_t)h * csh + 8 * sub) = make_uint2(lo, hi);
  if (sub == 0) exps[row] = e;
}

// ---- 4-bit cache: OCP FP4 (E2M1) elements, blocks of 32 values sharing one power-of-two
// scale 2^e (the block structure of the OCP Microscaling formats), e the smallest
// exponent with max|x| <= 6 * 2^e (0 for an all-zero block), clamped to [-125, 125] so
// that every element value times 2^e is a finite bf16 and 2^e a normal float. Elements
// round x * 2^-e (exact) to the nearest E2M1 value, ties to the even code, saturating at 6
// (reached only where e was clamped); a negative value that rounds to zero is coded +0.
// Element 2j of a row is the low nibble of byte j.

// E2M1 code of y: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0 .. 7); each comparison
// puts an exact midpoint on the side of the even code.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t c = a <= 0.25f ? 0u
                     : a < 0.75f ? 1u
                     : a <= 1.25f ? 2u
                     : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u
                     : a < 3.5f ? 5u
                     : a <= 5.0f ? 6u
                                 : 7u;
  return (y < 0.f && c != 0u) ? (c | 8u) : c;
}

// One thread per 32-value block: 4 threads per (token, head) row of 128 values, 64 rows
// per 256-thread workgroup. Reads 64 bytes, writes 16 bytes of codes and one exponent.
__global__ __launch_bounds__(256) void kv_quantize_mx4_kernel(const uint16_t* __restrict__ src, int64_t st,
                                                              int64_t sh, int T, int H, uint8_t* __restrict__ codes,
                                                              int64_t cst, int64_t csh, int8_t* __restrict__ exps) {
  const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int blk = threadIdx.x & 3;
  if (row >= (int64_t)T * H) return;
  const int64_t t = row / H;
  const int h = (int)(row % H);
  const uint16_t* xs = src + t * st + (int64_t)h * sh + 32 * blk;
  float x[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(xs + 8 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * q + 2 * j] = bf16_lo(w[j]);
      x[8 * q + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
  int e = 0;
  if (amax > 0.f) {
    int k;
    const float m = frexpf(amax, &k);  // amax = m * 2^k, m in [0.5, 1); 6 = 0.75 * 2^3
    e = m <= 0.75f ? k - 3 : k - 2;
    e = min(max(e, -125), 125);
  }
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) out[j >> 3] |= e2m1_code(ldexpf(x[j], -e)) << (4 * (j & 7));
  *reinterpret_cast<u32x4*>(codes + t * cst + (int64_t)h * csh + 16 * blk) = out;
  exps[row * 4 + blk] = (int8_t)e;
}

}  // namespace

hipError_t launch_kv_quantize_mx4(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                                  int64_t csh, int8_t* exps, hipStream_t stream) {
  const int64_t rows = (int64_t)T * H;
  hipLaunchKernelGGL(kv_quantize_mx4_kernel, dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), st, sh, T, H, static_cast<uint8_t*>(codes), cst, csh, exps);
  return hipGetLastError();
}

hipError_t launch_kv_quantize(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                              int64_t csh, int32_t* exps, hipStream_t stream) {
  const int64_t rows = (int64_t)T * H;
  hipLaunchKernelGGL(kv_quantize_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), st, sh, T, H, static_cast<uint8_t*>(codes), cst, csh, exps);
  return hipGetLastError();
}

}  // namespace tv

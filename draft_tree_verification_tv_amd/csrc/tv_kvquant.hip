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

// Rows per 16-lane group in both quantisers: all of a group's loads are issued before any
// row is converted, so each lane keeps that many 16-byte loads in flight. Source and codes
// are streamed (each load and store instruction covers whole 128-byte lines), so both
// carry the non-temporal hint.
constexpr int kQuantRows = 4;

// Row (token, head) index -> its element offset in the source and byte offset in the codes;
// rows < 2^31 (the host checks).
struct RowAt {
  int64_t src, codes;
};
__device__ __forceinline__ RowAt row_at(uint32_t row, int H, int64_t st, int64_t sh, int64_t cst, int64_t csh) {
  const uint32_t t = row / (uint32_t)H, h = row - t * (uint32_t)H;
  return {(int64_t)t * st + (int64_t)h * sh, (int64_t)t * cst + (int64_t)h * csh};
}

// 16 lanes per (token, head) row of 128 values, 8 per lane (one 16-byte load, one 8-byte
// store); kQuantRows rows per group, 16 * kQuantRows rows per 256-thread block (row
// 16 r + g of the block in group g, so that each load instruction covers consecutive rows).
__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ src, int64_t st, int64_t sh,
                                                          int T, int H, uint8_t* __restrict__ codes, int64_t cst,
                                                          int64_t csh, int32_t* __restrict__ exps) {
  const uint32_t rows = (uint32_t)T * (uint32_t)H;
  const uint32_t row0 = blockIdx.x * (16u * kQuantRows) + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  u32x4 w[kQuantRows];
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r) {
    const uint32_t row = row0 + 16u * r;
    w[r] = u32x4{0u, 0u, 0u, 0u};
    if (row < rows)
      w[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(src + row_at(row, H, st, sh, 0, 0).src + 8 * sub));
  }
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r) {
    const uint32_t row = row0 + 16u * r;
    if (row >= rows) break;  // whole 16-lane groups leave together
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(w[r][j]);
      x[2 * j + 1] = bf16_hi(w[r][j]);
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
    typedef uint32_t n32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(n32x2{lo, hi},
                                reinterpret_cast<n32x2*>(codes + row_at(row, H, 0, 0, cst, csh).codes + 8 * sub));
    if (sub == 0) exps[row] = e;
  }
}

// ---- 4-bit cache: OCP FP4 (E2M1) elements, blocks of 32 values sharing one power-of-two
// scale 2^e (the block structure of the OCP Microscaling formats), e the smallest
// exponent with max|x| <= 6 * 2^e (0 for an all-zero block), clamped to [-125, 125] so
// that every element value times 2^e is a finite bf16 and 2^e a normal float. Elements
// round x * 2^-e (exact) to the nearest E2M1 value, ties to the even code, saturating at 6
// (reached only where e was clamped); a negative value that rounds to zero is coded +0.
// Element 2j of a row is the low nibble of byte j.
constexpr int kMxExpLo = -125, kMxExpHi = 125;

// Eight E2M1 codes of a lane's eight bf16 values (four words of value pairs) with the
// block scale 2^e: the hardware conversion divides each value by the scale (exact, a
// power of two) and rounds to the nearest E2M1 value, ties to the even code, saturating
// at 6; pair j goes to byte j, its first value to the low nibble. A negative value that
// rounds to zero comes out as code 8 (-0) and is recoded +0: bit 0 of each nibble of
// t = w | w >> 1 | w >> 2 is the OR of that nibble's three magnitude bits.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// A word as two bf16 values. The word comes in by value: bit-casting a vector element in
// place (w[j] of an ext_vector) yields element 0 whatever j is, with this compiler.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2_t, x); }

__device__ __forceinline__ uint32_t e2m1_pack8(const u32x4& w, float scale) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, as_bf16x2(w[0]), scale, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(w[1]), scale, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(w[2]), scale, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(w[3]), scale, 3);
  const uint32_t zero = ~(c | (c >> 1) | (c >> 2)) & 0x11111111u;
  return c & ~(zero << 3);
}

// The FP8 quantiser's layout: 16 lanes per (token, head) row of 128 values, 8 per lane
// (one 16-byte load, one 4-byte store), so four lanes hold a 32-value block and exchange
// their maxima; kQuantRows rows per group as there.
__global__ __launch_bounds__(256) void kv_quantize_mx4_kernel(const uint16_t* __restrict__ src, int64_t st,
                                                              int64_t sh, int T, int H, uint8_t* __restrict__ codes,
                                                              int64_t cst, int64_t csh, int8_t* __restrict__ exps) {
  const uint32_t rows = (uint32_t)T * (uint32_t)H;
  const uint32_t row0 = blockIdx.x * (16u * kQuantRows) + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  u32x4 w[kQuantRows];
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r) {
    const uint32_t row = row0 + 16u * r;
    w[r] = u32x4{0u, 0u, 0u, 0u};
    if (row < rows)
      w[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(src + row_at(row, H, st, sh, 0, 0).src + 8 * sub));
  }
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r) {
    const uint32_t row = row0 + 16u * r;
    if (row >= rows) break;  // whole 16-lane groups leave together
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[r][j])), fabsf(bf16_hi(w[r][j]))));
    for (int off = 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    int e = 0;
    if (amax > 0.f) {
      int k;
      const float m = frexpf(amax, &k);  // amax = m * 2^k, m in [0.5, 1); 6 = 0.75 * 2^3
      e = m <= 0.75f ? k - 3 : k - 2;
      e = min(max(e, kMxExpLo), kMxExpHi);
    }
    const uint32_t c = e2m1_pack8(w[r], __int_as_float((e + 127) << 23));
    __builtin_nontemporal_store(c,
                                reinterpret_cast<uint32_t*>(codes + row_at(row, H, 0, 0, cst, csh).codes + 4 * sub));
    if ((sub & 3) == 0) exps[(int64_t)row * 4 + (sub >> 2)] = (int8_t)e;
  }
}

}  // namespace

hipError_t launch_kv_quantize_mx4(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                                  int64_t csh, int8_t* exps, hipStream_t stream) {
  const int64_t rows = (int64_t)T * H;
  hipLaunchKernelGGL(kv_quantize_mx4_kernel, dim3((unsigned)((rows + 16 * kQuantRows - 1) / (16 * kQuantRows))),
                     dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), st, sh, T, H, static_cast<uint8_t*>(codes), cst, csh, exps);
  return hipGetLastError();
}

hipError_t launch_kv_quantize(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                              int64_t csh, int32_t* exps, hipStream_t stream) {
  const int64_t rows = (int64_t)T * H;
  hipLaunchKernelGGL(kv_quantize_kernel, dim3((unsigned)((rows + 16 * kQuantRows - 1) / (16 * kQuantRows))),
                     dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), st, sh, T, H, static_cast<uint8_t*>(codes), cst, csh, exps);
  return hipGetLastError();
}

}  // namespace tv

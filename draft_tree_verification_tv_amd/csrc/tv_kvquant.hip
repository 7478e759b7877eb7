// FP8 (E4M3) key/value cache: the quantiser.
//
// The pages reach long contexts in small memory through a quantised KV cache (Lucebox-Hub
// review, aichain-blog.pages.dev, "2. DFlash"); the format here is self-defined: OCP E4M3
// codes (bias 7, largest finite 448, subnormals at exponent 0) with one power-of-two
// scale 2^e per (token, KV head) row, e the smallest exponent with max|x| <= 448 * 2^e.
// Every step is exact except the intended rounding: x * 2^-e (ldexp), then
// round-to-nearest-even onto the E4M3 grid (rintf on the value scaled to its binade's
// integer grid). Dequantised values code * 2^e are exact in bfloat16, which is what the
// FP8 attention path feeds to its MFMAs.
#include <cmath>

#include "tv_internal.h"

namespace tv {

namespace {

// E4M3 code of y, |y| <= 448: nearest code value, ties to the even mantissa.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)rintf(a * 0x1p9f);  // subnormal grid 2^-9; 8 is the smallest normal
  } else {
    int k;
    (void)frexpf(a, &k);                   // a in [2^(k-1), 2^k)
    int E = k - 1;
    uint32_t n = (uint32_t)rintf(ldexpf(a, 3 - E));  // in [8, 16]
    if (n == 16) {
      E += 1;
      n = 8;
    }
    code = ((uint32_t)(E + 7) << 3) | (n - 8);
  }
  if (y < 0.f && code) code |= 0x80u;
  return code;
}

// One wave per (token, head) row of 128 values, two per lane.
__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ src, int64_t st, int64_t sh,
                                                          int T, int H, uint8_t* __restrict__ codes, int64_t cst,
                                                          int64_t csh, int32_t* __restrict__ exps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T * H) return;
  const int t = row / H, h = row % H;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (int64_t)t * st + (int64_t)h * sh + 2 * lane);
  const float x0 = bf16_lo(w), x1 = bf16_hi(w);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int e = 0;
  if (amax > 0.f) {
    int k;
    const float m = frexpf(amax, &k);  // amax = m * 2^k, m in [0.5, 1); 448 = 0.875 * 2^9
    e = m <= 0.875f ? k - 9 : k - 8;
  }
  const uint32_t c0 = e4m3_rne(ldexpf(x0, -e));
  const uint32_t c1 = e4m3_rne(ldexpf(x1, -e));
  *reinterpret_cast<uint16_t*>(codes + (int64_t)t * cst + (int64_t)h * csh + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) exps[(int64_t)t * H + h] = e;
}

}  // namespace

hipError_t launch_kv_quantize(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                              int64_t csh, int32_t* exps, hipStream_t stream) {
  const int rows = T * H;
  hipLaunchKernelGGL(kv_quantize_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), st, sh, T, H, static_cast<uint8_t*>(codes), cst, csh, exps);
  return hipGetLastError();
}

}  // namespace tv

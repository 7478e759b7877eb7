// Measurement probes for the benchmark (libtv_probe.so; declarations in include/tv_probe.h).
// They compute nothing of the verify step: one streams bytes from HBM so that the
// attention kernel's bandwidth can be set against what a plain read achieves on the same
// chip and access pattern; one counts shader clocks against the constant-rate real-time
// counter to give the clock the chip actually runs at under a given load; one times MFMA
// and VALU instruction mixes in shader cycles (how far a wave overlaps the two); one runs
// MFMA streams with LDS reads and VALU work beside them on every CU at once, the mix of
// the attention loop without its dependencies, for the throughput such a mix can reach.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // independent 16-byte loads in flight per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads rows [w / cols * rows_per_wg, ...) of column w % cols: row r of column
// c is row_bytes = 2^row_shift bytes at base + r * row_stride + c * row_bytes. Every thread keeps
// kUnroll 16-byte loads in flight and folds them into an XOR, which the workgroup writes
// to sink[w] (so no load is dead).
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* __restrict__ base, int64_t rows,
                                                               int row_shift, int64_t row_stride, int cols,
                                                               int64_t rows_per_wg, uint32_t* __restrict__ sink) {
  const int w = blockIdx.x;
  const int col = w % cols;
  const int64_t r0 = (int64_t)(w / cols) * rows_per_wg;
  const int64_t r1 = r0 + rows_per_wg < rows ? r0 + rows_per_wg : rows;
  const int cshift = row_shift - 4;  // 16-byte chunks per row = 2^cshift
  const int chunks = (int)((r1 - r0) << cshift);
  const char* cb = base + r0 * row_stride + ((int64_t)col << row_shift);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int k0 = 0; k0 < chunks; k0 += kThreads * kUnroll) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int k = k0 + u * kThreads + (int)threadIdx.x;
      if (k >= chunks) k = chunks - 1;  // clamped: every load is in bounds and unconditional
      x[u] = *reinterpret_cast<const u32x4*>(cb + (int64_t)(k >> cshift) * row_stride + ((k & ((1 << cshift) - 1)) << 4));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kThreads / 64; ++i) r ^= red[i];
    sink[w] = r;
  }
}

// One wave: shader-clock cycles and real-time ticks over a spin of `ticks` real-time ticks.
// The spin ends when the real-time counter has advanced that far, so it always ends.
__global__ __launch_bounds__(64) void clock_kernel(uint64_t* __restrict__ out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  while (r1 - r0 < ticks) r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

// One workgroup: `iters` iterations of eight 32x32x16 bf16 MFMAs (four independent
// accumulators) and/or VALU work, in the instruction mix `MODE` names; each wave stores
// its shader-clock cycle count. Modes: 0 MFMA only; 1 64 fp32 FMAs per iteration (eight
// independent chains); 2 MFMA each followed by 8 FMAs; 3 MFMA each followed by 4 exp2 and
// 4 FMAs; 4 64 exp2 per iteration; 5 MFMA each followed by 2 exp2 and 6 FMAs. The
// interleaved modes are kept in that order by scheduling-group barriers.
template <int MODE>
__global__ __launch_bounds__(512) void coissue_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                      uint64_t* __restrict__ cyc, int iters) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(in[lane] * i);
    b[i] = (__bf16)(in[lane + 1] * i);
  }
  f32x16 acc[4];
  for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = in[j + lane];
  const float c0 = in[100], c1 = in[101];
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (MODE != 1 && MODE != 4) acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
      if (MODE == 1 || MODE == 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], c0, c1);
      }
      if (MODE == 3) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
#pragma unroll
        for (int j = 4; j < 8; ++j) x[j] = __builtin_fmaf(x[j], c0, c1);
      }
      if (MODE == 4) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
      }
      if (MODE == 5) {
#pragma unroll
        for (int j = 0; j < 2; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
#pragma unroll
        for (int j = 2; j < 8; ++j) x[j] = __builtin_fmaf(x[j], c0, c1);
      }
      if (MODE == 2 || MODE == 3 || MODE == 5) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
  for (int k = 0; k < 4; ++k)
    for (int e = 0; e < 16; ++e) sum += acc[k][e];
  for (int j = 0; j < 8; ++j) sum += x[j];
  out[threadIdx.x] = sum;
  if (lane == 0) cyc[threadIdx.x >> 6] = t1 - t0;
}

// Every CU at once: `iters` iterations of eight v_mfma_f32_32x32x16_bf16 on four
// independent accumulators. LSTEP 1: each MFMA's A operand is a fresh 16-byte LDS read per
// lane (1 KB per wave); LSTEP 2: every second one is (0.5 KB per MFMA); 0: none. LSTEP 3-5
// read 1 KB per MFMA in the attention tiles' layout (64 rows of 256 bytes, the K and V
// chunk swizzles, four 16 KB stages): 3, the attention loop's own mix, alternates a K
// fragment (one 128-bit read per lane, rows = lane % 32) with a V^T fragment (two
// ds_read_b64_tr_b16 per lane); 4 reads only V^T fragments, 5 only K fragments. LSTEP 6
// and 7 model a wave of 64 rows, where each fragment feeds two MFMAs (one per 32-row
// half): 6 reads K, -, V^T, - per four MFMAs (0.5 KB per MFMA); 7 reads K, K, V^T, - (the
// second K read standing for a Q fragment kept in LDS, 0.75 KB per MFMA). VALU: each
// MFMA is followed by one exp2 and four FMAs on independent values. Nothing depends on
// anything else, so this is the most such a mix can reach. Wave 0 of workgroup 0 records
// shader cycles and real-time ticks around its loop in clk[0], clk[1].
template <int LSTEP, bool VALU>
__global__ __launch_bounds__(512) void mix_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                  uint64_t* __restrict__ clk, int iters) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  __shared__ __align__(16) char lds[65536];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 65536 / 4; i += blockDim.x) reinterpret_cast<float*>(lds)[i] = in[i & 1023];
  __syncthreads();
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(in[lane] * i);
    b[i] = (__bf16)(in[lane + 1] * i);
  }
  float x[4];
  for (int j = 0; j < 4; ++j) x[j] = in[j + lane] * 1e-3f;
  const float c0 = in[100], c1 = in[101];
  uint64_t r0 = 0, t0 = 0;
  if (blockIdx.x == 0 && tid == 0) {
    r0 = __builtin_amdgcn_s_memrealtime();
    t0 = __builtin_amdgcn_s_memtime();
  }
  // Attention-tile offsets: K row ql, chunk 2*s + grp; V^T rows 4*grp + i16/4 (and +8),
  // head-dim columns db*32 + g16*16 + 4*(i16%4); both with their tiles' chunk swizzles.
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int ql = lane & 31, grp = lane >> 5, i16 = lane & 15, g16 = (lane >> 4) & 1;
  int koff[4], voff[4];
  for (int s = 0; s < 4; ++s) koff[s] = ql * 256 + (((2 * s + grp) ^ (ql & 15)) << 4);
  {
    const int row = 4 * grp + (i16 >> 2), sw = (0xCA60 >> ((row & 3) * 4)) & 15;
    for (int db = 0; db < 4; ++db)
      voff[db] = row * 256 + (((db * 4 + g16 * 2 + ((i16 & 3) >> 1)) ^ sw) << 4) + (i16 & 1) * 8;
  }
  f32x16 acc[4];
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
    const char* stage = lds + (it & 3) * 16384 + ((it >> 2) & 1) * 8192;  // + < 8 KB of rows
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      bf16x8 aa = a;
      const bool kread = LSTEP == 5 || (LSTEP == 3 && m % 2 == 0) || (LSTEP == 6 && m % 4 == 0) ||
                         (LSTEP == 7 && m % 4 < 2);
      const bool vread = LSTEP == 4 || (LSTEP == 3 && m % 2 == 1) || ((LSTEP == 6 || LSTEP == 7) && m % 4 == 2);
      if ((LSTEP == 1 || LSTEP == 2) && m % LSTEP == 0) {
        const int off = ((it * 8 + m) * 1024 + lane * 16 + wave * 64) & (65536 - 16);
        aa = *reinterpret_cast<const bf16x8*>(lds + off);
      } else if (kread) {
        aa = *reinterpret_cast<const bf16x8*>(stage + koff[(m >> 1) & 3]);
      } else if (vread) {
        const char* a0 = stage + voff[(m >> 1) & 3];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * 256));
        aa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, b, acc[m & 3], 0, 0, 0);
      if (VALU) {
        x[0] = __builtin_amdgcn_exp2f(x[0] * 1e-3f);
#pragma unroll
        for (int j = 1; j < 4; ++j) x[j] = __builtin_fmaf(x[j], c0, c1);
      }
    }
  }
  float sum = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 16; ++e) sum += acc[j][e];
  for (int j = 0; j < 4; ++j) sum += x[j];
  out[(int64_t)blockIdx.x * blockDim.x + tid] = sum;
  if (blockIdx.x == 0 && tid == 0) {
    clk[0] = __builtin_amdgcn_s_memtime() - t0;
    clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace

extern "C" {

int tv_probe_stream_read(const void* base, int64_t rows, int row_bytes, int64_t row_stride, int cols,
                         int64_t rows_per_wg, uint32_t* sink, void* stream) {
  if (!base || !sink || rows < 1 || cols < 1 || rows_per_wg < 1) return 1;
  int shift = 4;
  while (shift < 16 && (1 << shift) < row_bytes) ++shift;
  if (row_bytes != (1 << shift) || row_stride < (int64_t)row_bytes * cols || row_stride % 16 ||
      (reinterpret_cast<uintptr_t>(base) & 15u))
    return 1;
  if ((rows_per_wg << (shift - 4)) > INT32_MAX / 2) return 1;
  const int64_t groups = (rows + rows_per_wg - 1) / rows_per_wg;
  if (groups * cols > INT32_MAX) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)(groups * cols)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(base), rows, shift, row_stride,
                     cols, rows_per_wg, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int tv_probe_coissue(int mode, int threads, int iters, const float* in, float* out, uint64_t* cycles,
                     void* stream) {
  if (!in || !out || !cycles || iters < 1 || (threads != 64 && threads != 256 && threads != 512)) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(coissue_kernel<0>, dim3(1), dim3(threads), 0, st, in, out, cycles, iters); break;
    case 1: hipLaunchKernelGGL(coissue_kernel<1>, dim3(1), dim3(threads), 0, st, in, out, cycles, iters); break;
    case 2: hipLaunchKernelGGL(coissue_kernel<2>, dim3(1), dim3(threads), 0, st, in, out, cycles, iters); break;
    case 3: hipLaunchKernelGGL(coissue_kernel<3>, dim3(1), dim3(threads), 0, st, in, out, cycles, iters); break;
    case 4: hipLaunchKernelGGL(coissue_kernel<4>, dim3(1), dim3(threads), 0, st, in, out, cycles, iters); break;
    case 5: hipLaunchKernelGGL(coissue_kernel<5>, dim3(1), dim3(threads), 0, st, in, out, cycles, iters); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int tv_probe_clock(uint64_t* out, uint64_t ticks, void* stream) {
  if (!out || ticks < 1 || ticks > 100000000ull) return 1;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out, ticks);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int tv_probe_mix(int lds_step, int valu, int threads, int workgroups, int iters, const float* in, float* out,
                 uint64_t* clk, void* stream) {
  if (!in || !out || !clk || iters < 1 || workgroups < 1 || workgroups > 65536 || (threads != 256 && threads != 512) ||
      lds_step < 0 || lds_step > 7 || (valu != 0 && valu != 1))
    return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g(workgroups), b(threads);
  typedef void (*mix_fn)(const float*, float*, uint64_t*, int);
  static const mix_fn fns[2][8] = {
      {mix_kernel<0, false>, mix_kernel<1, false>, mix_kernel<2, false>, mix_kernel<3, false>,
       mix_kernel<4, false>, mix_kernel<5, false>, mix_kernel<6, false>, mix_kernel<7, false>},
      {mix_kernel<0, true>, mix_kernel<1, true>, mix_kernel<2, true>, mix_kernel<3, true>, mix_kernel<4, true>,
       mix_kernel<5, true>, mix_kernel<6, true>, mix_kernel<7, true>}};
  hipLaunchKernelGGL(fns[valu][lds_step], g, b, 0, st, in, out, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"

// Row argmax of the target logits (greedy verification compares each draft token with
// the temperature-0 sample, i.e. the argmax; DFlash contributor guide, discosf.com/news/
// 4742660, "Coding conventions"). Lowest index on ties, bit exact.
//
// HBM-bound scan. Each workgroup owns one slice of one row; every thread issues four
// independent 16-byte loads before touching any of them, so each CU keeps 64 KB in
// flight. Per vector only a max and one compare are spent; the element index is looked
// up once, in the winning vector, which is still in registers. Partial (value, index)
// pairs go to the workspace and the last workgroup of the row, found with a counter,
// reduces them and restores the counter to zero.
#include <climits>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;

struct Best {
  float v;
  int i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
  // b wins on a larger value, or an equal value at a lower index.
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ Best wave_reduce(Best x) {
  for (int off = 32; off > 0; off >>= 1) {
    Best o;
    o.v = __shfl_xor(x.v, off);
    o.i = __shfl_xor(x.i, off);
    x = better(x, o);
  }
  return x;
}

template <bool kF32>
__device__ __forceinline__ void unpack(const u32x4 w, float (&x)[8]) {
  if constexpr (kF32) {
    x[0] = __uint_as_float(w[0]);
    x[1] = __uint_as_float(w[1]);
    x[2] = __uint_as_float(w[2]);
    x[3] = __uint_as_float(w[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(w[j]);
      x[2 * j + 1] = bf16_hi(w[j]);
    }
  }
}

template <bool kF32>
__device__ __forceinline__ float load_one(const char* row, int e) {
  if constexpr (kF32) return reinterpret_cast<const float*>(row)[e];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[e] << 16);
}

template <bool kF32, bool kVec>
__global__ __launch_bounds__(kBlock) void argmax_kernel(const char* __restrict__ logits, int V,
                                                        int64_t row_bytes, int chunks, int chunk_len,
                                                        int32_t* __restrict__ tok,
                                                        float* __restrict__ part_v,
                                                        int* __restrict__ part_i,
                                                        unsigned* __restrict__ counters) {
  constexpr int EPV = kVec ? (kF32 ? 4 : 8) : 1;  // elements per 16-byte load
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const char* rp = logits + (int64_t)row * row_bytes;
  const int begin = c * chunk_len;
  const int end = min(V, begin + chunk_len);

  Best b{-INFINITY, INT_MAX};
  if constexpr (kVec) {
    // kUnroll independent 16-byte loads per thread, issued before any compare. Thread
    // tid owns vectors begin + (u * kBlock + tid) * EPV, ascending in u.
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = begin + (u * kBlock + (int)threadIdx.x) * EPV;
      raw[u] = u32x4{0u, 0u, 0u, 0u};
      if (e + EPV <= end) raw[u] = *reinterpret_cast<const u32x4*>(rp + (int64_t)e * (kF32 ? 4 : 2));
    }
    int bu = -1;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = begin + (u * kBlock + (int)threadIdx.x) * EPV;
      if (e + EPV <= end) {
        float x[8];
        unpack<kF32>(raw[u], x);
        float m = x[0];
#pragma unroll
        for (int j = 1; j < EPV; ++j) m = fmaxf(m, x[j]);
        if (bu < 0 || m > b.v) {
          b.v = m;
          bu = u;
        }
      }
    }
    // Element index inside the winning vector (first element equal to the maximum).
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u == bu) {
        float x[8];
        unpack<kF32>(raw[u], x);
        const int e = begin + (u * kBlock + (int)threadIdx.x) * EPV;
#pragma unroll
        for (int j = EPV - 1; j >= 0; --j)
          if (x[j] == b.v) b.i = e + j;
      }
    }
    // A vector cut by the end of the row is read element by element (it is the
    // thread's last and highest-indexed vector, so ascending order is kept).
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = begin + (u * kBlock + (int)threadIdx.x) * EPV;
      if (e < end && e + EPV > end) {
        for (int j = e; j < end; ++j) {
          const float x = load_one<kF32>(rp, j);
          if (b.i == INT_MAX || x > b.v) {
            b.v = x;
            b.i = j;
          }
        }
      }
    }
    if (b.i == INT_MAX) b.v = -INFINITY;
  } else {
    for (int e = begin + (int)threadIdx.x; e < end; e += kBlock) {
      const float x = load_one<kF32>(rp, e);
      if (b.i == INT_MAX || x > b.v) {
        b.v = x;
        b.i = e;
      }
    }
    if (b.i == INT_MAX) b.v = -INFINITY;
  }

  __shared__ float sv[kBlock / 64];
  __shared__ int si[kBlock / 64];
  __shared__ bool last;
  b = wave_reduce(b);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = b.v;
    si[wave] = b.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Best r{sv[0], si[0]};
    for (int w = 1; w < kBlock / 64; ++w) r = better(r, Best{sv[w], si[w]});
    if (chunks == 1) {
      tok[row] = r.i == INT_MAX ? -1 : r.i;
      last = false;
    } else {
      part_v[(int64_t)row * chunks + c] = r.v;
      part_i[(int64_t)row * chunks + c] = r.i;
      __threadfence();
      last = atomicAdd(&counters[row], 1u) == (unsigned)(chunks - 1);
    }
  }
  __syncthreads();
  if (!last) return;
  // Last workgroup of this row: reduce the row's partials.
  __threadfence();
  Best r{-INFINITY, INT_MAX};
  for (int j = threadIdx.x; j < chunks; j += kBlock) {
    const float v = __hip_atomic_load(&part_v[(int64_t)row * chunks + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int ix = __hip_atomic_load(&part_i[(int64_t)row * chunks + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r = better(r, Best{v, ix});
  }
  r = wave_reduce(r);
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = r.v;
    si[wave] = r.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Best f{sv[0], si[0]};
    for (int w = 1; w < kBlock / 64; ++w) f = better(f, Best{sv[w], si[w]});
    tok[row] = f.i == INT_MAX ? -1 : f.i;
    atomicExch(&counters[row], 0u);
  }
}

}  // namespace

ArgmaxPlan argmax_plan(int N, int V, int dtype, bool vec) {
  // One slice = kUnroll 16-byte loads per thread: 8192 bf16 or 4096 fp32 elements. The
  // scalar path (rows not 16-byte aligned) uses 4096-element slices.
  (void)N;
  ArgmaxPlan p;
  p.chunk_len = (vec && dtype == TV_BF16) ? kBlock * 8 * kUnroll : kBlock * 4 * kUnroll;
  p.chunks = (V + p.chunk_len - 1) / p.chunk_len;
  return p;
}

size_t argmax_workspace_bytes(int N, int V) {
  const ArgmaxPlan p = argmax_plan(N, V, TV_F32, false);  // the most slices of any path
  const size_t parts = (size_t)N * p.chunks;
  size_t bytes = parts * sizeof(float);
  bytes = (bytes + 255) / 256 * 256;
  bytes += parts * sizeof(int);
  bytes = (bytes + 255) / 256 * 256;
  bytes += (size_t)N * sizeof(unsigned);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_argmax(const void* logits, int dtype, int N, int V, int64_t row_stride, int32_t* tok,
                         void* workspace, hipStream_t stream) {
  const int esize = dtype == TV_F32 ? 4 : 2;
  const int64_t row_bytes = row_stride * esize;
  const bool vec = ((uintptr_t)logits % 16 == 0) && (row_bytes % 16 == 0);
  const ArgmaxPlan p = argmax_plan(N, V, dtype, vec);
  const size_t parts = (size_t)N * argmax_plan(N, V, TV_F32, false).chunks;
  char* ws = static_cast<char*>(workspace);
  float* part_v = reinterpret_cast<float*>(ws);
  size_t off = (parts * sizeof(float) + 255) / 256 * 256;
  int* part_i = reinterpret_cast<int*>(ws + off);
  off += (parts * sizeof(int) + 255) / 256 * 256;
  unsigned* counters = reinterpret_cast<unsigned*>(ws + off);

  const dim3 grid(p.chunks, N);
  const char* lg = static_cast<const char*>(logits);
  if (dtype == TV_F32) {
    if (vec)
      hipLaunchKernelGGL((argmax_kernel<true, true>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes,
                         p.chunks, p.chunk_len, tok, part_v, part_i, counters);
    else
      hipLaunchKernelGGL((argmax_kernel<true, false>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes,
                         p.chunks, p.chunk_len, tok, part_v, part_i, counters);
  } else {
    if (vec)
      hipLaunchKernelGGL((argmax_kernel<false, true>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes,
                         p.chunks, p.chunk_len, tok, part_v, part_i, counters);
    else
      hipLaunchKernelGGL((argmax_kernel<false, false>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes,
                         p.chunks, p.chunk_len, tok, part_v, part_i, counters);
  }
  return hipGetLastError();
}

}  // namespace tv

// Row argmax of the target logits (greedy verification compares each draft token with
// the temperature-0 sample, i.e. the argmax; DFlash contributor guide, discosf.com/news/
// 4742660, "Coding conventions"). Lowest index on ties, bit exact.
//
// HBM-bound scan. Each workgroup owns one slice of one row and streams it with 16-byte
// loads. Per thread, only the running maximum and the position of the first vector that
// raised it are tracked (a max over the vector plus one compare); the element index is
// recovered once at the end by re-reading that single vector. Partial (value, index)
// pairs go to the workspace and the last workgroup of the row, found with a counter,
// reduces them and restores the counter to zero.
#include <climits>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kBlock = 256;
constexpr int kTargetWGs = 1024;

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

template <bool kF32, bool kVec>
__device__ __forceinline__ void load_vec(const char* row, int e, float (&x)[8]) {
  if constexpr (kF32) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + (int64_t)e * 4);
    x[0] = __uint_as_float(w[0]);
    x[1] = __uint_as_float(w[1]);
    x[2] = __uint_as_float(w[2]);
    x[3] = __uint_as_float(w[3]);
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + (int64_t)e * 2);
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
  constexpr int EPV = kVec ? (kF32 ? 4 : 8) : 1;  // elements per load
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const char* rp = logits + (int64_t)row * row_bytes;
  const int begin = c * chunk_len;
  const int end = min(V, begin + chunk_len);

  float bv = -INFINITY;
  int bvec = INT_MAX;  // start of the first vector holding bv
  int e = begin + threadIdx.x * EPV;
  if (e < end) bvec = e;
  if constexpr (kVec) {
    // Full vectors, two in flight per iteration.
    for (; e + EPV <= end; e += kBlock * EPV) {
      float x[8];
      load_vec<kF32, kVec>(rp, e, x);
      float m = x[0];
#pragma unroll
      for (int j = 1; j < EPV; ++j) m = fmaxf(m, x[j]);
      if (m > bv) {
        bv = m;
        bvec = e;
      }
    }
  }
  // Ragged tail (or the whole slice when rows are not 16-byte aligned).
  for (; e < end; e += kBlock * EPV) {
    const int lim = min(EPV, end - e);
    float m = load_one<kF32>(rp, e);
    for (int j = 1; j < lim; ++j) m = fmaxf(m, load_one<kF32>(rp, e + j));
    if (m > bv) {
      bv = m;
      bvec = e;
    }
  }
  Best b{bv, INT_MAX};
  if (bvec != INT_MAX) {
    const int lim = min(EPV, end - bvec);
    for (int j = lim - 1; j >= 0; --j)
      if (load_one<kF32>(rp, bvec + j) == bv) b.i = bvec + j;
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
    const float v = __builtin_nontemporal_load(&part_v[(int64_t)row * chunks + j]);
    const int ix = __builtin_nontemporal_load(&part_i[(int64_t)row * chunks + j]);
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

ArgmaxPlan argmax_plan(int N, int V) {
  ArgmaxPlan p;
  int chunks = (kTargetWGs + N - 1) / N;
  const int max_chunks = V / 4096 > 0 ? V / 4096 : 1;  // keep slices >= 4096 elements
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  int len = (V + chunks - 1) / chunks;
  len = (len + 7) / 8 * 8;
  p.chunks = (V + len - 1) / len;
  p.chunk_len = len;
  return p;
}

size_t argmax_workspace_bytes(int N, int V) {
  const ArgmaxPlan p = argmax_plan(N, V);
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
  const ArgmaxPlan p = argmax_plan(N, V);
  const size_t parts = (size_t)N * p.chunks;
  char* ws = static_cast<char*>(workspace);
  float* part_v = reinterpret_cast<float*>(ws);
  size_t off = (parts * sizeof(float) + 255) / 256 * 256;
  int* part_i = reinterpret_cast<int*>(ws + off);
  off += (parts * sizeof(int) + 255) / 256 * 256;
  unsigned* counters = reinterpret_cast<unsigned*>(ws + off);

  const int esize = dtype == TV_F32 ? 4 : 2;
  const int64_t row_bytes = row_stride * esize;
  const bool vec = ((uintptr_t)logits % 16 == 0) && (row_bytes % 16 == 0);
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

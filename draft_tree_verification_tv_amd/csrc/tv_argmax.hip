// Row argmax of the target logits (greedy verification compares each draft token with
// the temperature-0 sample, i.e. the argmax; DFlash contributor guide, discosf.com/news/
// 4742660, "Coding conventions"). Lowest index on ties, bit exact.
//
// HBM-bound scan in two launches:
//   1. argmax_partial: grid (slices, rows). Every thread issues four independent 16-byte
//      loads (addresses clamped into the slice, so no load is conditional and all four
//      are in flight together), keeps only a per-vector max and one compare, and looks up
//      the element index once, in the winning vector that is still in registers. The
//      workgroup's (value, index) goes to the workspace as one 64-bit ordered key (or
//      straight to tok when a row is a single slice).
//   2. argmax_final (one wave per row) or, for tv_argmax_accept, argmax_accept_kernel
//      (one workgroup: the largest key of every row, then the acceptance walk).
// The key orders (value, index) so that the largest key is the row maximum at its lowest
// index: the high word is the value's bits mapped to an unsigned order (-0.0 first made
// +0.0, so the two tie as floats do), the low word the complement of the index. The kernel
// boundary orders the two launches, so no atomics, fences or counters are needed and the
// workspace needs no initialisation. A one-launch form, in which each workgroup folds its
// key into the row's with an atomic maximum and the workgroup completing the last row
// walks the tree, was measured slower: its chain of device-scope atomics takes longer than
// the kernel boundary.
#include <climits>
#include <cmath>

#include "tv_accept_wave.h"
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

// This thread's best (value, index) over its part of elements [begin, end) of the row at
// rp; {-inf, INT_MAX} when it has no element.
template <bool kF32, bool kVec>
__device__ __forceinline__ Best slice_scan(const char* __restrict__ rp, int begin, int end) {
  constexpr int EPV = kVec ? (kF32 ? 4 : 8) : 1;  // elements per 16-byte load
  constexpr int ESZ = kF32 ? 4 : 2;
  const int tid = threadIdx.x;
  Best b{-INFINITY, INT_MAX};
  bool have = false;
  if constexpr (kVec) {
    if (end - begin >= EPV) {
      u32x4 raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e = begin + (u * kBlock + tid) * EPV;
        const int ea = (e + EPV <= end) ? e : begin;  // clamped: always a full vector in the slice
        // the logits are read once: each wave's load covers 1 KB of whole lines, streamed
        raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp + (int64_t)ea * ESZ));
      }
      int bu = -1;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e = begin + (u * kBlock + tid) * EPV;
        float x[8];
        unpack<kF32>(raw[u], x);
        float m = x[0];
#pragma unroll
        for (int j = 1; j < EPV; ++j) m = fmaxf(m, x[j]);
        if (e + EPV <= end && (bu < 0 || m > b.v)) {
          b.v = m;
          bu = u;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (u == bu) {
          float x[8];
          unpack<kF32>(raw[u], x);
          const int e = begin + (u * kBlock + tid) * EPV;
#pragma unroll
          for (int j = EPV - 1; j >= 0; --j)
            if (x[j] == b.v) b.i = e + j;
        }
      }
      have = b.i != INT_MAX;
    }
    // A vector cut by the end of the row is read element by element; it is the
    // thread's highest-indexed vector, so ascending order is kept.
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = begin + (u * kBlock + tid) * EPV;
      if (e < end && e + EPV > end) {
        for (int j = e; j < end; ++j) {
          const float x = load_one<kF32>(rp, j);
          if (!have || x > b.v) {
            b.v = x;
            b.i = j;
            have = true;
          }
        }
      }
    }
  } else {
    for (int e = begin + tid; e < end; e += kBlock) {
      const float x = load_one<kF32>(rp, e);
      if (!have || x > b.v) {
        b.v = x;
        b.i = e;
        have = true;
      }
    }
  }
  if (!have) b = Best{-INFINITY, INT_MAX};

  return b;
}

// Workgroup reduction of slice_scan results; the result is valid in thread 0.
__device__ __forceinline__ Best block_best(Best b) {
  __shared__ float sv[kBlock / 64];
  __shared__ int si[kBlock / 64];
  b = wave_reduce(b);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = b.v;
    si[wave] = b.i;
  }
  __syncthreads();
  Best r{sv[0], si[0]};
  for (int w = 1; w < kBlock / 64; ++w) r = better(r, Best{sv[w], si[w]});
  return r;
}

// 64-bit key ordering (value, index) as described at the top of the file.
__device__ __forceinline__ uint64_t order_key(Best b) {
  const float v = b.v == 0.f ? 0.f : b.v;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)b.i;
}

// The token a row's largest key stands for (-1 for a row without elements).
__device__ __forceinline__ int32_t key_token(uint64_t key) {
  const uint32_t idx = ~(uint32_t)key;
  return (key == 0ull || idx == (uint32_t)INT_MAX) ? -1 : (int32_t)idx;
}

// Thread 0 stores the workgroup result of slice c of row `row`.
__device__ __forceinline__ void store_slice(Best r, int row, int c, int chunks, int32_t* __restrict__ tok,
                                            uint64_t* __restrict__ part) {
  if (threadIdx.x == 0) {
    if (chunks == 1)
      tok[row] = r.i == INT_MAX ? -1 : r.i;
    else
      part[(int64_t)row * chunks + c] = order_key(r);
  }
}

template <bool kF32, bool kVec>
__global__ __launch_bounds__(kBlock) void argmax_partial(const char* __restrict__ logits, int V, int64_t row_bytes,
                                                         int chunks, int chunk_len, int32_t* __restrict__ tok,
                                                         uint64_t* __restrict__ part) {
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const char* rp = logits + (int64_t)row * row_bytes;
  const int begin = c * chunk_len;
  store_slice(block_best(slice_scan<kF32, kVec>(rp, begin, min(V, begin + chunk_len))), row, c, chunks, tok, part);
}

// One wave per row: the row's largest slice key.
__global__ __launch_bounds__(256) void argmax_final(int N, int chunks, const uint64_t* __restrict__ part,
                                                    int32_t* __restrict__ tok) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  uint64_t k = 0;
  for (int j = lane; j < chunks; j += 64) {
    const uint64_t x = part[(int64_t)row * chunks + j];
    k = x > k ? x : k;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  if (lane == 0) tok[row] = key_token(k);
}

// ---- sampled targets (temperature > 0)
//
// The target's token for node i is a sample from softmax(logits[i] / T), drawn as the
// lowest index of the largest logit / T + G with Gumbel noise G = -ln(-ln u). The uniforms
// come from Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC 2011): key (seed lo, seed hi), counter (v / 4, node, offset lo, offset
// hi); word v % 4 gives u = ((word >> 9) + 0.5) / 2^23, exact in float32.
//
// The kernel ranks log2-domain scores, logit * log2(e) / T - log2(-log2 u). That is
// (score - ln ln 2) / ln 2 for the natural-log score above: an increasing map, so the
// argmax is the same, and it costs one fma and two hardware log2 instructions per entry.
// u >= 2^-24 and -log2 u >= 2^-24 / ln 2, so neither logarithm sees a denormal.

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

struct SampleKey {
  uint32_t k0, k1, o0, o1;  // seed and offset halves
  float c;                  // log2(e) / temperature
};

__device__ __forceinline__ float gumbel_score(float x, uint32_t word, float c) {
  const float u = ((float)(word >> 9) + 0.5f) * 0x1p-23f;
  return __builtin_fmaf(x, c, -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u)));
}

// Grid (slices, rows), 256 threads; the slice layout and outputs are those of
// argmax_partial. Each thread scores eight consecutive entries per step (two Philox
// blocks); a row that is not 16-byte aligned is read element by element.
// This thread's best (Gumbel score, index) over its entries of [begin, end) of row `row`.
// Entries [e, e + 8): e is a multiple of 8 relative to the row, so the two Philox blocks
// are (e / 4) and (e / 4 + 1).
template <bool kF32, bool kVec>
__device__ __forceinline__ Best sample_scan(const char* __restrict__ rp, int begin, int end, int row,
                                            const SampleKey& key) {
  constexpr int ESZ = kF32 ? 4 : 2;
  const int tid = threadIdx.x;
  Best b{-INFINITY, INT_MAX};
  for (int e = begin + tid * 8; e < end; e += kBlock * 8) {
    float x[8];
    if (kVec && e + 8 <= end) {
      if constexpr (kF32) {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(rp + (int64_t)e * ESZ);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(rp + (int64_t)e * ESZ + 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = __uint_as_float(w0[j]);
          x[4 + j] = __uint_as_float(w1[j]);
        }
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(rp + (int64_t)e * ESZ);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = bf16_lo(w[j]);
          x[2 * j + 1] = bf16_hi(w[j]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (e + j < end) ? load_one<kF32>(rp, e + j) : -INFINITY;
    }
    const u32x4 r0 = philox4x32_10((uint32_t)(e >> 2), (uint32_t)row, key.o0, key.o1, key.k0, key.k1);
    const u32x4 r1 = philox4x32_10((uint32_t)(e >> 2) + 1u, (uint32_t)row, key.o0, key.o1, key.k0, key.k1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (e + j < end) {
        const float sc = gumbel_score(x[j], j < 4 ? r0[j] : r1[j - 4], key.c);
        if (sc > b.v || b.i == INT_MAX) {
          b.v = sc;
          b.i = e + j;
        }
      }
    }
  }

  return b;
}

template <bool kF32, bool kVec>
__global__ __launch_bounds__(kBlock) void sample_partial(const char* __restrict__ logits, int V, int64_t row_bytes,
                                                         int chunks, int chunk_len, SampleKey key,
                                                         int32_t* __restrict__ tok, uint64_t* __restrict__ part) {
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const char* rp = logits + (int64_t)row * row_bytes;
  const int begin = c * chunk_len;
  store_slice(block_best(sample_scan<kF32, kVec>(rp, begin, min(V, begin + chunk_len), row, key)), row, c, chunks,
              tok, part);
}

// One workgroup finishes the verify step: thread i takes node row i's largest slice key
// (loads batched 32 slices at a time, all unconditional, indices clamped: a repeated key
// cannot change the maximum), keeps the token in LDS and runs the acceptance walk on the
// tokens (the walk of tv_accept). The draft and parent entries and the first batch of keys
// are loaded together, ahead of the tree preprocessing, so that their round trips overlap.
// With a single slice per row the slice kernel already wrote tok.
__global__ __launch_bounds__(kBlock) void argmax_accept_kernel(
    int N, int chunks, const uint64_t* __restrict__ part, int32_t* tok, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ draft, int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ accept_tokens, int32_t* __restrict__ bonus, int32_t* dev_error) {
  constexpr int kBatch = 32;  // a bf16 row of up to 262144 values in one round trip
  __shared__ uint64_t anc[kMaxNodes * kAncWords];
  __shared__ int par[kMaxNodes];
  __shared__ int jmp[kMaxNodes];
  __shared__ uint64_t okw[kAncWords];
  __shared__ uint32_t red[kBlock / 64];
  __shared__ int32_t tok_s[kMaxNodes];
  const int i = threadIdx.x;
  const int draft_i = i < N ? draft[i] : 0;
  const int parent_i = i < N ? parent[i] : -1;
  const bool reduce = i < N && chunks > 1;
  const uint64_t* pk = part + (int64_t)(reduce ? i : 0) * chunks;
  uint64_t k[kBatch];
  if (reduce) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) k[u] = pk[min(u, chunks - 1)];
  }
  tree_prep_lds_from(parent_i, N, anc, par, jmp, dev_error);

  if (i < N) {
    int32_t t;
    if (chunks > 1) {
      uint64_t best = 0;
      for (int j0 = 0; j0 < chunks; j0 += kBatch) {
        if (j0 > 0) {
#pragma unroll
          for (int u = 0; u < kBatch; ++u) k[u] = pk[min(j0 + u, chunks - 1)];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) best = k[u] > best ? k[u] : best;
      }
      t = key_token(best);
      tok[i] = t;
    } else {
      t = tok[i];
    }
    tok_s[i] = t;
  }
  __syncthreads();
  accept_block<kBlock>(anc, par, tok_s, draft_i, N, okw, red, accept_len, accept_nodes, accept_tokens, bonus);
}

// The same for at most 64 nodes: one wave (lane i = node row i), no LDS and no barrier.
__global__ __launch_bounds__(64) void argmax_accept_wave_kernel(
    int N, int chunks, const uint64_t* __restrict__ part, int32_t* tok, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ draft, int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ accept_tokens, int32_t* __restrict__ bonus, int32_t* dev_error) {
  constexpr int kBatch = 32;
  const int i = threadIdx.x;
  const bool valid = i < N;
  const int draft_i = valid ? draft[i] : 0;
  const int parent_i = valid ? parent[i] : -1;
  int t = 0;
  if (valid) {
    if (chunks > 1) {
      const uint64_t* pk = part + (int64_t)i * chunks;
      uint64_t best = 0;
      for (int j0 = 0; j0 < chunks; j0 += kBatch) {
        uint64_t k[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) k[u] = pk[min(j0 + u, chunks - 1)];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) best = k[u] > best ? k[u] : best;
      }
      t = key_token(best);
      tok[i] = t;
    } else {
      t = tok[i];
    }
  }
  accept_wave(parent_i, draft_i, t, N, accept_len, accept_nodes, accept_tokens, bonus, dev_error);
}

// Argmax + accept finish: one wave for trees of at most 64 nodes, else one workgroup.
void launch_finish(int N, int chunks, const uint64_t* part, int32_t* tok, const int32_t* parent, const int32_t* draft,
                   int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens, int32_t* bonus,
                   int32_t* dev_error, hipStream_t stream) {
  if (N <= 64)
    hipLaunchKernelGGL(argmax_accept_wave_kernel, dim3(1), dim3(64), 0, stream, N, chunks, part, tok, parent, draft,
                       accept_len, accept_nodes, accept_tokens, bonus, dev_error);
  else
    hipLaunchKernelGGL(argmax_accept_kernel, dim3(1), dim3(kBlock), 0, stream, N, chunks, part, tok, parent, draft,
                       accept_len, accept_nodes, accept_tokens, bonus, dev_error);
}

}  // namespace

ArgmaxPlan argmax_plan(int N, int V, int dtype, bool vec) {
  // One slice = kUnroll 16-byte loads per thread: 8192 bf16 or 4096 fp32 elements. The
  // scalar path (rows not 16-byte aligned) uses 4096-element slices. (Eight loads per
  // thread, with half as many workgroups, measured slower: 7.7 against 6.5 us for
  // [64, 152064] bf16.)
  (void)N;
  ArgmaxPlan p;
  p.chunk_len = (vec && dtype == TV_BF16) ? kBlock * 8 * kUnroll : kBlock * 4 * kUnroll;
  p.chunks = (V + p.chunk_len - 1) / p.chunk_len;
  return p;
}

// Workspace: one 64-bit key per (row, slice), sized for the most slices any path uses.
size_t argmax_workspace_bytes(int N, int V) {
  const ArgmaxPlan p = argmax_plan(N, V, TV_F32, false);
  return ((size_t)N * p.chunks * sizeof(uint64_t) + 255) / 256 * 256;
}

hipError_t launch_argmax_partial(const void* logits, int dtype, int N, int V, int64_t row_bytes, bool vec,
                                 const ArgmaxPlan& p, int32_t* tok, uint64_t* part, hipStream_t stream) {
  const dim3 grid(p.chunks, N);
  const char* lg = static_cast<const char*>(logits);
  if (dtype == TV_F32) {
    if (vec)
      hipLaunchKernelGGL((argmax_partial<true, true>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, tok, part);
    else
      hipLaunchKernelGGL((argmax_partial<true, false>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, tok, part);
  } else {
    if (vec)
      hipLaunchKernelGGL((argmax_partial<false, true>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, tok, part);
    else
      hipLaunchKernelGGL((argmax_partial<false, false>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, tok, part);
  }
  return hipGetLastError();
}

hipError_t launch_argmax(const void* logits, int dtype, int N, int V, int64_t row_stride, int32_t* tok,
                         void* workspace, hipStream_t stream) {
  const int esize = dtype == TV_F32 ? 4 : 2;
  const int64_t row_bytes = row_stride * esize;
  const bool vec = ((uintptr_t)logits % 16 == 0) && (row_bytes % 16 == 0);
  const ArgmaxPlan p = argmax_plan(N, V, dtype, vec);
  uint64_t* part = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_argmax_partial(logits, dtype, N, V, row_bytes, vec, p, tok, part, stream);
  if (e != hipSuccess || p.chunks == 1) return e;
  hipLaunchKernelGGL(argmax_final, dim3((N + 3) / 4), dim3(256), 0, stream, N, p.chunks, part, tok);
  return hipGetLastError();
}

hipError_t launch_argmax_accept(const void* logits, int dtype, int N, int V, int64_t row_stride,
                                const int32_t* parent, const int32_t* draft, int32_t* tok,
                                int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                                int32_t* bonus, void* workspace, int32_t* dev_error,
                                hipStream_t stream) {
  const int esize = dtype == TV_F32 ? 4 : 2;
  const int64_t row_bytes = row_stride * esize;
  const bool vec = ((uintptr_t)logits % 16 == 0) && (row_bytes % 16 == 0);
  const ArgmaxPlan p = argmax_plan(N, V, dtype, vec);
  uint64_t* part = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_argmax_partial(logits, dtype, N, V, row_bytes, vec, p, tok, part, stream);
  if (e != hipSuccess) return e;
  launch_finish(N, p.chunks, part, tok, parent, draft, accept_len, accept_nodes, accept_tokens, bonus, dev_error,
                stream);
  return hipGetLastError();
}

hipError_t launch_sample_accept(const void* logits, int dtype, int N, int V, int64_t row_stride, float temperature,
                                uint64_t seed, uint64_t offset, const int32_t* parent, const int32_t* draft,
                                int32_t* tok, int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                                int32_t* bonus, void* workspace, int32_t* dev_error, hipStream_t stream) {
  const int esize = dtype == TV_F32 ? 4 : 2;
  const int64_t row_bytes = row_stride * esize;
  const bool vec = ((uintptr_t)logits % 16 == 0) && (row_bytes % 16 == 0);
  const ArgmaxPlan p = argmax_plan(N, V, dtype, vec);
  uint64_t* part = static_cast<uint64_t*>(workspace);
  SampleKey key{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)offset, (uint32_t)(offset >> 32),
                (float)(1.4426950408889634 / (double)temperature)};
  const dim3 grid(p.chunks, N);
  const char* lg = static_cast<const char*>(logits);
  if (dtype == TV_F32) {
    if (vec)
      hipLaunchKernelGGL((sample_partial<true, true>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, key, tok, part);
    else
      hipLaunchKernelGGL((sample_partial<true, false>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, key, tok, part);
  } else {
    if (vec)
      hipLaunchKernelGGL((sample_partial<false, true>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, key, tok, part);
    else
      hipLaunchKernelGGL((sample_partial<false, false>), grid, dim3(kBlock), 0, stream, lg, V, row_bytes, p.chunks,
                         p.chunk_len, key, tok, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_finish(N, p.chunks, part, tok, parent, draft, accept_len, accept_nodes, accept_tokens, bonus, dev_error,
                stream);
  return hipGetLastError();
}

}  // namespace tv

// Internal declarations shared by the libtv translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kMaxNodes = TV_MAX_NODES;
constexpr int kAncWords = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Tree preprocessing into LDS (shared by tree attention and acceptance).
//
// On return, for every node i < N:
//   anc[i*4 + w]  bit j set <=> node 64*w + j is i or one of its ancestors;
//   par[i]        parent[i] clamped to -1 when outside [-1, i-1].
// A clamped entry stores TV_ERR_BAD_TREE into *dev_error when dev_error is non-null.
// Ancestor sets are built by pointer jumping: anc[i] always holds the path from i up to
// (not including) jmp[i]; each round doubles the jump, so 8 rounds cover depth 256.
// Requires blockDim.x >= N; every thread of the block must call it (it synchronises).
__device__ __forceinline__ void tree_prep_lds(const int32_t* __restrict__ parent, int N,
                                              uint64_t* anc, int* par, int* jmp,
                                              int32_t* dev_error) {
  const int i = threadIdx.x;
  if (i < N) {
    int p = parent[i];
    if (p < -1 || p >= i) {
      p = -1;
      if (dev_error) *dev_error = TV_ERR_BAD_TREE;
    }
    par[i] = p;
    jmp[i] = p;
#pragma unroll
    for (int w = 0; w < kAncWords; ++w) anc[i * kAncWords + w] = (w == (i >> 6)) ? (1ull << (i & 63)) : 0ull;
  }
  __syncthreads();
  for (int round = 0; round < 8; ++round) {
    uint64_t a[kAncWords];
    int next = -1;
    if (i < N) {
      const int j = jmp[i];
#pragma unroll
      for (int w = 0; w < kAncWords; ++w) a[w] = anc[i * kAncWords + w];
      if (j >= 0) {
#pragma unroll
        for (int w = 0; w < kAncWords; ++w) a[w] |= anc[j * kAncWords + w];
        next = jmp[j];
      }
    }
    __syncthreads();
    if (i < N) {
#pragma unroll
      for (int w = 0; w < kAncWords; ++w) anc[i * kAncWords + w] = a[w];
      jmp[i] = next;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ int anc_popcount(const uint64_t* anc, int i) {
  int c = 0;
#pragma unroll
  for (int w = 0; w < kAncWords; ++w) c += __popcll(anc[i * kAncWords + w]);
  return c;
}

// Launch helpers implemented in the .hip files. Return hipSuccess or the launch error.
hipError_t launch_tree_prep(const int32_t* parent, int N, uint64_t* anc, int32_t* depth,
                            int32_t* dev_error, hipStream_t stream);
hipError_t launch_accept(const int32_t* parent, const int32_t* draft, const int32_t* tok, int N,
                         int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                         int32_t* bonus, int32_t* dev_error, hipStream_t stream);

struct ArgmaxPlan {
  int chunks;     // workgroups per row
  int chunk_len;  // elements per workgroup (multiple of 8)
};
ArgmaxPlan argmax_plan(int N, int V, int dtype, bool vec);
size_t argmax_workspace_bytes(int N, int V);
hipError_t launch_argmax(const void* logits, int dtype, int N, int V, int64_t row_stride,
                         int32_t* tok, void* workspace, hipStream_t stream);

struct AttnPlan {
  int G, M;        // q heads per KV head; stacked rows per KV head (G * N)
  int RT;          // row tiles of up to 256 stacked rows
  int NW;          // waves per workgroup: 2, 4 or 8 (32 rows each)
  int S;           // KV splits actually launched
  int KS;          // keys per split (multiple of the key tile)
  int T;           // L + N
};
AttnPlan attn_plan(int N, int L, int Hq, int Hkv, int num_splits, int num_cus);
size_t attn_workspace_bytes(const AttnPlan& p, int Hkv);
hipError_t launch_tree_attn(const AttnPlan& plan, const void* q, const void* k, const void* v,
                            int64_t st, int64_t sh, const int32_t* parent, int N, int L, int Hq,
                            int Hkv, float scale, void* out, float* lse, void* workspace,
                            int32_t* dev_error, hipStream_t stream);

}  // namespace tv

// Internal declarations shared by the libtv translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
// (not including) jmp[i]; each round doubles the jump. A path holds at most N nodes
// (parent[i] < i), so ceil(log2 N) rounds complete every set.
// Requires blockDim.x >= N; every thread of the block must call it (it synchronises).
// tree_prep_lds_from takes thread i's entry parent[i] already loaded (ignored for i >= N),
// so that a caller can have other loads in flight behind it; tree_prep_lds loads it.
__device__ __forceinline__ void tree_prep_lds_from(int parent_i, int N, uint64_t* anc, int* par, int* jmp,
                                                   int32_t* dev_error) {
  const int i = threadIdx.x;
  if (i < N) {
    int p = parent_i;
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
  const int rounds = N > 1 ? 32 - __clz(N - 1) : 0;  // ceil(log2 N), uniform
  for (int round = 0; round < rounds; ++round) {
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

__device__ __forceinline__ void tree_prep_lds(const int32_t* __restrict__ parent, int N, uint64_t* anc, int* par,
                                              int* jmp, int32_t* dev_error) {
  const int i = threadIdx.x;
  tree_prep_lds_from(i < N ? parent[i] : -1, N, anc, par, jmp, dev_error);
}

__device__ __forceinline__ int anc_popcount(const uint64_t* anc, int i) {
  int c = 0;
#pragma unroll
  for (int w = 0; w < kAncWords; ++w) c += __popcll(anc[i * kAncWords + w]);
  return c;
}

// Largest 32-bit key over the block (kThreads threads); `red` holds kThreads/64 words.
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(x, off);
    x = o > x ? o : x;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  uint32_t r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = red[w] > r ? red[w] : r;
  __syncthreads();
  return r;
}

// Longest accepted path of one tree, computed by one workgroup of kThreads >= N threads
// after tree_prep_lds has filled anc/par. Thread i handles node i: `draft_i` is draft[i]
// and tok[i] (any address space) the target's argmax for node i.
//   ok[i]       draft[i] == tok[i];
//   accepted    every node on the path from the prefix to i is ok (anc[i] within ok);
//   result      the deepest accepted node, ties to the lowest index; its path in
//               root-to-leaf (= ascending index) order, then -1 padding;
//   bonus       tok of the lowest-index child of the end node (of the prefix when nothing
//               is accepted), -1 when there is none.
template <int kThreads>
__device__ __forceinline__ void accept_block(const uint64_t* anc, const int* par, const int32_t* tok, int draft_i,
                                             int N, uint64_t* okw, uint32_t* red, int32_t* accept_len,
                                             int32_t* accept_nodes, int32_t* accept_tokens, int32_t* bonus) {
  const int i = threadIdx.x;
  const int wave = i >> 6;
  const bool ok = (i < N) && (draft_i == tok[i]);
  const uint64_t ball = __ballot(ok);
  if ((i & 63) == 0 && wave < kAncWords) okw[wave] = ball;
  __syncthreads();

  bool elig = i < N;
  if (elig) {
#pragma unroll
    for (int w = 0; w < kAncWords; ++w) elig = elig && ((anc[i * kAncWords + w] & ~okw[w]) == 0ull);
  }
  // Longest path first, then the lowest end index: key = depth << 16 | (0xFFFF - i).
  const uint32_t key = elig ? ((uint32_t)anc_popcount(anc, i) << 16) | (0xFFFFu - (uint32_t)i) : 0u;
  const uint32_t best = block_max_u32<kThreads>(key, red);
  const int len = (int)(best >> 16);
  const int end = best ? (int)(0xFFFFu - (best & 0xFFFFu)) : -1;

  if (i < N) {
    bool on_path = false;
    int pos = 0;
    if (end >= 0) {
      const int w = i >> 6, b = i & 63;
      on_path = (anc[end * kAncWords + w] >> b) & 1ull;
      // Nodes on the path in ascending index order are in root-to-leaf order because
      // parent[i] < i.
      for (int x = 0; x < w; ++x) pos += __popcll(anc[end * kAncWords + x]);
      pos += __popcll(anc[end * kAncWords + w] & ((1ull << b) - 1ull));
    }
    if (on_path) {
      accept_nodes[pos] = i;
      accept_tokens[pos] = draft_i;
    }
    if (i >= len) {
      accept_nodes[i] = -1;
      accept_tokens[i] = -1;
    }
  }

  const uint32_t child = (i < N && par[i] == end) ? (uint32_t)(0xFFFFu - (uint32_t)i) : 0u;
  const uint32_t first_child = block_max_u32<kThreads>(child, red);
  if (i == 0) {
    *accept_len = len;
    if (bonus) *bonus = first_child ? tok[0xFFFFu - first_child] : -1;
  }
}


// Launch helpers implemented in the .hip files. Return hipSuccess or the launch error.
hipError_t launch_tree_prep(const int32_t* parent, int N, uint64_t* anc, int32_t* depth,
                            int32_t* dev_error, hipStream_t stream);
hipError_t launch_accept(const int32_t* parent, const int32_t* draft, const int32_t* tok, int N,
                         int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                         int32_t* bonus, int32_t* dev_error, hipStream_t stream);

hipError_t launch_sample_accept(const void* logits, int dtype, int N, int V, int64_t row_stride, float temperature,
                                uint64_t seed, uint64_t offset, const int32_t* parent, const int32_t* draft,
                                int32_t* tok, int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                                int32_t* bonus, void* workspace, int32_t* dev_error, hipStream_t stream);
hipError_t launch_kv_quantize_mx4(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                                  int64_t csh, int8_t* exps, hipStream_t stream);
hipError_t launch_kv_quantize(const void* src, int64_t st, int64_t sh, int T, int H, void* codes, int64_t cst,
                              int64_t csh, int32_t* exps, hipStream_t stream);
hipError_t launch_kv_commit(void* k, void* v, int64_t st, int64_t sh, int Hkv, int D, int L, int N,
                            const int32_t* accept_len, const int32_t* accept_nodes, int32_t* new_len,
                            int32_t* dev_error, hipStream_t stream);

struct ArgmaxPlan {
  int chunks;     // workgroups per row
  int chunk_len;  // elements per workgroup (multiple of 8)
};
ArgmaxPlan argmax_plan(int N, int V, int dtype, bool vec);
size_t argmax_workspace_bytes(int N, int V);
hipError_t launch_argmax(const void* logits, int dtype, int N, int V, int64_t row_stride,
                         int32_t* tok, void* workspace, hipStream_t stream);
hipError_t launch_argmax_accept(const void* logits, int dtype, int N, int V, int64_t row_stride,
                                const int32_t* parent, const int32_t* draft, int32_t* tok,
                                int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                                int32_t* bonus, void* workspace, int32_t* dev_error,
                                hipStream_t stream);

struct AttnPlan {
  int G, M;        // q heads per KV head; stacked rows per KV head (G * N)
  int RT;          // row tiles of RWV * 32 stacked rows
  int RWV;         // row-waves per workgroup (1, 2, 4 or 8); the other 8 / RWV split keys
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
hipError_t launch_tree_attn_mx4(const AttnPlan& plan, const void* q, const void* kc, const void* vc,
                                const int8_t* ek, const int8_t* ev, int64_t st, int64_t sh,
                                const int32_t* parent, int N, int L, int Hq, int Hkv, float scale, void* out,
                                float* lse, void* workspace, int32_t* dev_error, hipStream_t stream);
hipError_t launch_tree_attn_fp8(const AttnPlan& plan, const void* q, const void* kc, const void* vc,
                                const int32_t* ek, const int32_t* ev, int64_t st, int64_t sh,
                                const int32_t* parent, int N, int L, int Hq, int Hkv, float scale, void* out,
                                float* lse, void* workspace, int32_t* dev_error, hipStream_t stream);

}  // namespace tv

// Tree preprocessing and the longest-accepted-path walk (single workgroup each).
//
// Acceptance follows the verify rule of speculative decoding: drafted tokens the target
// agrees with are kept, the rest dropped (DFlash contributor guide, discosf.com/news/
// 4742660, "What is DFlash?"); on a DDTree the kept tokens form a root-to-node path
// (Lucebox-Hub review, aichain-blog.pages.dev, "2. DFlash"). The longest such path wins,
// ties to the lowest end index.
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void tree_prep_kernel(const int32_t* __restrict__ parent, int N,
                                                           uint64_t* __restrict__ anc_out,
                                                           int32_t* __restrict__ depth_out,
                                                           int32_t* dev_error) {
  __shared__ uint64_t anc[kMaxNodes * kAncWords];
  __shared__ int par[kMaxNodes];
  __shared__ int jmp[kMaxNodes];
  tree_prep_lds(parent, N, anc, par, jmp, dev_error);
  const int i = threadIdx.x;
  if (i < N) {
    if (anc_out) {
#pragma unroll
      for (int w = 0; w < kAncWords; ++w) anc_out[i * kAncWords + w] = anc[i * kAncWords + w];
    }
    if (depth_out) depth_out[i] = anc_popcount(anc, i);
  }
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(x, off);
    x = o > x ? o : x;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  uint32_t r = red[0];
  for (int w = 1; w < kBlock / 64; ++w) r = red[w] > r ? red[w] : r;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kBlock) void accept_kernel(const int32_t* __restrict__ parent,
                                                        const int32_t* __restrict__ draft,
                                                        const int32_t* __restrict__ tok, int N,
                                                        int32_t* __restrict__ accept_len,
                                                        int32_t* __restrict__ accept_nodes,
                                                        int32_t* __restrict__ accept_tokens,
                                                        int32_t* __restrict__ bonus,
                                                        int32_t* dev_error) {
  __shared__ uint64_t anc[kMaxNodes * kAncWords];
  __shared__ int par[kMaxNodes];
  __shared__ int jmp[kMaxNodes];
  __shared__ uint64_t okw[kAncWords];
  __shared__ uint32_t red[kBlock / 64];

  tree_prep_lds(parent, N, anc, par, jmp, dev_error);
  const int i = threadIdx.x;
  const int wave = i >> 6;

  // Match mask: bit i set when node i's draft equals the target's argmax.
  const bool ok = (i < N) && (draft[i] == tok[i]);
  const uint64_t ball = __ballot(ok);
  if ((i & 63) == 0) okw[wave] = ball;
  __syncthreads();

  // A node is accepted when every node on its path matches: anc[i] is a subset of okw.
  bool elig = i < N;
  if (elig) {
#pragma unroll
    for (int w = 0; w < kAncWords; ++w) elig = elig && ((anc[i * kAncWords + w] & ~okw[w]) == 0ull);
  }
  // Longest path first, then the lowest end index: key = depth << 16 | (0xFFFF - i).
  const uint32_t key = elig ? ((uint32_t)anc_popcount(anc, i) << 16) | (0xFFFFu - (uint32_t)i) : 0u;
  const uint32_t best = block_max_u32(key, red);
  const int len = (int)(best >> 16);
  const int end = best ? (int)(0xFFFFu - (best & 0xFFFFu)) : -1;

  if (i < N) {
    bool on_path = false;
    int pos = 0;
    if (end >= 0) {
      const int w = i >> 6, b = i & 63;
      on_path = (anc[end * kAncWords + w] >> b) & 1ull;
      // Nodes on the path in ascending index order are in root-to-leaf order
      // because parent[i] < i.
      for (int x = 0; x < w; ++x) pos += __popcll(anc[end * kAncWords + x]);
      pos += __popcll(anc[end * kAncWords + w] & ((1ull << b) - 1ull));
    }
    if (on_path) {
      accept_nodes[pos] = i;
      accept_tokens[pos] = draft[i];
    }
    if (i >= len) {
      accept_nodes[i] = -1;
      accept_tokens[i] = -1;
    }
  }

  // Bonus: the target's argmax at the first child of the path's last node.
  const uint32_t child = (i < N && par[i] == end) ? (uint32_t)(0xFFFFu - (uint32_t)i) : 0u;
  const uint32_t first_child = block_max_u32(child, red);
  if (i == 0) {
    *accept_len = len;
    if (bonus) *bonus = first_child ? tok[0xFFFFu - first_child] : -1;
  }
}

}  // namespace

hipError_t launch_tree_prep(const int32_t* parent, int N, uint64_t* anc, int32_t* depth,
                            int32_t* dev_error, hipStream_t stream) {
  hipLaunchKernelGGL(tree_prep_kernel, dim3(1), dim3(kBlock), 0, stream, parent, N, anc, depth,
                     dev_error);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* parent, const int32_t* draft, const int32_t* tok, int N,
                         int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                         int32_t* bonus, int32_t* dev_error, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(kBlock), 0, stream, parent, draft, tok, N,
                     accept_len, accept_nodes, accept_tokens, bonus, dev_error);
  return hipGetLastError();
}

}  // namespace tv

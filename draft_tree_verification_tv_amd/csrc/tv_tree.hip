// Tree preprocessing and the longest-accepted-path walk (single workgroup each).
//
// Acceptance follows the verify rule of speculative decoding: drafted tokens the target
// agrees with are kept, the rest dropped (DFlash contributor guide, discosf.com/news/
// 4742660, "What is DFlash?"); on a DDTree the kept tokens form a root-to-node path
// (Lucebox-Hub review, aichain-blog.pages.dev, "2. DFlash"). The longest such path wins,
// ties to the lowest end index.
#include "tv_accept_wave.h"
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
  const int i = threadIdx.x;
  const int draft_i = i < N ? draft[i] : 0;
  tree_prep_lds(parent, N, anc, par, jmp, dev_error);
  accept_block<kBlock>(anc, par, tok, draft_i, N, okw, red, accept_len, accept_nodes, accept_tokens, bonus);
}

// At most 64 nodes: one wave, no LDS and no barrier.
__global__ __launch_bounds__(64) void accept_wave_kernel(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ tok, int N,
                                                         int32_t* __restrict__ accept_len,
                                                         int32_t* __restrict__ accept_nodes,
                                                         int32_t* __restrict__ accept_tokens,
                                                         int32_t* __restrict__ bonus, int32_t* dev_error) {
  const int i = threadIdx.x;
  const bool valid = i < N;
  accept_wave(valid ? parent[i] : -1, valid ? draft[i] : 0, valid ? tok[i] : 0, N, accept_len, accept_nodes,
              accept_tokens, bonus, dev_error);
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
  if (N <= 64)
    hipLaunchKernelGGL(accept_wave_kernel, dim3(1), dim3(64), 0, stream, parent, draft, tok, N, accept_len,
                       accept_nodes, accept_tokens, bonus, dev_error);
  else
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(kBlock), 0, stream, parent, draft, tok, N,
                       accept_len, accept_nodes, accept_tokens, bonus, dev_error);
  return hipGetLastError();
}

}  // namespace tv

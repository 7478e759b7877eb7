// Commit of the accepted path into the KV cache.
//
// Verification keeps the drafted tokens the target agreed with and drops the rest (DFlash
// contributor guide, discosf.com/news/4742660, "What is DFlash?"); on a tree the kept
// tokens are the accepted root-to-node path (Lucebox-Hub review, aichain-blog.pages.dev,
// "2. DFlash"). Their keys and values, written at rows L + node by the verify pass, move to
// rows L + 0, 1, ... in path order so that the cache holds the committed sequence.
//
// Each thread owns one column -- (K or V) x KV head x 16-byte chunk of the head dim -- and
// walks the path in ascending order. Path nodes increase and path[j] >= j, so a row is
// only ever written after every read of it (reads of a batch are issued before its
// writes, and later batches read rows beyond every earlier destination); columns are
// independent, so no synchronisation is needed between threads or workgroups.
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kBlock = 256;
constexpr int kBatch = 16;

__global__ __launch_bounds__(kBlock) void kv_commit_kernel(char* __restrict__ k, char* __restrict__ v,
                                                           int64_t st_b, int64_t sh_b, int Hkv, int cpr, int L,
                                                           int N, const int32_t* __restrict__ accept_len,
                                                           const int32_t* __restrict__ accept_nodes,
                                                           int32_t* new_len, int32_t* dev_error) {
  __shared__ int nodes[kMaxNodes];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int len = *accept_len;
  const bool len_ok = len >= 0 && len <= N;
  if (tid == 0) bad = len_ok ? 0 : 1;
  __syncthreads();
  if (len_ok && tid < len) {
    const int nd = accept_nodes[tid];
    nodes[tid] = nd;
    if (nd < tid || nd >= N) bad = 1;
  }
  __syncthreads();
  if (len_ok && tid > 0 && tid < len && nodes[tid] <= nodes[tid - 1]) bad = 1;
  __syncthreads();
  if (bad) {
    if (blockIdx.x == 0 && tid == 0 && dev_error) *dev_error = TV_ERR_INVALID_ARG;
    return;
  }
  if (blockIdx.x == 0 && tid == 0 && new_len) *new_len = L + len;

  const int col = blockIdx.x * kBlock + tid;
  if (col >= 2 * Hkv * cpr) return;
  const int per_tensor = Hkv * cpr;
  const int tensor = col / per_tensor;
  const int h = (col % per_tensor) / cpr;
  const int c = col % cpr;
  char* base = (tensor ? v : k) + h * sh_b + c * 16;
  const char* rbase = base + (int64_t)L * st_b;
  char* wbase = base + (int64_t)L * st_b;
  for (int j0 = 0; j0 < len; j0 += kBatch) {
    u32x4 buf[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = min(j0 + u, len - 1);
      buf[u] = *reinterpret_cast<const u32x4*>(rbase + (int64_t)nodes[j] * st_b);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u;
      if (j < len && nodes[j] != j) *reinterpret_cast<u32x4*>(wbase + (int64_t)j * st_b) = buf[u];
    }
  }
}

}  // namespace

hipError_t launch_kv_commit(void* k, void* v, int64_t st, int64_t sh, int Hkv, int D, int L, int N,
                            const int32_t* accept_len, const int32_t* accept_nodes, int32_t* new_len,
                            int32_t* dev_error, hipStream_t stream) {
  const int cpr = D / 8;
  const int cols = 2 * Hkv * cpr;
  const int grid = (cols + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(grid), dim3(kBlock), 0, stream, static_cast<char*>(k),
                     static_cast<char*>(v), st * 2, sh * 2, Hkv, cpr, L, N, accept_len, accept_nodes, new_len,
                     dev_error);
  return hipGetLastError();
}

}  // namespace tv

// Longest-accepted-path walk for trees of at most 64 nodes, by a single wave (used by the
// accept and argmax + accept kernels when N <= 64).
#pragma once

#include "tv_internal.h"

namespace tv {

// Lane src's 64-bit value, as two 32-bit shuffles.
__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)x, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(x >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// The walk of accept_block (tv_internal.h) for a tree of at most 64 nodes, by one wave
// with lane i = node i and no LDS or barrier: the ancestor sets come from pointer jumping
// over register shuffles (round r: anc_i |= anc_jmp(i), jmp(i) = jmp(jmp(i)), every lane
// reading the values of the previous round), then the rule of accept_block. parent_i,
// draft_i and tok_i are lane i's entries (ignored for lanes >= N); a parent outside
// [-1, i-1] is read as -1 and reported, as tree_prep_lds does.
__device__ __forceinline__ void accept_wave(int parent_i, int draft_i, int tok_i, int N, int32_t* accept_len,
                                            int32_t* accept_nodes, int32_t* accept_tokens, int32_t* bonus,
                                            int32_t* dev_error) {
  const int i = threadIdx.x;  // 0 .. 63
  const bool valid = i < N;
  int p = -1;
  if (valid) {
    p = parent_i;
    if (p < -1 || p >= i) {
      p = -1;
      if (dev_error) *dev_error = TV_ERR_BAD_TREE;
    }
  }
  uint64_t anc = valid ? (1ull << i) : 0ull;
  int jmp = p;
  const int rounds = N > 1 ? 32 - __clz(N - 1) : 0;  // ceil(log2 N), uniform
  for (int r = 0; r < rounds; ++r) {
    const int src = jmp >= 0 ? jmp : i;
    const uint64_t a = shfl_u64(anc, src);
    const int nj = __shfl(jmp, src);
    if (jmp >= 0) {
      anc |= a;
      jmp = nj;
    }
  }

  const uint64_t okmask = __ballot(valid && draft_i == tok_i);
  const bool elig = valid && (anc & ~okmask) == 0ull;
  // Longest path first, then the lowest end index: key = depth << 16 | (0xFFFF - i).
  uint32_t key = elig ? ((uint32_t)__popcll(anc) << 16) | (0xFFFFu - (uint32_t)i) : 0u;
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)key, off);
    key = o > key ? o : key;
  }
  const int len = (int)(key >> 16);
  const int end = key ? (int)(0xFFFFu - (key & 0xFFFFu)) : -1;
  const uint64_t anc_end = shfl_u64(anc, end >= 0 ? end : 0);
  if (valid) {
    if (end >= 0 && ((anc_end >> i) & 1ull)) {
      // Nodes on the path in ascending index order are in root-to-leaf order.
      const int pos = __popcll(anc_end & ((1ull << i) - 1ull));
      accept_nodes[pos] = i;
      accept_tokens[pos] = draft_i;
    }
    if (i >= len) {
      accept_nodes[i] = -1;
      accept_tokens[i] = -1;
    }
  }
  const uint64_t kids = __ballot(valid && p == end);
  const int first = kids ? __ffsll((unsigned long long)kids) - 1 : -1;
  const int first_tok = __shfl(tok_i, first >= 0 ? first : 0);
  if (i == 0) {
    *accept_len = len;
    if (bonus) *bonus = first >= 0 ? first_tok : -1;
  }
}

}  // namespace tv

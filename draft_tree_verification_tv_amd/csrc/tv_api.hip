// C ABI of libtv: host-side validation, plans and launches. Declarations and the
// contract of every entry point are in include/tv.h.
//
// A versioned ABI query and static descriptive strings follow the plugin-ABI pattern of
// the ROCmFPX page (bittide.aicompass.dev article, "plugin system" section): a caller can
// refuse a library whose version does not match its header.
#include <atomic>
#include <cmath>

#include "tv_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int status_of(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_HIP; }

// Whether the rows (t, h), t < T, h < H, of w units at t * st + h * sh are pairwise
// disjoint in one of the two layouts accepted for a cache that is written: token-major
// (the heads of a token side by side, then the next token) or head-major (the tokens of a
// head side by side, then the next head). Strides are non-negative.
bool rows_disjoint(int64_t st, int64_t sh, int64_t T, int64_t H, int64_t w) {
  if (st < 0 || sh < 0) return false;
  if (T <= 0 || H <= 0 || (T == 1 && H == 1)) return true;
  if (H == 1) return st >= w;
  if (T == 1) return sh >= w;
  // 128-bit products: no stride or count the caller passes can overflow them
  const bool token_major = sh >= w && (__int128)st >= (__int128)(H - 1) * sh + w;
  const bool head_major = st >= w && (__int128)sh >= (__int128)(T - 1) * st + w;
  return token_major || head_major;
}

// Whether rows x cols entries of w elements of esize bytes, entry (r, c) at element
// r * st + c * sh (strides non-negative), span at most 2^56 bytes. No real allocation is
// larger, and every address the kernels form inside such a span stays far from 64-bit
// overflow.
bool span_ok(int64_t rows, int64_t st, int64_t cols, int64_t sh, int64_t w, int64_t esize) {
  if (rows <= 0 || cols <= 0) return true;
  const __int128 end = (__int128)(rows - 1) * st + (__int128)(cols - 1) * sh + w;
  return end * esize <= ((__int128)1 << 56);
}

bool attn_args_ok(int N, int L, int Hq, int Hkv, int num_splits) {
  return N >= 1 && N <= TV_MAX_NODES && L >= 0 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0 &&
         num_splits >= 0 && num_splits <= 1024 && (int64_t)L + N <= INT32_MAX - 64 &&
         (int64_t)Hq * N <= (1 << 24);
}

// Host checks shared by the bf16-cache attention entry points.
int attn_bf16_args_status(const void* q, const void* k, const void* v, int64_t kv_stride_t, int64_t kv_stride_h,
                          const int32_t* parent, int N, int L, int Hq, int Hkv, int D, float scale, int num_splits,
                          const void* out, const float* lse) {
  if (!q || !k || !v || !parent || !out) return TV_ERR_INVALID_ARG;
  if (!attn_args_ok(N, L, Hq, Hkv, num_splits)) return TV_ERR_INVALID_ARG;
  if (D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return TV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return TV_ERR_INVALID_ARG;
  if (kv_stride_t < 0 || kv_stride_h < 0 || kv_stride_t % 8 || kv_stride_h % 8) return TV_ERR_INVALID_ARG;
  if (!span_ok((int64_t)L + N, kv_stride_t, Hkv, kv_stride_h, D, 2)) return TV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return TV_ERR_INVALID_ARG;
  // One KV head's rows must be addressable with 32-bit byte offsets.
  if ((__int128)((int64_t)L + N) * kv_stride_t * 2 + 4096 > (__int128)UINT32_MAX) return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

// ---- allocation-free attention: the split partials live in a static device array.
//
// `scratch` is a file-scope device array: in host code its name is only a stand-in, so
// the device address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels receive that address, never the name.
static __device__ __align__(256) char scratch[TV_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

hipError_t scratch_on_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // Concurrent first calls on one device may both look it up; they store the same value.
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int tv_abi_version(void) { return TV_ABI_VERSION; }

const char* tv_status_string(int status) {
  switch (status) {
    case TV_OK: return "ok";
    case TV_ERR_INVALID_ARG: return "invalid argument";
    case TV_ERR_BAD_TREE: return "parent[] entry outside [-1, i-1]";
    case TV_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 128)";
    case TV_ERR_WORKSPACE: return "workspace missing or too small";
    case TV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int tv_validate_tree_host(const int32_t* parent_host, int N) {
  if (!parent_host || N < 1 || N > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  for (int i = 0; i < N; ++i)
    if (parent_host[i] < -1 || parent_host[i] >= i) return TV_ERR_BAD_TREE;
  return TV_OK;
}

int tv_tree_prep(const int32_t* parent, int N, uint64_t* anc, int32_t* depth, int32_t* dev_error,
                 void* stream) {
  if (!parent || N < 1 || N > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  return status_of(tv::launch_tree_prep(parent, N, anc, depth, dev_error, static_cast<hipStream_t>(stream)));
}

size_t tv_tree_attn_workspace_size(int N, int L, int Hq, int Hkv, int D, int num_splits) {
  if (!attn_args_ok(N, L, Hq, Hkv, num_splits) || D != TV_HEAD_DIM) return 0;
  const tv::AttnPlan p = tv::attn_plan(N, L, Hq, Hkv, num_splits, cu_count());
  return tv::attn_workspace_bytes(p, Hkv);
}

int tv_tree_attn(const void* q, const void* k, const void* v, int64_t kv_stride_t, int64_t kv_stride_h,
                 const int32_t* parent, int N, int L, int Hq, int Hkv, int D, float scale, int num_splits,
                 void* out, float* lse, void* workspace, size_t workspace_bytes, int32_t* dev_error,
                 void* stream) {
  const int st = attn_bf16_args_status(q, k, v, kv_stride_t, kv_stride_h, parent, N, L, Hq, Hkv, D, scale,
                                       num_splits, out, lse);
  if (st != TV_OK) return st;
  const tv::AttnPlan p = tv::attn_plan(N, L, Hq, Hkv, num_splits, cu_count());
  const size_t need = tv::attn_workspace_bytes(p, Hkv);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TV_ERR_WORKSPACE;
  return status_of(tv::launch_tree_attn(p, q, k, v, kv_stride_t, kv_stride_h, parent, N, L, Hq, Hkv, scale, out,
                                        lse, workspace, dev_error, static_cast<hipStream_t>(stream)));
}

int tv_tree_attn_noalloc(const void* q, const void* k, const void* v, int64_t kv_stride_t, int64_t kv_stride_h,
                         const int32_t* parent, int N, int L, int Hq, int Hkv, int D, float scale, int num_splits,
                         void* out, float* lse, int32_t* dev_error, void* stream) {
  const int st = attn_bf16_args_status(q, k, v, kv_stride_t, kv_stride_h, parent, N, L, Hq, Hkv, D, scale,
                                       num_splits, out, lse);
  if (st != TV_OK) return st;
  const tv::AttnPlan p = tv::attn_plan(N, L, Hq, Hkv, num_splits, cu_count());
  if (tv::attn_workspace_bytes(p, Hkv) > (size_t)TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return TV_ERR_HIP;
  return status_of(tv::launch_tree_attn(p, q, k, v, kv_stride_t, kv_stride_h, parent, N, L, Hq, Hkv, scale, out,
                                        lse, ws, dev_error, static_cast<hipStream_t>(stream)));
}

int tv_tree_attn_fp8(const void* q, const void* k_codes, const void* v_codes, const int32_t* k_exps,
                     const int32_t* v_exps, int64_t kv_stride_t, int64_t kv_stride_h, const int32_t* parent,
                     int N, int L, int Hq, int Hkv, int D, float scale, int num_splits, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (!q || !k_codes || !v_codes || !k_exps || !v_exps || !parent || !out) return TV_ERR_INVALID_ARG;
  if (!attn_args_ok(N, L, Hq, Hkv, num_splits)) return TV_ERR_INVALID_ARG;
  if (D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return TV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(out)) return TV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_exps) & 3u) || (reinterpret_cast<uintptr_t>(v_exps) & 3u))
    return TV_ERR_INVALID_ARG;
  if (kv_stride_t < 0 || kv_stride_h < 0 || kv_stride_t % 16 || kv_stride_h % 16) return TV_ERR_INVALID_ARG;
  if (!span_ok((int64_t)L + N, kv_stride_t, Hkv, kv_stride_h, D, 1)) return TV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return TV_ERR_INVALID_ARG;
  // One KV head's code rows and the exponent arrays must be addressable with 32-bit
  // byte offsets.
  if ((__int128)((int64_t)L + N) * kv_stride_t + 4096 > (__int128)UINT32_MAX) return TV_ERR_UNSUPPORTED;
  if ((__int128)((int64_t)L + N) * Hkv * 4 > (__int128)UINT32_MAX) return TV_ERR_UNSUPPORTED;
  const tv::AttnPlan p = tv::attn_plan(N, L, Hq, Hkv, num_splits, cu_count());
  const size_t need = tv::attn_workspace_bytes(p, Hkv);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TV_ERR_WORKSPACE;
  return status_of(tv::launch_tree_attn_fp8(p, q, k_codes, v_codes, k_exps, v_exps, kv_stride_t, kv_stride_h,
                                            parent, N, L, Hq, Hkv, scale, out, lse, workspace, dev_error,
                                            static_cast<hipStream_t>(stream)));
}

int tv_tree_attn_mx4(const void* q, const void* k_codes, const void* v_codes, const int8_t* k_exps,
                     const int8_t* v_exps, int64_t kv_stride_t, int64_t kv_stride_h, const int32_t* parent,
                     int N, int L, int Hq, int Hkv, int D, float scale, int num_splits, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (!q || !k_codes || !v_codes || !k_exps || !v_exps || !parent || !out) return TV_ERR_INVALID_ARG;
  if (!attn_args_ok(N, L, Hq, Hkv, num_splits)) return TV_ERR_INVALID_ARG;
  if (D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return TV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(out)) return TV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_exps) & 3u) || (reinterpret_cast<uintptr_t>(v_exps) & 3u))
    return TV_ERR_INVALID_ARG;
  if (kv_stride_t < 0 || kv_stride_h < 0 || kv_stride_t % 16 || kv_stride_h % 16) return TV_ERR_INVALID_ARG;
  if (!span_ok((int64_t)L + N, kv_stride_t, Hkv, kv_stride_h, D / 2, 1)) return TV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return TV_ERR_INVALID_ARG;
  // One KV head's code rows and the exponent words must be addressable with 32-bit byte
  // offsets.
  if ((__int128)((int64_t)L + N) * kv_stride_t + 4096 > (__int128)UINT32_MAX) return TV_ERR_UNSUPPORTED;
  if ((__int128)((int64_t)L + N) * Hkv * 4 > (__int128)UINT32_MAX) return TV_ERR_UNSUPPORTED;
  const tv::AttnPlan p = tv::attn_plan(N, L, Hq, Hkv, num_splits, cu_count());
  const size_t need = tv::attn_workspace_bytes(p, Hkv);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TV_ERR_WORKSPACE;
  return status_of(tv::launch_tree_attn_mx4(p, q, k_codes, v_codes, k_exps, v_exps, kv_stride_t, kv_stride_h,
                                            parent, N, L, Hq, Hkv, scale, out, lse, workspace, dev_error,
                                            static_cast<hipStream_t>(stream)));
}

size_t tv_argmax_workspace_size(int N, int V) {
  if (N < 1 || V < 1 || V >= INT32_MAX) return 0;
  return tv::argmax_workspace_bytes(N, V);
}

int tv_argmax(const void* logits, int dtype, int N, int V, int64_t row_stride, int32_t* tok, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!logits || !tok) return TV_ERR_INVALID_ARG;
  if (N < 1 || N > 65535 || V < 1 || V >= INT32_MAX || row_stride < V) return TV_ERR_INVALID_ARG;
  if (!span_ok(N, row_stride, 1, 0, V, dtype == TV_F32 ? 4 : 2)) return TV_ERR_INVALID_ARG;
  if (dtype != TV_BF16 && dtype != TV_F32) return TV_ERR_INVALID_ARG;
  const size_t need = tv::argmax_workspace_bytes(N, V);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TV_ERR_WORKSPACE;
  return status_of(tv::launch_argmax(logits, dtype, N, V, row_stride, tok, workspace,
                                     static_cast<hipStream_t>(stream)));
}

int tv_accept(const int32_t* parent, const int32_t* draft, const int32_t* tok, int N, int32_t* accept_len,
              int32_t* accept_nodes, int32_t* accept_tokens, int32_t* bonus, int32_t* dev_error, void* stream) {
  if (!parent || !draft || !tok || !accept_len || !accept_nodes || !accept_tokens) return TV_ERR_INVALID_ARG;
  if (N < 1 || N > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  return status_of(tv::launch_accept(parent, draft, tok, N, accept_len, accept_nodes, accept_tokens, bonus,
                                     dev_error, static_cast<hipStream_t>(stream)));
}

int tv_argmax_accept(const void* logits, int dtype, int N, int V, int64_t row_stride, const int32_t* parent,
                     const int32_t* draft, int32_t* tok, int32_t* accept_len, int32_t* accept_nodes,
                     int32_t* accept_tokens, int32_t* bonus, void* workspace, size_t workspace_bytes,
                     int32_t* dev_error, void* stream) {
  if (!logits || !tok || !parent || !draft || !accept_len || !accept_nodes || !accept_tokens)
    return TV_ERR_INVALID_ARG;
  if (N < 1 || N > TV_MAX_NODES || V < 1 || V >= INT32_MAX || row_stride < V) return TV_ERR_INVALID_ARG;
  if (!span_ok(N, row_stride, 1, 0, V, dtype == TV_F32 ? 4 : 2)) return TV_ERR_INVALID_ARG;
  if (dtype != TV_BF16 && dtype != TV_F32) return TV_ERR_INVALID_ARG;
  const size_t need = tv::argmax_workspace_bytes(N, V);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TV_ERR_WORKSPACE;
  return status_of(tv::launch_argmax_accept(logits, dtype, N, V, row_stride, parent, draft, tok, accept_len,
                                            accept_nodes, accept_tokens, bonus, workspace, dev_error,
                                            static_cast<hipStream_t>(stream)));
}

int tv_kv_commit(void* k, void* v, int64_t kv_stride_t, int64_t kv_stride_h, int Hkv, int D, int L, int N,
                 const int32_t* accept_len, const int32_t* accept_nodes, int32_t* new_len, int32_t* dev_error,
                 void* stream) {
  if (!k || !v || !accept_len || !accept_nodes) return TV_ERR_INVALID_ARG;
  if (N < 1 || N > TV_MAX_NODES || L < 0 || Hkv < 1 || D < 8 || D % 8 != 0 || D > 4096) return TV_ERR_INVALID_ARG;
  if (kv_stride_t % 8 != 0 || kv_stride_h % 8 != 0 || !rows_disjoint(kv_stride_t, kv_stride_h, (int64_t)L + N, Hkv, D))
    return TV_ERR_INVALID_ARG;
  if (!span_ok((int64_t)L + N, kv_stride_t, Hkv, kv_stride_h, D, 2)) return TV_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v)) return TV_ERR_INVALID_ARG;
  return status_of(tv::launch_kv_commit(k, v, kv_stride_t, kv_stride_h, Hkv, D, L, N, accept_len, accept_nodes,
                                        new_len, dev_error, static_cast<hipStream_t>(stream)));
}

int tv_sample_accept(const void* logits, int dtype, int N, int V, int64_t row_stride, float temperature,
                     uint64_t seed, uint64_t offset, const int32_t* parent, const int32_t* draft, int32_t* tok,
                     int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens, int32_t* bonus,
                     void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (!logits || !tok || !parent || !draft || !accept_len || !accept_nodes || !accept_tokens)
    return TV_ERR_INVALID_ARG;
  if (N < 1 || N > TV_MAX_NODES || V < 1 || V >= INT32_MAX - 8 || row_stride < V) return TV_ERR_INVALID_ARG;
  if (!span_ok(N, row_stride, 1, 0, V, dtype == TV_F32 ? 4 : 2)) return TV_ERR_INVALID_ARG;
  if (dtype != TV_BF16 && dtype != TV_F32) return TV_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !std::isfinite(temperature) ||
      !std::isfinite((float)(1.4426950408889634 / (double)temperature)))
    return TV_ERR_INVALID_ARG;
  const size_t need = tv::argmax_workspace_bytes(N, V);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TV_ERR_WORKSPACE;
  return status_of(tv::launch_sample_accept(logits, dtype, N, V, row_stride, temperature, seed, offset, parent,
                                            draft, tok, accept_len, accept_nodes, accept_tokens, bonus, workspace,
                                            dev_error, static_cast<hipStream_t>(stream)));
}

int tv_kv_quantize_fp8(const void* src, int64_t src_stride_t, int64_t src_stride_h, int T, int Hkv, int D,
                       void* codes, int64_t codes_stride_t, int64_t codes_stride_h, int32_t* exps, void* stream) {
  if (!src || !codes || !exps) return TV_ERR_INVALID_ARG;
  if (T < 0 || Hkv < 1 || (int64_t)T * Hkv > INT32_MAX - 4) return TV_ERR_INVALID_ARG;
  if (D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
  if (src_stride_t < 0 || src_stride_h < 0 || src_stride_t % 8 || src_stride_h % 8) return TV_ERR_INVALID_ARG;
  if (codes_stride_t % 8 || codes_stride_h % 8 || !rows_disjoint(codes_stride_t, codes_stride_h, T, Hkv, D))
    return TV_ERR_INVALID_ARG;
  if (!span_ok(T, src_stride_t, Hkv, src_stride_h, D, 2) || !span_ok(T, codes_stride_t, Hkv, codes_stride_h, D, 1))
    return TV_ERR_INVALID_ARG;
  if (!aligned16(src) || ((uintptr_t)codes % 8) || ((uintptr_t)exps % 4)) return TV_ERR_INVALID_ARG;
  if (T == 0) return TV_OK;
  return status_of(tv::launch_kv_quantize(src, src_stride_t, src_stride_h, T, Hkv, codes, codes_stride_t,
                                          codes_stride_h, exps, static_cast<hipStream_t>(stream)));
}

int tv_kv_quantize_mx4(const void* src, int64_t src_stride_t, int64_t src_stride_h, int T, int Hkv, int D,
                       void* codes, int64_t codes_stride_t, int64_t codes_stride_h, int8_t* exps, void* stream) {
  if (!src || !codes || !exps) return TV_ERR_INVALID_ARG;
  if (T < 0 || Hkv < 1 || (int64_t)T * Hkv > INT32_MAX / 4) return TV_ERR_INVALID_ARG;
  if (D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
  if (src_stride_t < 0 || src_stride_h < 0 || src_stride_t % 8 || src_stride_h % 8) return TV_ERR_INVALID_ARG;
  if (codes_stride_t % 16 || codes_stride_h % 16 || !rows_disjoint(codes_stride_t, codes_stride_h, T, Hkv, D / 2))
    return TV_ERR_INVALID_ARG;
  if (!span_ok(T, src_stride_t, Hkv, src_stride_h, D, 2) || !span_ok(T, codes_stride_t, Hkv, codes_stride_h, D / 2, 1))
    return TV_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(codes)) return TV_ERR_INVALID_ARG;
  if (T == 0) return TV_OK;
  return status_of(tv::launch_kv_quantize_mx4(src, src_stride_t, src_stride_h, T, Hkv, codes, codes_stride_t,
                                              codes_stride_h, exps, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

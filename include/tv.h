/*
 * tv.h -- C ABI of libtv: target-side verification of a speculative draft tree on
 * AMD Instinct MI355X (gfx950).
 *
 * The method. A drafter proposes a block of tokens; the target model checks the whole
 * block in one pass, keeps the tokens it agrees with and drops the rest (DFlash
 * contributor guide, discosf.com/news/4742660, section "What is DFlash?"). With DDTree
 * verification the block is a tree of alternative continuations that the target scores
 * in one forward pass (Lucebox-Hub review, aichain-blog.pages.dev, section "2. DFlash";
 * Lucebox Hub tips page, d9249.github.io/tips/lucebox-hub, section "Lucebox Hub
 * overview"). Greedy verification compares each draft token with the target's
 * temperature-0 sample, the argmax of its logits (DFlash contributor guide, section
 * "Coding conventions", `sample(logits, temperature=0.0)`).
 *
 * This library computes the data-parallel part of one verify step:
 *   tv_tree_prep  parent[] -> ancestor bitmasks and depths            (integer)
 *   tv_tree_attn  tree-masked attention of N nodes over a bf16 KV cache
 *   tv_argmax     row argmax of the target logits                      (bit exact)
 *   tv_accept     longest accepted root-to-node path                   (bit exact)
 *   tv_argmax_accept   the two above in one call
 *   tv_sample_accept   the same with sampled targets (temperature > 0)
 *   tv_kv_commit  moves the accepted nodes' K/V rows behind the context   (bit exact)
 *   tv_kv_quantize_fp8   bf16 cache -> FP8 (E4M3) codes + per-row scales      (bit exact)
 *   tv_kv_quantize_mx4   bf16 cache -> 4-bit (E2M1) codes + per-32 scales     (bit exact)
 *   tv_tree_attn_mx4     tree attention over that 4-bit cache
 *   tv_tree_attn_fp8     tree attention over that FP8 cache
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the name ends in _host. The caller owns every
 *     buffer; the library never allocates or frees.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls only
 *     enqueue work and never synchronise the host; results appear in stream order.
 *   - Every call returns a tv_status. Arguments that the host can check are checked
 *     before anything is enqueued; a failed check enqueues nothing. Strides and sizes
 *     that together describe more than 2^56 bytes of one array (no allocation is that
 *     large) are refused with TV_ERR_INVALID_ARG.
 *   - A tree is given as parent[N] (int32, device): parent[i] in [-1, i-1], -1 meaning
 *     "child of the committed prefix". Node order is therefore topological. A kernel
 *     that meets an entry outside that range treats it as -1 and, when `dev_error` is
 *     non-NULL, stores TV_ERR_BAD_TREE there (it never writes TV_OK; clear it first).
 *     tv_validate_tree_host() gives the same check synchronously on a host copy.
 *   - Thread safety: calls from any host threads, on different streams, may run
 *     concurrently as long as they do not share output or workspace buffers. The only
 *     state kept between calls is per-device information filled in on first use (the
 *     compute-unit count, whether a kernel's large-LDS launch attribute has been set),
 *     held in atomics; concurrent first calls at worst repeat that idempotent setup.
 */
#ifndef TV_H_
#define TV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_ABI_VERSION 1
#define TV_MAX_NODES 256   /* ancestor sets are 4 x 64-bit words */
#define TV_HEAD_DIM 128    /* the only head dimension the kernels are built for */

typedef enum {
  TV_OK = 0,
  TV_ERR_INVALID_ARG = 1, /* null pointer, size out of range, misaligned buffer */
  TV_ERR_BAD_TREE = 2,    /* parent[] entry outside [-1, i-1] */
  TV_ERR_UNSUPPORTED = 3, /* valid request the kernels are not built for (D != 128) */
  TV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  TV_ERR_HIP = 5          /* the HIP runtime refused a launch */
} tv_status;

typedef enum { TV_BF16 = 0, TV_F32 = 1 } tv_dtype;

/* ABI version compiled into the library; equals TV_ABI_VERSION of a matching header. */
int tv_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* tv_status_string(int status);

/* Synchronous host check of a parent array (host memory). TV_OK, TV_ERR_BAD_TREE, or
 * TV_ERR_INVALID_ARG for a NULL pointer or N outside [1, TV_MAX_NODES]. */
int tv_validate_tree_host(const int32_t* parent_host, int N);

/*
 * Tree preprocessing. For every node i:
 *   anc[i][w]  bit j of word w is set when node 64*w + j is i or an ancestor of i
 *              (uint64 [N][4], little-endian word order; bits >= N are zero);
 *   depth[i]   number of nodes on the path from the prefix to i (1 for a child of the
 *              prefix) = popcount of anc[i].
 * Either output may be NULL (then it is not written). 1 <= N <= TV_MAX_NODES.
 * The same routine runs inside tv_tree_attn and tv_accept; this entry point exposes it.
 */
int tv_tree_prep(const int32_t* parent, int N, uint64_t* anc, int32_t* depth,
                 int32_t* dev_error, void* stream);

/*
 * Tree-masked attention (one layer's verify attention).
 *
 * Node i's query attends to every context key t in [0, L) and to the tree keys L + j
 * for j = i and every ancestor j of i -- the one-pass tree forward read as masked
 * softmax attention. Query head h reads KV head h / (Hq / Hkv).
 *
 *   q        bf16 [N][Hq][D], contiguous, 16-byte aligned.
 *   k, v     bf16; element (t, kvh, d) at base + t*kv_stride_t + kvh*kv_stride_h + d
 *            (strides in elements, non-negative multiples of 8; d contiguous; 16-byte
 *            aligned base). Token-major ([T][Hkv][D]) and head-major ([Hkv][T][D])
 *            caches are both served through the strides. Rows t in [0, L) are the
 *            context, rows L + i are tree node i's own key and value. Only rows
 *            [0, L + N) are read.
 *   parent   int32 [N] (see conventions).
 *   scale    softmax scale applied to q.k (1/sqrt(D) for standard attention).
 *   num_splits  number of KV splits per (KV head, row tile); 0 = library's choice.
 *   out      bf16 [N][Hq][D] (round to nearest even), contiguous, 16-byte aligned.
 *   lse      optional fp32 [N][Hq], natural-log sum of exp of the scaled scores.
 *   workspace   device scratch of at least tv_tree_attn_workspace_size(...) bytes with
 *               the same num_splits; 16-byte aligned. Contents need no initialisation.
 * Limits: 1 <= N <= TV_MAX_NODES, L >= 0, D == TV_HEAD_DIM, Hkv >= 1, Hq % Hkv == 0,
 * num_splits in [0, 1024], scale > 0 and finite; (L + N) * kv_stride_t * 2 bytes must stay
 * below 4 GiB (TV_ERR_UNSUPPORTED otherwise). Accumulation is fp32; each KV split's
 * normalised partial output passes through the workspace as bf16 (its log-sum-exp as
 * fp32). Inputs are never modified.
 */
size_t tv_tree_attn_workspace_size(int N, int L, int Hq, int Hkv, int D, int num_splits);

int tv_tree_attn(const void* q, const void* k, const void* v, int64_t kv_stride_t,
                 int64_t kv_stride_h, const int32_t* parent, int N, int L, int Hq,
                 int Hkv, int D, float scale, int num_splits, void* out, float* lse,
                 void* workspace, size_t workspace_bytes, int32_t* dev_error,
                 void* stream);

/*
 * Tree attention that allocates nothing, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and limits are those of tv_tree_attn without the workspace (the same
 * kernels, so the same outputs bit for bit). The split partials go to a static device
 * buffer of TV_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends; the call itself allocates nothing. A call whose partials need
 * more (tv_tree_attn_workspace_size(...) > TV_NOALLOC_SCRATCH_BYTES, e.g. forced split
 * counts far above the default) returns TV_ERR_WORKSPACE and enqueues nothing. Every call
 * on one device shares that device's buffer: calls that can overlap on one device (other
 * streams, other host threads) race on it and must be ordered by the caller. The buffer
 * needs no initialisation (each call writes every partial it reads).
 */
#define TV_NOALLOC_SCRATCH_BYTES (32u << 20)

int tv_tree_attn_noalloc(const void* q, const void* k, const void* v, int64_t kv_stride_t,
                         int64_t kv_stride_h, const int32_t* parent, int N, int L, int Hq,
                         int Hkv, int D, float scale, int num_splits, void* out, float* lse,
                         int32_t* dev_error, void* stream);

/*
 * Tree attention over an FP8 key/value cache (the quantised cache of Lucebox-Hub review,
 * section "2. DFlash"; format of tv_kv_quantize_fp8). Computes tv_tree_attn on the
 * dequantised cache k[t][h][d] = decode(k_codes[t][h][d]) * 2^k_exps[t * Hkv + h] (and
 * likewise v), which is exact in bf16: the result is the bf16 call's on those values.
 *   k_codes, v_codes   uint8 E4M3 codes; element (t, kvh, d) at base + t*kv_stride_t +
 *                      kvh*kv_stride_h + d (strides in bytes, multiples of 16; d
 *                      contiguous; 16-byte aligned base). NaN codes (0x7F, 0xFF) are not
 *                      allowed.
 *   k_exps, v_exps     int32 [>= L + N][Hkv], contiguous, 4-byte aligned; each in
 *                      [-117, 119] (what tv_kv_quantize_fp8 gives for rows whose largest
 *                      magnitude lies in [2^-125, 2^127]). An exponent outside is clamped
 *                      into the range and, when dev_error is non-NULL, TV_ERR_INVALID_ARG
 *                      is stored there.
 *   The other arguments, the workspace (tv_tree_attn_workspace_size) and the limits are
 *   those of tv_tree_attn, with (L + N) * kv_stride_t and (L + N) * Hkv * 4 bytes below
 *   4 GiB.
 */
int tv_tree_attn_fp8(const void* q, const void* k_codes, const void* v_codes,
                     const int32_t* k_exps, const int32_t* v_exps, int64_t kv_stride_t,
                     int64_t kv_stride_h, const int32_t* parent, int N, int L, int Hq,
                     int Hkv, int D, float scale, int num_splits, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t* dev_error,
                     void* stream);

/*
 * Tree attention over a 4-bit key/value cache (the sub-8-bit cache of Lucebox-Hub review,
 * section "2. DFlash"; format of tv_kv_quantize_mx4). Computes tv_tree_attn on the
 * dequantised cache k[t][h][d] = decode(code of d) * 2^k_exps[(t * Hkv + h) * 4 + d / 32]
 * (and likewise v), which is exact in bf16: the result is the bf16 call's on those values.
 *   k_codes, v_codes   uint8, two E2M1 codes per byte (value 2j in the low nibble of byte
 *                      j); row (t, kvh) of D / 2 bytes at base + t*kv_stride_t +
 *                      kvh*kv_stride_h (strides in bytes, multiples of 16; 16-byte aligned
 *                      base).
 *   k_exps, v_exps     int8 [>= L + N][Hkv][4], contiguous, 4-byte aligned; each in
 *                      [-125, 125] (what tv_kv_quantize_mx4 writes). An exponent outside is
 *                      clamped into the range and, when dev_error is non-NULL,
 *                      TV_ERR_INVALID_ARG is stored there.
 *   The other arguments, the workspace (tv_tree_attn_workspace_size) and the limits are
 *   those of tv_tree_attn, with (L + N) * kv_stride_t and (L + N) * Hkv * 4 bytes below
 *   4 GiB. Above 16 stacked rows per KV head the call always runs the 256-row kernel.
 */
int tv_tree_attn_mx4(const void* q, const void* k_codes, const void* v_codes,
                     const int8_t* k_exps, const int8_t* v_exps, int64_t kv_stride_t,
                     int64_t kv_stride_h, const int32_t* parent, int N, int L, int Hq,
                     int Hkv, int D, float scale, int num_splits, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t* dev_error,
                     void* stream);

/*
 * Row argmax: tok[i] = the lowest index u with logits[i][u] equal to the row maximum
 * (float comparison, so -0.0 and +0.0 tie). Rows holding NaN give an unspecified index.
 *   logits   dtype TV_BF16 or TV_F32, row i at base + i*row_stride elements.
 *   tok      int32 [N].
 *   workspace   at least tv_argmax_workspace_size(N, V) bytes, 16-byte aligned, used for
 *               per-slice partial results. Contents need no initialisation.
 * Limits: N >= 1, 1 <= V < 2^31 - 1, row_stride >= V.
 */
size_t tv_argmax_workspace_size(int N, int V);

int tv_argmax(const void* logits, int dtype, int N, int V, int64_t row_stride,
              int32_t* tok, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Longest accepted path. Node i matches when draft[i] == tok[i]; a node is accepted when
 * it and all its ancestors match. The result is the longest accepted root-to-node path;
 * among equally long paths the one ending at the lowest node index.
 *   accept_len     int32 [1]: path length (0 when nothing is accepted).
 *   accept_nodes   int32 [N]: path nodes root to leaf, then -1 padding.
 *   accept_tokens  int32 [N]: draft tokens of those nodes, then -1 padding.
 *   bonus          optional int32 [1]: tok of the lowest-index child of the path's last
 *                  node (of the prefix when nothing is accepted), -1 if it has none.
 * Limits: 1 <= N <= TV_MAX_NODES. Runs as a single workgroup (a single wave for N <= 64).
 */
int tv_accept(const int32_t* parent, const int32_t* draft, const int32_t* tok, int N,
              int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
              int32_t* bonus, int32_t* dev_error, void* stream);

/*
 * Argmax and acceptance in one call: tok = row argmax of the logits (exactly as
 * tv_argmax), then the longest accepted path on those tokens (exactly as tv_accept). Both
 * steps of greedy verification follow the passages cited for tv_argmax and tv_accept; one
 * workgroup (one wave for N <= 64) finishes the row reductions and walks the tree, so the
 * pair costs one launch fewer than two separate calls and tok never leaves the chip before
 * the walk.
 *   logits, dtype, V, row_stride, tok, workspace   as for tv_argmax (same workspace size).
 *   parent, draft, accept_len, accept_nodes, accept_tokens, bonus, dev_error   as for
 *            tv_accept.
 * Limits: 1 <= N <= TV_MAX_NODES and the limits of tv_argmax.
 */
int tv_argmax_accept(const void* logits, int dtype, int N, int V, int64_t row_stride,
                     const int32_t* parent, const int32_t* draft, int32_t* tok,
                     int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                     int32_t* bonus, void* workspace, size_t workspace_bytes,
                     int32_t* dev_error, void* stream);

/*
 * Sampled verification (temperature > 0). The pages' sampling call takes a temperature,
 * 0 meaning the argmax (DFlash contributor guide, section "Coding conventions"); here the
 * target's token for node i is a sample from softmax(logits[i] / T):
 *     tok[i] = lowest index of the largest  logits[i][v] / T - ln(-ln u(i, v))
 * (Gumbel-max). u(i, v) comes from Philox-4x32-10 (Salmon et al., SC 2011) with key
 * (seed low, seed high) and counter (v / 4, i, offset low, offset high): word v % 4 of the
 * output gives u = ((word >> 9) + 0.5) / 2^23. The same (seed, offset) repeats the draw;
 * advance offset between steps. Acceptance then follows tv_accept on these tokens.
 * The kernel ranks the equivalent scores logits[i][v] * log2(e) / T - log2(-log2 u) in
 * float32 (one fma and two hardware log2 per entry), so among scores equal after float32
 * rounding the lowest index wins.
 *   temperature  > 0, finite, with log2(e) / T finite in float32 (else TV_ERR_INVALID_ARG).
 *   Other arguments and limits as for tv_argmax_accept (same workspace size).
 */
int tv_sample_accept(const void* logits, int dtype, int N, int V, int64_t row_stride,
                     float temperature, uint64_t seed, uint64_t offset, const int32_t* parent,
                     const int32_t* draft, int32_t* tok, int32_t* accept_len,
                     int32_t* accept_nodes, int32_t* accept_tokens, int32_t* bonus,
                     void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream);

/*
 * Commit of the accepted path (the step after acceptance). Verification keeps the drafted
 * tokens the target agreed with and drops the rest (DFlash contributor guide, section
 * "What is DFlash?"); the kept tokens' keys and values, written at cache rows L + node by
 * the verify pass, move in place to rows L + 0, 1, ... in path order:
 *     for j in [0, *accept_len): row L + j <- row L + accept_nodes[j]   (K and V, all heads)
 * Other rows are not touched; the committed sequence then has length L + *accept_len.
 *   k, v         the cache of tv_tree_attn (same strides; any 2-byte element type; rows
 *                [0, L + N) valid); modified in place. 16-byte aligned.
 *   kv_stride_t, kv_stride_h, Hkv, D   as for tv_tree_attn (D a multiple of 8, <= 4096),
 *                with the rows (t, h), t < L + N, pairwise disjoint in a token-major
 *                (kv_stride_h >= D, kv_stride_t >= (Hkv - 1) * kv_stride_h + D) or a
 *                head-major (kv_stride_t >= D, kv_stride_h >= (L + N - 1) * kv_stride_t + D)
 *                layout; TV_ERR_INVALID_ARG otherwise.
 *   accept_len, accept_nodes   device int32, as tv_accept writes them.
 *   new_len      optional int32 [1]: receives L + *accept_len.
 *   dev_error    optional: receives TV_ERR_INVALID_ARG when *accept_len is outside [0, N]
 *                or the nodes are not increasing indices with accept_nodes[j] in [j, N);
 *                the cache is then left unchanged.
 * Limits: 1 <= N <= TV_MAX_NODES, L >= 0.
 */
int tv_kv_commit(void* k, void* v, int64_t kv_stride_t, int64_t kv_stride_h, int Hkv, int D,
                 int L, int N, const int32_t* accept_len, const int32_t* accept_nodes,
                 int32_t* new_len, int32_t* dev_error, void* stream);

/*
 * FP8 key/value cache: quantiser. Long contexts fit small memory through a quantised KV
 * cache (Lucebox-Hub review, section "2. DFlash"); the format is this library's own. Each
 * (token, head) row of D values gets one exponent e, the smallest integer with
 * max|x| <= 448 * 2^e (e = 0 for an all-zero row), and each value the OCP E4M3 code
 * (bias 7, no infinities, largest finite 448) nearest to x * 2^-e, ties to the even
 * mantissa, -0 coded as +0. The row dequantises to decode(code) * 2^e, which is exact in
 * bfloat16.
 *   src          bf16 [T][Hkv][D], strides src_stride_t / src_stride_h in elements
 *                (non-negative multiples of 8), D contiguous; 16-byte aligned. Values
 *                must be finite.
 *   codes        uint8 [T][Hkv][D] out, strides codes_stride_t / codes_stride_h in bytes
 *                (multiples of 8), D contiguous; 8-byte aligned. Its rows must be pairwise
 *                disjoint in a token-major or a head-major layout (the rule of
 *                tv_kv_commit with T rows of D bytes).
 *   exps         int32 [T * Hkv] out (row t * Hkv + h), 4-byte aligned.
 * Limits: T >= 0 (T = 0 enqueues nothing), Hkv >= 1, D = TV_HEAD_DIM (else
 * TV_ERR_UNSUPPORTED).
 */
int tv_kv_quantize_fp8(const void* src, int64_t src_stride_t, int64_t src_stride_h, int T,
                       int Hkv, int D, void* codes, int64_t codes_stride_t,
                       int64_t codes_stride_h, int32_t* exps, void* stream);

/*
 * 4-bit key/value cache: quantiser. A quantised cache of under 8 bits per value, as the
 * pages' 256K-context cache is (Lucebox-Hub review, section "2. DFlash"); the format is
 * this library's own, in the block structure of the OCP Microscaling formats: each run of
 * 32 consecutive values of a (token, head) row shares one exponent e, the smallest integer
 * with max|x| <= 6 * 2^e (e = 0 for an all-zero block) clamped to [-125, 125], and each
 * value becomes the OCP FP4 E2M1 code (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) nearest to
 * x * 2^-e, ties to the even code, saturating at 6 (only where e was clamped), -0 coded
 * as +0. The block dequantises to decode(code) * 2^e, which is exact in bfloat16.
 *   src          bf16 [T][Hkv][D], strides src_stride_t / src_stride_h in elements
 *                (non-negative multiples of 8), D contiguous; 16-byte aligned. Values
 *                must be finite.
 *   codes        uint8 [T][Hkv][D / 2] out, two codes per byte (value 2j in the low
 *                nibble of byte j), strides codes_stride_t / codes_stride_h in bytes
 *                (multiples of 16), D / 2 contiguous; 16-byte aligned. Its rows must be
 *                pairwise disjoint in a token-major or a head-major layout (the rule of
 *                tv_kv_commit with T rows of D / 2 bytes).
 *   exps         int8 [T * Hkv * D / 32] out (block b of row (t, h) at (t * Hkv + h) * 4 + b).
 * Limits: T >= 0 (T = 0 enqueues nothing), Hkv >= 1, D = TV_HEAD_DIM (else
 * TV_ERR_UNSUPPORTED).
 */
int tv_kv_quantize_mx4(const void* src, int64_t src_stride_t, int64_t src_stride_h, int T,
                       int Hkv, int D, void* codes, int64_t codes_stride_t,
                       int64_t codes_stride_h, int8_t* exps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_H_ */

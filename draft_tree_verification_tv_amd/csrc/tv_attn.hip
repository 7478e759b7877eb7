// Tree-masked attention for verifying a speculative draft tree on gfx950.
//
// The target scores every node of the draft tree in one forward pass (Lucebox-Hub
// review, aichain-blog.pages.dev, "2. DFlash"; Lucebox Hub tips page, "Lucebox Hub
// overview"). Read as attention: node i's query sees the whole committed context and the
// tree keys of i and its ancestors; nothing else.
//
// Design (split-KV flash decoding, MFMA form):
//   * Rows. For KV head h the G = Hq/Hkv query heads of all N nodes are stacked into
//     M = G*N rows (row r -> node r/G, q head h*G + r%G), so one K/V tile read from HBM
//     is used by every row that needs it. A workgroup owns up to 256 rows, 32 per wave.
//   * Splits. The key sequence [0, L+N) is cut into S ranges; each workgroup streams one
//     range for one (KV head, row tile) and writes a normalised fp32 partial output and
//     its log2-sum-exp. attn_merge_kernel combines the partials.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the
//     accumulator layout gives every lane one query row (16 keys per 32-key block), so the
//     online-softmax statistics are lane-local (plus one exchange with lane ^ 32), and
//     P^T feeds the P.V product as the B operand straight from registers. O^T = V^T P^T
//     accumulates in 64 fp32 registers per lane.
//   * Memory pipeline. K and V tiles (64 keys x 128 dims, bf16) are copied HBM -> LDS by
//     global_load_lds_dwordx4 (no registers involved) into a ring of four stages, three
//     tiles ahead of their use; each wave waits only for its own copies of the tile it needs
//     next and the barrier drains LDS traffic only, so up to 96 KB per CU stay in flight.
//     Both tiles are row-major with a 16-byte-chunk XOR swizzle: K rows are read as 128-bit
//     MFMA A operands; V is read with ds_read_b64_tr_b16, whose 4x16 in-register transpose
//     hands each lane four consecutive keys of one head-dim column -- exactly the k-run the
//     P.V MFMA needs -- so V needs no transposition pass.
//   * Software pipeline. Every wave walks its keys in 32-key blocks. While it turns block j
//     into probabilities it already issues the score MFMAs of block j+1 (into the other of
//     two score buffers), then block j's P.V MFMAs: MFMA and VALU work of one wave overlap,
//     and the two waves sharing a SIMD fill each other's stalls.
//   * Softmax. exp2 with the scale folded into one FMA. The reference maximum is raised
//     only when a block exceeds it by more than 2^8 (lazy rescaling), so the 64-register
//     rescale of O is off the common path. Row sums use the unrounded fp32 probabilities
//     (so the exported log-sum-exp is exact to fp32); P is rounded to bf16 only as the
//     MFMA operand. The two lanes holding a row exchange maxima and sums with
//     permlane32_swap.
//   * Tree keys (rows L..L+N-1) are masked with per-node ancestor bitmasks built in LDS by
//     the workgroups whose range reaches them.
//   * Work items are remapped so that consecutive ones (the splits of one KV head) land
//     on the same XCD.
#include <cmath>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int D = TV_HEAD_DIM;
constexpr int KT = 64;                         // keys per tile
constexpr int TILE_ROWS = 256;                 // stacked rows per workgroup (8 waves x 32)
constexpr int ROWB = D * 2;                    // bytes per K or V row (256)
constexpr int TILE_B = KT * ROWB;              // 16 KB per K (or V) tile
constexpr int STAGE_B = 2 * TILE_B;            // K + V
constexpr int NSTAGE = 4;                      // LDS ring: tiles t-1 .. t+2
constexpr int TREE_ANC_BYTES = kMaxNodes * kAncWords * 8;
constexpr int TREE_BYTES = TREE_ANC_BYTES + 2 * kMaxNodes * 4;
constexpr int SMEM_BYTES = NSTAGE * STAGE_B + TREE_BYTES;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleTh = 8.0f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t st, sh;  // KV strides in elements
  const int32_t* parent;
  int N, L, T, Hq, G, M;
  int RT, S, KS;
  float c;  // scale * log2(e)
  float* part_o;
  float* part_lse;
  int32_t* dev_error;
  int remap;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte-chunk swizzles. K: chunk c of row r lives at chunk c ^ (r & 15), so the 16 rows
// a 128-bit read phase touches hit 16 different chunks. V: chunk c of row r lives at
// c ^ swz_v(r) with swz_v = {0, 6, 10, 12}[r & 3]; the transposed reads touch 4
// consecutive rows x 4 chunks per half-wave, which this maps onto distinct chunks (and
// onto distinct chunk pairs modulo 8).
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return (0xCA60 >> ((r & 3) * 4)) & 15; }

// Asynchronous 16-byte-per-lane copy from global memory straight into LDS
// (global_load_lds_dwordx4): lane i's 16 bytes at gbase + goff land at LDS byte
// lds + 16*i. No VGPR receives data, so nothing can be overwritten while the copy is in
// flight; completion is tracked by vmcnt. M0 carries the LDS address and is restored.
// An LDS-DMA load that follows an SALU write of M0 needs one wait state (s_nop 0), or
// it may still see the previous M0 and write the wrong LDS block.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t goff, const void* gbase) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(goff), "s"(gbase)
      : "memory");
}

// Workgroup barrier that waits for this wave's LDS traffic and for all but its newest
// kPending vector-memory operations (the copies of the tile after next stay in flight).
// No release fence: outstanding global loads are deliberately not drained.
template <int kPending>
__device__ __forceinline__ void barrier_keep(void) {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kPending) : "memory");
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_split_kernel(SplitParams p) {
  constexpr int BLK = KT / 4;            // 1 KB blocks per K (or V) tile
  constexpr int BPW = BLK / NW;          // blocks of each per wave
  constexpr int DPT = 2 * BPW;           // copies per wave per tile
  static_assert(BLK % NW == 0, "waves must divide the tile");

  extern __shared__ __align__(16) char smem[];
  uint64_t* anc = reinterpret_cast<uint64_t*>(smem + NSTAGE * STAGE_B);
  int* par = reinterpret_cast<int*>(smem + NSTAGE * STAGE_B + TREE_ANC_BYTES);
  int* jmp = par + kMaxNodes;

  // ---- work item
  int w = blockIdx.x;
  if (p.remap) {
    const int per = gridDim.x >> 3;
    w = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  const int rt = w % p.RT;
  const int s = (w / p.RT) % p.S;
  const int h = w / (p.RT * p.S);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int grp = lane >> 5;
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;

  const int r = rt * TILE_ROWS + wave * 32 + ql;
  const bool rvalid = r < p.M;
  const int node = rvalid ? r / p.G : 0;
  const int qh = h * p.G + (rvalid ? r % p.G : 0);

  // ---- query fragments (B operand of S^T = K Q^T): dims s8*16 + grp*8 .. +7
  bf16x8 qf[8];
  {
    const uint16_t* qrow = p.q + ((int64_t)node * p.Hq + qh) * D + grp * 8;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (rvalid) x = *reinterpret_cast<const u32x4*>(qrow + s8 * 16);
      qf[s8] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int kbeg = s * p.KS;
  const int kend = min(kbeg + p.KS, p.T);
  const int ntiles = (kend - kbeg + KT - 1) / KT;
  if (kend > p.L) tree_prep_lds(p.parent, p.N, anc, par, jmp, p.dev_error);

  const uint16_t* kbase = p.k + (int64_t)h * p.sh;
  const uint16_t* vbase = p.v + (int64_t)h * p.sh;

  // ---- per-lane LDS offsets
  int koff[8];  // K row ql, chunk 2*s8 + grp
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) koff[s8] = ql * ROWB + (((2 * s8 + grp) ^ swz_k(ql)) << 4);
  int voff[4];  // V rows 4*grp + i16/4 (+8), head-dim columns db*32 + g16*16 + 4*(i16%4)
  {
    const int row = 4 * grp + (i16 >> 2);
    const int sw = swz_v(row);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = db * 4 + g16 * 2 + ((i16 & 3) >> 1);
      voff[db] = row * ROWB + ((chunk ^ sw) << 4) + (i16 & 1) * 8;
    }
  }

  // ---- HBM -> LDS copies. A tile's K (and V) is 16 blocks of 4 rows x 256 bytes; wave w
  // copies blocks w, w + NW, ... of both. Lane i of a block copy fills LDS row
  // 4b + i/16, physical chunk i%16, so it loads logical chunk (i%16) ^ swizzle(row).
  // Offsets within one KV head are 32-bit (the host guarantees (L+N) rows fit).
  const char* kb8 = reinterpret_cast<const char*>(kbase);
  const char* vb8 = reinterpret_cast<const char*>(vbase);
  const uint32_t rowstride_b = (uint32_t)p.st * 2u;
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
  uint32_t dk[BPW], dv[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int row = 4 * (wave + j * NW) + (lane >> 4);
    const int pc = lane & 15;
    dk[j] = (uint32_t)row * rowstride_b + (uint32_t)((pc ^ swz_k(row)) << 4);
    dv[j] = (uint32_t)row * rowstride_b + (uint32_t)((pc ^ swz_v(row)) << 4);
  }

  auto issue = [&](int t) __attribute__((always_inline)) {
    const int kt0 = kbeg + t * KT;
    const uint32_t st_lds = lds_base + (uint32_t)((t & (NSTAGE - 1)) * STAGE_B);
    if (kt0 + KT <= p.T) {
      const uint32_t base = (uint32_t)kt0 * rowstride_b;
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const uint32_t blk = (uint32_t)((wave + j * NW) * 1024);
        dma16(st_lds + blk, base + dk[j], kb8);
        dma16(st_lds + TILE_B + blk, base + dv[j], vb8);
      }
    } else {
      // Last tile of the sequence: rows past L+N re-read row L+N-1 (always masked).
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int row = 4 * (wave + j * NW) + (lane >> 4);
        const int pc = lane & 15;
        const uint32_t grow = (uint32_t)min(kt0 + row, p.T - 1) * rowstride_b;
        const uint32_t blk = (uint32_t)((wave + j * NW) * 1024);
        dma16(st_lds + blk, grow + (uint32_t)((pc ^ swz_k(row)) << 4), kb8);
        dma16(st_lds + TILE_B + blk, grow + (uint32_t)((pc ^ swz_v(row)) << 4), vb8);
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_ref = -INFINITY;  // reference maximum of the row, log2 domain (scaled)
  float lsum = 0.f;         // this lane's part of the row sum, relative to m_ref
  f32x16 sc[2];             // scores of two consecutive 32-key blocks
  bf16x8 pb[2];             // P^T fragments of the current block (two 16-key steps)

  // Scheduling masks for __builtin_amdgcn_sched_group_barrier.

  // S^T of 32-key block kb of the tile in `stage` into sc[c]: 8 K fragments, 8 MFMAs.
  auto qk = [&](int stage, int kb, int c) __attribute__((always_inline)) {
    const char* Ks = smem + stage * STAGE_B + kb * 32 * ROWB;
    sc[c] = f32x16{};
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      sc[c] = mfma32(*reinterpret_cast<const bf16x8*>(Ks + koff[s8]), qf[s8], sc[c]);
  };

  // O^T += V^T P^T over 32-key block kb of the tile in `stage`; V^T fragments come from
  // the row-major V tile through transposed reads (two per MFMA).
  auto pv = [&](int stage, int kb) __attribute__((always_inline)) {
    const char* Vs = smem + stage * STAGE_B + TILE_B + kb * 32 * ROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char* a0 = Vs + (i >> 2) * 16 * ROWB + voff[i & 3];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * ROWB));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[i & 3] = mfma32(a, pb[i >> 2], o[i & 3]);
    }
  };

  // Keys past the context: tree keys by ancestry, anything past L+N never. The block's 32
  // keys kb0 .. kb0+31 map to a 32-bit window of the row's ancestor set (bit b <-> node
  // kb0 + b - L), with context keys (kb0 + b < L) always set; nodes >= N have no ancestor
  // bit, so keys past L+N come out clear.
  auto mask = [&](int kb0, int c) __attribute__((always_inline)) {
    if (kb0 + 32 <= p.L) return;
    const int d = kb0 - p.L;  // > -32 here
    const uint64_t* a = anc + node * kAncWords;
    uint32_t win;
    if (d >= 0) {
      const int wi = d >> 6, sh = d & 63;
      const uint64_t lo = wi < kAncWords ? a[wi] : 0ull;
      const uint64_t hi = (sh > 32 && wi + 1 < kAncWords) ? a[wi + 1] : 0ull;
      win = (uint32_t)((lo >> sh) | (sh > 32 ? hi << (64 - sh) : 0ull));
    } else {
      win = (uint32_t)((a[0] << (-d)) | ((1ull << (-d)) - 1ull));
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int b = 8 * (e >> 2) + 4 * grp + (e & 3);  // key within the block
      if (!((win >> b) & 1u)) sc[c][e] = -INFINITY;
    }
  };

  // Lazy online-softmax rescale to the maximum of block sc[c]: the reference maximum moves
  // only when a block exceeds it by more than 2^8. A row's 32 keys are split between lanes
  // l and l ^ 32, whose maxima permlane32_swap exchanges (max(r0, r1) is the row maximum
  // in both).
  auto rescale = [&](int c) __attribute__((always_inline)) {
    // One v_max3 per two new scores (8 instructions for 16).
    float m = fmaxf(fmaxf(sc[c][0], sc[c][1]), sc[c][2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) m = fmaxf(fmaxf(m, sc[c][e]), sc[c][e + 1]);
    m = fmaxf(m, sc[c][15]);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const float mt = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * p.c;
    const bool need = mt > m_ref + kRescaleTh;
    if (__any(need)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = need ? exp2f(m_ref - m_new) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m_ref = m_new;
    }
  };

  // Probabilities of block sc[c] relative to m_ref: unrounded fp32 row sums, bf16 P^T
  // fragments for the P.V MFMAs.
  auto probs = [&](int c) __attribute__((always_inline)) {
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      bf16x2 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c][th * 8 + 2 * j], p.c, -mu));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c][th * 8 + 2 * j + 1], p.c, -mu));
        b[j] = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
        lsum += p0 + p1;
      }
      pb[th] = bf16x8{b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
    }
  };

  // Barrier closing tile t: tile t+2 has landed; tile t+3 (if any) stays in flight.
  auto wait_step = [&](int t) __attribute__((always_inline)) {
    if (t + 3 < ntiles)
      barrier_keep<DPT>();
    else
      barrier_keep<0>();
  };

  // Tiles whose 64 keys all precede L need no mask.
  const int nplain = p.L > kbeg ? min(ntiles, (p.L - kbeg) / KT) : 0;

  // Sub-step over 32-key block (t, kb) with a successor block (tn, kb ^ 1): the
  // successor's score MFMAs, this block's softmax and this block's P.V MFMAs form one
  // scheduling region, so the compiler interleaves MFMAs with the softmax VALU work; then
  // the successor is masked (if it reaches past the context) and the running maximum
  // updated. The score buffer index equals kb.
  auto sub = [&](int t, auto kbc, int tn) __attribute__((always_inline)) {
    constexpr int kb = decltype(kbc)::value;
    constexpr int kbn = kb ^ 1;
    qk(tn & (NSTAGE - 1), kbn, kbn);
    probs(kb);
    pv(t & (NSTAGE - 1), kb);
    if (tn >= nplain) mask(kbeg + tn * KT + kbn * 32, kbn);
    rescale(kbn);
  };

  // ---- prologue: tiles 0, 1, 2 start streaming; tiles 0 and 1 must land.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // query loads are not tile copies
  for (int t = 0; t < 3 && t < ntiles; ++t) issue(t);
  if (ntiles > 2)
    barrier_keep<DPT>();
  else
    barrier_keep<0>();
  qk(0, 0, 0);
  if (nplain == 0) mask(kbeg, 0);
  rescale(0);

  // Tile t: block 0 (successor: block 1 of tile t), block 1 (successor: block 0 of tile
  // t+1); the barrier after each tile guarantees tile t+2 and keeps tile t+3 in flight.
  // Stage reuse: tile t+3 overwrites tile t-1, whose last reads were in tile t-1's blocks.
  for (int t = 0; t + 1 < ntiles; ++t) {
    if (t + 3 < ntiles) issue(t + 3);
    sub(t, std::integral_constant<int, 0>{}, t);
    sub(t, std::integral_constant<int, 1>{}, t + 1);
    wait_step(t);
  }
  {
    const int t = ntiles - 1;
    sub(t, std::integral_constant<int, 0>{}, t);
    probs(1);
    pv(t & (NSTAGE - 1), 1);
  }

  // ---- partial result of this split
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float lse2 = lsum > 0.f ? m_ref + __log2f(lsum) : -INFINITY;
  if (rvalid) {
    const int64_t base = ((int64_t)(h * p.RT + rt) * p.S + s) * TILE_ROWS + wave * 32 + ql;
    float* po = p.part_o + base * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 val = {o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                           o[db][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>(po + db * 32 + 8 * i + 4 * grp) = val;
      }
    }
    if (grp == 0) p.part_lse[base] = lse2;
  }
}

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int N, Hq, G, RT, S;
};

// One wave per (node, q head) row, two head-dim values per lane:
// lse = M + log2 sum_s 2^(lse_s - M), out = sum_s 2^(lse_s - lse) * out_s.
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams mp) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= mp.N * mp.Hq) return;
  const int n = row / mp.Hq;
  const int qh = row % mp.Hq;
  const int h = qh / mp.G;
  const int r = n * mp.G + qh % mp.G;
  const int rt = r / TILE_ROWS;
  const int64_t base0 = (int64_t)(h * mp.RT + rt) * mp.S * TILE_ROWS + (r % TILE_ROWS);
  const float* lse_p = mp.part_lse + base0;
  const float* o_p = mp.part_o + base0 * D + 2 * lane;

  float mx = -INFINITY;
  for (int s = lane; s < mp.S; s += 64) mx = fmaxf(mx, lse_p[(int64_t)s * TILE_ROWS]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));

  f32x2 acc = {0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    int s = 0;
    for (; s + 8 <= mp.S; s += 8) {
      float l8[8];
      f32x2 x8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        l8[u] = lse_p[(int64_t)(s + u) * TILE_ROWS];
        x8[u] = *reinterpret_cast<const f32x2*>(o_p + (int64_t)(s + u) * TILE_ROWS * D);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = exp2f(l8[u] - mx);
        wsum += wgt;
        acc += wgt * x8[u];
      }
    }
    for (; s < mp.S; ++s) {
      const float wgt = exp2f(lse_p[(int64_t)s * TILE_ROWS] - mx);
      wsum += wgt;
      acc += wgt * *reinterpret_cast<const f32x2*>(o_p + (int64_t)s * TILE_ROWS * D);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const bf16x2 ob = __builtin_convertvector((f32x2{acc[0] * inv, acc[1] * inv}), bf16x2);
  *reinterpret_cast<bf16x2*>(mp.out + (int64_t)row * D + 2 * lane) = ob;
  if (mp.lse && lane == 0) mp.lse[row] = mx == -INFINITY ? -INFINITY : (mx + __log2f(wsum)) * kLn2;
}

template <int NW>
hipError_t launch_split(const SplitParams& sp, int nwg, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_split_kernel<NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(attn_split_kernel<NW>, dim3(nwg), dim3(NW * 64), SMEM_BYTES, stream, sp);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int N, int L, int Hq, int Hkv, int num_splits, int num_cus) {
  AttnPlan p;
  p.G = Hq / Hkv;
  p.M = p.G * N;
  p.RT = (p.M + TILE_ROWS - 1) / TILE_ROWS;
  const int rows = p.M < TILE_ROWS ? p.M : TILE_ROWS;
  p.NW = rows <= 64 ? 2 : rows <= 128 ? 4 : 8;
  p.T = L + N;
  const int tiles = (p.T + KT - 1) / KT;
  int S = num_splits;
  if (S <= 0) {
    // One workgroup per CU (the four LDS stages and the tree masks take 138 KB): enough
    // splits to give every CU a workgroup, down to one 64-key tile per split. Short
    // sequences are latency-bound, so filling the chip beats saving partial-output
    // traffic; long ones get long splits anyway.
    const int units = Hkv * p.RT;
    S = (num_cus + units - 1) / units;
  }
  if (S > tiles) S = tiles;
  if (S < 1) S = 1;
  const int tps = (tiles + S - 1) / S;
  p.KS = tps * KT;
  p.S = (p.T + p.KS - 1) / p.KS;
  return p;
}

size_t attn_workspace_bytes(const AttnPlan& p, int Hkv) {
  const size_t rows = (size_t)Hkv * p.RT * p.S * TILE_ROWS;
  size_t bytes = rows * D * sizeof(float);
  bytes = (bytes + 255) / 256 * 256;
  bytes += rows * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_tree_attn(const AttnPlan& plan, const void* q, const void* k, const void* v, int64_t st,
                            int64_t sh, const int32_t* parent, int N, int L, int Hq, int Hkv, float scale,
                            void* out, float* lse, void* workspace, int32_t* dev_error, hipStream_t stream) {
  const size_t rows = (size_t)Hkv * plan.RT * plan.S * TILE_ROWS;
  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + (rows * D * sizeof(float) + 255) / 256 * 256);

  SplitParams sp;
  sp.q = static_cast<const uint16_t*>(q);
  sp.k = static_cast<const uint16_t*>(k);
  sp.v = static_cast<const uint16_t*>(v);
  sp.st = st;
  sp.sh = sh;
  sp.parent = parent;
  sp.N = N;
  sp.L = L;
  sp.T = plan.T;
  sp.Hq = Hq;
  sp.G = plan.G;
  sp.M = plan.M;
  sp.RT = plan.RT;
  sp.S = plan.S;
  sp.KS = plan.KS;
  sp.c = scale * kLog2e;
  sp.part_o = part_o;
  sp.part_lse = part_lse;
  sp.dev_error = dev_error;
  const int nwg = Hkv * plan.RT * plan.S;
  sp.remap = (nwg % 8 == 0) ? 1 : 0;

  hipError_t e;
  switch (plan.NW) {
    case 2: e = launch_split<2>(sp, nwg, stream); break;
    case 4: e = launch_split<4>(sp, nwg, stream); break;
    default: e = launch_split<8>(sp, nwg, stream); break;
  }
  if (e != hipSuccess) return e;

  MergeParams mp;
  mp.part_o = part_o;
  mp.part_lse = part_lse;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse;
  mp.N = N;
  mp.Hq = Hq;
  mp.G = plan.G;
  mp.RT = plan.RT;
  mp.S = plan.S;
  const int rows_out = N * Hq;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((rows_out + 3) / 4), dim3(256), 0, stream, mp);
  return hipGetLastError();
}

}  // namespace tv

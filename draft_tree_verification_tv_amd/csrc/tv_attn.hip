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
//     is used by every row that needs it. A workgroup always runs 8 waves: RWV row-waves
//     of 32 rows times KSW key-waves (8x1 for M > 128; 4x2, 2x4, 1x8 for fewer rows).
//     Key-wave k takes every KSW-th 32-key block of the split with its own online
//     softmax; the key-waves' partial results are merged in LDS at the end (a tree of
//     log2 KSW rounds), so small trees and single-token decode still keep two waves busy
//     on every SIMD. With a single row-wave each 32-key block has one reader, so every
//     wave streams its own blocks (K into registers, V through a private LDS stage; an
//     FP8 cache is widened in registers on the way) with no shared ring and no barrier.
//   * Splits. The key sequence [0, L+N) is cut into S ranges; each workgroup streams one
//     range for one (KV head, row tile) and writes a normalised partial output (bf16)
//     and its log2-sum-exp (fp32). attn_merge_small_kernel (up to 64 splits, one memory
//     round trip) or attn_merge_kernel combines the partials.
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
//     and the two waves sharing a SIMD fill each other's stalls. In the 256-row kernel the
//     K fragments of block j+2 are read before block j's P.V, so score MFMAs find their
//     operands in registers.
//   * Softmax. exp2 with the scale folded into one FMA, against a lazy reference maximum
//     that moves only when a block would exceed it by more than 2^8; whether it must is
//     read off the probabilities themselves (a lane's sum of 16 above 2^8), so the block
//     maximum and the 64-register rescale of O are off the common path. Row sums use the
//     unrounded fp32 probabilities (so the exported log-sum-exp is exact to fp32); P is
//     rounded to bf16 only as the MFMA operand. The two lanes holding a row exchange
//     maxima and sums with permlane32_swap.
//   * Tree keys (rows L..L+N-1) are masked with per-node ancestor bitmasks built in LDS by
//     the workgroups whose range reaches them.
//   * Work items are remapped so that consecutive ones (the splits of one KV head) land
//     on the same XCD.
//   * FP8 cache (E4M3 codes with one power-of-two exponent per token and head; the
//     quantised KV cache of Lucebox-Hub review, "2. DFlash", in a self-defined format).
//     Codes and exponents stream into a ring of raw stages (half the HBM bytes of bf16);
//     each tile is widened once per workgroup into bf16 stages with the same swizzles,
//     code * 2^e exactly (v_cvt_scalef32_pk_bf16_fp8), two steps ahead for K and one for
//     V, inside the same one-barrier-per-tile pipeline. The MFMA and softmax code is
//     shared with the bf16 kernel, so both compute the same function of the bf16 values.
#include <atomic>
#include <type_traits>
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
// bf16 ring layout: the four K stages first, then the four V stages, so every stage of
// either lies within 64 KB of its first one (ds_read immediate offsets reach it).
constexpr int V_OFF = NSTAGE * TILE_B;
constexpr int TREE_ANC_BYTES = kMaxNodes * kAncWords * 8;
constexpr int TREE_BYTES = TREE_ANC_BYTES + 2 * kMaxNodes * 4;
constexpr int SMEM_BYTES = NSTAGE * STAGE_B + TREE_BYTES;
// FP8 cache: raw stages of [K codes 8 KB][V codes 8 KB][K exps 256 B][V exps 256 B], then
// three bf16 K stages, two bf16 V stages, the tree masks.
constexpr int F8_ROWB = D;                                  // bytes per code row
constexpr int F8_TILE_B = KT * F8_ROWB;                     // 8 KB
constexpr int F8_RAW_B = 2 * F8_TILE_B + 2 * KT * 4;
constexpr int F8_NRAW = 4;
constexpr int F8_KB_OFF = F8_NRAW * F8_RAW_B;
constexpr int F8_VB_OFF = F8_KB_OFF + 3 * TILE_B;
constexpr int F8_TREE_OFF = F8_VB_OFF + 2 * TILE_B;
constexpr int F8_SMEM_BYTES = F8_TREE_OFF + TREE_BYTES;
static_assert(F8_SMEM_BYTES <= 160 * 1024, "FP8 stages exceed the LDS");
// Row exponents for which every code * 2^e is a normal bf16 (or zero) and 2^e a normal
// fp32: smallest code 2^-9, largest 448.
constexpr int kExpMin = -117;
constexpr int kExpMax = 119;
// 4-bit cache (E2M1 codes, one int8 exponent per 32 values): raw stages of [K codes 4 KB]
// [V codes 4 KB][K exponents 256 B][V exponents 256 B] inside the FP8 raw-stage stride; an
// exponent e in [-125, 125] keeps every code * 2^e a finite bf16 and 2^e a normal float.
constexpr int MX_ROWB = D / 2;                              // code bytes per row
constexpr int MX_TILE_B = KT * MX_ROWB;                     // 4 KB
constexpr int kMxExpMin = -125;
constexpr int kMxExpMax = 125;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCheck = 256.0f;  // largest probability (and 16-key partial sum) kept

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct SplitParams {
  const uint16_t* q;
  const void* k;   // bf16 values, or E4M3 codes
  const void* v;
  const int32_t* ek;  // FP8 only: row exponents [T][Hkv]
  const int32_t* ev;
  int Hkv;
  int64_t st, sh;  // KV strides in elements
  const int32_t* parent;
  int N, L, T, Hq, G, M;
  int RT, S, KS;
  float c;  // scale * log2(e)
  __bf16* part_o;  // normalised partial outputs, bf16
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
// kStream: the cache is streamed, each K/V byte read once per call (or by the few
// row-tile workgroups of one split), so the copy carries the non-temporal hint at device
// scope (sc1 nt) and does not displace other data in the caches. Only for copies whose
// rows cover whole 128-byte lines (bf16 rows of 256 bytes, FP8 rows of 128): a copy of
// part of a line would drop the line that the neighbouring head's workgroup reads next.
template <bool kStream>
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t goff, const void* gbase) {
  uint32_t saved;
  if constexpr (kStream)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3 sc1 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(goff), "s"(gbase)
        : "memory");
  else
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

// The same with 4 bytes per lane (lane i lands at lds + 4*i).
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t goff, const void* gbase) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(goff), "s"(gbase)
      : "memory");
}

// A pointer whose value is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* ptr) {
  const uint64_t x = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier that waits for this wave's LDS traffic and for all but its newest
// kPending vector-memory operations (the copies of the tile after next stay in flight).
// No release fence: outstanding global loads are deliberately not drained.
template <int kPending>
__device__ __forceinline__ void barrier_keep(void) {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kPending) : "memory");
}

template <int RWV, int KSW, bool kF8, bool kMX = false>
__global__ __launch_bounds__(RWV * KSW * 64) void attn_split_kernel(SplitParams p) {
  constexpr int NW = RWV * KSW;
  constexpr int ROWS = RWV * 32;  // stacked rows per workgroup
  static_assert(NW == 8, "eight waves per workgroup");
  static_assert(!kMX || (kF8 && RWV >= 2), "the 4-bit cache runs the shared-ring kernels");
  // Copies per wave per tile: bf16, 16 blocks of 1 KB for each of K and V; FP8, 8 blocks
  // of codes for each plus one copy of 128 / NW exponents; 4-bit, one of the 4 + 4 code
  // blocks plus one copy of 16 exponent words.
  constexpr int BLK = kF8 ? KT / 8 : KT / 4;
  constexpr int BPW = BLK / NW;
  constexpr int DPT = kMX ? 2 : 2 * BPW + (kF8 ? 1 : 0);
  constexpr int EPW = 2 * KT / NW;      // FP8: exponents copied per wave
  constexpr int TREE_OFF = kF8 ? F8_TREE_OFF : NSTAGE * STAGE_B;
  static_assert(BLK % NW == 0, "waves must divide the tile");

  extern __shared__ __align__(16) char smem[];
  uint64_t* anc = reinterpret_cast<uint64_t*>(smem + TREE_OFF);
  int* par = reinterpret_cast<int*>(smem + TREE_OFF + TREE_ANC_BYTES);
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

  const int rw = wave % RWV;  // row-wave
  const int kw = wave / RWV;  // key-wave
  const int r = rt * ROWS + rw * 32 + ql;
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

  constexpr int ESZ = kF8 ? 1 : 2;  // bytes per cache element
  const char* kb8 = static_cast<const char*>(p.k) + (int64_t)h * p.sh * ESZ;
  const char* vb8 = static_cast<const char*>(p.v) + (int64_t)h * p.sh * ESZ;

  // ---- per-lane LDS offsets
  int koff[8];  // K row ql, chunk 2*s8 + grp
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) koff[s8] = ql * ROWB + (((2 * s8 + grp) ^ swz_k(ql)) << 4);
  // V rows 4*grp + i16/4 (+8), head-dim columns db*32 + g16*16 + 4*(i16%4); the offset
  // of the V stages is included, so the per-stage part fits the ds_read immediate.
  constexpr int VBASE = kF8 ? F8_VB_OFF : V_OFF;
  int voff[4];
  {
    const int row = 4 * grp + (i16 >> 2);
    const int sw = swz_v(row);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = db * 4 + g16 * 2 + ((i16 & 3) >> 1);
      voff[db] = VBASE + row * ROWB + ((chunk ^ sw) << 4) + (i16 & 1) * 8;
    }
  }

  // ---- HBM -> LDS copies. bf16: a tile's K (and V) is 16 blocks of 4 rows x 256 bytes;
  // wave w copies blocks w, w + NW, ... of both. Lane i of a block copy fills LDS row
  // 4b + i/16, physical chunk i%16, so it loads logical chunk (i%16) ^ swizzle(row).
  // FP8: 8 blocks of 8 rows x 128 bytes each, unswizzled (lane i: row 8b + i/8, chunk
  // i%8); wave w also copies exponents (w % (NW/2)) * EPW .. + EPW - 1 of the tile, of K
  // for the first half of the waves and of V for the second.
  // Offsets within one KV head are 32-bit (the host guarantees (L+N) rows fit).
  const uint32_t rowstride_b = (uint32_t)p.st * (uint32_t)ESZ;
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
  uint32_t dk[BPW], dv[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    if constexpr (kF8) {
      const int row = 8 * (wave + j * NW) + (lane >> 3);
      dk[j] = dv[j] = (uint32_t)row * rowstride_b + (uint32_t)((lane & 7) << 4);
    } else {
      const int row = 4 * (wave + j * NW) + (lane >> 4);
      const int pc = lane & 15;
      dk[j] = (uint32_t)row * rowstride_b + (uint32_t)((pc ^ swz_k(row)) << 4);
      dv[j] = (uint32_t)row * rowstride_b + (uint32_t)((pc ^ swz_v(row)) << 4);
    }
  }
  const int32_t* ebase = nullptr;
  int ekey = 0;  // exponent copied by this lane
  if constexpr (kF8) {
    ebase = uniform_ptr(wave < NW / 2 ? p.ek : p.ev);
    ekey = (wave % (NW / 2)) * EPW + lane;
  }

  auto issue_f8 = [&](int t) __attribute__((always_inline)) {
    const int kt0 = kbeg + t * KT;
    const uint32_t raw = lds_base + (uint32_t)((t & (F8_NRAW - 1)) * F8_RAW_B);
    if (kt0 + KT <= p.T) {
      const uint32_t base = (uint32_t)kt0 * rowstride_b;
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const uint32_t blk = (uint32_t)((wave + j * NW) * 1024);
        dma16<true>(raw + blk, base + dk[j], kb8);
        dma16<true>(raw + F8_TILE_B + blk, base + dv[j], vb8);
      }
    } else {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int row = 8 * (wave + j * NW) + (lane >> 3);
        const uint32_t off = (uint32_t)min(kt0 + row, p.T - 1) * rowstride_b + (uint32_t)((lane & 7) << 4);
        const uint32_t blk = (uint32_t)((wave + j * NW) * 1024);
        dma16<true>(raw + blk, off, kb8);
        dma16<true>(raw + F8_TILE_B + blk, off, vb8);
      }
    }
    if (lane < EPW) {
      const uint32_t key = (uint32_t)min(kt0 + ekey, p.T - 1);
      dma4(raw + 2 * F8_TILE_B + wave * EPW * 4, (key * (uint32_t)p.Hkv + (uint32_t)h) * 4u, ebase);
    }
  };

  auto issue_bf16 = [&](int t) __attribute__((always_inline)) {
    const int kt0 = kbeg + t * KT;
    const uint32_t st_lds = lds_base + (uint32_t)((t & (NSTAGE - 1)) * TILE_B);
    if (kt0 + KT <= p.T) {
      const uint32_t base = (uint32_t)kt0 * rowstride_b;
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const uint32_t blk = (uint32_t)((wave + j * NW) * 1024);
        dma16<true>(st_lds + blk, base + dk[j], kb8);
        dma16<true>(st_lds + V_OFF + blk, base + dv[j], vb8);
      }
    } else {
      // Last tile of the sequence: rows past L+N re-read row L+N-1 (always masked).
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int row = 4 * (wave + j * NW) + (lane >> 4);
        const int pc = lane & 15;
        const uint32_t grow = (uint32_t)min(kt0 + row, p.T - 1) * rowstride_b;
        const uint32_t blk = (uint32_t)((wave + j * NW) * 1024);
        dma16<true>(st_lds + blk, grow + (uint32_t)((pc ^ swz_k(row)) << 4), kb8);
        dma16<true>(st_lds + V_OFF + blk, grow + (uint32_t)((pc ^ swz_v(row)) << 4), vb8);
      }
    }
  };
  // 4-bit: wave w copies code block w % 4 (16 rows x 64 bytes; lane i: row 16 (w % 4) +
  // i / 4, 16-byte chunk i % 4) of K (w < 4) or V, and 16 exponent words (4 int8 per row)
  // as the FP8 path copies its exponents. Rows past L + N repeat row L + N - 1.
  const char* cbase = nullptr;
  if constexpr (kMX) cbase = uniform_ptr(wave < NW / 2 ? kb8 : vb8);
  auto issue_mx = [&](int t) __attribute__((always_inline)) {
    const int kt0 = kbeg + t * KT;
    const uint32_t raw = lds_base + (uint32_t)((t & (F8_NRAW - 1)) * F8_RAW_B);
    const int row = 16 * (wave & 3) + (lane >> 2);
    const uint32_t off = (uint32_t)min(kt0 + row, p.T - 1) * rowstride_b + (uint32_t)((lane & 3) << 4);
    dma16<false>(raw + (uint32_t)((wave >> 2) * MX_TILE_B + (wave & 3) * 1024), off, cbase);
    if (lane < EPW) {
      const uint32_t key = (uint32_t)min(kt0 + ekey, p.T - 1);
      dma4(raw + 2 * MX_TILE_B + wave * EPW * 4, (key * (uint32_t)p.Hkv + (uint32_t)h) * 4u, ebase);
    }
  };
  auto issue = [&](int t) __attribute__((always_inline)) {
    if constexpr (kMX)
      issue_mx(t);
    else if constexpr (kF8)
      issue_f8(t);
    else
      issue_bf16(t);
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_ref = -INFINITY;  // reference maximum of the row, log2 domain (scaled)
  float lsum = 0.f;         // this lane's part of the row sum, relative to m_ref
  f32x16 sc[2];             // scores of two consecutive 32-key blocks
  bf16x8 pb[2];             // P^T fragments of the current block (two 16-key steps)

  // bf16 tiles of tile t in LDS.
  auto kstage = [&](int t) __attribute__((always_inline)) -> const char* {
    if constexpr (kF8)
      return smem + F8_KB_OFF + (t % 3) * TILE_B;
    else
      return smem + (t & (NSTAGE - 1)) * TILE_B;
  };
  // V stage of tile t relative to VBASE (pv adds VBASE through voff).
  auto vstage = [&](int t) __attribute__((always_inline)) -> const char* {
    if constexpr (kF8)
      return smem + (t & 1) * TILE_B;
    else
      return smem + (t & (NSTAGE - 1)) * TILE_B;
  };

  // S^T of 32-key block kb of the K tile at Kt: 8 K fragments, 8 MFMAs.
  auto qk_v = [&](const char* Kt, int kb) __attribute__((always_inline)) -> f32x16 {
    const char* Ks = Kt + kb * 32 * ROWB;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      acc = mfma32(*reinterpret_cast<const bf16x8*>(Ks + koff[s8]), qf[s8], acc);
    return acc;
  };
  auto qk = [&](const char* Kt, int kb, int c) __attribute__((always_inline)) { sc[c] = qk_v(Kt, kb); };

  // O^T += V^T P^T over 32-key block kb of the V tile at Vt + VBASE; V^T fragments come
  // from the row-major V tile through transposed reads (two per MFMA).
  auto pv = [&](const char* Vt, int kb) __attribute__((always_inline)) {
    const char* Vs = Vt + kb * 32 * ROWB;
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
    // Element e holds key 8 * (e / 4) + 4 * grp + e % 4 of the block. The bf16 kernels
    // shift the window by 4 * grp once, leaving a constant bit per element (16 fewer live
    // registers); the FP8 kernels keep the per-element shift, measured faster there.
    if constexpr (kF8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int b = 8 * (e >> 2) + 4 * grp + (e & 3);
        if (!((win >> b) & 1u)) sc[c][e] = -INFINITY;
      }
    } else {
      const uint32_t wl = win >> (4 * grp);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (!(wl & (1u << (8 * (e >> 2) + (e & 3))))) sc[c][e] = -INFINITY;
      }
    }
  };

  // Probabilities of block sc[c] relative to the reference m_ref (0 while it is unset):
  // bf16 P^T fragments for the P.V MFMAs; returns this lane's unrounded fp32 sum of its
  // 16 probabilities.
  auto probs = [&](int c) __attribute__((always_inline)) -> float {
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;
    float bs = 0.f;
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      bf16x2 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c][th * 8 + 2 * j], p.c, -mu));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c][th * 8 + 2 * j + 1], p.c, -mu));
        b[j] = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
        bs += p0 + p1;
      }
      pb[th] = bf16x8{b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
    }
    return bs;
  };

  // Online softmax of block sc[c] with a lazy reference maximum. The probabilities are
  // formed against the current reference first; the block needs a new reference only if
  // one of them exceeds 2^8, and then its lane's partial sum does too. So only when some
  // lane's sum exceeds 2^8 (or is infinite), or the reference is still unset, does the
  // wave take the exact path: the row maximum (lanes l and l ^ 32 hold a row's 32 keys
  // and exchange maxima through permlane32_swap), the reference raised to it, the row sum
  // and O (which holds the earlier blocks) rescaled, the probabilities formed again.
  // Probabilities therefore stay below 2^8 and the reference within 8 of the maximum;
  // the common path needs no maximum at all.
  auto softmax = [&](int c) __attribute__((always_inline)) {
    float bs = probs(c);
    const bool need = m_ref == -INFINITY || bs > kCheck;
    if (__any(need)) {
      // One v_max3 per two scores (8 instructions for 16).
      float m = fmaxf(fmaxf(sc[c][0], sc[c][1]), sc[c][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) m = fmaxf(fmaxf(m, sc[c][e]), sc[c][e + 1]);
      m = fmaxf(m, sc[c][15]);
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      const float mt = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * p.c;
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m_ref = m_new;
      bs = probs(c);
    }
    lsum += bs;
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

  // Sub-step over 32-key block (t, kb) with a successor block (tn, kb ^ 1), whose K tile
  // is at Kn (V of tile t at Vt): the successor's score MFMAs, this block's softmax and
  // this block's P.V MFMAs form one scheduling region, so the compiler interleaves MFMAs
  // with the softmax VALU work; then the successor is masked (if it reaches past the
  // context) and the running maximum updated. The score buffer index equals kb.
  auto sub = [&](int t, auto kbc, int tn, const char* Kn, const char* Vt) __attribute__((always_inline)) {
    constexpr int kb = decltype(kbc)::value;
    constexpr int kbn = kb ^ 1;
    qk(Kn, kbn, kbn);
    softmax(kb);
    pv(Vt, kb);
    if (tn >= nplain) mask(kbeg + tn * KT + kbn * 32, kbn);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  // Key-waves (KSW > 1): this wave owns half kbw of every tile t with t % KP == kph.
  // Its block's scores are computed one step ahead (tile t+1 has landed by then) into
  // sc[0]; at its own step it forms the probabilities and the P.V product. With KP == 1
  // both happen in every step, the next block's scores going to a temporary first so that
  // its MFMAs can overlap this block's softmax.
  constexpr int KP = KSW > 1 ? KSW / 2 : 1;
  const int kph = kw % KP;
  const int kbw = kw / KP;
  auto key_step = [&](int t) __attribute__((always_inline)) {
    if constexpr (KP == 1) {
      if (t + 1 < ntiles) {
        const f32x16 nx = qk_v(kstage(t + 1), kbw);
        softmax(0);
        pv(vstage(t), kbw);
        sc[0] = nx;
        if (t + 1 >= nplain) mask(kbeg + (t + 1) * KT + kbw * 32, 0);
      } else {
        softmax(0);
        pv(vstage(t), kbw);
      }
    } else {
      if ((t & (KP - 1)) == kph) {
        softmax(0);
        pv(vstage(t), kbw);
      }
      if (t + 1 < ntiles && ((t + 1) & (KP - 1)) == kph) {
        qk(kstage(t + 1), kbw, 0);
        if (t + 1 >= nplain) mask(kbeg + (t + 1) * KT + kbw * 32, 0);
      }
    }
  };
  // First scores of a key-wave whose first block lies in tile 0 (tiles 0 and 1 landed).
  auto key_prologue = [&]() __attribute__((always_inline)) {
    if (kph == 0) {
      qk(kstage(0), kbw, 0);
      if (nplain == 0) mask(kbeg + kbw * 32, 0);
    }
  };

  // FP8: widen the K (or V) codes of raw tile t into its bf16 stage. Thread i converts
  // 16 codes (row i/8, dims 16*(i%8) ..) with the row's scale 2^e and writes the two bf16
  // chunks to their swizzled places. Exponents outside [kExpMin, kExpMax] are clamped and
  // reported.
  bool bad_exp = false;
  // 4-bit: thread i widens 16 codes (row i/8, dims 16*(i%8) .., 8 bytes) with their
  // block's scale 2^e (byte (i%8)/2 of the row's exponent word) into the same two chunks.
  auto widen_mx = [&](int t, bool is_v) __attribute__((always_inline)) {
    const char* raw = smem + (t & (F8_NRAW - 1)) * F8_RAW_B + (is_v ? MX_TILE_B : 0);
    const uint32_t* ex = reinterpret_cast<const uint32_t*>(smem + (t & (F8_NRAW - 1)) * F8_RAW_B + 2 * MX_TILE_B) +
                         (is_v ? KT : 0);
    char* dst = const_cast<char*>(is_v ? vstage(t) + VBASE : kstage(t));
    const int row = tid >> 3, c8 = tid & 7;
    const uint2 w = *reinterpret_cast<const uint2*>(raw + row * MX_ROWB + c8 * 8);
    int e = (int)(int8_t)(uint8_t)(ex[row] >> (8 * (c8 >> 1)));
    bad_exp |= e < kMxExpMin || e > kMxExpMax;
    e = min(max(e, kMxExpMin), kMxExpMax);
    const float sc = __int_as_float((e + 127) << 23);
    u32x4 lo, hi;
    lo[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, sc, 0));
    lo[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, sc, 1));
    lo[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, sc, 2));
    lo[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, sc, 3));
    hi[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.y, sc, 0));
    hi[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.y, sc, 1));
    hi[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.y, sc, 2));
    hi[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.y, sc, 3));
    const int sw = is_v ? swz_v(row) : swz_k(row);
    *reinterpret_cast<u32x4*>(dst + row * ROWB + (((2 * c8) ^ sw) << 4)) = lo;
    *reinterpret_cast<u32x4*>(dst + row * ROWB + (((2 * c8 + 1) ^ sw) << 4)) = hi;
  };
  auto widen = [&](int t, bool is_v) __attribute__((always_inline)) {
    if constexpr (kMX) {
      widen_mx(t, is_v);
      return;
    }
    const char* raw = smem + (t & (F8_NRAW - 1)) * F8_RAW_B + (is_v ? F8_TILE_B : 0);
    const int* ex = reinterpret_cast<const int*>(smem + (t & (F8_NRAW - 1)) * F8_RAW_B + 2 * F8_TILE_B) +
                    (is_v ? KT : 0);
    char* dst = const_cast<char*>(is_v ? vstage(t) + VBASE : kstage(t));
#pragma unroll
    for (int pass = 0; pass < 8 / NW; ++pass) {
      const int idx = pass * NW * 64 + tid;
      const int row = idx >> 3, c8 = idx & 7;
      const u32x4 w = *reinterpret_cast<const u32x4*>(raw + row * F8_ROWB + c8 * 16);
      int e = ex[row];
      bad_exp |= e < kExpMin || e > kExpMax;
      e = min(max(e, kExpMin), kExpMax);
      const float sc = __int_as_float((e + 127) << 23);
      u32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        lo[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], sc, false));
        lo[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], sc, true));
        hi[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j + 2], sc, false));
        hi[2 * j + 1] =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j + 2], sc, true));
      }
      const int sw = is_v ? swz_v(row) : swz_k(row);
      *reinterpret_cast<u32x4*>(dst + row * ROWB + (((2 * c8) ^ sw) << 4)) = lo;
      *reinterpret_cast<u32x4*>(dst + row * ROWB + (((2 * c8 + 1) ^ sw) << 4)) = hi;
    }
  };

  if constexpr (kF8 && RWV == 1) {
    // ---- FP8, one row-wave: each wave streams its own 32-key blocks b = wave, wave + 8,
    // ... with no shared ring and no barrier. K codes come into registers and are widened
    // there (code * 2^e, the row's exponent, per lane) into the MFMA A fragments; V codes
    // come into registers, are widened and written to a private 8 KB bf16 stage in the
    // transposed-read layout. The wave's own LDS accesses stay in order, so one stage
    // suffices. Codes and exponents of the next block are in flight during this one.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    constexpr int VB = 32 * ROWB;
    const int nblk = (kend - kbeg + 31) / 32;
    char* vst = smem + wave * VB;
    const int32_t* ekp = uniform_ptr(p.ek);
    const int32_t* evp = uniform_ptr(p.ev);
    const int vr = lane >> 1, vh = lane & 1;  // V widening: key row vr, codes vh*64 .. +63
    auto scale_of = [&](int e) __attribute__((always_inline)) -> float {
      bad_exp |= e < kExpMin || e > kExpMax;
      e = min(max(e, kExpMin), kExpMax);
      return __int_as_float((e + 127) << 23);
    };
    struct Raw {
      uint2 k[8];
      u32x4 v[4];
      int ek, ev;
    };
    auto load_raw = [&](int b, Raw& r) __attribute__((always_inline)) {
      const int kk = min(kbeg + b * 32 + ql, p.T - 1);
      const char* krow = kb8 + (uint32_t)kk * rowstride_b + grp * 8;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) r.k[s8] = *reinterpret_cast<const uint2*>(krow + s8 * 16);
      const int kv = min(kbeg + b * 32 + vr, p.T - 1);
      const char* vrow = vb8 + (uint32_t)kv * rowstride_b + vh * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.v[j] = *reinterpret_cast<const u32x4*>(vrow + j * 16);
      r.ek = ekp[(int64_t)kk * p.Hkv + h];
      r.ev = evp[(int64_t)kv * p.Hkv + h];
    };
    auto compute_raw = [&](int b, const Raw& r) __attribute__((always_inline)) {
      // V: widen and store (after the previous block's transposed reads, in LDS order)
      const float svv = scale_of(r.ev);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 lo, hi;
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          lo[2 * q2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2], svv, false));
          lo[2 * q2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2], svv, true));
          hi[2 * q2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2 + 2], svv, false));
          hi[2 * q2 + 1] =
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2 + 2], svv, true));
        }
        const int c = vh * 8 + 2 * j;  // logical 16-byte chunks c, c + 1 of row vr
        *reinterpret_cast<u32x4*>(vst + vr * ROWB + ((c ^ swz_v(vr)) << 4)) = lo;
        *reinterpret_cast<u32x4*>(vst + vr * ROWB + (((c + 1) ^ swz_v(vr)) << 4)) = hi;
      }
      // K: widen into the A fragments and score
      const float skk = scale_of(r.ek);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        u32x4 kw;
        kw[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.k[s8].x, skk, false));
        kw[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.k[s8].x, skk, true));
        kw[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.k[s8].y, skk, false));
        kw[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.k[s8].y, skk, true));
        acc = mfma32(__builtin_bit_cast(bf16x8, kw), qf[s8], acc);
      }
      sc[0] = acc;
      if (kbeg + b * 32 + 32 > p.L) mask(kbeg + b * 32, 0);
      softmax(0);
      pv(vst - VBASE, 0);
    };
    Raw r0, r1;
    int b = wave;
    if (b < nblk) load_raw(b, r0);
    for (; b < nblk; b += 16) {
      if (b + 8 < nblk) load_raw(b + 8, r1);
      compute_raw(b, r0);
      if (b + 8 >= nblk) break;
      if (b + 16 < nblk) load_raw(b + 16, r0);
      compute_raw(b + 8, r1);
    }
    if (__any(bad_exp) && lane == 0 && p.dev_error) *p.dev_error = TV_ERR_INVALID_ARG;
  } else if constexpr (kF8) {
    // ---- FP8: raw tiles 0..3 start streaming.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // query loads are not tile copies
    for (int t = 0; t < 4 && t < ntiles; ++t) issue(t);
    if constexpr (KSW > 1) {
      // Raw tiles 0..2 must land; K of tiles 0, 1 and V of tile 0 are widened and the LDS
      // barrier publishes them.
      if (ntiles > 3)
        barrier_keep<DPT>();
      else
        barrier_keep<0>();
      widen(0, false);
      if (ntiles > 1) widen(1, false);
      widen(0, true);
      if (ntiles > 3)
        barrier_keep<DPT>();
      else
        barrier_keep<0>();
      key_prologue();
      for (int t = 0; t < ntiles; ++t) {
        if (t + 4 < ntiles) issue(t + 4);
        if (t + 2 < ntiles) widen(t + 2, false);
        if (t + 1 < ntiles) widen(t + 1, true);
        key_step(t);
        if (t + 1 < ntiles) {
          if (t + 4 < ntiles)
            barrier_keep<DPT>();
          else
            barrier_keep<0>();
        }
      }
    } else {
    // Only raw tile 0 must land before its K and V are widened; the barrier that publishes
    // them also waits for raw tile 1.
    if (ntiles > 3)
      barrier_keep<3 * DPT>();
    else if (ntiles > 2)
      barrier_keep<2 * DPT>();
    else if (ntiles > 1)
      barrier_keep<DPT>();
    else
      barrier_keep<0>();
    widen(0, false);
    widen(0, true);
    if (ntiles > 3)
      barrier_keep<2 * DPT>();
    else if (ntiles > 2)
      barrier_keep<DPT>();
    else
      barrier_keep<0>();
    qk(kstage(0), 0, 0);
    if (nplain == 0) mask(kbeg, 0);

    // Step t: raw tile t+4 starts (into the stage of raw tile t, fully widened by step
    // t-1); K of tile t+2 and V of tile t+1 are widened (their raw tiles landed by the
    // previous barrier; their bf16 stages last held K of tile t-1 and V of tile t-1);
    // tile t is consumed. The barrier guarantees raw tile t+3 and keeps t+4 in flight.
    // Step 0 is peeled: raw tile 4 goes into the stage of raw tile 0 (widened before the
    // last barrier), tile 1 is widened first, and a barrier midway publishes it (and
    // waits for raw tile 2) before the second block scores tile 1's keys; K of tile 2 is
    // widened last.
    int t = 0;
    if (ntiles > 1) {
      if (4 < ntiles) issue(4);
      widen(1, false);
      widen(1, true);
      sub(0, B0{}, 0, kstage(0), vstage(0));
      if (ntiles > 4)
        barrier_keep<2 * DPT>();
      else if (ntiles > 3)
        barrier_keep<DPT>();
      else
        barrier_keep<0>();
      sub(0, B1{}, 1, kstage(1), vstage(0));
      if (2 < ntiles) widen(2, false);
      if (4 < ntiles)
        barrier_keep<DPT>();
      else
        barrier_keep<0>();
      t = 1;
    }
    for (; t + 1 < ntiles; ++t) {
      if (t + 4 < ntiles) issue(t + 4);
      if (t + 2 < ntiles) widen(t + 2, false);
      sub(t, B0{}, t, kstage(t), vstage(t));
      widen(t + 1, true);  // between the blocks, so the two widening bursts are apart
      sub(t, B1{}, t + 1, kstage(t + 1), vstage(t));
      if (t + 4 < ntiles)
        barrier_keep<DPT>();
      else
        barrier_keep<0>();
    }
    {
      const int t = ntiles - 1;
      sub(t, B0{}, t, kstage(t), vstage(t));
      softmax(1);
      pv(vstage(t), 1);
    }
    }
    if (__any(bad_exp) && lane == 0 && p.dev_error) *p.dev_error = TV_ERR_INVALID_ARG;
  } else if constexpr (RWV == 1) {
    // ---- one row-wave (M <= 32): every 32-key block has a single reader, so each wave
    // streams its own blocks b = wave, wave + 8, ... with no shared ring and no barrier.
    // K goes straight into registers as MFMA A fragments (two buffers, one block ahead);
    // V is copied into two private 8 KB LDS stages for the transposed reads. Splits are
    // whole 64-key tiles, so a block never crosses into the next split; past the last key
    // the loads repeat row T-1, which the mask hides. A block is 16 memory operations (8 K
    // loads, 8 V copies): waiting for vmcnt(16) after issuing the next block's leaves
    // exactly this block landed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    constexpr int VB = 32 * ROWB;  // one V block
    const int nblk = (kend - kbeg + 31) / 32;
    const uint32_t vpriv = lds_base + (uint32_t)(wave * 2 * VB);
    const char* vprivp = smem + wave * 2 * VB;
    bf16x8 kf0[8], kf1[8];
    auto load_block = [&](int b, bf16x8(&kf)[8], int stage) __attribute__((always_inline)) {
      const int key = min(kbeg + b * 32 + ql, p.T - 1);
      const char* row = kb8 + (uint32_t)key * rowstride_b + grp * 16;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) kf[s8] = *reinterpret_cast<const bf16x8*>(row + s8 * 32);
      // The stage's previous block was read by transposed LDS reads whose data may not
      // have returned yet; the copies below overwrite it, so those reads finish first.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int pc = lane & 15;
        const uint32_t grow = (uint32_t)min(kbeg + b * 32 + r, p.T - 1) * rowstride_b;
        dma16<true>(vpriv + (uint32_t)(stage * VB + j * 1024), grow + (uint32_t)((pc ^ swz_v(r)) << 4), vb8);
      }
    };
    auto compute_block = [&](int b, const bf16x8(&kf)[8], int stage) __attribute__((always_inline)) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) acc = mfma32(kf[s8], qf[s8], acc);
      sc[0] = acc;
      if (kbeg + b * 32 + 32 > p.L) mask(kbeg + b * 32, 0);
      softmax(0);
      pv(vprivp + stage * VB - VBASE, 0);
    };
    int b = wave;
    if (b < nblk) load_block(b, kf0, 0);
    for (; b < nblk; b += 16) {
      if (b + 8 < nblk) {
        load_block(b + 8, kf1, 1);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      compute_block(b, kf0, 0);
      if (b + 8 >= nblk) break;
      if (b + 16 < nblk) {
        load_block(b + 16, kf0, 0);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      compute_block(b + 8, kf1, 1);
    }
  } else if constexpr (KSW > 1) {
    // ---- key-waves: tiles 0, 1, 2 start streaming; tiles 0 and 1 must land.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    for (int t = 0; t < 3 && t < ntiles; ++t) issue(t);
    if (ntiles > 2)
      barrier_keep<DPT>();
    else
      barrier_keep<0>();
    key_prologue();
    for (int t = 0; t < ntiles; ++t) {
      if (t + 3 < ntiles) issue(t + 3);
      key_step(t);
      if (t + 1 < ntiles) wait_step(t);
    }
  } else {
  // ---- prologue: tiles 0, 1, 2 start streaming; only tile 0 must land before the first
  // scores. Step 0 waits for tile 1 (its second block scores tile 1's keys) midway.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // query loads are not tile copies
  for (int t = 0; t < 3 && t < ntiles; ++t) issue(t);
  if (ntiles > 2)
    barrier_keep<2 * DPT>();
  else if (ntiles > 1)
    barrier_keep<DPT>();
  else
    barrier_keep<0>();
  // The K fragments of the next block to score are read from LDS one sub-step ahead, into
  // kf, right after this block's softmax and before its P.V product, so the score MFMAs of
  // a sub-step never wait for LDS. Within step t the block after the successor lies in
  // tile t or t+1, both landed by the barrier that closed step t-1 (step 0 waits for tile
  // 1 midway, before its first read of it).
  bf16x8 kf[8];
  auto kload = [&](const char* Kt, int kb) __attribute__((always_inline)) {
    const char* Ks = Kt + kb * 32 * ROWB;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) kf[s8] = *reinterpret_cast<const bf16x8*>(Ks + koff[s8]);
  };
  // Sub-step over block (t, kb) with successor (tn, kb ^ 1), whose fragments are in kf: the
  // successor's score MFMAs beside this block's softmax (one scheduling region), then the
  // reads of the block after the successor (block kbnn of the K tile at Knn, if nn), this
  // block's P.V MFMAs, and the successor's mask.
  auto sub_kf = [&](int t, auto kbc, int tn, const char* Knn, int kbnn, bool nn, const char* Vt)
                    __attribute__((always_inline)) {
    constexpr int kb = decltype(kbc)::value;
    constexpr int kbn = kb ^ 1;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) acc = mfma32(kf[s8], qf[s8], acc);
    sc[kbn] = acc;
    softmax(kb);
    __builtin_amdgcn_sched_barrier(0);
    if (nn) kload(Knn, kbnn);
    pv(Vt, kb);
    if (tn >= nplain) mask(kbeg + tn * KT + kbn * 32, kbn);
  };
  qk(kstage(0), 0, 0);
  if (nplain == 0) mask(kbeg, 0);
  kload(kstage(0), 1);

  // Tile t: block 0 (successor: block 1 of tile t; reads block 0 of tile t+1), block 1
  // (successor: block 0 of tile t+1; reads block 1 of tile t+1); the barrier after each
  // tile guarantees tile t+2 and keeps tile t+3 in flight. Stage reuse: tile t+3
  // overwrites tile t-1, whose last reads were in tile t-1's blocks. Unrolled by the ring
  // length so that stage offsets are constants (folded into the ds_read offsets); the up
  // to three steps left over use computed stages.
  auto step = [&](int t, auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    if (t + 3 < ntiles) issue(t + 3);
    const char* K1 = smem + ((st + 1) & (NSTAGE - 1)) * TILE_B;
    const char* V0 = smem + st * TILE_B;
    sub_kf(t, B0{}, t, K1, 0, true, V0);
    sub_kf(t, B1{}, t + 1, K1, 1, true, V0);
    wait_step(t);
  };
  int t = 0;
  if (ntiles > 1) {
    // Step 0: tile 1 must land before the block after block 0's successor is read.
    if (3 < ntiles) issue(3);
    sub_kf(0, B0{}, 0, nullptr, 0, false, vstage(0));
    if (ntiles > 3)
      barrier_keep<2 * DPT>();
    else if (ntiles > 2)
      barrier_keep<DPT>();
    else
      barrier_keep<0>();
    kload(kstage(1), 0);
    sub_kf(0, B1{}, 1, kstage(1), 1, true, vstage(0));
    wait_step(0);
    t = 1;
  }
  for (; t + 4 < ntiles; t += 4) {
    step(t, std::integral_constant<int, 1>{});
    step(t + 1, std::integral_constant<int, 2>{});
    step(t + 2, std::integral_constant<int, 3>{});
    step(t + 3, std::integral_constant<int, 0>{});
  }
  for (; t + 1 < ntiles; ++t) {
    if (t + 3 < ntiles) issue(t + 3);
    sub_kf(t, B0{}, t, kstage(t + 1), 0, true, vstage(t));
    sub_kf(t, B1{}, t + 1, kstage(t + 1), 1, true, vstage(t));
    wait_step(t);
  }
  {
    const int t = ntiles - 1;
    sub_kf(t, B0{}, t, nullptr, 0, false, vstage(t));
    softmax(1);
    pv(vstage(t), 1);
  }
  }

  // ---- key-waves: merge the KSW partial states of each row in LDS (the ring is free:
  // every copy has landed and every wave has finished its reads at the barrier), as a
  // tree: in each round the upper half of the remaining key-waves leaves O (64 values per
  // lane, lane-major with a 68-float pitch so that the 16-byte accesses of 16 lanes cover
  // all 64 banks once), its reference maximum and its row-sum part, and the lower half
  // rescales both states to the common maximum and adds them. log2(KSW) rounds.
  if constexpr (KSW > 1) {
    constexpr int PITCH = 68;
    constexpr int SLOT = 64 * PITCH + 128;  // floats per (row-wave, writer)
    float* ms = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int half = KSW / 2; half >= 1; half /= 2) {
      barrier_keep<0>();
      if (kw >= half && kw < 2 * half) {
        float* b = ms + ((kw - half) * RWV + rw) * SLOT;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<f32x4*>(b + lane * PITCH + db * 16 + i) =
                f32x4{o[db][i], o[db][i + 1], o[db][i + 2], o[db][i + 3]};
        b[64 * PITCH + lane] = m_ref;
        b[64 * PITCH + 64 + lane] = lsum;
      }
      barrier_keep<0>();
      if (kw < half) {
        const float* b = ms + (kw * RWV + rw) * SLOT;
        const float mk = b[64 * PITCH + lane];
        const float lk = b[64 * PITCH + 64 + lane];
        const float mn = fmaxf(m_ref, mk);
        const float a0 = m_ref == -INFINITY ? 0.f : exp2f(m_ref - mn);
        const float ak = mk == -INFINITY ? 0.f : exp2f(mk - mn);
        lsum = lsum * a0 + lk * ak;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; i += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(b + lane * PITCH + db * 16 + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[db][i + j] = o[db][i + j] * a0 + v[j] * ak;
          }
        m_ref = mn;
      }
    }
  }

  // ---- partial result of this split
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float lse2 = lsum > 0.f ? m_ref + __log2f(lsum) : -INFINITY;
  if (rvalid && kw == 0) {
    const int64_t base = ((int64_t)(h * p.RT + rt) * p.S + s) * TILE_ROWS + rw * 32 + ql;
    __bf16* po = p.part_o + base * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 val = {o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                           o[db][4 * i + 3] * inv};
        *reinterpret_cast<bf16x4*>(po + db * 32 + 8 * i + 4 * grp) = __builtin_convertvector(val, bf16x4);
      }
    }
    if (grp == 0) p.part_lse[base] = lse2;
  }
}

// ---- At most 16 stacked rows (single-token decode, small trees): 16x16x32 MFMA tiles.
//
// A 32-row tile would leave at least half of every MFMA and of the softmax work on empty
// rows here; 16-row tiles (v_mfma_f32_16x16x32_bf16) halve both. The memory side is the
// single-row-wave stream of attn_split_kernel: each of the eight waves streams its own
// 32-key blocks (K straight into registers as MFMA A fragments, V through two private LDS
// stages for the transposed reads), one block ahead, with no shared ring and no barrier.
// The query, and for the split that reaches the tree the parent entries, are loaded
// together with the first key block, so their round trips overlap.
//
// FP8 cache (kF8): K and V codes and their row exponents come into registers one block
// ahead; K is widened there (code * 2^e, the key's exponent) into the A fragments, V is
// widened and written to one private 8 KB stage per wave in the transposed-read layout
// (the wave's own LDS accesses stay in order, so the previous block's reads precede the
// writes), then the block proceeds as for bf16.
//
// Layouts. Scores S^T = K Q^T per 16-key half: lane l holds keys 4(l/16) + i (i < 4) of
// query row l % 16, so a row's 32 keys sit in four lanes (l, l^16, l^32, l^48). The P.V
// product O^T += V^T P^T takes each lane's own eight probabilities as its B fragment, the
// reduction order of the 32 keys being (4g .. 4g+3, 16+4g .. 16+4g+3) for lane group g;
// two transposed LDS reads give the V^T A fragment in that same order. O^T accumulates in
// 8 x 4 fp32 registers per lane (dims 16 db + 4 g + i of row l % 16).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// V swizzle of the 16-row kernel: chunk c of key row r lives at chunk c ^ 2(r & 7). A
// half-wave of transposed reads touches rows r0 .. r0 + 7 and the two chunks of one
// 16-dim column block, which this maps onto all 16 chunks (all 64 banks) once.
__device__ __forceinline__ int swz_v16(int r) { return (r & 7) << 1; }

constexpr int R16_STAGES = 2;
constexpr int R16_VB = 32 * ROWB;                    // one 32-key V block, 8 KB
constexpr int R16_TREE_OFF = 8 * R16_STAGES * R16_VB;
constexpr int R16_SMEM_BYTES = R16_TREE_OFF + TREE_BYTES;
static_assert(R16_SMEM_BYTES <= 160 * 1024, "16-row kernel LDS");

template <bool kF8, bool kMX = false>
__global__ __launch_bounds__(512) void attn_rows16_kernel(SplitParams p) {
  constexpr int NW = 8;
  extern __shared__ __align__(16) char smem[];
  uint64_t* anc = reinterpret_cast<uint64_t*>(smem + R16_TREE_OFF);
  int* par = reinterpret_cast<int*>(smem + R16_TREE_OFF + TREE_ANC_BYTES);
  int* jmp = par + kMaxNodes;

  // ---- work item (RT == 1: one row tile)
  int w = blockIdx.x;
  if (p.remap) {
    const int per = gridDim.x >> 3;
    w = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  const int s = w % p.S;
  const int h = w / p.S;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const bool rvalid = i16 < p.M;
  const int node = rvalid ? i16 / p.G : 0;
  const int qh = h * p.G + (rvalid ? i16 % p.G : 0);

  const int kbeg = s * p.KS;
  const int kend = min(kbeg + p.KS, p.T);
  const bool tree = kend > p.L;  // uniform over the workgroup
  const int nblk = (kend - kbeg + 31) / 32;

  // ---- loads whose round trips overlap the first key block: parent entries, query
  const int parent_i = (tree && tid < p.N) ? p.parent[tid] : -1;
  bf16x8 qf[4];  // B fragments of S^T: row i16, dims 32c + 8g .. + 7
  {
    const uint16_t* qrow = p.q + ((int64_t)node * p.Hq + qh) * D + g * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (rvalid) x = *reinterpret_cast<const u32x4*>(qrow + c * 32);
      qf[c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  constexpr int ESZ = kF8 ? 1 : 2;  // bytes per cache element
  const char* kb8 = static_cast<const char*>(p.k) + (int64_t)h * p.sh * ESZ;
  const char* vb8 = static_cast<const char*>(p.v) + (int64_t)h * p.sh * ESZ;
  const uint32_t rowstride_b = (uint32_t)p.st * (uint32_t)ESZ;
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
  const uint32_t vpriv = lds_base + (uint32_t)(wave * R16_STAGES * R16_VB);
  const char* vprivp = smem + wave * R16_STAGES * R16_VB;
  // transposed-read offsets: key row 4g + i16/4 (the second read adds 16 rows), 8-byte
  // piece i16 % 4 of the 32-byte span of dims 16 db .. 16 db + 15
  int voff[8];
  {
    const int row = 4 * g + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      voff[db] = row * ROWB + (((2 * db + ((i16 & 3) >> 1)) ^ swz_v16(row)) << 4) + (i16 & 1) * 8;
  }

  // One 32-key block: 8 K fragment loads (keys 16 hh + i16, dims 32 c + 8 g) and 8 V copies
  // of 4 rows each (lane -> row 4 j + lane / 16, physical chunk lane % 16, which holds
  // logical chunk (lane % 16) ^ swz_v16(row)). Keys past T - 1 repeat row T - 1 (masked).
  // 16 memory operations per block.
  auto load_block = [&](int b, bf16x8(&kf)[8], int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int key = min(kbeg + b * 32 + 16 * hh + i16, p.T - 1);
      const char* row = kb8 + (uint32_t)key * rowstride_b + g * 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) kf[4 * hh + c] = *reinterpret_cast<const bf16x8*>(row + c * 64);
    }
    // the stage's previous block was read by transposed LDS reads; they finish first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int pc = lane & 15;
      const uint32_t grow = (uint32_t)min(kbeg + b * 32 + r, p.T - 1) * rowstride_b;
      dma16<true>(vpriv + (uint32_t)(stage * R16_VB + j * 1024), grow + (uint32_t)((pc ^ swz_v16(r)) << 4), vb8);
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{};
  float m_ref = -INFINITY;  // reference maximum of the row (log2 domain, scaled), equal in its four lanes
  float lsum = 0.f;         // this lane's part of the row sum relative to m_ref
  bf16x8 pb;                // P^T fragment of the current block

  // probabilities against the reference (0 while unset); returns the lane's fp32 sum
  auto probs = [&](const float (&sc)[8]) __attribute__((always_inline)) -> float {
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;
    float bs = 0.f;
    bf16x2 b2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * j], p.c, -mu));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * j + 1], p.c, -mu));
      b2[j] = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
      bs += p0 + p1;
    }
    pb = bf16x8{b2[0][0], b2[0][1], b2[1][0], b2[1][1], b2[2][0], b2[2][1], b2[3][0], b2[3][1]};
    return bs;
  };

  auto compute_block = [&](int b, const bf16x8(&kf)[8], int stage) __attribute__((always_inline)) {
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s0 = mfma16(kf[c], qf[c], s0);
      s1 = mfma16(kf[4 + c], qf[c], s1);
    }
    float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    const int kb0 = kbeg + b * 32;
    if (kb0 + 32 > p.L) {
      // 32-bit window of the row's ancestor set: bit bb <-> key kb0 + bb (context keys set)
      const int d = kb0 - p.L;
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
      for (int e = 0; e < 8; ++e) {
        const int bb = 16 * (e >> 2) + 4 * g + (e & 3);
        if (!((win >> bb) & 1u)) sc[e] = -INFINITY;
      }
    }
    // online softmax with the lazy reference of attn_split_kernel: the exact path (row
    // maximum over the four lanes of the row, rescale) only when some lane's block sum
    // exceeds 2^8 or the reference is unset
    float bs = probs(sc);
    const bool need = m_ref == -INFINITY || bs > kCheck;
    if (__any(need)) {
      float m = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
      for (int e = 3; e < 7; e += 2) m = fmaxf(fmaxf(m, sc[e]), sc[e + 1]);
      m = fmaxf(m, sc[7]);
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      const float m_new = fmaxf(m_ref, m * p.c);
      const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      m_ref = m_new;
      bs = probs(sc);
    }
    lsum += bs;
    const char* Vs = vprivp + stage * R16_VB;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + voff[db]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + voff[db] + 16 * ROWB));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = mfma16(a, pb, o[db]);
    }
  };

  if constexpr (!kF8) {
    bf16x8 kf0[8], kf1[8];
    int b = wave;
    if (b < nblk) load_block(b, kf0, 0);
    if (tree) tree_prep_lds_from(parent_i, p.N, anc, par, jmp, p.dev_error);
    // Block b + 8's 16 operations are issued before block b's are awaited: vmcnt(16)
    // leaves exactly them in flight (older loads, the query's included, have landed).
    for (; b < nblk; b += 16) {
      if (b + 8 < nblk) {
        load_block(b + 8, kf1, 1);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      compute_block(b, kf0, 0);
      if (b + 8 >= nblk) break;
      if (b + 16 < nblk) {
        load_block(b + 16, kf0, 0);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      compute_block(b + 8, kf1, 1);
    }
  } else {
    // Codes and exponents of one 32-key block in registers: K for keys 16 hh + i16, dims
    // 32 c + 8 g .. + 7 (8 codes each); V for key row vr = lane / 2, dims 64 vh .. + 63.
    // All loads go to registers, so the compiler's own waits order them.
    const int32_t* ekp = uniform_ptr(p.ek);
    const int32_t* evp = uniform_ptr(p.ev);
    const int vr = lane >> 1, vh = lane & 1;
    bool bad_exp = false;
    auto scale_of = [&](int e) __attribute__((always_inline)) -> float {
      bad_exp |= e < kExpMin || e > kExpMax;
      e = min(max(e, kExpMin), kExpMax);
      return __int_as_float((e + 127) << 23);
    };
    struct RawF8 {
      uint2 k[8];
      int ek[2];
      u32x4 v[4];
      int ev;
    };
    // 4-bit: K 8 codes (4 bytes) per fragment and the key's word of 4 block exponents;
    // V 64 codes (32 bytes) of row vr and that row's exponent word.
    struct RawMX {
      uint32_t k[8];
      uint32_t ek[2];
      u32x4 v[2];
      uint32_t ev;
    };
    using Raw = std::conditional_t<kMX, RawMX, RawF8>;
    auto mx_scale = [&](uint32_t word, int b) __attribute__((always_inline)) -> float {
      int e = (int)(int8_t)(uint8_t)(word >> (8 * b));
      bad_exp |= e < kMxExpMin || e > kMxExpMax;
      e = min(max(e, kMxExpMin), kMxExpMax);
      return __int_as_float((e + 127) << 23);
    };
    auto cvt4 = [&](uint32_t w, float sc) __attribute__((always_inline)) -> u32x4 {
      return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3))};
    };
    auto load_raw_mx = [&](int b, RawMX& r) __attribute__((always_inline)) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = min(kbeg + b * 32 + 16 * hh + i16, p.T - 1);
        const char* row = kb8 + (uint32_t)key * rowstride_b + g * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.k[4 * hh + c] = *reinterpret_cast<const uint32_t*>(row + c * 16);
        r.ek[hh] = (uint32_t)ekp[(int64_t)key * p.Hkv + h];
      }
      const int kv = min(kbeg + b * 32 + vr, p.T - 1);
      const char* vrow = vb8 + (uint32_t)kv * rowstride_b + vh * 32;
      r.v[0] = *reinterpret_cast<const u32x4*>(vrow);
      r.v[1] = *reinterpret_cast<const u32x4*>(vrow + 16);
      r.ev = (uint32_t)evp[(int64_t)kv * p.Hkv + h];
    };
    auto compute_raw_mx = [&](int b, const RawMX& r) __attribute__((always_inline)) {
      // V: dims 64 vh + 32 j + 8 q .. + 7 (block 2 vh + j) become logical chunk 8 vh + 4 j + q
      char* vst = smem + wave * R16_STAGES * R16_VB;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sv = mx_scale(r.ev, 2 * vh + j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 8 * vh + 4 * j + q;
          *reinterpret_cast<u32x4*>(vst + vr * ROWB + ((c ^ swz_v16(vr)) << 4)) = cvt4(r.v[j][q], sv);
        }
      }
      // K: fragment (hh, c) holds dims 32 c + 8 g .. + 7 of key 16 hh + i16 (block c)
      bf16x8 kf[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kf[4 * hh + c] = __builtin_bit_cast(bf16x8, cvt4(r.k[4 * hh + c], mx_scale(r.ek[hh], c)));
      compute_block(b, kf, 0);
    };
    auto load_raw_f8 = [&](int b, RawF8& r) __attribute__((always_inline)) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = min(kbeg + b * 32 + 16 * hh + i16, p.T - 1);
        const char* row = kb8 + (uint32_t)key * rowstride_b + g * 8;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.k[4 * hh + c] = *reinterpret_cast<const uint2*>(row + c * 32);
        r.ek[hh] = ekp[(int64_t)key * p.Hkv + h];
      }
      const int kv = min(kbeg + b * 32 + vr, p.T - 1);
      const char* vrow = vb8 + (uint32_t)kv * rowstride_b + vh * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.v[j] = *reinterpret_cast<const u32x4*>(vrow + j * 16);
      r.ev = evp[(int64_t)kv * p.Hkv + h];
    };
    auto compute_raw_f8 = [&](int b, const RawF8& r) __attribute__((always_inline)) {
      // V: widen 64 codes of row vr and write them as logical chunks 8 vh .. 8 vh + 7
      char* vst = smem + wave * R16_STAGES * R16_VB;
      const float svv = scale_of(r.ev);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 lo, hi;
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          lo[2 * q2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2], svv, false));
          lo[2 * q2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2], svv, true));
          hi[2 * q2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2 + 2], svv, false));
          hi[2 * q2 + 1] =
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[j][q2 + 2], svv, true));
        }
        const int c = vh * 8 + 2 * j;
        *reinterpret_cast<u32x4*>(vst + vr * ROWB + ((c ^ swz_v16(vr)) << 4)) = lo;
        *reinterpret_cast<u32x4*>(vst + vr * ROWB + (((c + 1) ^ swz_v16(vr)) << 4)) = hi;
      }
      // K: widen into the A fragments
      bf16x8 kf[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float skk = scale_of(r.ek[hh]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint2 u = r.k[4 * hh + c];
          u32x4 kw;
          kw[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, skk, false));
          kw[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, skk, true));
          kw[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, skk, false));
          kw[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, skk, true));
          kf[4 * hh + c] = __builtin_bit_cast(bf16x8, kw);
        }
      }
      compute_block(b, kf, 0);
    };
    auto load_raw = [&](int b, Raw& r) __attribute__((always_inline)) {
      if constexpr (kMX)
        load_raw_mx(b, r);
      else
        load_raw_f8(b, r);
    };
    auto compute_raw = [&](int b, const Raw& r) __attribute__((always_inline)) {
      if constexpr (kMX)
        compute_raw_mx(b, r);
      else
        compute_raw_f8(b, r);
    };
    Raw r0, r1;
    int b = wave;
    if (b < nblk) load_raw(b, r0);
    if (tree) tree_prep_lds_from(parent_i, p.N, anc, par, jmp, p.dev_error);
    for (; b < nblk; b += 16) {
      if (b + 8 < nblk) load_raw(b + 8, r1);
      compute_raw(b, r0);
      if (b + 8 >= nblk) break;
      if (b + 16 < nblk) load_raw(b + 16, r0);
      compute_raw(b + 8, r1);
    }
    if (__any(bad_exp) && lane == 0 && p.dev_error) *p.dev_error = TV_ERR_INVALID_ARG;
  }

  // ---- the eight waves' states meet in LDS (the V stages are free after the barrier):
  // each wave leaves O (16 rows x 128 dims, row pitch 132 floats), its references and its
  // row sums; then wave w combines rows 2w and 2w + 1 (lane -> row 2w + lane / 32, dims
  // 4 (lane % 32) .. + 3) and writes the split's normalised partial output.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  constexpr int OP = 132;
  constexpr int WSLOT = 16 * OP + 32;
  float* ms = reinterpret_cast<float*>(smem);
  barrier_keep<0>();
  {
    float* mine = ms + wave * WSLOT;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(mine + i16 * OP + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      mine[16 * OP + i16] = m_ref;
      mine[16 * OP + 16 + i16] = lsum;
    }
  }
  barrier_keep<0>();
  const int orow = 2 * wave + (lane >> 5);
  const int od = 4 * (lane & 31);
  float mk[NW];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    mk[k] = ms[k * WSLOT + 16 * OP + orow];
    M = fmaxf(M, mk[k]);
  }
  float L = 0.f;
  f32x4 acc = f32x4{};
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const float a = mk[k] == -INFINITY ? 0.f : exp2f(mk[k] - M);
    L += a * ms[k * WSLOT + 16 * OP + 16 + orow];
    acc += a * *reinterpret_cast<const f32x4*>(ms + k * WSLOT + orow * OP + od);
  }
  if (orow < p.M) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int64_t base = ((int64_t)h * p.RT * p.S + s) * TILE_ROWS + orow;
    *reinterpret_cast<bf16x4*>(p.part_o + base * D + od) = __builtin_convertvector(acc * inv, bf16x4);
    if ((lane & 31) == 0) p.part_lse[base] = L > 0.f ? M + __log2f(L) : -INFINITY;
  }
}

struct MergeParams {
  const __bf16* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int N, Hq, G, RT, S;
  int rows;  // stacked rows per workgroup of the split kernel
};

// One wave per (node, q head) row, two head-dim values per lane:
// lse = M + log2 sum_s 2^(lse_s - M), out = sum_s 2^(lse_s - lse) * out_s.
// Lane s of a 64-split chunk holds split s's weight; the partial outputs are read in
// batches of 16 independent loads (addresses clamped into the chunk, weight 0 past its
// end), so a row costs a few memory round trips whatever the split count.
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams mp) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= mp.N * mp.Hq) return;
  const int n = row / mp.Hq;
  const int qh = row % mp.Hq;
  const int h = qh / mp.G;
  const int r = n * mp.G + qh % mp.G;
  const int rt = r / mp.rows;
  const int64_t base0 = (int64_t)(h * mp.RT + rt) * mp.S * TILE_ROWS + (r % mp.rows);
  const float* lse_p = mp.part_lse + base0;
  const __bf16* o_p = mp.part_o + base0 * D + 2 * lane;

  float mx = -INFINITY;
  for (int s = lane; s < mp.S; s += 64) mx = fmaxf(mx, lse_p[(int64_t)s * TILE_ROWS]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));

  f32x2 acc = {0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s0 = 0; s0 < mp.S; s0 += 64) {
      const int cnt = min(64, mp.S - s0);
      const float w = lane < cnt ? exp2f(lse_p[(int64_t)(s0 + lane) * TILE_ROWS] - mx) : 0.f;
      wsum += w;
      for (int j = 0; j < cnt; j += 16) {
        f32x2 x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int sj = s0 + min(j + u, cnt - 1);
          x[u] = __builtin_convertvector(
              __builtin_nontemporal_load(reinterpret_cast<const bf16x2*>(o_p + (int64_t)sj * TILE_ROWS * D)), f32x2);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
          acc += (j + u < cnt ? wu : 0.f) * x[u];
        }
      }
    }
    for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const bf16x2 ob = __builtin_convertvector((f32x2{acc[0] * inv, acc[1] * inv}), bf16x2);
  *reinterpret_cast<bf16x2*>(mp.out + (int64_t)row * D + 2 * lane) = ob;
  if (mp.lse && lane == 0) mp.lse[row] = mx == -INFINITY ? -INFINITY : (mx + __log2f(wsum)) * kLn2;
}

// The same merge for up to 64 splits in one memory round trip: the split log-sum-exps and
// all NB * 16 partial-output loads (addresses clamped to the last split) are issued before
// any of them is used.
template <int NB>
__global__ __launch_bounds__(256) void attn_merge_small_kernel(MergeParams mp) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= mp.N * mp.Hq) return;
  const int n = row / mp.Hq;
  const int qh = row % mp.Hq;
  const int h = qh / mp.G;
  const int r = n * mp.G + qh % mp.G;
  const int rt = r / mp.rows;
  const int64_t base0 = (int64_t)(h * mp.RT + rt) * mp.S * TILE_ROWS + (r % mp.rows);
  const float* lse_p = mp.part_lse + base0;
  const __bf16* o_p = mp.part_o + base0 * D + 2 * lane;
  const int S = mp.S;  // 1 .. NB * 16

  const float l = lane < S ? lse_p[(int64_t)lane * TILE_ROWS] : -INFINITY;
  f32x2 x[NB * 16];
#pragma unroll
  for (int u = 0; u < NB * 16; ++u)
    x[u] = __builtin_convertvector(
        __builtin_nontemporal_load(reinterpret_cast<const bf16x2*>(o_p + (int64_t)min(u, S - 1) * TILE_ROWS * D)),
        f32x2);

  float mx = l;
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float w = (lane < S && mx != -INFINITY) ? exp2f(l - mx) : 0.f;
  float wsum = w;
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  f32x2 acc = {0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NB * 16; ++u) {
    const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
    acc += wu * x[u];  // lanes >= S carry weight 0
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const bf16x2 ob = __builtin_convertvector((f32x2{acc[0] * inv, acc[1] * inv}), bf16x2);
  *reinterpret_cast<bf16x2*>(mp.out + (int64_t)row * D + 2 * lane) = ob;
  if (mp.lse && lane == 0) mp.lse[row] = mx == -INFINITY ? -INFINITY : (mx + __log2f(wsum)) * kLn2;
}

// The kernels take more than 64 KB of dynamic LDS, which a function attribute must allow
// on every device before the first launch there. Per kernel, one bit per device records
// that it was set; the word is atomic, so concurrent first calls from several host threads
// at worst set the (idempotent) attribute twice. Devices past the 64 bits set it on every
// call.
template <typename Kernel>
hipError_t allow_dynamic_lds(Kernel kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

template <int RWV, bool kF8, bool kMX = false>
hipError_t launch_split(const SplitParams& sp, int nwg, hipStream_t stream) {
  constexpr int KSW = 8 / RWV;
  constexpr int smem = kF8 ? F8_SMEM_BYTES : SMEM_BYTES;
  static std::atomic<uint64_t> attr_devices{0};
  hipError_t e = allow_dynamic_lds(&attn_split_kernel<RWV, KSW, kF8, kMX>, smem, attr_devices);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_split_kernel<RWV, KSW, kF8, kMX>), dim3(nwg), dim3(512), smem, stream, sp);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int N, int L, int Hq, int Hkv, int num_splits, int num_cus) {
  AttnPlan p;
  p.G = Hq / Hkv;
  p.M = p.G * N;
  // Row-waves: the power of two of 32-row waves that covers min(M, 256) rows; the rest of
  // the eight waves split the keys.
  const int rows = p.M < TILE_ROWS ? p.M : TILE_ROWS;
  p.RWV = rows <= 32 ? 1 : rows <= 64 ? 2 : rows <= 128 ? 4 : 8;
  p.RT = (p.M + p.RWV * 32 - 1) / (p.RWV * 32);
  p.T = L + N;
  // Split lengths are whole 64-key tiles for attn_split_kernel; the 16-row kernel
  // streams 32-key blocks, so its splits need only be whole blocks.
  const int gran = p.M <= 16 ? 32 : KT;
  const int tiles = (p.T + gran - 1) / gran;
  int S = num_splits;
  if (S <= 0) {
    // One workgroup per CU (the four LDS stages and the tree masks take 138 KB): enough
    // splits to give every CU a workgroup, down to one tile (block) per split. Short
    // sequences are latency-bound, so filling the chip beats saving partial-output
    // traffic; long ones get long splits anyway.
    const int units = Hkv * p.RT;
    S = (num_cus + units - 1) / units;
  }
  if (S > tiles) S = tiles;
  if (S < 1) S = 1;
  const int tps = (tiles + S - 1) / S;
  p.KS = tps * gran;
  p.S = (p.T + p.KS - 1) / p.KS;
  return p;
}

size_t attn_workspace_bytes(const AttnPlan& p, int Hkv) {
  const size_t rows = (size_t)Hkv * p.RT * p.S * TILE_ROWS;
  size_t bytes = rows * D * sizeof(__bf16);  // partial outputs
  bytes = (bytes + 255) / 256 * 256;
  bytes += rows * sizeof(float);              // partial log2-sum-exps
  return (bytes + 255) / 256 * 256;
}

namespace {

// Cache formats: bf16 values, FP8 codes with a row exponent, 4-bit codes with an exponent
// per 32 values (always the 16-row or the 256-row kernel).
enum CacheFmt { kBf16 = 0, kFp8 = 1, kMx4 = 2 };

hipError_t launch_attn(const AttnPlan& plan, int fmt, const void* q, const void* k, const void* v,
                       const int32_t* ek, const int32_t* ev, int64_t st, int64_t sh, const int32_t* parent, int N,
                       int L, int Hq, int Hkv, float scale, void* out, float* lse, void* workspace,
                       int32_t* dev_error, hipStream_t stream) {
  const size_t rows = (size_t)Hkv * plan.RT * plan.S * TILE_ROWS;
  char* ws = static_cast<char*>(workspace);
  __bf16* part_o = reinterpret_cast<__bf16*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + (rows * D * sizeof(__bf16) + 255) / 256 * 256);

  SplitParams sp;
  sp.q = static_cast<const uint16_t*>(q);
  sp.k = k;
  sp.v = v;
  sp.ek = ek;
  sp.ev = ev;
  sp.Hkv = Hkv;
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
  int merge_rows = plan.RWV * 32;  // stacked rows per split workgroup
  if (plan.M <= 16 && fmt == kBf16) {
    static std::atomic<uint64_t> attr_devices{0};
    e = allow_dynamic_lds(&attn_rows16_kernel<false>, R16_SMEM_BYTES, attr_devices);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(attn_rows16_kernel<false>, dim3(nwg), dim3(512), R16_SMEM_BYTES, stream, sp);
      e = hipGetLastError();
    }
  } else if (plan.M <= 16 && fmt == kFp8) {
    static std::atomic<uint64_t> attr_devices{0};
    e = allow_dynamic_lds(&attn_rows16_kernel<true>, R16_SMEM_BYTES, attr_devices);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(attn_rows16_kernel<true>, dim3(nwg), dim3(512), R16_SMEM_BYTES, stream, sp);
      e = hipGetLastError();
    }
  } else if (plan.M <= 16) {
    static std::atomic<uint64_t> attr_devices{0};
    e = allow_dynamic_lds(&attn_rows16_kernel<true, true>, R16_SMEM_BYTES, attr_devices);
    if (e == hipSuccess) {
      hipLaunchKernelGGL((attn_rows16_kernel<true, true>), dim3(nwg), dim3(512), R16_SMEM_BYTES, stream, sp);
      e = hipGetLastError();
    }
  } else if (fmt == kMx4) {
    // The shared-ring kernels (two, four or eight row-waves); 17-32 rows take the two
    // row-wave one (one row tile per KV head either way, so RT, S and the workspace are
    // those of the plan).
    switch (plan.RWV) {
      case 1:
      case 2: e = launch_split<2, true, true>(sp, nwg, stream); merge_rows = 64; break;
      case 4: e = launch_split<4, true, true>(sp, nwg, stream); break;
      default: e = launch_split<8, true, true>(sp, nwg, stream); break;
    }
  } else if (fmt == kFp8) {
    switch (plan.RWV) {
      case 1: e = launch_split<1, true>(sp, nwg, stream); break;
      case 2: e = launch_split<2, true>(sp, nwg, stream); break;
      case 4: e = launch_split<4, true>(sp, nwg, stream); break;
      default: e = launch_split<8, true>(sp, nwg, stream); break;
    }
  } else {
    switch (plan.RWV) {
      case 1: e = launch_split<1, false>(sp, nwg, stream); break;
      case 2: e = launch_split<2, false>(sp, nwg, stream); break;
      case 4: e = launch_split<4, false>(sp, nwg, stream); break;
      default: e = launch_split<8, false>(sp, nwg, stream); break;
    }
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
  mp.rows = merge_rows;
  const int rows_out = N * Hq;
  const dim3 mgrid((rows_out + 3) / 4);
  switch ((plan.S + 15) / 16) {
    case 1: hipLaunchKernelGGL(attn_merge_small_kernel<1>, mgrid, dim3(256), 0, stream, mp); break;
    case 2: hipLaunchKernelGGL(attn_merge_small_kernel<2>, mgrid, dim3(256), 0, stream, mp); break;
    case 3: hipLaunchKernelGGL(attn_merge_small_kernel<3>, mgrid, dim3(256), 0, stream, mp); break;
    case 4: hipLaunchKernelGGL(attn_merge_small_kernel<4>, mgrid, dim3(256), 0, stream, mp); break;
    default: hipLaunchKernelGGL(attn_merge_kernel, mgrid, dim3(256), 0, stream, mp); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_attn(const AttnPlan& plan, const void* q, const void* k, const void* v, int64_t st,
                            int64_t sh, const int32_t* parent, int N, int L, int Hq, int Hkv, float scale,
                            void* out, float* lse, void* workspace, int32_t* dev_error, hipStream_t stream) {
  return launch_attn(plan, kBf16, q, k, v, nullptr, nullptr, st, sh, parent, N, L, Hq, Hkv, scale, out, lse,
                     workspace, dev_error, stream);
}

hipError_t launch_tree_attn_fp8(const AttnPlan& plan, const void* q, const void* kc, const void* vc,
                                const int32_t* ek, const int32_t* ev, int64_t st, int64_t sh,
                                const int32_t* parent, int N, int L, int Hq, int Hkv, float scale, void* out,
                                float* lse, void* workspace, int32_t* dev_error, hipStream_t stream) {
  return launch_attn(plan, kFp8, q, kc, vc, ek, ev, st, sh, parent, N, L, Hq, Hkv, scale, out, lse, workspace,
                     dev_error, stream);
}

hipError_t launch_tree_attn_mx4(const AttnPlan& plan, const void* q, const void* kc, const void* vc,
                                const int8_t* ek, const int8_t* ev, int64_t st, int64_t sh,
                                const int32_t* parent, int N, int L, int Hq, int Hkv, float scale, void* out,
                                float* lse, void* workspace, int32_t* dev_error, hipStream_t stream) {
  // a row's four int8 block exponents travel as one 32-bit word
  return launch_attn(plan, kMx4, q, kc, vc, reinterpret_cast<const int32_t*>(ek), reinterpret_cast<const int32_t*>(ev),
                     st, sh, parent, N, L, Hq, Hkv, scale, out, lse, workspace, dev_error, stream);
}

}  // namespace tv

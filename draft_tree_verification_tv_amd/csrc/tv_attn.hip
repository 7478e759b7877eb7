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
//     is used by every row that needs it. A workgroup owns up to 256 rows (32 per wave).
//   * Splits. The key sequence [0, L+N) is cut into S ranges; each workgroup streams one
//     range for one (KV head, row tile) and writes a normalised fp32 partial output and
//     its log2-sum-exp. A second kernel merges the partials.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the
//     accumulator layout puts one query row per lane (16 keys per lane per 32-key
//     block), so the running max / sum of the online softmax are lane-local (plus one
//     exchange with lane ^ 32) and P^T can feed the P.V product as the B operand
//     straight from registers. O^T = V^T P^T accumulates in 64 fp32 registers per lane.
//   * LDS. K is staged row-major (272-byte rows: 16 bytes of padding keep the 128-bit
//     MFMA operand reads conflict free). V is staged transposed (one row per head-dim
//     index, keys contiguous) with the keys of each 16-key group permuted so that the
//     eight keys a lane needs for one MFMA are one 16-byte read. Two stages; the next
//     tile's global loads are in flight while the current tile is multiplied.
//   * Softmax. exp2 with the scale folded into one FMA; the reference maximum is only
//     raised when a tile exceeds it by more than 2^8 (lazy rescaling), which keeps the
//     per-tile rescale of the 64 output registers off the common path.
//   * Tree keys (rows L..L+N-1) are masked with per-node ancestor bitmasks built in LDS
//     by the workgroups whose range reaches them.
//   * Workgroup order is remapped so that consecutive work items (the splits of one KV
//     head) run on the same XCD and share its L2.
#include <cmath>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int D = TV_HEAD_DIM;
constexpr int KT = 64;                 // keys per LDS tile
constexpr int TILE_ROWS = 256;         // stacked rows per workgroup (8 waves x 32)
constexpr int KROW = D * 2 + 16;       // bytes per staged K row
constexpr int VROW = KT * 2 + 16;      // bytes per staged V^T row
constexpr int K_BYTES = KT * KROW;
constexpr int V_BYTES = D * VROW;
constexpr int STAGE = K_BYTES + V_BYTES;
constexpr int TREE_ANC_BYTES = kMaxNodes * kAncWords * 8;
constexpr int TREE_BYTES = TREE_ANC_BYTES + 2 * kMaxNodes * 4;
constexpr int SMEM_BYTES = 2 * STAGE + TREE_BYTES;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleTh = 8.0f;

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

// Position of the first key of quad qd (keys 4qd..4qd+3 of a tile) in a staged V^T row.
// Within each 16-key group the middle quads swap, so that a lane's eight keys for one
// MFMA step (4g..4g+3 and 8+4g..8+4g+3) are contiguous.
__device__ __forceinline__ int vt_pos(int qd) {
  return (qd >> 2) * 16 + (qd & 1) * 8 + ((qd >> 1) & 1) * 4;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_split_kernel(SplitParams p) {
  constexpr int NT = NW * 64;
  constexpr int KCH = KT * (D / 8);            // 16-byte K chunks per tile
  constexpr int KPT = (KCH + NT - 1) / NT;     // per thread
  constexpr int VIT = (KT / 4) * (D / 8);      // (4-key quad, 8-dim chunk) items per tile
  constexpr int VPT = (VIT + NT - 1) / NT;

  extern __shared__ __align__(16) char smem[];
  uint64_t* anc = reinterpret_cast<uint64_t*>(smem + 2 * STAGE);
  int* par = reinterpret_cast<int*>(smem + 2 * STAGE + TREE_ANC_BYTES);
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
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int grp = lane >> 5;

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

  u32x4 kreg[KPT];
  u32x4 vreg[VPT][4];

  auto gload = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      const int key = kt0 + (c >> 4);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (c < KCH && key < p.T)
        x = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * p.st + (c & 15) * 8);
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int it = tid + i * NT;
      const int dc = it & 15;
      const int qd = it >> 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kt0 + qd * 4 + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (it < VIT && key < p.T)
          x = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.st + dc * 8);
        vreg[i][j] = x;
      }
    }
  };

  auto lds_store = [&](int buf) {
    char* Ks = smem + buf * STAGE;
    char* Vs = Ks + K_BYTES;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KROW + (c & 15) * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int it = tid + i * NT;
      if (it < VIT) {
        const int dc = it & 15;
        const int qd = it >> 4;
        char* dst = Vs + (dc * 8) * VROW + vt_pos(qd) * 2;
        // 4 keys x 8 dims -> 8 rows (one per dim) of 4 keys.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a0 = vreg[i][0][e], a1 = vreg[i][1][e], a2 = vreg[i][2][e], a3 = vreg[i][3][e];
          uint2 lo, hi;
          lo.x = (a0 & 0xFFFFu) | (a1 << 16);
          lo.y = (a2 & 0xFFFFu) | (a3 << 16);
          hi.x = (a0 >> 16) | (a1 & 0xFFFF0000u);
          hi.y = (a2 >> 16) | (a3 & 0xFFFF0000u);
          *reinterpret_cast<uint2*>(dst + (2 * e) * VROW) = lo;
          *reinterpret_cast<uint2*>(dst + (2 * e + 1) * VROW) = hi;
        }
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_ref = -INFINITY;
  float lsum = 0.f;

  if (ntiles > 0) {
    gload(kbeg);
    lds_store(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = kbeg + t * KT;
    if (t + 1 < ntiles) gload(kt0 + KT);

    const char* Ks = smem + (t & 1) * STAGE;
    const char* Vs = Ks + K_BYTES;

    // S^T for two 32-key blocks
    f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + ql) * KROW + s8 * 32 + grp * 16);
        sc[kb] = mfma32(a, qf[s8], sc[kb]);
      }
    }

    // Mask keys past the context: tree keys by ancestry, anything past L+N always.
    if (kt0 + KT > p.L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt0 + kb * 32 + 8 * (e >> 2) + 4 * grp + (e & 3);
          bool vis = key < p.L;
          if (!vis && key < p.T) {
            const int j = key - p.L;
            vis = (anc[node * kAncWords + (j >> 6)] >> (j & 63)) & 1ull;
          }
          if (!vis) sc[kb][e] = -INFINITY;
        }
      }
    }

    // Online softmax (log2 domain), lazily rescaled.
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, fmaxf(sc[0][e], sc[1][e]));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    mt *= p.c;
    const bool need = mt > m_ref + kRescaleTh;
    if (__any(need)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = need ? exp2f(m_ref - m_new) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m_ref = m_new;
    }
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;

    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        f32x2 pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][th * 8 + 2 * j], p.c, -mu));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][th * 8 + 2 * j + 1], p.c, -mu));
          lsum += p0 + p1;
          pr[j] = f32x2{p0, p1};
        }
        const bf16x2 b0 = __builtin_convertvector(pr[0], bf16x2);
        const bf16x2 b1 = __builtin_convertvector(pr[1], bf16x2);
        const bf16x2 b2 = __builtin_convertvector(pr[2], bf16x2);
        const bf16x2 b3 = __builtin_convertvector(pr[3], bf16x2);
        pb[kb * 2 + th] = bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + (db * 32 + ql) * VROW + ks * 32 + grp * 16);
        o[db] = mfma32(a, pb[ks], o[db]);
      }
    }

    if (t + 1 < ntiles) lds_store((t + 1) & 1);
    __syncthreads();
  }

  // ---- partial result of this split
  lsum += __shfl_xor(lsum, 32);
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

// One (node, q head) row per 32 threads; each thread merges 4 head-dim values:
// lse = M + log2 sum_s 2^(lse_s - M), out = sum_s 2^(lse_s - lse) * out_s.
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams mp) {
  const int row = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= mp.N * mp.Hq) return;
  const int n = row / mp.Hq;
  const int qh = row % mp.Hq;
  const int h = qh / mp.G;
  const int r = n * mp.G + qh % mp.G;
  const int rt = r / TILE_ROWS;
  const int64_t base0 = (int64_t)(h * mp.RT + rt) * mp.S * TILE_ROWS + (r % TILE_ROWS);
  float mx = -INFINITY;
  for (int s = 0; s < mp.S; ++s) mx = fmaxf(mx, mp.part_lse[base0 + (int64_t)s * TILE_ROWS]);
  const int d0 = (threadIdx.x & 31) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < mp.S; ++s) {
      const int64_t b = base0 + (int64_t)s * TILE_ROWS;
      const float wgt = exp2f(mp.part_lse[b] - mx);
      wsum += wgt;
      const f32x4 x = *reinterpret_cast<const f32x4*>(mp.part_o + b * D + d0);
      acc += wgt * x;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const bf16x2 lo = __builtin_convertvector((f32x2{acc[0] * inv, acc[1] * inv}), bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2{acc[2] * inv, acc[3] * inv}), bf16x2);
  uint2 packed;
  packed.x = __builtin_bit_cast(uint32_t, lo);
  packed.y = __builtin_bit_cast(uint32_t, hi);
  *reinterpret_cast<uint2*>(mp.out + (int64_t)row * D + d0) = packed;
  if (mp.lse && (threadIdx.x & 31) == 0)
    mp.lse[row] = mx == -INFINITY ? -INFINITY : (mx + __log2f(wsum)) * kLn2;
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
  p.NW = (rows + 31) / 32;
  if (p.NW < 2) p.NW = 2;
  p.T = L + N;
  const int tiles = (p.T + KT - 1) / KT;
  int S = num_splits;
  if (S <= 0) {
    // One workgroup per CU for 8-wave groups (register bound), two for smaller groups
    // (LDS bound); at least 8 tiles per split so partial traffic stays small.
    const int per_cu = p.NW > 4 ? 1 : 2;
    const int units = Hkv * p.RT;
    S = (num_cus * per_cu + units - 1) / units;
    const int cap = tiles / 8 > 0 ? tiles / 8 : 1;
    if (S > cap) S = cap;
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
    case 3: e = launch_split<3>(sp, nwg, stream); break;
    case 4: e = launch_split<4>(sp, nwg, stream); break;
    case 5: e = launch_split<5>(sp, nwg, stream); break;
    case 6: e = launch_split<6>(sp, nwg, stream); break;
    case 7: e = launch_split<7>(sp, nwg, stream); break;
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
  hipLaunchKernelGGL(attn_merge_kernel, dim3((rows_out + 7) / 8), dim3(256), 0, stream, mp);
  return hipGetLastError();
}

}  // namespace tv

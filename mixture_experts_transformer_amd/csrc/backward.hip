// Backward of the GPT-OSS MoE block on gfx950 (bf16 expert weights), with the top-k
// selection of the forward held fixed.
//
// torchtitan GPT-OSS guide, section "Grouped matrix multiplication": the block is trained,
// and the gradient of its SwiGLU variant is unit tested against a reference.  The selection
// is piecewise constant in the inputs, so gradients reach the router only through the
// softmax gates.  Per assignment a = t*k + j (expert e, gate g, row p of e's group):
//
//   u  = x[t] W1[e]^T + b1[e]                          (recomputed: the forward's mlp1 kernel)
//   dh' = dout[t] W2[e]                                 (the forward's mlp2 kernel, W2 as stored)
//   dg[a] = <dh', h(u)> + <dout[t], b2[e]>              (= <dout[t], z[a]>, z the ungated mlp2 output)
//   du = SwiGLU'(u) * (g dh')
//   dx[t] += du W1[e]                                   (the forward's mlp2 kernel, W1 as stored)
//   dW2[e] = sum_p (g dout[t])^T h,  dW1[e] = sum_p du^T x[t]   (per-expert GEMMs, K = rows)
//   db2[e] = sum_p g dout[t],  db1[e] = sum_p du
//   router: dl = g (dg - sum_j g_j dg_j) on the selected experts; dWr[e] = sum dl x[t],
//   dbr[e] = sum dl, dx[t] += sum_j dl_j Wr[e_j].
//
// The three products over routed rows are the forward's grouped GEMMs (grouped_gemm_kernel):
// mlp1 with an epilogue that stores u instead of h, and mlp2 with unit gates and zero biases
// for dh' and for du W1 (their weights read as stored, [K][N], through transposing LDS reads;
// dout enters as a bf16 pair, hi and lo against the same weight tile).  The weight gradients contract
// over an expert's rows, so their operands are written transposed, per expert, in a layout
// whose expert blocks are padded to 64 rows with zeros, and multiplied by bwd_gemm_kernel.
// Everything runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  No float atomics:
// every sum runs in a fixed order, so the gradients are bitwise reproducible.
#include "device_common.h"

namespace moe {

namespace {

constexpr float BW_ALPHA = 1.702f;
constexpr float BW_LIMIT = 7.0f;
constexpr float BW_NEG_ALPHA_LOG2E = -BW_ALPHA * 1.4426950408889634f;

// ------------------------------------------------------------------------------ GEMM tile
// Weight-gradient tiles for experts with few rows (K of 64 or 128), where a tile is one or two
// matrix steps and then 128 KB of fp32 stores: 256 x 128 outputs, 8 waves in a 4 x 2 grid of
// 64 x 64, K in steps of 64 (whole 128-byte row segments) staged to one LDS stage through
// registers, two workgroups per CU so one tile's loads and matrix work overlap another's
// stores.  Experts with many rows take the grouped GEMM kernel's weight-gradient mode
// (launch_wgrad_tiles: 256 x 256 tiles fed by direct-to-LDS copies).
constexpr int BG_BK = 64, BG_CPR = BG_BK / 8;
template <int BM_, int BN_, int WM_, int WN_, int WPE_>
struct WTile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WM_, WAVES_N = WN_, WPE = WPE_;
  static constexpr int NW = WM_ * WN_, THREADS = 64 * NW;
  static constexpr int WTM = BM / WM_, WTN = BN / WN_;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_BYTES = BM * BG_BK * 2, B_BYTES = BN * BG_BK * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int ALD = BM * BG_CPR / THREADS;   // 16-byte A chunks per thread and stage
  static constexpr int BLD = BN * BG_CPR / THREADS;   // B chunks
  static_assert(ALD * THREADS == BM * BG_CPR && BLD * THREADS == BN * BG_CPR, "load split");
};
using WTileSmall = WTile<256, 128, 4, 2, 4>;

struct BwdGemmArgs {
  const int32_t* poff;      // [E+1] padded column offsets, then [E] the experts by decreasing
                            //   padded row count
  const uint16_t* a;        // A operand rows (bf16, K contiguous), lda elements apart
  const uint16_t* b;        // B operand rows, ldb elements apart
  int lda, ldb;
  int E, M, N;
  int n_tiles, m_tiles;
  float* c;                 // [E][M][N]
};

// Per-expert weight gradient C[e] = A_e B_e^T: A_e = rows of a transposed activation and B_e
// rows of another, both restricted to expert e's padded columns [poff[e], poff[e + 1]) (the
// K of the product: the expert's rows, zero past its count).
//
// Matrix-core mapping as in the forward's grouped GEMM: in MFMA step ks of a stage, lane l
// feeds row l & 31 and the 8 K elements of chunk 4 (l >> 5) + ks of each operand, and output
// register q of lane l is C[8 (q >> 2) + 4 (l >> 5) + (q & 3)][l & 31].
template <class W>
__global__ __launch_bounds__(W::THREADS, W::WPE) void bwd_gemm_kernel(BwdGemmArgs p) {
  constexpr int BM = W::BM, BN = W::BN, FM = W::FM, FN = W::FN, ALD = W::ALD, BLD = W::BLD;
  constexpr int THREADS = W::THREADS, STAGE = W::STAGE, A_BYTES = W::A_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / W::WAVES_N, wn = wave % W::WAVES_N;
  const int kg = lane >> 5;

  // ---- which tile: the tiles cost their expert's row count, so the largest experts go
  // first (dispatched first and spread over every XCD) and the Zipf head does not trail;
  // in groups of four row tiles so neighbouring workgroups share operand rows
  int e, m0, n_tile, rows;
  {
    constexpr int GM = 4;
    const int mt_total = p.E * p.m_tiles;
    const int total = mt_total * p.n_tiles;
    const int lin = blockIdx.x;
    if (lin >= total) return;
    const int gsize = GM * p.n_tiles;
    const int g = lin / gsize;
    const int first_m = g * GM;
    const int gm = min(mt_total - first_m, GM);
    const int m_tile = first_m + (lin % gsize) % gm;
    n_tile = (lin % gsize) / gm;
    // the expert of rank m_tile / m_tiles in decreasing padded row count
    e = p.poff[p.E + 1 + m_tile / p.m_tiles];
    m0 = (m_tile % p.m_tiles) * BM;
    rows = min(BM, p.M - m0);
  }
  const int K = p.poff[e + 1] - p.poff[e];
  const int n0 = n_tile * BN;
  const int nk = K / BG_BK;

  // ---- this thread's copy rows: chunk c of tile rows (tid / CPR) + (THREADS / CPR) j
  const int cch = tid % BG_CPR;
  const uint16_t* arow[ALD];
  const uint16_t* brow[BLD];
  int ar[ALD], br[BLD];
#pragma unroll
  for (int j = 0; j < ALD; ++j) {
    const int r = tid / BG_CPR + (THREADS / BG_CPR) * j;
    ar[j] = r;
    arow[j] = p.a + (int64_t)min(m0 + r, p.M - 1) * p.lda + p.poff[e] + cch * 8;
  }
#pragma unroll
  for (int j = 0; j < BLD; ++j) {
    const int r = tid / BG_CPR + (THREADS / BG_CPR) * j;
    br[j] = r;
    brow[j] = p.b + (int64_t)min(n0 + r, p.N - 1) * p.ldb + p.poff[e] + cch * 8;
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Stage kt of this thread's rows into register set R, and register set R into LDS slot s
  // (macros, not lambdas: a call that is not inlined would leave the staging arrays in
  // memory).
  u32x4 ra0[ALD], rb0[BLD];
#define BW_GLOAD(kt, RA, RB)                                                                     \
  do {                                                                                           \
    const int ko_ = (kt) * BG_BK;                                                                \
    _Pragma("unroll") for (int j = 0; j < ALD; ++j) RA[j] = *(const u32x4*)(arow[j] + ko_);      \
    _Pragma("unroll") for (int j = 0; j < BLD; ++j) RB[j] = *(const u32x4*)(brow[j] + ko_);      \
  } while (0)
#define BW_LSTORE(slot, RA, RB)                                                                  \
  do {                                                                                           \
    uint8_t* s_ = smem + (slot) * STAGE;                                                         \
    _Pragma("unroll") for (int j = 0; j < ALD; ++j)                                              \
      *(u32x4*)(s_ + swz<BG_CPR>(ar[j], cch)) = RA[j];                                           \
    _Pragma("unroll") for (int j = 0; j < BLD; ++j)                                              \
      *(u32x4*)(s_ + A_BYTES + swz<BG_CPR>(br[j], cch)) = RB[j];                                 \
  } while (0)
  // a wave whose rows are all padding skips its matrix instructions
  const bool active = wm * W::WTM < rows;
  const int arow0 = wm * W::WTM + (lane & 31);
  const int brow0 = wn * W::WTN + (lane & 31);
#define BW_COMPUTE(slot)                                                                         \
  do {                                                                                           \
    if (active) {                                                                                \
      const uint8_t* sa = smem + (slot) * STAGE;                                                 \
      const uint8_t* sb = sa + A_BYTES;                                                          \
      _Pragma("unroll") for (int ks = 0; ks < BG_BK / 16; ++ks) {                                \
        const int cc = kg * (BG_BK / 16) + ks;                                                   \
        bf16x8 fa[FM], fb[FN];                                                                   \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                           \
          fa[i] = *(const bf16x8*)(sa + swz<BG_CPR>(arow0 + 32 * i, cc));                        \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
          fb[j] = *(const bf16x8*)(sb + swz<BG_CPR>(brow0 + 32 * j, cc));                        \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                           \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0); \
      }                                                                                          \
    }                                                                                            \
  } while (0)
  // The loads are unconditional (past the last stage they fetch the last stage again): with
  // loads under a condition the compiler's wait counts assume the newest loads may be the
  // ones a store needs, and the stores then wait for everything in flight.
  // one LDS stage: stage kt + 1 loads into the register set while stage kt is multiplied
  if (nk > 0) {
    BW_GLOAD(0, ra0, rb0);
    for (int kt = 0; kt < nk; ++kt) {
      __syncthreads();                      // the previous stage's reads are done
      BW_LSTORE(0, ra0, rb0);
      __syncthreads();
      BW_GLOAD(min(kt + 1, nk - 1), ra0, rb0);
      BW_COMPUTE(0);
    }
  }
#undef BW_GLOAD
#undef BW_LSTORE
#undef BW_COMPUTE

  // ---- epilogue: row rr of the tile for register q of fragment i, column for fragment j
  float* const dst = p.c + (int64_t)e * p.M * p.N;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * W::WTN + 32 * j + (lane & 31);
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = wm * W::WTM + 32 * i + 8 * (q >> 2) + 4 * kg + (q & 3);
        if (rr < rows) dst[(int64_t)(m0 + rr) * p.N + n] = acc[i][j][q];
      }
  }
}

// dst[e] = A_e B_e^T for every expert: M x N outputs per expert.  Few rows per expert: the
// single-stage tile above; many: the forward's grouped GEMM kernel in its weight-gradient
// mode (direct-to-LDS copies, 256 x 256 tiles)
template <class W>
static hipError_t launch_wgrad_t(BwdGemmArgs g, hipStream_t st) {
  g.m_tiles = (g.M + W::BM - 1) / W::BM;
  g.n_tiles = (g.N + W::BN - 1) / W::BN;
  const int64_t tiles = (int64_t)g.E * g.m_tiles * g.n_tiles;
  hipLaunchKernelGGL(bwd_gemm_kernel<W>, dim3((unsigned)tiles), dim3(W::THREADS), 0, st, g);
  return hipGetLastError();
}
hipError_t launch_wgrad(const BwdGemmArgs& g, bool small, hipStream_t st) {
  if (small) return launch_wgrad_t<WTileSmall>(g, st);
  return launch_wgrad_tiles(g.a, g.b, g.lda, g.poff, g.E, g.M, g.N, g.c, st);
}

// ------------------------------------------------------------------------------ routing helpers
// Padded column offsets of the experts in the transposed activations: expert e's rows
// occupy columns [poff[e], poff[e + 1]), its count rounded up to a multiple of 64.  Then
// poff[E + 1 + r] = the expert of rank r by decreasing padded count (ties: lower index), the
// order in which the weight-gradient tiles are dispatched.
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                          int32_t* __restrict__ poff) {
  __shared__ int s[257];
  const int tid = threadIdx.x;
  if (tid < E) {
    const int c = offsets[tid + 1] - offsets[tid];
    s[tid + 1] = (max(c, 0) + BG_BK - 1) / BG_BK * BG_BK;
  }
  if (tid == 0) s[0] = 0;
  __syncthreads();
  if (tid < E) {
    const int kc = s[tid + 1];
    int rk = 0;
    for (int o = 0; o < E; ++o) rk += (s[o + 1] > kc || (s[o + 1] == kc && o < tid)) ? 1 : 0;
    poff[E + 1 + rk] = tid;
  }
  __syncthreads();
  if (tid == 0)
    for (int i = 1; i <= E; ++i) s[i] += s[i - 1];
  __syncthreads();
  for (int i = tid; i <= E; i += 256) poff[i] = s[i];
}

// padmap[col] = routed row p in column col of the transposed layout, or -1 for padding.
__global__ __launch_bounds__(256) void pad_map_kernel(const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ poff, int E, int ldt,
                                                      int32_t* __restrict__ padmap) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= ldt) return;
  int lo = 0, hi = E;                      // the expert e with poff[e] <= col < poff[e + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (poff[mid] <= col) lo = mid;
    else hi = mid;
  }
  int v = -1;
  if (col < poff[E]) {
    const int r = col - poff[lo];
    if (r < offsets[lo + 1] - offsets[lo]) v = offsets[lo] + r;
  }
  padmap[col] = v;
}

// ------------------------------------------------------------------------------ conversions
static __device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)*(const uint16_t*)&x | ((uint32_t)*(const uint16_t*)&y << 16);
}
// dout rows in routed order as bf16 pairs: hi[p] and lo[p] of dout[token of perm[p]], hi the
// nearest bf16 and lo the nearest bf16 of what hi leaves (hi + lo: about 16 significant bits),
// the two parts of the A operand of dh' = dout W2^T.
__global__ __launch_bounds__(256) void gather_dout_pair_kernel(const float4* __restrict__ dout,
                                                               const int32_t* __restrict__ perm, int A, int k,
                                                               int D4, uint2* __restrict__ hi,
                                                               uint2* __restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)A * D4) return;
  const int64_t p = i / D4;
  const int c = (int)(i - p * D4);
  int a = perm[p];
  a = ((unsigned)a < (unsigned)A) ? a : 0;
  const float4 v = dout[(int64_t)(a / k) * D4 + c];
  const float h0 = (float)(__bf16)v.x, h1 = (float)(__bf16)v.y, h2 = (float)(__bf16)v.z, h3 = (float)(__bf16)v.w;
  hi[i] = uint2{pack_bf16x2(h0, h1), pack_bf16x2(h2, h3)};
  lo[i] = uint2{pack_bf16x2(v.x - h0, v.y - h1), pack_bf16x2(v.z - h2, v.w - h3)};
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// The clamped SwiGLU's backward on routed row p (one workgroup per row): from u (fp32, gate
// half then linear half) and dh' (fp32, the ungated mlp2 input gradient at slot row a =
// perm[p]), h = gc sigmoid(ALPHA gc) (lc + 1) with gc = min(gate, LIMIT), lc = clamp(lin);
// du_gate = g dh' (sigmoid + ALPHA gc sigmoid (1 - sigmoid)) (lc + 1) where gate <= LIMIT,
// du_lin = g dh' gc sigmoid where -LIMIT <= lin <= LIMIT; writes h and du (bf16) and
// dg[a] = sum_f dh' h (fixed-order tree over the workgroup).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ u, const float* __restrict__ dhp,
                                                         const int32_t* __restrict__ perm,
                                                         const float* __restrict__ gates, int A, int F,
                                                         uint16_t* __restrict__ h, uint16_t* __restrict__ du,
                                                         float* __restrict__ dg) {
  __shared__ float red[256];
  const int64_t p = blockIdx.x;
  int a = perm[p];
  a = ((unsigned)a < (unsigned)A) ? a : 0;
  const float g = gates[a];
  const float* const ur = u + p * 2 * F;
  const float* const dr = dhp + (int64_t)a * F;
  float s = 0.f;
  for (int f = threadIdx.x * 4; f < F; f += 1024) {
    const f32x4 ug4 = *(const f32x4*)(ur + f), ul4 = *(const f32x4*)(ur + F + f);
    const f32x4 d4 = *(const f32x4*)(dr + f);
    float hv[4], dgv[4], dlv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float ug = ug4[c], ul = ul4[c];
      const float gc = fminf(ug, BW_LIMIT);
      const float lc = fminf(fmaxf(ul, -BW_LIMIT), BW_LIMIT);
      // sigmoid(ALPHA gc) = 1 / (1 + 2^(-ALPHA log2(e) gc))
      const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gc * BW_NEG_ALPHA_LOG2E));
      hv[c] = gc * sg * (lc + 1.0f);
      s += d4[c] * hv[c];
      const float dh = g * d4[c];
      const float dgc = sg + BW_ALPHA * gc * sg * (1.0f - sg);    // d(gc sigmoid(ALPHA gc)) / d gc
      dgv[c] = (ug <= BW_LIMIT) ? dh * dgc * (lc + 1.0f) : 0.f;
      dlv[c] = (ul >= -BW_LIMIT && ul <= BW_LIMIT) ? dh * gc * sg : 0.f;
    }
    *(uint2*)(h + p * F + f) = uint2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
    *(uint2*)(du + p * 2 * F + f) = uint2{pack_bf16x2(dgv[0], dgv[1]), pack_bf16x2(dgv[2], dgv[3])};
    *(uint2*)(du + p * 2 * F + F + f) = uint2{pack_bf16x2(dlv[0], dlv[1]), pack_bf16x2(dlv[2], dlv[3])};
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dg[a] = red[0];
}

// 64 x 64 bf16 tiles through LDS with 16-byte global accesses: phase 1 puts tile row r
// (8-element chunks) in LDS row r, phase 2 writes output row c as eight 8-element chunks,
// each gathered from one LDS column.  Row stride 72 elements keeps LDS rows 16-byte aligned.
constexpr int TP_LD = 72;
static __device__ __forceinline__ void tile_out(const uint16_t (*t)[TP_LD], int c, int ch, uint16_t* dst) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = (uint32_t)t[ch * 8 + 2 * q][c] | ((uint32_t)t[ch * 8 + 2 * q + 1][c] << 16);
  *(u32x4*)dst = v;
}

// Transposed, expert-padded copy of routed rows: dst[c][col] = scale(col) src[row(col)][c]
// for the C columns of the rows (C a multiple of 64), zero where padmap[col] < 0.
// SRC_TOKEN: the source row is the token of the routed row's assignment (x, dout), else the
// routed row itself (du, h).  GATE: scaled by the assignment's gate (dz = g dout).  SRC_F32:
// fp32 source.
template <bool SRC_TOKEN, bool GATE, bool SRC_F32>
__global__ __launch_bounds__(256) void gather_transpose_kernel(const void* __restrict__ src, int C, int ld_src,
                                                               const int32_t* __restrict__ padmap,
                                                               const int32_t* __restrict__ perm,
                                                               const float* __restrict__ gates, int k, int A,
                                                               int ldt, uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint16_t t[64][TP_LD];
  const int col0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, ch = i & 7;          // r: column of the padded layout (a routed row)
    const int prow = padmap[col0 + r];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (prow >= 0) {
      int64_t srow = prow;
      float sc = 1.f;
      if (SRC_TOKEN || GATE) {
        int a = perm[prow];
        a = ((unsigned)a < (unsigned)A) ? a : 0;
        if (SRC_TOKEN) srow = a / k;
        if (GATE) sc = gates[a];
      }
      if (SRC_F32) {
        const float* sp = (const float*)src + srow * ld_src + c0 + ch * 8;
        const f32x4 lo = *(const f32x4*)sp, hi = *(const f32x4*)(sp + 4);
        v[0] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
        v[1] = pack_bf16x2(lo[2] * sc, lo[3] * sc);
        v[2] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
        v[3] = pack_bf16x2(hi[2] * sc, hi[3] * sc);
      } else {
        v = *(const u32x4*)((const uint16_t*)src + srow * ld_src + c0 + ch * 8);
        if (GATE) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[q] = pack_bf16x2(bf16_to_f32(v[q] & 0xFFFFu) * sc, bf16_to_f32(v[q] >> 16) * sc);
        }
      }
    }
    *(u32x4*)&t[r][ch * 8] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int c = i >> 3, ch = i & 7;
    tile_out(t, c, ch, dst + (int64_t)(c0 + c) * ldt + col0 + ch * 8);
  }
}

// ------------------------------------------------------------------------------ router
// One workgroup per token: dg_j = <dh', h> (from the SwiGLU backward) + <dout[t], b2[e_j]>,
// then the softmax backward over the k selected logits, dl_j = g_j (dg_j - sum_i g_i dg_i).
// The dot products take the slots four at a time: thread i reads four consecutive elements
// of dout's row (16 bytes) and of each slot's b2 row (8 bytes) at 256-element steps, the
// workgroup's partial sums meet in LDS in a fixed order, and wave 0 finishes the token (lane
// l keeps dg_j for the slots j = l + 64 m, k <= 256).
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ dgh,
                                                         const float* __restrict__ dout,
                                                         const uint16_t* __restrict__ b2,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ gates, int T, int D, int E,
                                                         int k, float* __restrict__ dl) {
  constexpr int JG = 4;                     // slots per pass over dout's row
  __shared__ float part[JG][4];
  __shared__ float dgs[256];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float4* const drow = (const float4*)(dout + (int64_t)t * D);
  for (int j0 = 0; j0 < k; j0 += JG) {
    const uint2* brow[JG];
#pragma unroll
    for (int jj = 0; jj < JG; ++jj) {
      const int j = min(j0 + jj, k - 1);
      const int e = min(max(idx[(int64_t)t * k + j], 0), E - 1);
      brow[jj] = (const uint2*)(b2 + (int64_t)e * D);
    }
    float v[JG];
#pragma unroll
    for (int jj = 0; jj < JG; ++jj) v[jj] = 0.f;
    for (int c = tid; c < D / 4; c += 256) {    // D is a multiple of 64
      const float4 o = drow[c];
#pragma unroll
      for (int jj = 0; jj < JG; ++jj) {
        if (j0 + jj < k) {
          const uint2 w = brow[jj][c];
          v[jj] += o.x * __uint_as_float(w.x << 16) + o.y * __uint_as_float(w.x & 0xFFFF0000u) +
                   o.z * __uint_as_float(w.y << 16) + o.w * __uint_as_float(w.y & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < JG; ++jj) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v[jj] += __shfl_xor(v[jj], off);
      if (lane == 0) part[jj][wave] = v[jj];
    }
    __syncthreads();
    if (tid < JG && j0 + tid < k) {
      const int a = t * k + j0 + tid;
      dgs[j0 + tid] = dgh[a] + ((part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]));
    }
    __syncthreads();
  }
  if (wave == 0) {
    float sgd = 0.f;
    for (int j = 0; j < k; ++j) sgd += gates[t * k + j] * dgs[j];
    for (int j = lane; j < k; j += 64) dl[t * k + j] = gates[t * k + j] * (dgs[j] - sgd);
  }
}

// Per expert, sums over its routed rows.  The rows are split into EX_CHUNKS fixed chunks in
// group order; pass 1 sums each chunk per column, pass 2 adds the chunks in order:
//   dwr[e][d] = sum dl x[t][d];  db2[e][d] = sum g dout[t][d];  db1[e][c] = sum du[p][c].
constexpr int EX_CHUNKS = 32;
__global__ __launch_bounds__(256) void expert_partial_kernel(const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ perm,
                                                             const float* __restrict__ gates,
                                                             const float* __restrict__ dl,
                                                             const uint16_t* __restrict__ x,
                                                             const float* __restrict__ dout,
                                                             const uint16_t* __restrict__ du, int D, int F, int k,
                                                             int A, int E, float* __restrict__ pw,
                                                             float* __restrict__ pb2, float* __restrict__ pb1) {
  const int e = blockIdx.y, r = blockIdx.z;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int G = 2 * F;
  const int p0 = offsets[e], cnt = offsets[e + 1] - p0;
  const int len = (cnt + EX_CHUNKS - 1) / EX_CHUNKS;
  const int lo = p0 + min(cnt, r * len), hi = p0 + min(cnt, (r + 1) * len);
  const int64_t slot = (int64_t)r * E + e;
  if (c < D) {
    float sw = 0.f, sb = 0.f;
#pragma unroll 4
    for (int pp = lo; pp < hi; ++pp) {
      int a = perm[pp];
      a = ((unsigned)a < (unsigned)A) ? a : 0;
      const int64_t t = a / k;
      sw += dl[a] * bf16_to_f32(x[t * D + c]);
      sb += gates[a] * dout[t * D + c];
    }
    pw[slot * D + c] = sw;
    pb2[slot * D + c] = sb;
  }
  if (c < G) {
    float s = 0.f;
#pragma unroll 4
    for (int pp = lo; pp < hi; ++pp) s += bf16_to_f32(du[(int64_t)pp * G + c]);
    pb1[slot * G + c] = s;
  }
}

__global__ __launch_bounds__(256) void expert_reduce_kernel(const float* __restrict__ pw,
                                                            const float* __restrict__ pb2,
                                                            const float* __restrict__ pb1, int D, int F, int E,
                                                            float* __restrict__ dwr, float* __restrict__ db2,
                                                            float* __restrict__ db1) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int G = 2 * F;
  if (c < D) {
    float sw = 0.f, sb = 0.f;
    for (int r = 0; r < EX_CHUNKS; ++r) {
      sw += pw[((int64_t)r * E + e) * D + c];
      sb += pb2[((int64_t)r * E + e) * D + c];
    }
    dwr[(int64_t)e * D + c] = sw;
    db2[(int64_t)e * D + c] = sb;
  }
  if (c < G) {
    float s = 0.f;
    for (int r = 0; r < EX_CHUNKS; ++r) s += pb1[((int64_t)r * E + e) * G + c];
    db1[(int64_t)e * G + c] = s;
  }
}

// dbr[e] = sum of dl over the expert's rows: 256 threads stride the rows, then a fixed tree.
__global__ __launch_bounds__(256) void router_bias_grad_kernel(const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ perm,
                                                               const float* __restrict__ dl, int A,
                                                               float* __restrict__ dbr) {
  __shared__ float s[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  float v = 0.f;
  for (int pp = offsets[e] + tid; pp < offsets[e + 1]; pp += 256) {
    int a = perm[pp];
    a = ((unsigned)a < (unsigned)A) ? a : 0;
    v += dl[a];
  }
  s[tid] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s[tid] += s[tid + w];
    __syncthreads();
  }
  if (tid == 0) dbr[e] = s[0];
}

// dx[t][d] = sum_j dxs[t k + j][d] + sum_j dl[t k + j] Wr[e_j][d], slots in order; four
// columns per thread (dxs rows are ld_dxs floats apart).
__global__ __launch_bounds__(256) void dx_combine_kernel(const float* __restrict__ dxs, int ld_dxs,
                                                         const float* __restrict__ dl,
                                                         const int32_t* __restrict__ idx,
                                                         const uint16_t* __restrict__ wr, int T, int D, int E,
                                                         int k, float* __restrict__ dx) {
  const int D4 = D / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * D4) return;
  const int64_t t = i / D4;
  const int d = (int)(i - t * D4) * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) s += *(const f32x4*)(dxs + (t * k + j) * ld_dxs + d);
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    const int e = min(max(idx[a], 0), E - 1);
    const float g = dl[a];
    const uint2 w = *(const uint2*)(wr + (int64_t)e * D + d);
    s[0] += g * bf16_to_f32(w.x & 0xFFFFu);
    s[1] += g * bf16_to_f32(w.x >> 16);
    s[2] += g * bf16_to_f32(w.y & 0xFFFFu);
    s[3] += g * bf16_to_f32(w.y >> 16);
  }
  *(f32x4*)(dx + t * D + d) = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

unsigned blocks_for(int64_t n, int per = 256) { return (unsigned)((n + per - 1) / per); }

#define BW_CHECK(expr)                          \
  do {                                          \
    const hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return e_;            \
  } while (0)

}  // namespace

int bwd_padded_cols(int64_t A, int64_t E) {
  const int64_t v = A + E * (BG_BK - 1);
  return (int)((v + 63) / 64 * 64);
}
int bwd_sum_chunks() { return EX_CHUNKS; }

hipError_t launch_backward(const BwdArgs& b, hipStream_t st, const BwdSide* side) {
  const int T = b.T, D = b.D, E = b.E, k = b.k, F = b.F, G = 2 * F;
  const int A = T * k;
  const int ldt = bwd_padded_cols(A, E);
  const int DF = D > F ? D : F;
  // The memory-bound side work (activation transposes, the dout pair, the router and bias
  // gradients) goes to the side stream, when there is one, beside the grouped products on
  // st; events order the two where one reads what the other writes.  Without a side stream
  // everything runs on st in the same order.
  hipStream_t sb = side ? side->stream : st;
  auto fork = [&](hipStream_t from, hipStream_t to, int i) -> hipError_t {
    if (!side) return hipSuccess;
    const hipError_t e = hipEventRecord(side->ev[i], from);
    return e != hipSuccess ? e : hipStreamWaitEvent(to, side->ev[i], 0);
  };
  // 1. padded layout of the routed rows per expert (weight gradients)
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, st, b.offsets, E, b.poff);
  BW_CHECK(hipGetLastError());
  hipLaunchKernelGGL(pad_map_kernel, dim3(blocks_for(ldt)), dim3(256), 0, st, b.offsets, b.poff, E, ldt, b.padmap);
  BW_CHECK(hipGetLastError());
  // 2. unit gates and zero biases for the forward's mlp2 kernel used as a plain grouped GEMM
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(A)), dim3(256), 0, st, b.ones, (int64_t)A, 1.0f);
  BW_CHECK(hipGetLastError());
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for((int64_t)E * DF / 2)), dim3(256), 0, st, (float*)b.zeros,
                     (int64_t)E * DF / 2, 0.0f);
  BW_CHECK(hipGetLastError());
  BW_CHECK(fork(st, sb, 0));
  // 3. (side) transposed, padded x and dz = g dout (operands of the weight gradients)
  hipLaunchKernelGGL((gather_transpose_kernel<true, false, false>), dim3(ldt / 64, blocks_for(D, 64)), dim3(256), 0,
                     sb, (const void*)b.x, D, D, b.padmap, b.perm, b.gates, k, A, ldt, b.xT);
  BW_CHECK(hipGetLastError());
  hipLaunchKernelGGL((gather_transpose_kernel<true, true, true>), dim3(ldt / 64, blocks_for(D, 64)), dim3(256), 0,
                     sb, (const void*)b.dout, D, D, b.padmap, b.perm, b.gates, k, A, ldt, b.dzT);
  BW_CHECK(hipGetLastError());
  // 4. (side) dout rows in routed order as bf16 pairs
  uint16_t* const dout_lo = b.dout_perm + (int64_t)A * D;
  hipLaunchKernelGGL(gather_dout_pair_kernel, dim3(blocks_for((int64_t)A * D / 4)), dim3(256), 0, sb,
                     (const float4*)b.dout, b.perm, A, k, D / 4, (uint2*)b.dout_perm, (uint2*)dout_lo);
  BW_CHECK(hipGetLastError());

  const int cfg = expert_tile_config(A, E);
  // 5. recompute u = x W1^T + b1 (the forward's mlp1, storing u)
  ExpertArgs f{};
  f.x = b.x; f.w1 = b.w1; f.b1 = b.b1; f.gates = b.gates; f.offsets = b.offsets; f.perm = b.perm;
  f.u_out = b.u; f.T = T; f.D = D; f.E = E; f.k = k; f.F = F; f.fmt = 0;
  BW_CHECK(launch_mlp1(f, cfg, st));
  BW_CHECK(fork(sb, st, 1));                // the dout pair (and the transposes) are written
  // 6. dh' = (dout hi + lo) W2 at the slot rows: the forward's mlp2 with K = D, N = F, reading
  // W2 [E][D][F] as stored, both parts of A against each staged tile of W2
  ExpertArgs m{};
  m.h = b.dout_perm; m.h_lo = dout_lo; m.w2 = b.w2; m.b2 = b.zeros; m.gates = b.ones; m.offsets = b.offsets;
  m.perm = b.perm; m.y = b.dxs; m.T = T; m.D = F; m.E = E; m.k = k; m.F = D; m.fmt = 0; m.w2_kn_rows = D;
  BW_CHECK(launch_mlp2(m, cfg, st));
  // 7. the SwiGLU backward: h, du, dg (dh' sits in dxs until step 8 overwrites it)
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)A), dim3(256), 0, st, b.u, b.dxs, b.perm, b.gates, A, F, b.h,
                     b.du, b.dgsum);
  BW_CHECK(hipGetLastError());
  BW_CHECK(fork(st, sb, 2));                // h, du and dg are written
  // 9. (side) transposed, padded h and du
  hipLaunchKernelGGL((gather_transpose_kernel<false, false, false>), dim3(ldt / 64, blocks_for(F, 64)), dim3(256), 0,
                     sb, (const void*)b.h, F, F, b.padmap, b.perm, b.gates, k, A, ldt, b.hT);
  BW_CHECK(hipGetLastError());
  hipLaunchKernelGGL((gather_transpose_kernel<false, false, false>), dim3(ldt / 64, blocks_for(G, 64)), dim3(256), 0,
                     sb, (const void*)b.du, G, G, b.padmap, b.perm, b.gates, k, A, ldt, b.duT);
  BW_CHECK(hipGetLastError());
  BW_CHECK(side ? hipEventRecord(side->ev[3], sb) : hipSuccess);
  // 11. (side) router: dg and the softmax backward, then the per-expert sums (read h, du,
  // dg, dout and x only)
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)T), dim3(256), 0, sb, b.dgsum, b.dout, b.b2, b.idx,
                     b.gates, T, D, E, k, b.dl);
  BW_CHECK(hipGetLastError());
  const unsigned wblk = blocks_for(G > D ? G : D);
  hipLaunchKernelGGL(expert_partial_kernel, dim3(wblk, E, EX_CHUNKS), dim3(256), 0, sb, b.offsets, b.perm, b.gates,
                     b.dl, b.x, b.dout, b.du, D, F, k, A, E, b.part_w, b.part_b2, b.part_b1);
  BW_CHECK(hipGetLastError());
  hipLaunchKernelGGL(expert_reduce_kernel, dim3(wblk, E), dim3(256), 0, sb, b.part_w, b.part_b2, b.part_b1, D, F, E,
                     b.dwr, b.db2, b.db1);
  BW_CHECK(hipGetLastError());
  hipLaunchKernelGGL(router_bias_grad_kernel, dim3(E), dim3(256), 0, sb, b.offsets, b.perm, b.dl, A, b.dbr);
  BW_CHECK(hipGetLastError());
  BW_CHECK(side ? hipEventRecord(side->ev[4], sb) : hipSuccess);
  // 8. dx contributions du W1[e] at the slot rows: the forward's mlp2 with K = 2F, N = D,
  // reading W1 [E][2F][D] as stored
  m.h = b.du; m.h_lo = nullptr; m.w2 = b.w1; m.y = b.dxs; m.D = D; m.F = G; m.w2_kn_rows = G;
  BW_CHECK(launch_mlp2(m, cfg, st));
  BW_CHECK(side ? hipStreamWaitEvent(st, side->ev[3], 0) : hipSuccess);   // hT, duT (and xT, dzT)
  // 10. weight gradients per expert: dW2[e] = dz^T h, dW1[e] = du^T x
  // (few rows per expert, the forward's streaming regime: tiles that are mostly stores)
  const bool small = cfg == 0;
  BwdGemmArgs w{};
  w.poff = b.poff; w.E = E;
  w.a = b.dzT; w.lda = ldt; w.b = b.hT; w.ldb = ldt; w.M = D; w.N = F; w.c = b.dw2;
  BW_CHECK(launch_wgrad(w, small, st));
  w.a = b.duT; w.b = b.xT; w.M = G; w.N = D; w.c = b.dw1;
  BW_CHECK(launch_wgrad(w, small, st));
  BW_CHECK(side ? hipStreamWaitEvent(st, side->ev[4], 0) : hipSuccess);   // dl, and the side's end
  // 12. dx
  hipLaunchKernelGGL(dx_combine_kernel, dim3(blocks_for((int64_t)T * D / 4)), dim3(256), 0, st, b.dxs, D, b.dl,
                     b.idx, b.wr, T, D, E, k, b.dx);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for(n)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace moe

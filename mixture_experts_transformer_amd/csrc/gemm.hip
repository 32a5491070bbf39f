// Expert stage of the GPT-OSS MoE block on gfx950: the two grouped GEMMs and the combine.
//
// torchtitan GPT-OSS guide, section "Grouped matrix multiplication": every expert's
// rows form one group delimited by the int32 cumulative counts, and each group is
// multiplied by its expert's weight stored (experts, out, in).  Here one launch covers
// all groups: the grid is a static upper bound on the number of (row tile, column tile)
// pairs (no host round trip on the counts) and each workgroup locates its expert and
// row range from the offsets, exiting when it is past the last tile.
//
//   mlp1: rows gathered from x through the permutation (token = assignment / k),
//         C = X_e . W1[e]^T + b1[e] over the G = 2F outputs; the tile pairs gate column f
//         with linear column F + f, so the GPT-OSS SwiGLU (gate clamped above at LIMIT,
//         times sigmoid(ALPHA * gate); linear clamped to [-LIMIT, LIMIT], plus one) is
//         applied in registers and only h [A][F] is written.
//   mlp2: C = H_e . W2[e]^T + b2[e], scaled by the assignment's gate weight and stored at
//         the assignment's slot row (t*k + j), so the combine reads a token's k rows
//         contiguously.
//   combine: out[t] = sum_j y[t*k + j] in slot order, fp32, no atomics.
//
// Matrix-core mapping: v_mfma_f32_16x16x32_bf16.  Operands are K-contiguous (rows of x,
// h and the weights), so each lane feeds the instruction with one 16-byte LDS read per
// operand: lane l supplies row l & 15 and K elements 8 (l >> 4) .. +7; output register r
// of lane l is C[4 (l >> 4) + r][l & 15].  Tiles are staged in LDS with the 16-byte chunks
// of each 128-byte row XOR-swizzled by (row & 7), so the eight rows a group of lanes
// reads land in eight different bank groups.  LDS is double buffered: the next K step is
// fetched into registers while the current one feeds the matrix cores, one barrier per
// K step.
//
// MXFP4 weights (GPT-OSS-in-Transformers blog, MXFP4 paragraph: E2M1 values, one scale
// per 32 elements) are decoded while a tile moves from registers to LDS with the gfx950
// conversion v_cvt_scalef32_pk_bf16_fp4 (two codes per instruction, low nibble first,
// multiplied by the block's power-of-two scale).  Every E2M1 value times 2^(s-127) with
// s in [2, 252] is an exact bf16, so the matrix cores see the weights without rounding.
// mlp1's inputs are bf16 and exact; h is written as a bf16 pair (hi + lo) and mlp2 runs
// both parts through the matrix cores against the same decoded weight tile, which keeps
// h at 16 significant bits where a single bf16 would cost the output its accuracy.
#include "moe_internal.h"

namespace moe {

constexpr float SWIGLU_ALPHA = 1.702f;
constexpr float SWIGLU_LIMIT = 7.0f;

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_;      // routed rows per tile
  static constexpr int BN = BN_;      // weight rows per tile (mlp1: gate + linear halves)
  static constexpr int BK = 64;       // K per pipeline step (2 MFMA K-steps of 32)
  static constexpr int WAVES_M = WM_;
  static constexpr int WAVES_N = WN_;
  static constexpr int THREADS = 64 * WM_ * WN_;
  static constexpr int WTM = BM / WM_;
  static constexpr int WTN = BN / WN_;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static_assert(BM % (16 * WM_) == 0 && BN % (16 * WN_) == 0, "tile/wave mismatch");
};

// Configuration 0: few rows per expert (weight streaming); 1: many rows (matrix-core bound).
using SmallTile = Tile<32, 64, 1, 2>;
using LargeTile = Tile<256, 192, 2, 2>;
using LargeTileHiLo = Tile<128, 192, 2, 2>;   // mlp2 with the two h parts

struct GemmArgs {
  const uint16_t* a;        // mlp1: x [T][K]; mlp2: h (hi) [A][K]
  const uint16_t* a_lo;     // mlp2 + MXFP4: h lo [A][K]
  const int32_t* perm;
  const int32_t* offsets;
  const float* gates;
  const uint8_t* w;         // weights (bf16 or MXFP4 buffer)
  const uint16_t* bias;     // [E][N]
  uint16_t* h;              // mlp1 output
  uint16_t* h_lo;
  float* y;                 // mlp2 output
  int E, k, K, N, F;
  int A;                    // routed rows (T * k)
  int n_tiles, max_m_tiles;
};

// ------------------------------------------------------------------------------ helpers
static __device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
static __device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Locate row tile m in the flat list of all experts' tiles (experts ascending, BM rows
// each, the last tile of an expert possibly partial).  Wave-wide: lane l looks at
// experts 4l..4l+3.  Returns false past the last tile.
template <int BM>
static __device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int m,
                                                 int& e_out, int& row0_out, int& cnt_out) {
  const int lane = threadIdx.x & 63;
  int tl[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    const int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    tl[i] = (c + BM - 1) / BM;
    s += tl[i];
  }
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  const int excl = incl - s;
  const uint64_t hit = __ballot(m >= excl && m < incl);
  if (hit == 0) return false;
  const int src = __ffsll((long long)hit) - 1;
  int e = -1, r0 = 0, base = excl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e < 0 && m < base + tl[i]) {
      e = lane * 4 + i;
      r0 = (m - base) * BM;
    }
    base += tl[i];
  }
  e_out = __shfl(e, src);
  row0_out = __shfl(r0, src);
  cnt_out = offsets[e_out + 1] - offsets[e_out];
  return true;
}

// LDS byte offset of 16-byte chunk c (0..7) of row r in a [rows][64 bf16] tile.  The chunk
// index is XOR-swizzled with (r & 7) ^ (r >> 3 & 1): the 16 rows that 16 lanes read with the
// same chunk index then occupy 16 distinct 16-byte bank groups whether the LDS serves 8 or
// 16 lanes of a 128-bit read per cycle.
static __device__ __forceinline__ int swz(int r, int c) {
  return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

// Decode 32 MXFP4 codes (16 bytes) with E8M0 byte s into 32 bf16 (four 16-byte chunks).
static __device__ __forceinline__ void decode_fp4x32(const u32x4 q, uint32_t s, u32x4 out[4]) {
  const float scale = __uint_as_float(s << 23);   // 2^(s-127), s in [1, 254]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = q[i];
    out[i] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3))};
  }
}

// ------------------------------------------------------------------------------ kernel
// MODE 1: mlp1 (+SwiGLU), MODE 2: mlp2 (+bias, gate).  FMT 0: bf16 weights, 1: MXFP4.
//
// Per-thread load assignment is fixed for the whole K loop: thread t moves 16-byte chunk
// t + i * THREADS of the A tile (row = chunk / 8, column chunk = chunk % 8) and likewise of
// the B tile, so a wave moves eight whole 128-byte row segments per instruction.  Sources
// are kept as 32-bit element offsets (or -1 for rows outside the group / columns outside
// the matrix, which load zeros) so nothing leaves registers.
template <int MODE, int FMT, class C>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TH = C::THREADS;
  constexpr int FM = C::FM, FN = C::FN;
  constexpr int AP = (MODE == 2 && FMT == 1) ? 2 : 1;      // A parts (h hi, h lo)
  constexpr int A_TILE = BM * BK * 2;                       // bytes per A part
  constexpr int B_TILE = BN * BK * 2;
  constexpr int STAGE = AP * A_TILE + B_TILE;
  constexpr int A_IT = BM * 8 / TH;                         // 16-byte chunks per thread per part
  static_assert(BM * 8 % TH == 0, "A chunks must divide evenly");
  constexpr int B_CH = (FMT == 0) ? BN * 8 : BN * 2;        // bf16: 8 chunks/row; fp4: 2 x 16 B codes/row
  constexpr int B_IT = (B_CH + TH - 1) / TH;
  constexpr int PN = BN / 2;                                // mlp1: pairs per tile
  constexpr int WP = PN / C::WAVES_N;                       // mlp1: pairs per wave

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;

  // ---- tile order: XCD-contiguous ranges of the linear id, then groups of GM row tiles
  const int nb = gridDim.x;                 // multiple of 8
  const int lin = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int total = p.max_m_tiles * p.n_tiles;
  if (lin >= total) return;
  constexpr int GM = 4;
  const int gsize = GM * p.n_tiles;
  const int g = lin / gsize;
  const int first_m = g * GM;
  const int gm = min(p.max_m_tiles - first_m, GM);
  const int m_tile = first_m + (lin % gsize) % gm;
  const int n_tile = (lin % gsize) / gm;

  int e, row0, cnt;
  if (!find_tile<BM>(p.offsets, p.E, m_tile, e, row0, cnt)) return;
  const int gbase = p.offsets[e] + row0;    // routed row of tile row 0
  const int rows = min(BM, cnt - row0);
  // a routing passed in by the caller is trusted only this far: rows stay inside [0, A)
  if (gbase < 0 || rows <= 0 || gbase + rows > p.A) return;
  const int K = p.K;
  const int nk = K / BK;

  // ---- per-thread sources: element offsets (A: from p.a / p.a_lo; B: from the expert's
  // weight block), -1 = zero fill
  int a_off[A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int ch = tid + i * TH;
    const int r = ch >> 3, c = ch & 7;
    a_off[i] = -1;
    if (r < rows) {
      if (MODE == 1) {
        const int asg = p.perm[gbase + r];
        if ((unsigned)asg < (unsigned)p.A) a_off[i] = (asg / p.k) * K + c * 8;
      } else {
        a_off[i] = (gbase + r) * K + c * 8;
      }
    }
  }
  int b_off[B_IT];   // bf16: element offset within the expert; fp4: byte offset of the codes
  int s_off[B_IT];   // fp4: byte offset of the scale byte within the expert's scales
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int ch = tid + i * TH;
    b_off[i] = -1;
    s_off[i] = 0;
    const int rr = (FMT == 0) ? (ch >> 3) : (ch >> 1);
    const int c = (FMT == 0) ? (ch & 7) : (ch & 1);
    int wrow;
    bool ok;
    if (MODE == 1) {
      const int q = rr < PN ? rr : rr - PN;
      const int f = n_tile * PN + q;
      ok = f < p.F;
      wrow = rr < PN ? f : p.F + f;
    } else {
      wrow = n_tile * BN + rr;
      ok = wrow < p.N;
    }
    if (ch < B_CH && ok) {
      if (FMT == 0) {
        b_off[i] = wrow * K + c * 8;
      } else {
        b_off[i] = wrow * (K / 2) + c * 16;
        s_off[i] = wrow * (K / 32) + c;
      }
    }
  }
  const uint16_t* a_base = p.a;
  const uint16_t* a_lo_base = p.a_lo;
  const uint8_t* w_e;        // expert e's weight block (bf16: [N][K]; fp4: codes [N][K/2])
  const uint8_t* s_e = nullptr;
  if (FMT == 0) {
    w_e = p.w + (size_t)e * p.N * K * 2;
  } else {
    w_e = p.w + (size_t)e * p.N * (K / 2);
    s_e = p.w + (size_t)p.E * p.N * (K / 2) + (size_t)e * p.N * (K / 32);
  }

  u32x4 ra[AP][A_IT];
  u32x4 rb[B_IT];
  uint32_t rs[B_IT];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B-tile row of this wave's fragment j
  int brow[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (MODE == 1)
      brow[j] = (j < FN / 2) ? wn * WP + j * 16 : PN + wn * WP + (j - FN / 2) * 16;
    else
      brow[j] = wn * C::WTN + j * 16;
    brow[j] += lane & 15;
  }
  const int arow0 = wm * C::WTM + (lane & 15);

#define MOE_LOAD_GLOBAL(kt)                                                                      \
  do {                                                                                           \
    _Pragma("unroll") for (int i = 0; i < A_IT; ++i) {                                           \
      ra[0][i] = a_off[i] >= 0 ? *(const u32x4*)(a_base + a_off[i] + (kt) * BK) : zero4;        \
      if (AP == 2)                                                                               \
        ra[AP - 1][i] = a_off[i] >= 0 ? *(const u32x4*)(a_lo_base + a_off[i] + (kt) * BK) : zero4; \
    }                                                                                            \
    _Pragma("unroll") for (int i = 0; i < B_IT; ++i) {                                           \
      if (FMT == 0) {                                                                            \
        rb[i] = b_off[i] >= 0 ? *(const u32x4*)(w_e + 2 * (b_off[i] + (kt) * BK)) : zero4;       \
      } else {                                                                                   \
        rb[i] = b_off[i] >= 0 ? *(const u32x4*)(w_e + b_off[i] + (kt) * (BK / 2)) : zero4;       \
        rs[i] = b_off[i] >= 0 ? (uint32_t)s_e[s_off[i] + (kt) * (BK / 32)] : 127u;              \
      }                                                                                          \
    }                                                                                            \
  } while (0)

#define MOE_STORE_LDS(stage)                                                                     \
  do {                                                                                           \
    uint8_t* sa_ = smem + (stage) * STAGE;                                                       \
    uint8_t* sb_ = sa_ + AP * A_TILE;                                                            \
    _Pragma("unroll") for (int pa = 0; pa < AP; ++pa)                                            \
    _Pragma("unroll") for (int i = 0; i < A_IT; ++i) {                                           \
      const int ch = tid + i * TH;                                                               \
      *(u32x4*)(sa_ + pa * A_TILE + swz(ch >> 3, ch & 7)) = ra[pa][i];                           \
    }                                                                                            \
    _Pragma("unroll") for (int i = 0; i < B_IT; ++i) {                                           \
      const int ch = tid + i * TH;                                                               \
      if (ch < B_CH) {                                                                           \
        if (FMT == 0) {                                                                          \
          *(u32x4*)(sb_ + swz(ch >> 3, ch & 7)) = rb[i];                                         \
        } else {                                                                                 \
          u32x4 d_[4];                                                                           \
          decode_fp4x32(rb[i], rs[i], d_);                                                       \
          _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
            *(u32x4*)(sb_ + swz(ch >> 1, (ch & 1) * 4 + j)) = d_[j];                             \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
  } while (0)

  MOE_LOAD_GLOBAL(0);
  MOE_STORE_LDS(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_LOAD_GLOBAL(kt + 1);
    const uint8_t* sa = smem + cur * STAGE;
    const uint8_t* sb = sa + AP * A_TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cc = ks * 4 + (lane >> 4);
      bf16x8 fa[AP][FM];
      bf16x8 fb[FN];
#pragma unroll
      for (int pa = 0; pa < AP; ++pa)
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[pa][i] = *(const bf16x8*)(sa + pa * A_TILE + swz(arow0 + i * 16, cc));
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = *(const bf16x8*)(sb + swz(brow[j], cc));
#pragma unroll
      for (int pa = 0; pa < AP; ++pa)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[pa][i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_STORE_LDS(cur ^ 1);
    __syncthreads();
  }
#undef MOE_LOAD_GLOBAL
#undef MOE_STORE_LDS

  // ---- epilogue
  const uint16_t* bias = p.bias + (size_t)e * p.N;
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * C::WTM + i * 16 + 4 * (lane >> 4) + r;
        if (rl >= rows) continue;
        const size_t prow = (size_t)(gbase + rl) * p.F;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int f = n_tile * PN + wn * WP + j * 16 + (lane & 15);
          if (f >= p.F) continue;
          const float ug = acc[i][j][r] + bf16_to_f32(bias[f]);
          const float ul = acc[i][j + FN / 2][r] + bf16_to_f32(bias[p.F + f]);
          const float gc = fminf(ug, SWIGLU_LIMIT);
          const float lc = fminf(fmaxf(ul, -SWIGLU_LIMIT), SWIGLU_LIMIT);
          const float hv = gc / (1.0f + __expf(-SWIGLU_ALPHA * gc)) * (lc + 1.0f);
          const uint32_t hi = f32_to_bf16_rne(hv);
          p.h[prow + f] = (uint16_t)hi;
          if (FMT == 1) p.h_lo[prow + f] = (uint16_t)f32_to_bf16_rne(hv - bf16_to_f32(hi));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * C::WTM + i * 16 + 4 * (lane >> 4) + r;
        if (rl >= rows) continue;
        const int a = p.perm[gbase + rl];
        if ((unsigned)a >= (unsigned)p.A) continue;
        const float gw = p.gates[a];
        float* yrow = p.y + (size_t)a * p.N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int o = n_tile * BN + wn * C::WTN + j * 16 + (lane & 15);
          if (o < p.N) yrow[o] = gw * (acc[i][j][r] + bf16_to_f32(bias[o]));
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ launchers
int expert_tile_config(int64_t A, int64_t E) {
  // average routed rows per expert decides between weight streaming and matrix-core tiles
  return (A >= 128 * E) ? 1 : 0;
}

template <class C>
static int max_m_tiles(int64_t A, int E) {
  int64_t m = (A + (int64_t)E * (C::BM - 1)) / C::BM;
  if (m > A) m = A;
  return (int)m;
}

template <int MODE, int FMT, class C>
static hipError_t launch_gemm(GemmArgs g, int64_t A, hipStream_t st) {
  g.max_m_tiles = max_m_tiles<C>(A, g.E);
  const int64_t total = (int64_t)g.max_m_tiles * g.n_tiles;
  const int64_t blocks = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((grouped_gemm_kernel<MODE, FMT, C>), dim3((unsigned)blocks), dim3(C::THREADS), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_mlp1(const ExpertArgs& a, int cfg, hipStream_t st) {
  GemmArgs g{};
  g.a = a.x; g.a_lo = nullptr; g.perm = a.perm; g.offsets = a.offsets; g.gates = a.gates;
  g.w = (const uint8_t*)a.w1; g.bias = a.b1; g.h = a.h; g.h_lo = a.h_lo; g.y = nullptr;
  g.E = a.E; g.k = a.k; g.K = a.D; g.N = 2 * a.F; g.F = a.F;
  const int64_t A = (int64_t)a.T * a.k;
  g.A = (int)A;
  if (cfg == 0) {
    g.n_tiles = (a.F + SmallTile::BN / 2 - 1) / (SmallTile::BN / 2);
    return a.fmt == 0 ? launch_gemm<1, 0, SmallTile>(g, A, st) : launch_gemm<1, 1, SmallTile>(g, A, st);
  }
  g.n_tiles = (a.F + LargeTile::BN / 2 - 1) / (LargeTile::BN / 2);
  return a.fmt == 0 ? launch_gemm<1, 0, LargeTile>(g, A, st) : launch_gemm<1, 1, LargeTile>(g, A, st);
}

hipError_t launch_mlp2(const ExpertArgs& a, int cfg, hipStream_t st) {
  GemmArgs g{};
  g.a = a.h; g.a_lo = a.h_lo; g.perm = a.perm; g.offsets = a.offsets; g.gates = a.gates;
  g.w = (const uint8_t*)a.w2; g.bias = a.b2; g.h = nullptr; g.h_lo = nullptr; g.y = a.y;
  g.E = a.E; g.k = a.k; g.K = a.F; g.N = a.D; g.F = a.F;
  const int64_t A = (int64_t)a.T * a.k;
  g.A = (int)A;
  if (cfg == 0) {
    g.n_tiles = (a.D + SmallTile::BN - 1) / SmallTile::BN;
    return a.fmt == 0 ? launch_gemm<2, 0, SmallTile>(g, A, st) : launch_gemm<2, 1, SmallTile>(g, A, st);
  }
  if (a.fmt == 0) {
    g.n_tiles = (a.D + LargeTile::BN - 1) / LargeTile::BN;
    return launch_gemm<2, 0, LargeTile>(g, A, st);
  }
  g.n_tiles = (a.D + LargeTileHiLo::BN - 1) / LargeTileHiLo::BN;
  return launch_gemm<2, 1, LargeTileHiLo>(g, A, st);
}

// ------------------------------------------------------------------------------ combine
__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ y, int T, int D4, int k,
                                                      float4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * D4) return;
  const int64_t t = i / D4;
  const int64_t c = i - t * D4;
  const float4* src = y + (t * k) * D4 + c;
  float4 s = src[0];
  for (int j = 1; j < k; ++j) {
    const float4 v = src[(int64_t)j * D4];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  out[i] = s;
}

hipError_t launch_combine(const float* y, int T, int D, int k, float* out, hipStream_t st) {
  const int D4 = D / 4;
  const int64_t n = (int64_t)T * D4;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const float4*)y, T, D4, k, (float4*)out);
  return hipGetLastError();
}

}  // namespace moe

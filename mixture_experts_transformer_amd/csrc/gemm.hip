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
// Matrix-core mapping: v_mfma_f32_32x32x16_bf16 on K-contiguous operands (rows of x, h
// and the weights); operand tiles reach LDS by direct global->LDS copies through a ring of
// stages, details at the kernel.
//
// MXFP4 weights (GPT-OSS-in-Transformers blog, MXFP4 paragraph: E2M1 values, one scale
// per 32 elements) take one of two routes.
//   Few rows per expert (weight streaming): the codes are decoded from LDS into bf16
//   matrix-core operands with v_cvt_scalef32_pk_bf16_fp4 (two codes per instruction, low
//   nibble first, times the block's power-of-two scale; every E2M1 value times 2^(s-127)
//   with s in [2, 252] is an exact bf16).  h is written as a bf16 pair (hi + lo) and mlp2
//   runs both parts against the same decoded tile, keeping h at 16 significant bits where
//   a single bf16 would cost the output its accuracy.
//   Many rows per expert (matrix-core tiles): the scaled instruction
//   v_mfma_scale_f32_32x32x64_f8f6f4 takes the codes as its fp4 B operand and the scale
//   bytes as its B scales unchanged; the activations enter as pieces with their own
//   block scales (x: two fp8 E4M3 pieces from the split kernel; h: three fp6 E2M3 pieces
//   written by mlp1's epilogue, which the instruction multiplies at the FP6/FP4 rate), so
//   no weight is ever decoded.
//
// MXFP8 weights (E4M3 elements with the same block scales; the torchtitan guide's grouped
// GEMM section names MXFP8 converters as users of the scaled grouped-GEMM seam) are
// decoded like MXFP4 ones, with v_cvt_scalef32_pk_bf16_fp8 (E4M3 has 3 mantissa bits: exact
// in bf16 for scale bytes in [10, 246]), on streaming tiles and on matrix-core tiles alike;
// h goes into mlp2 as a bf16 pair there too.
#include "device_common.h"

namespace moe {

constexpr float SWIGLU_ALPHA = 1.702f;
constexpr float SWIGLU_LIMIT = 7.0f;
constexpr float SWIGLU_NEG_ALPHA_LOG2E = -SWIGLU_ALPHA * 1.4426950408889634f;

template <int BM_, int BN_, int WM_, int WN_, int NS_, int BK_, bool STREAM_ = false, int SUPER_ = 4, int WPE_ = 1>
struct Tile {
  static constexpr int WPE = WPE_;    // waves per SIMD the register allocation must allow
  static constexpr bool STREAM = STREAM_;   // weight-streaming tile order
  static constexpr int BM = BM_;      // routed rows per tile
  static constexpr int BN = BN_;      // weight rows per tile (mlp1: gate + linear halves)
  static constexpr int BK = BK_;      // K per pipeline stage (32 or 64)
  static constexpr int CPR = BK_ / 8; // 16-byte chunks per bf16 row segment
  static constexpr int NS = NS_;      // LDS stages; NS - 1 K steps are in flight
  static constexpr int SUPER = SUPER_; // MXFP4: K steps per code super-stage (32 code bytes each)
  static constexpr int WAVES_M = WM_;
  static constexpr int WAVES_N = WN_;
  static constexpr int NW = WM_ * WN_;
  static constexpr int THREADS = 64 * NW;
  static constexpr int WTM = BM / WM_;
  static constexpr int WTN = BN / WN_;
  static constexpr int FM = WTM / 32;  // 32x32 output blocks per wave
  static constexpr int FN = WTN / 32;
  static_assert(BM % (32 * WM_) == 0 && BN % (32 * WN_) == 0, "tile/wave mismatch");
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(SUPER_ == 1 || SUPER_ == 2 || SUPER_ == 4, "code super-stage");
  static_assert((BM * CPR) % 64 == 0 && (BN * CPR) % 64 == 0, "copy granularity");
};

// Tile shapes (the measured choices).
//
// Streaming tiles serve few routed rows per expert, where the weights' HBM stream bounds the
// loop: 64 routed rows x 128 weight rows, four waves side by side along the weight rows, two
// LDS stages of K = 64 (full 128-byte bf16 row segments).  With decoded formats (MXFP4,
// MXFP8) the registers are capped for four waves per SIMD, which measured a few percent
// faster; SUPER, the K steps whose codes one copy brings in, is 4 for MXFP4 mlp1 (32-byte
// code segments) and 2 for MXFP4 mlp2 (three workgroups per CU) and for MXFP8 (64 code bytes
// per row and stage: 128-byte windows).
template <int MODE, int FMT> using SmallTile =
    Tile<64, 128, 1, 4, 2, 64, true, (FMT == 0 || FMT >= 4 || (FMT == 1 && MODE == 1)) ? 4 : 2,
         (FMT == 0 || FMT >= 4) ? 1 : 4>;

// Matrix-core tiles serve many routed rows per expert: 256 x 256 outputs on eight waves
// (2 x 4, 128 x 64 each), two LDS stages of K = 64.
template <int MODE, int FMT> struct LargeTileSel {   // bf16 weights
  using type = Tile<256, 256, 2, 4, 2, 64, false>;
};
// the scaled-MFMA engine (activation pieces x MXFP4); mlp2 reads three pieces of h per
// stage, so its code super-stage is halved to fit LDS
template <> struct LargeTileSel<1, 2> {
  using type = Tile<256, 256, 2, 4, 2, 64, false, 4>;
};
template <> struct LargeTileSel<2, 2> {
  using type = Tile<256, 256, 2, 4, 2, 64, false, 2>;
};
// MXFP8 decoded to bf16 (128-byte code windows: 64 KB of codes per 256 weight rows); mlp2's
// h arrives as a bf16 pair, so its tile takes 128 rows to fit
template <> struct LargeTileSel<1, 3> {
  using type = Tile<256, 256, 2, 4, 2, 64, false, 2>;
};
template <> struct LargeTileSel<2, 3> {
  using type = Tile<128, 256, 2, 4, 2, 64, false, 2>;
};
// bf16 weights stored [K][N] with A as a bf16 pair (the backward's dout W2^T): 128 rows, as above
template <> struct LargeTileSel<2, 5> {
  using type = Tile<128, 256, 2, 4, 2, 64, false>;
};
template <int MODE, int FMT> using LargeTile = typename LargeTileSel<MODE, FMT>::type;

struct GemmArgs {
  const uint16_t* a;        // mlp1: x [T][K]; mlp2: h (hi) [A][K]
  const uint16_t* a_lo;     // mlp2 + MXFP4: h lo [A][K]
  const uint8_t* a8;        // scaled-MFMA engine: pieces of the A rows per 64-wide K stage
                            //   (x: fp8 [K/64][2][64], 128 bytes; h: fp6, 144 bytes as in mlp1's epilogue)
  const uint32_t* a8s;      //   and their scales [rows][a8s_stride] (piece p in byte p)
  int a8s_stride;           //   scale dwords per row (K / 32 rounded up to a multiple of 8)
  const int32_t* perm;
  const int32_t* offsets;
  const float* gates;
  const uint8_t* w;         // weights (bf16 or MXFP4 buffer)
  const uint16_t* bias;     // [E][N]
  uint16_t* h;              // mlp1 output
  float* u_out;             // mlp1, bf16 weights: when set, the pre-activation u [A][2F] (fp32,
                            //   gate half then linear half) is stored instead of h
  uint16_t* h_lo;
  uint8_t* h8;              // mlp1 output for the scaled-MFMA engine: three fp6 pieces of h
  uint32_t* h8s;            //   and their scales
  int h8s_stride;
  float* y;                 // mlp2 output
  int bt_rows;              // kernel format 4 (bf16 weights stored [rows][N], N contiguous): rows
                            //   per expert; K step k reads stored row k mod bt_rows
  int E, k, K, N, F;
  int A;                    // routed rows (T * k)
  int n_tiles, max_m_tiles;
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Transposing LDS read (ds_read_b64_tr_b16, gfx950), lane layout measured on the GPU: in
// each group of 16 lanes, lane s loads 4 consecutive 16-bit values from its own address and
// lane i of the group receives value i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
// With lane s of a group addressing stored row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3 of a
// [K][N] tile, lane i receives column c0 + i of rows r0 .. r0 + 3: four K values of one
// output column, as the matrix instruction's B operand wants them.
static __device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Direct global -> LDS copies.  They are written as inline assembly: the copies have no
// register results, their completion is waited for explicitly (vmcnt) before the barrier
// that publishes a stage, and a copy the compiler can see makes it treat every later LDS
// read as unordered and wait for all of them before the first use.  M0 carries the
// wave's LDS destination; lane L lands at M0 + size * L.  The compiler treats M0 as
// reserved and does not preserve it around the asm; that is sound because nothing else in
// these kernels uses M0 (tests/test_build.py checks the generated code for other uses).
// Saving and restoring it in the asm measured up to 12 % slower.
// Both are wave-uniform by construction; reading them from the first lane keeps them in
// scalar registers where the compiler cannot prove uniformity itself.
static __device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}
static __device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// The source is a wave-uniform base (scalar registers) plus a per-lane 32-bit byte offset,
// which keeps one vector register per copy slot instead of two.
// 16 bytes per lane: lane L fills LDS bytes [dst + 16 L, +16) from base + off.
// The LDS destination is a wave-uniform LDS byte address (kept as an integer: converting a
// generic pointer costs a null check per copy).
static __device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t dst_wave) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(dst_wave)), "v"(off), "s"(uniform_ptr(base))
               : "memory", "m0");
}
// The same with the non-temporal hint: for data read once whose every byte of a line is
// copied at once (streaming tiles: line-aligned bf16 weight rows and 128-byte code windows),
// so it does not displace what the L2 reuses (measured: streaming MXFP4 mlp1 -2 %; with
// 64-byte windows, whose line's other half is the next window, +8 %; the matrix-core tiles
// re-read weight tiles through the L2, +0.7 %).
static __device__ __forceinline__ void dma16_nt(const void* base, uint32_t off, uint32_t dst_wave) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(__builtin_amdgcn_readfirstlane(dst_wave)), "v"(off), "s"(uniform_ptr(base))
               : "memory", "m0");
}
// s_waitcnt vmcnt(N) with the LDS/export counters left alone (gfx9 encoding).
template <int N>
static __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
static __device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (0x7 << 4) | (0 << 8));
}
// Workgroup barrier without a memory fence: the waits above say what must have landed.
// The empty asm statements keep the compiler from moving memory accesses across it.
static __device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MXFP4 code super-stage in LDS: [rows][CCH 16-byte chunks], chunk c of row r stored at
// position c ^ code_swz(r), so the rows that one fragment read touches spread over the banks.
template <int CCH>
static __device__ __forceinline__ int code_swz(int r) {
  if (CCH == 8) return r & 7;
  if (CCH == 4) return (r >> 2) & 3;
  return (r >> 3) & 1;
}

// Decode 8 MXFP4 codes (one dword: element 2i in the low nibble of byte i) times the
// power-of-two scale into one bf16x8 matrix-core operand.
// Decode 8 MXFP8 codes (E4M3, element i in byte i of c0 c1) times a power-of-two scale:
// E4M3 has 3 mantissa bits, so with the scale bytes of the contract every value is an
// exact normal bf16.
static __device__ __forceinline__ bf16x8 decode_fp8x8(uint32_t c0, uint32_t c1, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, scale, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

static __device__ __forceinline__ bf16x8 decode_fp4x8(uint32_t codes, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// fp8 pieces (OCP E4M3: 3 mantissa bits, exponent bias 7, largest finite 448) of values
// that share one E8M0 scale per 32-element block.  The piece scale for a block whose
// largest remaining magnitude is m is the smallest power of two 2^(e - 127) with
// m / 2^(e - 127) <= 448, so no value rounds past the fp8 range: with m = 1.f 2^x,
// 2^(x - 8) maps m into [256, 512), and one more halving is needed when 1.f > 1.75.
static __device__ __forceinline__ int mx_scale_exp(float m) {
  if (!(m > 0.f)) return 0;                 // all-zero block (scale 2^-127)
  const uint32_t mb = __float_as_uint(m);
  const int x = (int)(mb >> 23) - 127;
  const int q = x - 8 + ((mb & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return min(max(q + 127, 0), 254);
}
static __device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(254 - e) << 23); }
static __device__ __forceinline__ float mx_scale(int e) {
  return e ? __uint_as_float((uint32_t)e << 23) : __uint_as_float(0x00400000u);   // 2^-127 is subnormal
}
// Four values times inv rounded to fp8 (nearest even), packed in order into one dword; when
// `residual`, what the codes represent (times scl) is subtracted from the values.
static __device__ __forceinline__ uint32_t mx_piece4(float* v, float inv, float scl, bool residual) {
  int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0, false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, pk, true);
  if (residual) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
    v[0] -= lo[0] * scl;
    v[1] -= lo[1] * scl;
    v[2] -= hi[0] * scl;
    v[3] -= hi[1] * scl;
  }
  return (uint32_t)pk;
}

// fp6 pieces (OCP E2M3: 3 mantissa bits, exponent bias 1, no infinity or NaN, largest 7.5,
// subnormal step 1/8) of h for the scaled engine's mlp2.  The scale for a block whose largest
// remaining magnitude is m = 1.f 2^x is the smallest power of two with m / 2^s <= 7.5:
// s = x - 2, one more when 1.f > 1.875.  It is kept at or above 2^-119 so that the scale and
// every decoded value stay normal fp32 (a block that small contributes nothing the output can
// hold), and an all-zero block takes 2^0.
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
static __device__ __forceinline__ int e2m3_scale_exp(float m) {
  if (!(m > 0.f)) return 127;
  const uint32_t mb = __float_as_uint(m);
  const int q = (int)(mb >> 23) - 2 + ((mb & 0x7FFFFFu) > 0x700000u ? 1 : 0);
  return min(max(q, 8), 254);
}
// v_cvt_scalef32_2xpk16_fp6_f32 (gfx950), measured on the GPU: code 2i is s0[i] / scale and
// code 2i + 1 is s1[i] / scale, each rounded to the nearest E2M3 value (ties to even), packed
// at bits 6 i of the six result dwords.  The instruction writes its result while it still
// reads its sources, so the result must not share their registers (early clobber); as inline
// assembly its neighbours get no hazard padding from the compiler, hence the s_nop on each side.
static __device__ __forceinline__ u32x6 fp6_encode32(f32x16 s0, f32x16 s1, float scale) {
  u32x6 r;
  asm("s_nop 1\n\tv_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3\n\ts_nop 1"
      : "=&v"(r) : "v"(s0), "v"(s1), "v"(scale));
  return r;
}
// v_cvt_scalef32_pk32_f32_fp6: value i = E2M3 code i (bits 6 i) times scale, exactly.
static __device__ __forceinline__ f32x32 fp6_decode32(u32x6 c, float scale) {
  f32x32 r;
  asm("s_nop 1\n\tv_cvt_scalef32_pk32_f32_fp6 %0, %1, %2\n\ts_nop 1" : "=&v"(r) : "v"(c), "v"(scale));
  return r;
}
// Three E2M3 pieces of this lane's 16 values v (one half of a 32-element block whose other
// half is in lane ^ 1): codes[pc] holds piece pc's 16 codes (value i at bits 6 i), byte pc of
// the result its E8M0 scale; piece pc rounds what the earlier ones left.  v is consumed.
static __device__ __forceinline__ uint32_t fp6_pieces16(float* v, uint32_t (*codes)[3]) {
  uint32_t sc = 0;
#pragma unroll
  for (int pc = 0; pc < 3; ++pc) {
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) m = fmaxf(m, fabsf(v[u]));
    m = fmaxf(m, __shfl_xor(m, 1));
    const int se = e2m3_scale_exp(m);
    sc |= (uint32_t)se << (8 * pc);
    const float scl = __uint_as_float((uint32_t)se << 23);
    f32x16 s0, s1;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      s0[u] = u < 8 ? v[2 * u] : 0.f;
      s1[u] = u < 8 ? v[2 * u + 1] : 0.f;
    }
    const u32x6 c = fp6_encode32(s0, s1, scl);
    codes[pc][0] = c[0];
    codes[pc][1] = c[1];
    codes[pc][2] = c[2];
    if (pc < 2) {
      const f32x32 d = fp6_decode32(c, scl);
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] -= d[u];
    }
  }
  return sc;
}

// ------------------------------------------------------------------------------ kernel
// s_waitcnt needs an immediate: dispatch a wave-uniform count to the matching wait.
static __device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define MOE_W(k) case k: wait_vmcnt<k>(); break;
    MOE_W(0) MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7)
    MOE_W(8) MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15)
    MOE_W(16) MOE_W(17) MOE_W(18) MOE_W(19) MOE_W(20) MOE_W(21) MOE_W(22) MOE_W(23)
    MOE_W(24) MOE_W(25) MOE_W(26) MOE_W(27) MOE_W(28) MOE_W(29) MOE_W(30) MOE_W(31)
    MOE_W(32) MOE_W(33) MOE_W(34) MOE_W(35) MOE_W(36) MOE_W(37) MOE_W(38) MOE_W(39)
    MOE_W(40) MOE_W(41) MOE_W(42) MOE_W(43) MOE_W(44) MOE_W(45) MOE_W(46) MOE_W(47)
#undef MOE_W
    default: wait_vmcnt<0>(); break;
  }
}

// MODE 1: mlp1 (+SwiGLU), MODE 2: mlp2 (+bias, gate), MODE 3: the backward's per-expert
// weight gradients (bf16 operands both K-contiguous, K an expert's padded rows, fp32 out).
// FMT 0: bf16 weights, 1: MXFP4.
//
// Matrix-core mapping: v_mfma_f32_32x32x16_bf16 (measured on gfx950 at about twice the
// sustained rate of the 16x16x32 form).  In MFMA step ks of a stage, lane l feeds row
// l & 31 and the 8 K elements  g BK/2 + 8 ks .. +7  (g = l >> 5) of each operand: each lane
// half covers one contiguous half of the stage's K range.  Output register r of lane l is
// C[8 (r >> 2) + 4 g + (r & 3)][l & 31].
//
// Pipeline: K advances BK at a time through an NS-stage ring in LDS, filled by direct
// global->LDS copies (no registers) issued NS-1 steps before use.  Before consuming a stage
// every wave waits until its own copies for it have landed (vmcnt counts, in issue order,
// exactly the copies issued after them) and the workgroup meets at a fence-free barrier,
// which also frees the stage consumed in the previous step.  Inside a stage the operand
// fragments of MFMA step ks + 1 are read while step ks multiplies, and the last step of a
// stage multiplies after the next stage's barrier, so LDS latency hides behind the
// matrix cores.
//
// bf16 stage: rows x BK with 16-byte chunks; copy instruction i fills LDS bytes
// [1024 i, +1024), lane L landing at row 1024 i / (16 CPR) + L / CPR, swizzle position
// L % CPR.  Rows past the group's end or the matrix edge copy a valid row (their results
// are never stored).
//
// MXFP4 B: full 128-byte row segments are what HBM serves efficiently, and one stage's
// codes are only 32 bytes per row, so the codes have their own ring of two super-stages of
// four stages (128 code bytes = 256 K elements per row, 16-byte chunks XOR-swizzled by
// row & 7).  A super-stage's copies are issued just before the group of its first stage,
// so that group's completion implies the codes'.  Each stage also copies, per row, the
// aligned dword holding the stage's two scale bytes.
//
// Epilogue: each wave moves its outputs through its own slice of the (then idle) LDS,
// 32 rows at a time, so that global stores are whole 8-byte (h) or 16-byte (y) chunks of
// rows instead of one element per lane.
template <int MODE, int FMT, class C>
__global__ __launch_bounds__(C::THREADS, C::WPE) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, CPR = C::CPR, NS = C::NS, NW = C::NW;
  // formats 4 and 5: bf16 weights stored [K][N] (N contiguous), staged as such and read into
  // the matrix-core operand with transposing LDS reads; otherwise as format 0.  Format 5 takes
  // A as a bf16 pair (a + a_lo), both parts against each staged weight tile.
  constexpr bool BT = FMT == 4 || FMT == 5;
  constexpr int WF = BT ? 0 : FMT;
  constexpr int FM = C::FM, FN = C::FN;
  constexpr bool MX = FMT == 2;                             // scaled MFMA on fp8/fp6 pieces
  // its A operand format: E4M3 (0) for the pieces of x in mlp1, E2M3 (2) for those of h in mlp2
  constexpr int ACB = MODE == 2 ? 2 : 0;
  constexpr bool DEC = FMT == 1 || FMT == 3;                // codes decoded to bf16 (MXFP4, MXFP8)
  constexpr int CBS = FMT == 3 ? 64 : 32;                   // code bytes per row and stage
  constexpr int KS = MX ? 1 : BK / 16;                      // MFMA K steps per stage
  // A parts: bf16 (1), h hi + lo (2), or pieces (x: 2 fp8, h: 3 fp6)
  constexpr int AP = MX ? (MODE == 1 ? 2 : 3) : ((MODE == 2 && (DEC || FMT == 5)) ? 2 : 1);
  constexpr int ROWB = CPR * 16;                            // bytes per bf16 row segment
  constexpr int APL = MX ? 1 : AP;                          // A parts in LDS (pieces share rows)
  // scaled engine, mlp2: h as three fp6 pieces packed into 144 bytes per row and stage (24
  // bytes per piece and K half)
  constexpr bool HC = MX && MODE == 2;
  constexpr int A_CPR = MX ? (HC ? 9 : 4 * AP) : CPR;     // 16-byte chunks per A row per stage
  constexpr int A_ROWB = A_CPR * 16;
  constexpr int A_CPC = BM * A_CPR / 64;                    // A copies per part and stage
  constexpr int A_BYTES = BM * A_ROWB;                      // per A part per stage
  static_assert((BM * A_CPR) % 64 == 0, "A stage must tile the copy instructions");
  static_assert(WF == 0 || BK == 64, "MXFP4 staging assumes 64-wide K steps");
  constexpr int SUPER = C::SUPER;                           // stages per MXFP4 code super-stage
  constexpr int NSB = 2;                                    // code super-stage slots
  // a slot is refilled NS - 1 steps ahead of its first use, after the barrier that ends
  // the last use of its previous super-stage
  static_assert(WF == 0 || SUPER * (NSB - 1) > NS - 2, "code ring too short for the stage ring");
  constexpr int CROW = CBS * SUPER;                         // code bytes per row per super-stage
  constexpr int CCH = CROW / 16;                            // 16-byte code chunks per row
  constexpr int B_STAGE_BYTES = (WF == 0) ? BN * ROWB : 0;  // bf16 B tile (MXFP4: none)
  constexpr int STAGE = APL * A_BYTES + B_STAGE_BYTES;
  constexpr int CODE_SLOT = BN * CROW;
  constexpr int CODE_BYTES = (WF != 0) ? NSB * CODE_SLOT : 0;
  constexpr int ROWS_PER_CP = 1024 / ROWB;                  // bf16 B rows per copy instruction
  constexpr int NA = APL * A_CPC;                           // per stage: A copies
  constexpr int NBS = (WF == 0) ? BN / ROWS_PER_CP : 0;    // per stage: B copies
  constexpr int NG = NA + NBS;                              // copies per stage group
  constexpr int NC = (WF != 0) ? BN * CROW / 1024 : 0;     // copies per code super-stage
  // scaled-MFMA engine: A scale dwords (two per row and stage) in a ring of super-stages
  // beside the codes, 8 SUPER bytes per row, chunks swizzled by row bit 3
  constexpr int ASL_ROW = MX ? 8 * SUPER : 16;
  constexpr int ASL_SLOT = BM * ASL_ROW;
  constexpr int ASL_BYTES = MX ? NSB * ASL_SLOT : 0;
  constexpr int NASC = MX ? BM * ASL_ROW / 1024 : 0;        // A scale copies per super-stage
  // MXFP4 weight scales travel per super-stage, beside the A scales: per row and super-stage
  // the 16 bytes that end at the 4-aligned address at or past the earlier of the super-stage's
  // last scale byte and the row's last one (a super-stage needs 2 SUPER <= 8 of them, so the
  // record covers them; stopping at the row keeps the last row's records inside the weight
  // buffer, whose size is a multiple of 4); one copy covers 64 rows
  constexpr int SCW_SLOT = (WF != 0) ? BN * 16 : 0;
  constexpr int SCW_BYTES = NSB * SCW_SLOT;
  constexpr int NSW = (WF != 0) ? BN / 64 : 0;             // scale copies per window
  constexpr int NCT = NC + NASC + NSW;
  static_assert(WF == 0 || (SUPER % 2 == 0 && SUPER <= 4), "scale records: even windows of <= 8 scale bytes");
  // with four-stage code super-stages the K loop is unrolled over one, which makes the
  // stage slot and the super-stage boundaries compile-time constants (measured: a few
  // percent there; elsewhere it costs registers, spills in the three-piece mlp2 tile)
  constexpr int UNR = (WF != 0 && SUPER >= 4 && SUPER % NS == 0) ? SUPER : 1;
  // Code windows aligned to their own size (64 or 128 bytes per row): each row's windows
  // start at the boundary at or below its codes (a row starts 32 s bytes past one when its
  // length is not a multiple of the window), so every 64-byte sector or 128-byte line is
  // fetched by one window instead of two.  Row r's stage kt then sits at position
  // kt + s(r) of the row's window sequence.  The windows need their own issue schedule
  // (below), which fits a two-stage ring.
  constexpr bool WALIGN = WF != 0 && (CROW == 64 || CROW == 128) && NS == 2;
  static_assert(!MX || (SUPER >= 2 && 1024 % ASL_ROW == 0), "A scale super-stage granularity");
  constexpr int PW_G = (NG + NW - 1) / NW;
  constexpr int PW_C = (NCT + NW - 1) / NW + (NCT == 0 ? 1 : 0);
  constexpr int PN = BN / 2;                                // mlp1: pairs per tile
  static_assert(BN % 32 == 0 && (BM * CPR) % 64 == 0 && (BN * CPR) % 64 == 0, "copy granularity");
  static_assert(WF == 0 || BN % 64 == 0, "scale copies cover 64 rows");

  constexpr int SMEM = NS * STAGE + CODE_BYTES + ASL_BYTES + SCW_BYTES;
  // epilogue slices (per wave, 32 output rows): mlp1 bf16 [32][pairs] (+ lo part), row
  // stride 2 P + 8 bytes so the four 16-lane groups of one store hit disjoint banks; mlp2
  // fp32 [32][WTN], row stride 4 WTN + 32 bytes so the two lane halves hit disjoint banks
  constexpr int EP_P = C::WTN / 2;
  // (scaled-MFMA engine, mlp1: fp32 [32][32 pairs], one MXFP8 block of h per row)
  constexpr int EP_S = (MODE == 1) ? (MX ? 4 * EP_P + 16 : 2 * EP_P + 8) : 4 * C::WTN + 32;
  constexpr int EP_REG = 32 * EP_S * ((MODE == 1 && DEC) ? 2 : 1);
  static_assert(!(MX && MODE == 1) || EP_P % 32 == 0, "whole 32-element blocks of h per wave and row");
  static_assert(MODE != 3 || (FMT == 0 && !C::STREAM), "weight gradients: bf16 matrix-core tiles");
  static_assert(NW * EP_REG <= SMEM, "epilogue slices exceed the operand ring");
  constexpr int ROWTAB = (MODE >= 2) ? BM * 8 : 0;          // mlp2: assignment and gate per tile row
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM + ROWTAB];
  uint8_t* const codes_lds = smem + NS * STAGE;
  uint8_t* const ascale_lds = codes_lds + CODE_BYTES;       // scaled-MFMA engine: A scales
  uint8_t* const wsc_lds = ascale_lds + ASL_BYTES;          // MXFP4 weight scale windows
  // the same regions as LDS byte addresses, for the copies
  const uint32_t smem_l = lds_addr(smem);
  const uint32_t codes_l = smem_l + NS * STAGE;
  const uint32_t ascale_l = codes_l + CODE_BYTES;
  const uint32_t wsc_l = ascale_l + ASL_BYTES;
  int* const tab_a = (int*)(smem + SMEM);
  float* const tab_g = (float*)(smem + SMEM + BM * 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;

  // ---- tile order over the tiles that exist (the grid is an upper bound).  The workgroups
  // of XCD x (block ids congruent to x mod 8) take the x-th eighth of the tiles, so each
  // XCD's L2 holds the A rows of only its own experts (streaming tiles: measured mlp2 -5 %
  // at T = 256, where all of h does not fit one L2) and every XCD gets an equal share
  // however many row tiles the routing produced.  Streaming tiles (few rows per expert):
  // column tiles fastest, so workgroups launched together read neighbouring rows of one
  // expert's weights.  Large tiles: in groups of GM row tiles, so the workgroups sharing an
  // XCD's L2 share operand tiles.
  int m_tile, n_tile;
  int e, row0, cnt;
  if constexpr (MODE == 3) {
    // weight gradients: per expert (in the order of decreasing K that offsets[E + 1 ..]
    // lists) max_m_tiles row tiles of the M output rows by n_tiles column tiles, in block
    // order, so the largest experts' tiles go first and spread over every XCD; in groups of
    // GM row tiles so neighbouring workgroups share operand rows
    const int mt = p.max_m_tiles;
    const int total = p.E * mt * p.n_tiles;
    const int lin = blockIdx.x;
    if (lin >= total) return;
    constexpr int GM = 4;
    const int gsize = GM * p.n_tiles;
    const int g = lin / gsize;
    const int first_m = g * GM;
    const int gm = min(p.E * mt - first_m, GM);
    m_tile = first_m + (lin % gsize) % gm;
    n_tile = (lin % gsize) / gm;
    e = p.offsets[p.E + 1 + m_tile / mt];
    if ((unsigned)e >= (unsigned)p.E) return;
    row0 = (m_tile % mt) * BM;
    cnt = p.A;
  } else {
  const TileScan ts = tile_scan<BM>(p.offsets, p.E);
  const int total = ts.total * p.n_tiles;
  if (C::STREAM) {
    const int share = (total + 7) >> 3;
    const int xl = blockIdx.x >> 3;
    const int lin = (blockIdx.x & 7) * share + xl;
    if (xl >= share || lin >= total) return;
    m_tile = lin / p.n_tiles;
    n_tile = lin % p.n_tiles;
  } else {
    const int share = (total + 7) >> 3;
    const int xl = blockIdx.x >> 3;
    const int lin = (blockIdx.x & 7) * share + xl;
    if (xl >= share || lin >= total) return;
    // row tiles per group: 1 for the forward's mlp2 (bf16 and scaled engine), the backward's
    // products of the same kind (formats 4, 5) and the scaled engine's mlp1, whose column
    // tiles of one row tile then run side by side and read each stage of its A rows as one
    // (measured: mlp2 C3 -4.5 %, X2 -2 %, C5 -1 %; scaled mlp1 X2 -3.8 %, C5 -0.9 %; C3
    // backward -0.7 %); 8 for the bf16 mlp1 (C3 -1.3 % against 4; +3 % with 1, +1.5 % with 2,
    // -1 % with 16); 4 elsewhere
    constexpr int GM = ((MODE == 2 && FMT != 3) || (MODE == 1 && FMT == 2)) ? 1
                       : (MODE == 1 && FMT == 0) ? 8 : 4;
    const int gsize = GM * p.n_tiles;
    const int g = lin / gsize;
    const int first_m = g * GM;
    const int gm = min(ts.total - first_m, GM);
    m_tile = first_m + (lin % gsize) % gm;
    n_tile = (lin % gsize) / gm;
  }

  if (!tile_lookup<BM>(ts, p.offsets, m_tile, e, row0, cnt)) return;
  }
  // routed row of tile row 0 (weight gradients: output row)
  const int gbase = MODE == 3 ? row0 : p.offsets[e] + row0;
  const int rows = min(BM, cnt - row0);
  // a routing passed in by the caller is trusted only this far: rows stay inside [0, A)
  if (gbase < 0 || rows <= 0 || gbase + rows > p.A) return;
  const int K = p.K;                        // weight gradients: the operands' row stride
  // weight gradients: K is the expert's padded row count, its columns from offsets[e]
  const int kcol0 = MODE == 3 ? p.offsets[e] : 0;
  const int nk = MODE == 3 ? (p.offsets[e + 1] - kcol0) / BK : K / BK;
  // mlp2: thread r < rows fetches tile row r's assignment now and its gate in the first K
  // step, for the epilogue (which then needs no dependent global loads)
  int rt_a = -1;
  float rt_g = 0.f;
  if (MODE == 2 && tid < rows) {
    const int a = p.perm[gbase + tid];
    rt_a = ((unsigned)a < (unsigned)p.A) ? a : -1;
  }
  if (MODE == 3 && tid < rows) {            // output row of expert e's gradient, unit scale
    rt_a = e * p.A + gbase + tid;
    rt_g = 1.f;
  }

  // A row behind tile row r (clamped into the group): mlp1 gathers token rows, mlp2 reads
  // the routed rows in place
  auto a_row = [&](int r) -> size_t {
    const int rc = min(r, rows - 1);
    if (MODE == 1) {
      int asg = p.perm[gbase + rc];
      asg = ((unsigned)asg < (unsigned)p.A) ? asg : 0;
      return (size_t)(asg / p.k);
    }
    return (size_t)(gbase + rc);
  };

  const uint8_t* w_e;
  size_t s_e_off = 0;                       // byte offset of expert e's scales in p.w
  if (BT) {
    w_e = p.w + (size_t)e * p.bt_rows * p.N * 2;
  } else if (MODE == 3) {
    w_e = p.w + (size_t)kcol0 * 2;
  } else if (WF == 0) {
    w_e = p.w + (size_t)e * p.N * K * 2;
  } else {
    w_e = p.w + (size_t)e * p.N * (K / 64 * CBS);
    s_e_off = (size_t)p.E * p.N * (K / 64 * CBS) + (size_t)e * p.N * (K / 32);
  }
  // scale records: offsets relative to 32 bytes before the expert's scales (a record can
  // start up to 24 bytes before a row's first scale byte)
  const uint8_t* const scbase = p.w + s_e_off - 32;
  const int s_al = (int)(s_e_off & 3);
  // code-window shift of a weight row (in 32-byte stages), 0 unless the buffer is aligned
  // to the window; windows start below the row, so copies are relative to w_e - CROW
  const bool walign = WALIGN && (((uintptr_t)p.w) & (CROW - 1)) == 0;
  // bf16 weight rows are whole 128-byte lines per stage when the buffer is line-aligned (K is
  // a multiple of 64); streaming tiles read each once and copy them with the non-temporal
  // hint, which keeps the A rows that every column tile re-reads in the L2 (measured at
  // T = 256: mlp1 -8 %, mlp2 -9 %)
  const bool wlines = WF == 0 && (((uintptr_t)p.w) & 127) == 0;
  const int bt_kt = BT ? p.bt_rows / 64 : 1;  // format 4: K steps before the stored rows repeat
  const size_t w_e_off = (size_t)(w_e - p.w);
  const uint8_t* const wbase = WALIGN ? w_e - CROW : w_e;
#define MOE_CSHIFT(wr) (walign ? (int)(((w_e_off + (size_t)(wr) * (K / 64 * CBS)) / CBS) & (SUPER - 1)) : 0)
  // start of super-stage w's 16-byte scale record of a row whose scales are [rs, re)
  // (offsets relative to the expert's scales): the super-stage's bytes end at
  // rs + 2 SUPER (w + 1), the record at the 4-aligned address at or past the earlier end
#define MOE_SCW_START(rs, re, w)                                                                 \
  ([&]() {                                                                                       \
    const int e_ = min((int)(rs) + 2 * SUPER * ((w) + 1), (int)(re));                            \
    return e_ + ((4 - ((s_al + e_) & 3)) & 3) - 16;                                              \
  }())
  // tile row -> weight row, clamped into the matrix.  mlp1 tiles interleave the halves in
  // 16-row groups: rows 32 j .. 32 j + 15 are gate rows of pairs 16 j .. 16 j + 15 and rows
  // 32 j + 16 .. 32 j + 31 the linear rows of the same pairs, so every 32-column output
  // fragment holds matching gate and linear columns in lanes n and n + 16.
#define MOE_WROW(rr)                                                                             \
  (MODE == 1 ? ((((rr) & 16) ? p.F : 0) + min(n_tile * PN + ((rr) >> 5) * 16 + ((rr) & 15), p.F - 1)) \
             : min(n_tile * BN + (rr), p.N - 1))

  // ---- this wave's copy slots: global byte source for K step 0 and LDS offset
  // source offsets relative to the slot kind's base: A rows (x, h, h lo or pieces), the
  // expert's bf16 weight rows, or the 4-aligned start of the expert's scale bytes
  uint32_t goff[PW_G];
  int gdst[PW_G];
#pragma unroll
  for (int j = 0; j < PW_G; ++j) {
    const int i = wave + j * NW;
    goff[j] = 0;
    gdst[j] = 0;
    if (i < NA) {
      const int part = i / A_CPC;
      const int ii = i % A_CPC;
      const int idx = ii * 64 + lane;                      // chunk of the part's stage tile
      const int r = idx / A_CPR;
      const int c = swz_pos<A_CPR>(r, idx % A_CPR);        // logical chunk at this position
      if (MX) {
        goff[j] = (uint32_t)(a_row(r) * (size_t)(HC ? 9 * K / 4 : AP * K) + c * 16);
      } else {
        goff[j] = (uint32_t)((a_row(r) * K + c * 8) * 2);
      }
      gdst[j] = part * A_BYTES + ii * 1024;
    } else if (i < NG) {
      const int ii = i - NA;
      if (BT) {
        // stored rows of the stage's 64 K values, BN columns each (16-byte chunks XOR-swizzled
        // by 4 (row & 3), so the transposing reads of four rows hit disjoint banks); columns
        // past the matrix edge copy valid ones (never stored)
        constexpr int RCH = BN / 8;
        const int r = ii * (64 / RCH) + lane / RCH;
        const int c = (lane % RCH) ^ (4 * (r & 3));
        goff[j] = (uint32_t)(((size_t)r * p.N + min(n_tile * BN + 8 * c, p.N - 8)) * 2);
        gdst[j] = APL * A_BYTES + ii * 1024;
      } else if (WF == 0) {
        const int r = ii * ROWS_PER_CP + lane / CPR;
        const int c = swz_pos<CPR>(r, lane % CPR);
        goff[j] = (uint32_t)(((size_t)MOE_WROW(r) * K + c * 8) * 2);
        gdst[j] = APL * A_BYTES + ii * 1024;
      }
    }
  }
  uint32_t coff[PW_C];                      // codes, A scales (window 0); weight scale rows: rs
  int cdst[PW_C];
  int cre[PW_C];                            // weight scale rows: re
#pragma unroll
  for (int j = 0; j < PW_C; ++j) {
    const int i = wave + j * NW;
    coff[j] = 0;
    cdst[j] = 0;
    cre[j] = 0;
    if (WF != 0 && i < NC) {
      const int r = i * (1024 / CROW) + lane / CCH;
      const int c = (lane % CCH) ^ code_swz<CCH>(r);
      const int wr = MOE_WROW(r);
      coff[j] = (uint32_t)((size_t)wr * (K / 64 * CBS) + (WALIGN ? CROW - CBS * MOE_CSHIFT(wr) : 0) + c * 16);
      cdst[j] = i * 1024;
    } else if (i < NC + NASC) {
      constexpr int CPS = ASL_ROW / 16;                    // chunks per row
      const int r = (i - NC) * (1024 / ASL_ROW) + lane / CPS;
      const int c = (lane % CPS) ^ (CPS > 1 ? (r >> 3) & (CPS - 1) : 0);
      coff[j] = (uint32_t)((a_row(r) * (size_t)p.a8s_stride + c * 4) * 4);
      cdst[j] = (i - NC) * 1024;
    } else if (i < NCT) {
      const int r = (i - NC - NASC) * 64 + lane;           // lane = weight row of the tile
      const int wr = MOE_WROW(r);
      coff[j] = (uint32_t)(wr * (K / 32));
      cre[j] = (wr + 1) * (K / 32);
      cdst[j] = (i - NC - NASC) * 1024;
    }
  }

  // every copy this wave issues is counted; mark[slot] = count right after the stage group
  // that filled the slot, so the wait for a stage is exact: vmcnt completes in issue order.
  // Both are wave-uniform (the wave index is read from the first lane).
  int issued = 0;
  int mark[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) mark[q] = 0;

#define MOE_ISSUE_GROUP(kt, slot)                                                                \
  do {                                                                                           \
    _Pragma("unroll") for (int j = 0; j < PW_G; ++j) {                                           \
      const int i_ = wave + j * NW;                                                              \
      if (i_ < NG && !(i_ < NA && (i_ % A_CPC) * 64 / A_CPR >= rows)) {                         \
        const uint32_t d_ = smem_l + (slot) * STAGE + gdst[j];                                   \
        if (i_ < NA) {                                                                           \
          const void* ab_ = MX ? (const void*)p.a8                                               \
                                : (i_ < A_CPC ? (const void*)(p.a + kcol0) : (const void*)p.a_lo); \
          dma16((const uint8_t*)ab_ + (size_t)(kt) * A_ROWB, goff[j], d_);                       \
        } else {                                                                                 \
          const uint8_t* ws_ = BT ? w_e + (size_t)((kt) % bt_kt) * 64 * p.N * 2                  \
                                  : w_e + (size_t)(kt) * ROWB;                                   \
          if (C::STREAM && wlines) dma16_nt(ws_, goff[j], d_);                                   \
          else dma16(ws_, goff[j], d_);                                                          \
        }                                                                                        \
        ++issued;                                                                                \
      }                                                                                          \
    }                                                                                            \
  } while (0)
// code window w of the tile's rows into slot w % NSB
#define MOE_ISSUE_WIN(w)                                                                         \
  do {                                                                                           \
    _Pragma("unroll") for (int j = 0; j < PW_C; ++j) {                                           \
      const int i_ = wave + j * NW;                                                              \
      if (WF != 0 && i_ < NC) {                                                                 \
        if (CROW == 128 && C::STREAM && walign)   /* whole lines, read once */                  \
          dma16_nt(wbase + (size_t)(w) * CROW, coff[j], codes_l + ((w) % NSB) * CODE_SLOT + cdst[j]); \
        else                                                                                     \
          dma16(wbase + (size_t)(w) * CROW, coff[j], codes_l + ((w) % NSB) * CODE_SLOT + cdst[j]); \
        ++issued;                                                                                \
      }                                                                                          \
    }                                                                                            \
  } while (0)
// the scales of super-stage sk: weight scale records, and A scales (scaled-MFMA engine)
#define MOE_ISSUE_ASC(sk)                                                                        \
  do {                                                                                           \
    _Pragma("unroll") for (int j = 0; j < PW_C; ++j) {                                           \
      const int i_ = wave + j * NW;                                                              \
      if (i_ >= NC && i_ < NC + NASC && ((i_ - NC) * (1024 / ASL_ROW)) < rows) {                 \
        dma16((const uint8_t*)p.a8s + (size_t)(sk) * ASL_ROW, coff[j],                           \
              ascale_l + ((sk) % NSB) * ASL_SLOT + cdst[j]);                                     \
        ++issued;                                                                                \
      } else if (i_ >= NC + NASC && i_ < NCT) {                                                  \
        dma16(scbase, (uint32_t)(MOE_SCW_START((int)coff[j], cre[j], sk) + 32),                  \
              wsc_l + ((sk) % NSB) * SCW_SLOT + cdst[j]);                                        \
        ++issued;                                                                                \
      }                                                                                          \
    }                                                                                            \
  } while (0)
  // everything a K step needs, codes first so the group's completion implies theirs.
  // Aligned code windows go out one window ahead instead: window w (stages S w - s .. of a
  // row with shift s, S = SUPER) right after the barrier of stage S (w - 1), when window
  // w - 2's slot is free, ahead of the group of stage S (w - 1) + 1, its first use.
#define MOE_ISSUE(kt)                                                                            \
  do {                                                                                           \
    if (WF != 0 && (kt) % SUPER == 0) {                                                         \
      if (!WALIGN) MOE_ISSUE_WIN((kt) / SUPER);                                                  \
      MOE_ISSUE_ASC((kt) / SUPER);                                                               \
    }                                                                                            \
    MOE_ISSUE_GROUP(kt, (kt) % NS);                                                              \
    mark[(kt) % NS] = issued;                                                                    \
  } while (0)
  const int nwin = (nk + SUPER - 2) / SUPER + 1;   // aligned windows any row needs
  // Wait for a stage's copies.  With two stages nothing is issued between the group of
  // the stage about to be consumed and this wait, so it is a plain vmcnt(0) (no count
  // dispatch on the scalar unit).
#define MOE_WAIT_STAGE(slot_)                                                                    \
  do {                                                                                           \
    if (NS == 2) wait_vmcnt<0>();                                                                \
    else wait_vmcnt_dyn(__builtin_amdgcn_readfirstlane(issued - mark[slot_]));                   \
  } while (0)
#define MOE_ISSUE_NEXT_WIN(kt)                                                                   \
  do {                                                                                           \
    if (WALIGN && (kt) % SUPER == 0 && (kt) / SUPER + 1 < nwin) MOE_ISSUE_WIN((kt) / SUPER + 1); \
  } while (0)

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int kg = lane >> 5;                 // which half of the stage's K range this lane feeds
  // B-tile row of this lane for fragment j
  int brow[FN];
  int csh[FN];                              // code-window shift of the fragment row
  int sidx[FN];                             // scale ring byte of the fragment row's first stage
                                            //   of a super-stage (K block kg), in slot 0
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    brow[j] = wn * C::WTN + j * 32 + (lane & 31);
    csh[j] = 0;
    sidx[j] = 0;
    if (WALIGN) csh[j] = MOE_CSHIFT(MOE_WROW(brow[j]));
    if (WF != 0) {
      const int rs = MOE_WROW(brow[j]) * (K / 32);
      sidx[j] = brow[j] * 16 + rs - MOE_SCW_START(rs, 1 << 30, 0) + kg;
    }
  }
  // the last super-stage's records stop at the row's end, so its bytes sit further into
  // the record: move the fragments' scale bytes there when it starts
  const int sk_last = (nk - 1) / SUPER;
#define MOE_SCALE_LAST(kt_)                                                                      \
  do {                                                                                           \
    if (WF != 0 && (kt_) == SUPER * sk_last) {                                                  \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                           \
        const int rs_ = MOE_WROW(brow[j]) * (K / 32);                                            \
        sidx[j] += MOE_SCW_START(rs_, 1 << 30, sk_last) - MOE_SCW_START(rs_, rs_ + K / 32, sk_last); \
      }                                                                                          \
    }                                                                                            \
  } while (0)
  // this lane's scale byte of fragment j for stage kt (K block kg) in the scale ring
#define MOE_SCALE_AT(kt_, j_)                                                                    \
  ((uint32_t)wsc_lds[(((kt_) / SUPER) % NSB) * SCW_SLOT + sidx[j_] + 2 * ((kt_) % SUPER)])
  // this lane's 32 codes of fragment j for stage kt in the code ring: 16-byte chunk h_ of
  // them (MXFP4: one chunk; MXFP8: two)
#define MOE_CODES_AT(kt_, j_, h_)                                                                \
  ([&]() {                                                                                       \
    const int t_ = (kt_) + csh[j_];                                                              \
    const int c_ = (CBS / 16) * (t_ % SUPER) + (CBS / 32) * kg + (h_);                           \
    return codes_lds + ((t_ / SUPER) % NSB) * CODE_SLOT + brow[j_] * CROW +                      \
           ((c_ ^ code_swz<CCH>(brow[j_])) << 4);                                               \
  }())
  const int arow0 = wm * C::WTM + (lane & 31);

  // prologue: NS - 1 stages in flight
  if (WALIGN) MOE_ISSUE_WIN(0);
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < nk) MOE_ISSUE(s0);

  // double-buffered operand fragments: buffer ks & 1 feeds MFMA step ks
  bf16x8 fa[2][AP][FM];
  bf16x8 fb[2][FN];
  u32x4 q4[FN];                             // MXFP4: this lane's 32 codes per fragment
  u32x4 q8[FN];                             // MXFP8: the second 16 of them (q4 the first)
  float scl[FN];
#define MOE_LOAD_FRAGS(buf, ks_, sa_, sb_, FA)                                                   \
  do {                                                                                           \
    const int cc_ = kg * KS + (ks_);        /* chunk (8 K elements) this lane feeds */           \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                             \
      if (BT) {                                                                                  \
        const int s_ = lane & 15;                                                                \
        const int col_ = wn * C::WTN + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (s_ & 3);           \
        const uint8_t* p_ = (sb_) + (32 * kg + 8 * (ks_) + (s_ >> 2)) * (2 * BN) +              \
                            ((((col_ >> 3) ^ (4 * (s_ >> 2))) << 4) | ((col_ & 7) * 2));         \
        const i16x4 t0_ = lds_read_tr16(p_);                                                     \
        const i16x4 t1_ = lds_read_tr16(p_ + 4 * (2 * BN));                                      \
        fb[buf][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0_, t1_, 0, 1, 2, 3, 4, 5, 6, 7)); \
      } else if (WF == 0) fb[buf][j] = *(const bf16x8*)((sb_) + swz<CPR>(brow[j], cc_));         \
      else if (FMT == 3) fb[buf][j] = (ks_) < 2 ? decode_fp8x8(q4[j][2 * (ks_)], q4[j][2 * (ks_) + 1], scl[j]) \
                                    : decode_fp8x8(q8[j][2 * (ks_) - 4], q8[j][2 * (ks_) - 3], scl[j]); \
      else fb[buf][j] = decode_fp4x8(q4[j][ks_], scl[j]);                                        \
    }                                                                                            \
    _Pragma("unroll") for (int pa = 0; pa < AP; ++pa)                                            \
    _Pragma("unroll") for (int i = 0; i < (FA); ++i)                                             \
      fa[buf][pa][i] = *(const bf16x8*)((sa_) + pa * A_BYTES + swz<CPR>(arow0 + i * 32, cc_));    \
  } while (0)
#define MOE_MMA(buf, FA, ACC)                                                                    \
  do {                                                                                           \
    _Pragma("unroll") for (int i = 0; i < (FA); ++i)                                             \
    _Pragma("unroll") for (int pa = 0; pa < AP; ++pa)                                            \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                               \
      ACC[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][pa][i], fb[buf][j], ACC[i][j], 0, 0, 0); \
  } while (0)
  // one scheduling group per MFMA step: the next step's LDS reads ahead of this step's MFMAs
#define MOE_SCHED(FA)                                                                            \
  do {                                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x100, (WF == 0 ? (BT ? 2 : 1) * FN : 0) + AP * (FA), 0); \
    __builtin_amdgcn_sched_group_barrier(0x008, AP * (FA) * FN, 0);                              \
  } while (0)

  // Matrix-core tiles: a stage's row copies go out between the previous stage's deferred
  // matrix instructions instead of in one burst after the barrier, so the matrix pipe works
  // while the copies queue for the CU's memory path (each 1 KB copy holds it ~16 cycles).
  constexpr bool ILV = !C::STREAM && NS == 2;
#define MOE_COPY_SLOT(kt_, j_)                                                                   \
  do {                                                                                           \
    const int i_ = wave + (j_) * NW;                                                             \
    if (i_ < NG && !(i_ < NA && (i_ % A_CPC) * 64 / A_CPR >= rows)) {                           \
      const uint32_t d_ = smem_l + ((kt_) % NS) * STAGE + gdst[j_];                              \
      if (i_ < NA) {                                                                             \
        const void* ab_ = MX ? (const void*)p.a8                                                 \
                             : (i_ < A_CPC ? (const void*)(p.a + kcol0) : (const void*)p.a_lo);  \
        dma16((const uint8_t*)ab_ + (size_t)(kt_) * A_ROWB, goff[j_], d_);                       \
      } else {                                                                                   \
        const uint8_t* ws_ = BT ? w_e + (size_t)((kt_) % bt_kt) * 64 * p.N * 2                   \
                                : w_e + (size_t)(kt_) * ROWB;                                    \
        dma16(ws_, goff[j_], d_);                                                                \
      }                                                                                          \
    }                                                                                            \
  } while (0)
// the K loop for FA active 32-row fragment rows per wave (the rest are padding), into ACC
#define MOE_MAIN_LOOP(FA, ACC)                                                                   \
  do {                                                                                           \
    for (int kt0 = 0; kt0 < nk; kt0 += UNR) {                                                    \
    _Pragma("unroll") for (int u_ = 0; u_ < UNR; ++u_) {                                         \
      const int kt = kt0 + u_;                                                                   \
      if (kt >= nk) break;                                                                       \
      const int slot = UNR > 1 ? u_ % NS : kt % NS;                                              \
      MOE_WAIT_STAGE(slot);                                                                      \
      wait_lgkmcnt0();                                                                           \
      barrier_nofence();                                                                         \
      if (MODE == 2 && kt == 0 && rt_a >= 0) rt_g = p.gates[rt_a];                               \
      MOE_ISSUE_NEXT_WIN(kt);                                                                    \
      if (kt + NS - 1 < nk) {                                                                    \
        if (!ILV) {                                                                              \
          MOE_ISSUE(kt + NS - 1);                                                                \
        } else if (WF != 0 && (kt + NS - 1) % SUPER == 0) {  /* codes, scales; rows below */     \
          if (!WALIGN) MOE_ISSUE_WIN((kt + NS - 1) / SUPER);                                     \
          MOE_ISSUE_ASC((kt + NS - 1) / SUPER);                                                  \
        }                                                                                        \
      }                                                                                          \
                                                                                                 \
      const uint8_t* sa = smem + slot * STAGE;                                                   \
      const uint8_t* sb = sa + AP * A_BYTES;                                                     \
      if (DEC) {                                                                                 \
        if (UNR == 1 || u_ == 0) MOE_SCALE_LAST(kt);                                             \
  _Pragma("unroll")                                                                              \
        for (int j = 0; j < FN; ++j) {                                                           \
          q4[j] = *(const u32x4*)MOE_CODES_AT(kt, j, 0);                                         \
          if (FMT == 3) q8[j] = *(const u32x4*)MOE_CODES_AT(kt, j, 1);                           \
          const uint32_t sc = MOE_SCALE_AT(kt, j);                                               \
          scl[j] = __uint_as_float(sc << 23);                                                    \
        }                                                                                        \
      }                                                                                          \
      MOE_LOAD_FRAGS(0, 0, sa, sb, FA);                                                          \
      if (ILV) {                                                                                 \
        /* the previous stage's last MFMA step, the next stage's copies in between */            \
        const bool cp_ = kt + 1 < nk;                                                            \
        _Pragma("unroll") for (int m_ = 0; m_ < AP * (FA) * FN || m_ < PW_G; ++m_) {             \
          if (m_ < AP * (FA) * FN && kt > 0) {                                                   \
            const int i_ = m_ / (AP * FN), pa_ = (m_ / FN) % AP, j_ = m_ % FN;                    \
            ACC[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                               \
                fa[(KS - 1) & 1][pa_][i_], fb[(KS - 1) & 1][j_], ACC[i_][j_], 0, 0, 0);          \
          }                                                                                      \
          if (m_ < PW_G) {                                                                       \
            __builtin_amdgcn_sched_barrier(0);                                                   \
            if (cp_) MOE_COPY_SLOT(kt + 1, m_);                                                  \
            __builtin_amdgcn_sched_barrier(0);                                                   \
          }                                                                                      \
        }                                                                                        \
      } else if (kt > 0) {                                                                       \
        MOE_MMA((KS - 1) & 1, FA, ACC);     /* last MFMA step of the previous stage */           \
      }                                                                                          \
      MOE_SCHED(FA);                                                                             \
  _Pragma("unroll")                                                                              \
      for (int ks = 0; ks < KS - 1; ++ks) {                                                      \
        MOE_LOAD_FRAGS((ks + 1) & 1, ks + 1, sa, sb, FA);                                        \
        MOE_MMA(ks & 1, FA, ACC);                                                                \
        MOE_SCHED(FA);                                                                           \
      }                                                                                          \
    }                                                                                            \
    }                                                                                            \
    if (nk > 0) MOE_MMA((KS - 1) & 1, FA, ACC);                                                  \
  } while (0)
  // scaled-MFMA engine: the A pieces of row block i_ (this lane's row, its two chunks per
  // piece; fp6 pieces of h: the 24 bytes of the piece for this lane's K half, the operand's
  // six dwords, in three 8-byte reads) from the stage at sa
#define MX_LOAD_A(dst, i_)                                                                       \
  do {                                                                                           \
    _Pragma("unroll") for (int pa = 0; pa < AP; ++pa) {                                          \
      const int r_ = arow0 + 32 * (i_);                                                          \
      if (HC) {                                                                                  \
        const uint8_t* f_ = sa + r_ * A_ROWB + 72 * kg + 24 * pa;                                \
        const i32x2 d0_ = *(const i32x2*)(f_);                                                   \
        const i32x2 d1_ = *(const i32x2*)(f_ + 8);                                               \
        const i32x2 d2_ = *(const i32x2*)(f_ + 16);                                              \
        const i32x4 d01_ = __builtin_shufflevector(d0_, d1_, 0, 1, 2, 3);                        \
        const i32x4 d2x_ = __builtin_shufflevector(d2_, d2_, 0, 1, -1, -1);                      \
        (dst)[pa] = __builtin_shufflevector(d01_, d2x_, 0, 1, 2, 3, 4, 5, -1, -1);               \
      } else {                                                                                   \
        const i32x4 lo_ = *(const i32x4*)(sa + swz<A_CPR>(r_, 2 * AP * kg + 2 * pa));            \
        const i32x4 hi_ = *(const i32x4*)(sa + swz<A_CPR>(r_, 2 * AP * kg + 2 * pa + 1));        \
        (dst)[pa] = __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7);                   \
      }                                                                                          \
    }                                                                                            \
  } while (0)
  // the scale dword of this lane's row and K block holds piece pa's scale in byte pa,
  // which op_sel selects
#define MX_MMA(ACC, i_, FA, FB, SA, SB)                                                               \
  do {                                                                                           \
    _Pragma("unroll") for (int pa = 0; pa < AP; ++pa)                                            \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                             \
      if (pa == 0)                                                                               \
        ACC[i_][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                             \
            (FA)[pa], (FB)[j], ACC[i_][j], ACB, 4, 0, (int)(SA), 0, (int)(SB)[j]);                  \
      else if (pa == 1)                                                                          \
        ACC[i_][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                             \
            (FA)[pa], (FB)[j], ACC[i_][j], ACB, 4, 1, (int)(SA), 0, (int)(SB)[j]);                  \
      else                                                                                       \
        ACC[i_][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                             \
            (FA)[pa], (FB)[j], ACC[i_][j], ACB, 4, 2, (int)(SA), 0, (int)(SB)[j]);                  \
    }                                                                                            \
  } while (0)
  if constexpr (!MX) {
    // Row blocks of 32 past the tile's rows hold only padding: their copies (above) and
    // matrix instructions are skipped.  When every wave's rows of a streaming tile fit in its
    // first block, that loop accumulates into an array of its own, so the unused block is not
    // carried through it.
    if (C::WAVES_M == 1 && FM == 2 && rows <= 32) {
      f32x16 acc1[1][FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc1[0][j][q] = 0.f;
      MOE_MAIN_LOOP(1, acc1);
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[0][j] = acc1[0][j];
    } else if (FM == 4 && rows - wm * C::WTM <= 3 * 32) {
      // the tile's last rows: this wave multiplies only the 32-row blocks that hold some
      // (at least one), as the full tile's loop does in every other respect
      const int wrows = rows - wm * C::WTM;
      if (wrows > 64) MOE_MAIN_LOOP(FM >= 3 ? 3 : FM, acc);
      else if (wrows > 32) MOE_MAIN_LOOP(FM >= 2 ? 2 : FM, acc);
      else MOE_MAIN_LOOP(1, acc);
    } else {
      MOE_MAIN_LOOP(FM, acc);
    }
  } else {
    // Scaled matrix-core engine, one 64-wide K step per stage.  Per stage a lane loads its B
    // codes and scale bytes and the A scale dwords of its row blocks, then the A pieces one
    // row block ahead of the block it multiplies.  The last row block of a stage multiplies
    // after the next stage's barrier, behind that stage's first loads.
#define MX_LOOP(FA, ACC)                                                                         \
  do {                                                                                           \
    i32x8 fap[AP], fbp[FN];                 /* deferred operands of the previous stage */        \
    uint32_t sap, sbp[FN];                                                                       \
    for (int kt0 = 0; kt0 < nk; kt0 += UNR) {                                                    \
    _Pragma("unroll") for (int u_ = 0; u_ < UNR; ++u_) {                                         \
      const int kt = kt0 + u_;                                                                   \
      if (kt >= nk) break;                                                                       \
      const int slot = UNR > 1 ? u_ % NS : kt % NS;                                              \
      MOE_WAIT_STAGE(slot);                                                                      \
      wait_lgkmcnt0();                                                                           \
      barrier_nofence();                                                                         \
      if (MODE == 2 && kt == 0 && rt_a >= 0) rt_g = p.gates[rt_a];                               \
      MOE_ISSUE_NEXT_WIN(kt);                                                                    \
      if (kt + NS - 1 < nk) {                                                                    \
        if (!ILV) {                                                                              \
          MOE_ISSUE(kt + NS - 1);                                                                \
        } else if ((kt + NS - 1) % SUPER == 0) {  /* the scales now, the rows below */           \
          if (!WALIGN) MOE_ISSUE_WIN((kt + NS - 1) / SUPER);                                     \
          MOE_ISSUE_ASC((kt + NS - 1) / SUPER);                                                  \
        }                                                                                        \
      }                                                                                          \
      const uint8_t* sa = smem + slot * STAGE;                                                   \
      const uint8_t* sas = ascale_lds + ((kt / SUPER) % NSB) * ASL_SLOT;                         \
      const uint8_t* sb = sa + A_BYTES;                                                          \
      i32x8 fb[FN];                                                                              \
      uint32_t sbv[FN];                                                                          \
      if (UNR == 1 || u_ == 0) MOE_SCALE_LAST(kt);                                               \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                           \
        const i32x4 q = *(const i32x4*)MOE_CODES_AT(kt, j, 0);                                      \
        fb[j] = __builtin_shufflevector(q, q, 0, 1, 2, 3, -1, -1, -1, -1);                       \
        sbv[j] = MOE_SCALE_AT(kt, j);                                                            \
      }                                                                                          \
      uint32_t sav[FA];                                                                          \
      const int dw = (kt % SUPER) * 2 + kg;  /* scale dword of this stage and K block */         \
      _Pragma("unroll") for (int i = 0; i < (FA); ++i) {                                         \
        const int r = arow0 + 32 * i;                                                            \
        const int pos = (dw >> 2) ^ (ASL_ROW > 16 ? (r >> 3) & (ASL_ROW / 16 - 1) : 0);          \
        sav[i] = *(const uint32_t*)(sas + r * ASL_ROW + pos * 16 + (dw & 3) * 4);                \
      }                                                                                          \
      i32x8 fa[2][AP];                                                                           \
      MX_LOAD_A(fa[0], 0);                                                                       \
      if (ILV) {                                                                                 \
        /* the previous stage's last row block, this stage's row copies in between */            \
        const bool cp_ = kt + NS - 1 < nk;                                                       \
        _Pragma("unroll") for (int m_ = 0; m_ < AP * FN || m_ < PW_G; ++m_) {                    \
          if (m_ < AP * FN && kt > 0) {                                                          \
            const int pa = m_ / FN, j = m_ % FN;                                                 \
            if (pa == 0)                                                                         \
              ACC[(FA) - 1][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                \
                  fap[pa], fbp[j], ACC[(FA) - 1][j], ACB, 4, 0, (int)sap, 0, (int)sbp[j]);         \
            else if (pa == 1)                                                                    \
              ACC[(FA) - 1][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                \
                  fap[pa], fbp[j], ACC[(FA) - 1][j], ACB, 4, 1, (int)sap, 0, (int)sbp[j]);         \
            else                                                                                 \
              ACC[(FA) - 1][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                \
                  fap[pa], fbp[j], ACC[(FA) - 1][j], ACB, 4, 2, (int)sap, 0, (int)sbp[j]);         \
          }                                                                                      \
          if (m_ < PW_G) {                                                                       \
            __builtin_amdgcn_sched_barrier(0);                                                   \
            if (cp_) MOE_COPY_SLOT(kt + NS - 1, m_);                                             \
            __builtin_amdgcn_sched_barrier(0);                                                   \
          }                                                                                      \
        }                                                                                        \
      } else if (kt > 0) {                                                                       \
        MX_MMA(ACC, (FA) - 1, fap, fbp, sap, sbp);                                               \
      }                                                                                          \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * FN + (FA) + 2 * AP, 0);                    \
      __builtin_amdgcn_sched_group_barrier(0x008, AP * FN, 0);                                   \
      _Pragma("unroll") for (int i = 0; i + 1 < (FA); ++i) {                                     \
        MX_LOAD_A(fa[(i + 1) & 1], i + 1);                                                       \
        MX_MMA(ACC, i, fa[i & 1], fb, sav[i], sbv);                                              \
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AP, 0);                                  \
        __builtin_amdgcn_sched_group_barrier(0x008, AP * FN, 0);                                 \
      }                                                                                          \
      _Pragma("unroll") for (int pa = 0; pa < AP; ++pa) fap[pa] = fa[((FA) - 1) & 1][pa];        \
      sap = sav[(FA) - 1];                                                                       \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                           \
        fbp[j] = fb[j];                                                                          \
        sbp[j] = sbv[j];                                                                         \
      }                                                                                          \
    }                                                                                            \
    }                                                                                            \
    MX_MMA(ACC, (FA) - 1, fap, fbp, sap, sbp);                                                   \
  } while (0)
    // as above: padding row blocks of a single-block group are skipped
    if (C::WAVES_M == 1 && FM == 2 && rows <= 32) {
      f32x16 acc1[1][FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc1[0][j][q] = 0.f;
      MX_LOOP(1, acc1);
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[0][j] = acc1[0][j];
    } else if (MODE == 1 && FM == 4 && rows - wm * C::WTM <= 32) {
      // a tile's last rows, at most one 32-row block in this wave's share (more variants, or
      // this one in the three-piece mlp2 loop, would not fit the registers)
      MX_LOOP(1, acc);
    } else {
      MX_LOOP(FM, acc);
    }
#undef MX_LOOP
  }
#undef MX_LOAD_A
#undef MX_MMA
#undef MOE_MAIN_LOOP
#undef MOE_COPY_SLOT
#undef MOE_LOAD_FRAGS
#undef MOE_MMA
#undef MOE_SCHED
#undef MOE_ISSUE
#undef MOE_ISSUE_GROUP
#undef MOE_ISSUE_WIN
#undef MOE_ISSUE_ASC
#undef MOE_ISSUE_NEXT_WIN
#undef MOE_WAIT_STAGE
#undef MOE_CODES_AT
#undef MOE_CSHIFT
#undef MOE_SCW_START
#undef MOE_SCALE_AT
#undef MOE_SCALE_LAST
#undef MOE_WROW

  // ---- epilogue.  Output register q of fragment (i, j) is row 8 (q >> 2) + 4 kg + (q & 3)
  // of the fragment's 32 rows, column lane & 31.
  if (MODE >= 2 && tid < BM) {
    tab_a[tid] = rt_a;
    tab_g[tid] = rt_g;
  }
  // copies still in flight (a code window issued for shifted rows that this tile has
  // none of) must land before the ring's memory becomes the epilogue slices
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  barrier_nofence();                        // every wave is done with the operand ring
  uint8_t* const ep = smem + wave * EP_REG;
  const uint16_t* bias = MODE == 3 ? nullptr : p.bias + (size_t)e * p.N;
  if (MODE == 1) {
    // Lane n < 16 of a fragment holds the gate column of pair 16 j + n, lane n + 16 the
    // linear column of the same pair.  v_permlane16_swap of registers q and q + 8 exchanges
    // odd 16-lane rows of the first with even rows of the second: afterwards a gate lane
    // holds (gate, linear) of register q's row and a linear lane those of register q + 8's,
    // so each lane evaluates SwiGLU for eight of the fragment's sixteen rows.
    const bool gate_lane = (lane & 16) == 0;
    const int rlane = 4 * kg + (gate_lane ? 0 : 16);      // row offset of this lane's results
    const int pl = lane & 15;
    const int f_wave = n_tile * PN + wn * EP_P;            // first pair of this wave
    float bg[FN], bl[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int f = f_wave + j * 16 + pl;
      bg[j] = (f < p.F) ? bf16_to_f32(bias[f]) : 0.f;
      bl[j] = (f < p.F) ? bf16_to_f32(bias[p.F + f]) : 0.f;
    }
    constexpr int CH = EP_P / 4;                           // 8-byte chunks per slice row
    if constexpr (FMT == 0) {
      if (p.u_out) {
        // the backward's recomputation of the pre-activation: u itself, fp32, no SwiGLU
        const size_t ldu = 2 * (size_t)p.F;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][q]),
                                                               __float_as_uint(acc[i][j][q + 8]), false, false);
              const int rl = wm * C::WTM + i * 32 + 8 * (q >> 2) + rlane + (q & 3);
              const int f = f_wave + j * 16 + pl;
              if (rl < rows && f < p.F) {
                float* const d = p.u_out + (size_t)(gbase + rl) * ldu + f;
                d[0] = __uint_as_float(sw[0]) + bg[j];
                d[p.F] = __uint_as_float(sw[1]) + bl[j];
              }
            }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][q]),
                                                           __float_as_uint(acc[i][j][q + 8]), false, false);
          const float ug = __uint_as_float(sw[0]) + bg[j];
          const float ul = __uint_as_float(sw[1]) + bl[j];
          const float gc = fminf(ug, SWIGLU_LIMIT);
          const float lc = fminf(fmaxf(ul, -SWIGLU_LIMIT), SWIGLU_LIMIT);
          // sigmoid(ALPHA gc) = 1 / (1 + 2^(-ALPHA log2(e) gc)), hardware exp2 and reciprocal
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gc * SWIGLU_NEG_ALPHA_LOG2E));
          const float hv = gc * sg * (lc + 1.0f);
          const int r = 8 * (q >> 2) + rlane + (q & 3);
          if (MX) {
            *(float*)(ep + r * EP_S + (j * 16 + pl) * 4) = hv;
          } else {
            const __bf16 hi = (__bf16)hv;                  // round to nearest even
            __bf16* d = (__bf16*)(ep + r * EP_S) + j * 16 + pl;
            d[0] = hi;
            if (DEC) d[32 * EP_S / 2] = (__bf16)(hv - (float)hi);
          }
        }
      }
      if constexpr (MX) {
        // three fp6 (E2M3) pieces of each 32-element block of the rows: lane l takes half
        // l & 1 of row l >> 1.  In the row's 144-byte record of a 64-wide K stage, the 24
        // bytes of piece pc of K block b (its 32 codes) are bytes 72 b + 24 pc .. + 23: what
        // a lane of mlp2's fragment loads for its K half; a lane writes 12 of them
        const int r = lane >> 1, hh = lane & 1;
        const int rl = wm * C::WTM + i * 32 + r;
        const size_t row = (size_t)(gbase + rl);
#pragma unroll
        for (int bb = 0; bb < EP_P / 32; ++bb) {
        const int f0 = f_wave + 32 * bb;
        float v[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 w4 = *(const f32x4*)(ep + r * EP_S + bb * 128 + hh * 64 + u * 16);
          v[4 * u] = w4[0]; v[4 * u + 1] = w4[1]; v[4 * u + 2] = w4[2]; v[4 * u + 3] = w4[3];
        }
        const bool st = rl < rows && f0 < p.F;
        uint32_t* const dst = (uint32_t*)(p.h8 + row * (size_t)(9 * p.F / 4) + (f0 >> 6) * 144 +
                                          ((f0 >> 5) & 1) * 72 + hh * 12);
        uint32_t codes[3][3];
        const uint32_t sc = fp6_pieces16(v, codes);
        if (st) {
#pragma unroll
          for (int pc = 0; pc < 3; ++pc) {
            dst[6 * pc] = codes[pc][0];
            dst[6 * pc + 1] = codes[pc][1];
            dst[6 * pc + 2] = codes[pc][2];
          }
        }
        if (st && hh == 0) p.h8s[row * p.h8s_stride + (f0 >> 5)] = sc;
        }
        continue;
      }
#pragma unroll
      for (int t = 0; t < (32 * CH + 63) / 64; ++t) {
        const int idx = lane + 64 * t;
        const int r = idx / CH, c = idx % CH;
        const int rl = wm * C::WTM + i * 32 + r;
        const int f0 = f_wave + c * 4;
        if (idx < 32 * CH && rl < rows && f0 < p.F) {
          const size_t at = (size_t)(gbase + rl) * p.F + f0;
          *(uint2*)(p.h + at) = *(const uint2*)(ep + r * EP_S + c * 8);
          if (DEC) *(uint2*)(p.h_lo + at) = *(const uint2*)(ep + 32 * EP_S + r * EP_S + c * 8);
        }
      }
    }
  } else {
    const int o_wave = n_tile * BN + wn * C::WTN;          // first output column of this wave
    float bo[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int o = o_wave + j * 32 + (lane & 31);
      bo[j] = (MODE == 2 && o < p.N) ? bf16_to_f32(bias[o]) : 0.f;
    }
    constexpr int CH = C::WTN / 4;                         // 16-byte chunks per slice row
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = 8 * (q >> 2) + 4 * kg + (q & 3);
          *(float*)(ep + r * EP_S + (j * 32 + (lane & 31)) * 4) = acc[i][j][q] + bo[j];
        }
#pragma unroll
      for (int t = 0; t < (32 * CH + 63) / 64; ++t) {
        const int idx = lane + 64 * t;
        const int r = idx / CH, c = idx % CH;
        const int rl = wm * C::WTM + i * 32 + r;
        const int o0 = o_wave + c * 4;
        if (idx < 32 * CH && rl < rows && o0 < p.N) {
          const int a = tab_a[rl];
          if (a >= 0) {
            const float gw = tab_g[rl];
            f32x4 v = *(const f32x4*)(ep + r * EP_S + c * 16);
            v *= gw;
            *(f32x4*)(p.y + (size_t)a * p.N + o0) = v;
          }
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
  g.n_tiles = MODE == 1 ? (g.F + C::BN / 2 - 1) / (C::BN / 2) : (g.N + C::BN - 1) / C::BN;
  const int64_t total = (int64_t)g.max_m_tiles * g.n_tiles;
  const int64_t blocks = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((grouped_gemm_kernel<MODE, FMT, C>), dim3((unsigned)blocks), dim3(C::THREADS), 0, st, g);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_any(const GemmArgs& g, int fmt, int cfg, int64_t A, hipStream_t st) {
  if (fmt == 2) return launch_gemm<MODE, 2, LargeTile<MODE, 2>>(g, A, st);
  if (fmt == 0)
    return cfg == 0 ? launch_gemm<MODE, 0, SmallTile<MODE, 0>>(g, A, st) : launch_gemm<MODE, 0, LargeTile<MODE, 0>>(g, A, st);
  if constexpr (MODE == 2) {
    // bf16 weights stored [K][N] (the backward's products with W2 and W1 as stored)
    if (fmt == 4)
      return cfg == 0 ? launch_gemm<MODE, 4, SmallTile<MODE, 4>>(g, A, st)
                      : launch_gemm<MODE, 4, LargeTile<MODE, 4>>(g, A, st);
    if (fmt == 5)
      return cfg == 0 ? launch_gemm<MODE, 5, SmallTile<MODE, 5>>(g, A, st)
                      : launch_gemm<MODE, 5, LargeTile<MODE, 5>>(g, A, st);
  }
  // MXFP8 (kernel format 3) decodes to bf16: matrix-core tiles at many rows per expert,
  // streaming tiles otherwise
  if (fmt == 3)
    return cfg != 0 ? launch_gemm<MODE, 3, LargeTile<MODE, 3>>(g, A, st)
                    : launch_gemm<MODE, 3, SmallTile<MODE, 3>>(g, A, st);
  // MXFP4 on matrix-core tiles runs on the scaled engine (fmt 2)
  if (cfg != 0) return hipErrorInvalidValue;
  return launch_gemm<MODE, 1, SmallTile<MODE, 1>>(g, A, st);
}

// Streaming tiles keep the decoded-bf16 path: with few rows per expert the stage loop is
// bound by memory latency, and the scaled engine's wider tiles (a whole 32-element block of
// h per wave) measured slower there.
bool mx_engine(int fmt, int cfg) { return fmt == 1 && cfg == 1; }

// Kernel format of a weight format (0 bf16, 1 MXFP4, 2 MXFP8) and tile configuration:
// 0 bf16, 1 MXFP4 decoded, 2 MXFP4 on the scaled engine, 3 MXFP8 decoded.
static int kernel_format(int fmt, int cfg) { return fmt == 2 ? 3 : (mx_engine(fmt, cfg) ? 2 : fmt); }

// Weight gradients C[e] = A_e B_e^T on the matrix-core tiles: A and B bf16 [M][ld] and [N][ld]
// (K contiguous), expert e's K the columns [poff[e], poff[e + 1]) (multiples of 64, zero
// past its rows), poff[E + 1 + r] the expert of rank r by decreasing K; C fp32 [E][M][N].
hipError_t launch_wgrad_tiles(const uint16_t* a, const uint16_t* b, int ld, const int32_t* poff, int E, int M,
                              int N, float* c, hipStream_t st) {
  using C = LargeTile<3, 0>;
  GemmArgs g{};
  g.a = a; g.w = (const uint8_t*)b; g.K = ld; g.offsets = poff; g.E = E; g.A = M; g.N = N; g.y = c;
  g.max_m_tiles = (M + C::BM - 1) / C::BM;
  g.n_tiles = (N + C::BN - 1) / C::BN;
  const int64_t total = (int64_t)E * g.max_m_tiles * g.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_kernel<3, 0, C>), dim3((unsigned)total), dim3(C::THREADS), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_mlp1(const ExpertArgs& a, int cfg, hipStream_t st) {
  GemmArgs g{};
  g.a = a.x; g.a_lo = nullptr; g.perm = a.perm; g.offsets = a.offsets; g.gates = a.gates;
  g.a8 = a.xq; g.a8s = a.xs; g.a8s_stride = mx_scale_stride(a.D);
  g.h8 = a.hq; g.h8s = a.hs; g.h8s_stride = mx_scale_stride(a.F);
  g.w = (const uint8_t*)a.w1; g.bias = a.b1; g.h = a.h; g.h_lo = a.h_lo; g.y = nullptr; g.u_out = a.u_out;
  g.E = a.E; g.k = a.k; g.K = a.D; g.N = 2 * a.F; g.F = a.F;
  const int64_t A = (int64_t)a.T * a.k;
  g.A = (int)A;
  return launch_any<1>(g, kernel_format(a.fmt, cfg), cfg, A, st);
}

hipError_t launch_mlp2(const ExpertArgs& a, int cfg, hipStream_t st) {
  GemmArgs g{};
  g.a = a.h; g.a_lo = a.h_lo; g.perm = a.perm; g.offsets = a.offsets; g.gates = a.gates;
  g.a8 = a.hq; g.a8s = a.hs; g.a8s_stride = mx_scale_stride(a.F);
  g.w = (const uint8_t*)a.w2; g.bias = a.b2; g.h = nullptr; g.h_lo = nullptr; g.y = a.y;
  g.E = a.E; g.k = a.k; g.K = a.F; g.N = a.D; g.F = a.F;
  g.bt_rows = a.w2_kn_rows;
  const int64_t A = (int64_t)a.T * a.k;
  g.A = (int)A;
  if (a.w2_kn_rows > 0) {
    if (a.fmt != 0 || a.w2_kn_rows % 64 != 0) return hipErrorInvalidValue;
    return launch_any<2>(g, a.h_lo ? 5 : 4, cfg, A, st);
  }
  return launch_any<2>(g, kernel_format(a.fmt, cfg), cfg, A, st);
}

// ------------------------------------------------------------------------------ fp8 pieces
// Activations for the scaled matrix-core engine, whose A operand is fp8 E4M3 with one
// E8M0 scale per 32 K elements (OCP microscaling formats: E4M3 has 3 mantissa bits,
// exponent bias 7, largest finite 448).  Every 32-element block of a row is written as NP
// pieces, v ~ sum_p q_p 2^(s_p - 127): piece p rounds (to nearest even) what the earlier
// pieces left, divided by a power of two chosen from the block's largest remainder m,
// 2^(s - 127) = the smallest power of two with m / 2^(s - 127) <= 448, so no value rounds
// past the fp8 range.  Each piece keeps four significant bits of every value within the
// block's normal range; two pieces hold a bf16 value (eight bits) exactly unless it is
// far below its block's largest.
//
// Layout: one 64-element group of a row (64 NP bytes) per stage of the matrix-core loop,
// as 16-byte chunks indexed c = 2 NP h + 2 p + t: piece p, elements 32 t + 16 h .. +15 of
// the group.  Lane half h of the matrix instruction takes elements 16h..16h+15 and
// 32+16h..32+16h+15 of a K step, so each lane reads two consecutive chunks per piece, and
// the two lane halves read chunks 2 NP apart (different LDS banks under the row swizzle).
// Row r, group g starts at byte (r K / 64 + g) 64 NP.  Scales: one dword per row and
// 32-element block at rec[r * RS + b], piece p's E8M0 scale in byte p; RS = K / 32 rounded
// up to a multiple of 8, the padding zero, so that the matrix-core loop can copy whole
// 16-byte chunks of four stages.
//
// One thread per 32-element block.
int mx_scale_stride(int K) { return (K / 32 + 7) & ~7; }

template <int NP>
__global__ __launch_bounds__(256) void mx_split_kernel(const uint16_t* __restrict__ src, int64_t nblk, int K,
                                                       int RS, uint8_t* __restrict__ q, uint32_t* __restrict__ rec) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nblk) return;
  const int nb = K >> 5;
  const int64_t row = gid / nb;
  const int b = (int)(gid - row * nb);
  const uint4* s4 = (const uint4*)(src + row * K + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = s4[i];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(ww[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
    }
  }
  uint32_t sc[NP];
  uint8_t* const dst = q + row * NP * K + (b >> 1) * (NP * 64) + (b & 1) * 16;
#pragma unroll
  for (int pc = 0; pc < NP; ++pc) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    const int e = mx_scale_exp(m);
    sc[pc] = (uint32_t)e;
    const float inv = mx_inv_scale(e), scl = mx_scale(e);
    uint32_t o[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) o[w] = mx_piece4(v + 4 * w, inv, scl, pc + 1 < NP);
    *(uint4*)(dst + pc * 32) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(dst + NP * 32 + pc * 32) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  uint32_t r = 0;
#pragma unroll
  for (int pc = 0; pc < NP; ++pc) r |= sc[pc] << (8 * pc);
  uint32_t* const rrow = rec + row * RS;
  rrow[b] = r;
  if (b == nb - 1)
    for (int pad = nb; pad < RS; ++pad) rrow[pad] = 0;
}

hipError_t launch_mx_split(const uint16_t* src, int64_t rows, int K, uint8_t* q, uint32_t* rec, hipStream_t st) {
  const int64_t nblk = rows * (K / 32);
  const unsigned blocks = (unsigned)((nblk + 255) / 256);
  hipLaunchKernelGGL(mx_split_kernel<2>, dim3(blocks), dim3(256), 0, st, src, nblk, K, mx_scale_stride(K), q, rec);
  return hipGetLastError();
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
// the same sum for a fixed slot count: every slot's load is issued before the first add
template <int K>
__global__ __launch_bounds__(256) void combine_k_kernel(const float4* __restrict__ y, int T, int D4,
                                                        float4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * D4) return;
  const int64_t t = i / D4;
  const int64_t c = i - t * D4;
  const float4* src = y + (t * K) * D4 + c;
  float4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = src[(int64_t)j * D4];
  float4 s = v[0];
#pragma unroll
  for (int j = 1; j < K; ++j) {
    s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
  }
  out[i] = s;
}

hipError_t launch_combine(const float* y, int T, int D, int k, float* out, hipStream_t st) {
  const int D4 = D / 4;
  const int64_t n = (int64_t)T * D4;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (k == 4)
    hipLaunchKernelGGL(combine_k_kernel<4>, grid, dim3(256), 0, st, (const float4*)y, T, D4, (float4*)out);
  else if (k == 2)
    hipLaunchKernelGGL(combine_k_kernel<2>, grid, dim3(256), 0, st, (const float4*)y, T, D4, (float4*)out);
  else
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, (const float4*)y, T, D4, k, (float4*)out);
  return hipGetLastError();
}

}  // namespace moe

// Internal declarations shared by the kernel sources and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum Stage { ST_ROUTER = 0, ST_TOPK = 1, ST_PERMUTE = 2, ST_MLP1 = 3, ST_MLP2 = 4, ST_COMBINE = 5, ST_SPLIT = 6 };

// ---------------------------------------------------------------- routing
// Number of K splits the router uses for T tokens of width D (>= 1).
int router_ksplit(int64_t T, int64_t D);

// fp64 partial dot products partial[s][t][e] over the s-th K range.
hipError_t launch_router_partial(const uint16_t* x, const uint16_t* wr, int T, int D, int E,
                                 int ksplit, double* partial, hipStream_t st);
// Sum of partials + bias -> fp32 logits, top-k (ties to lower index), softmax gates.  With
// ebias (fp32 [E], or null) the selection key is the fp32 sum logit + ebias[e]; the gates
// stay the softmax of the selected logits.
hipError_t launch_topk(const double* partial, int ksplit, const uint16_t* br, const float* ebias, int T,
                       int E, int k, float* logits, int32_t* idx, float* gates, hipStream_t st);
// One load-balancing step of the expert bias (fp32 [E], in place) from the counts (int32 [E]).
hipError_t launch_bias_update(const int32_t* counts, int E, float coeff, float* bias, hipStream_t st);
// counts, exclusive offsets and the stable per-expert permutation of the A assignments.
// hist: workspace of permute_groups(A) * E int32 (unused when permute_groups(A) == 1).
int permute_groups(int64_t A);
hipError_t launch_permute(const int32_t* idx, int A, int E, int32_t* hist, int32_t* counts,
                          int32_t* offsets, int32_t* perm, hipStream_t st);

// ---------------------------------------------------------------- experts
struct ExpertArgs {
  const uint16_t* x;        // [T][D] bf16
  const void* w1;           // bf16 [E][2F][D] or MXFP4 buffer
  const uint16_t* b1;       // [E][2F]
  const void* w2;           // bf16 [E][D][F] or MXFP4 buffer
  const uint16_t* b2;       // [E][D]
  const float* gates;       // [A]
  const int32_t* offsets;   // [E+1]
  const int32_t* perm;      // [A]
  uint16_t* h;              // [A][F] bf16 (hi part for MXFP4)
  uint16_t* h_lo;           // [A][F] bf16 low part (MXFP4 only)
  // scaled-MFMA engine (h and h_lo unused): fp8 pieces of x (two) and of h (three), each
  // row stored as 64-element groups of 64 bytes per piece, and their scales, one dword per
  // row and 32-element block (piece p in byte p), mx_scale_stride(K) dwords per row
  uint8_t* xq;              // [T][2 D]
  uint32_t* xs;             // [T][mx_scale_stride(D)]
  uint8_t* hq;              // [A][3 F]
  uint32_t* hs;             // [A][mx_scale_stride(F)]
  float* y;                 // [A][D] fp32, row a = assignment id
  float* out;               // [T][D] fp32
  int T, D, E, k, F, fmt;
};

// Tile configuration chosen for a routed-row count (the same choice for every stage).
int expert_tile_config(int64_t A, int64_t E);
// Whether the expert GEMMs run on the scaled matrix-core engine (MXFP4 weights,
// matrix-core tiles): mlp1 then reads x as fp8 pieces written by launch_mx_split and
// writes h as fp8 pieces, which mlp2 reads.
bool mx_engine(int fmt, int cfg);
// Scale dwords per row of the pieces of a K-wide row (K / 32 rounded up to a multiple of 8).
int mx_scale_stride(int K);
// Two fp8 pieces of each bf16 row of src [rows][K] and their scales, for mlp1's A rows.
hipError_t launch_mx_split(const uint16_t* src, int64_t rows, int K, uint8_t* q, uint32_t* rec, hipStream_t st);
hipError_t launch_mlp1(const ExpertArgs& a, int cfg, hipStream_t st);
hipError_t launch_mlp2(const ExpertArgs& a, int cfg, hipStream_t st);
hipError_t launch_combine(const float* y, int T, int D, int k, float* out, hipStream_t st);

}  // namespace moe

// Device helpers shared by the expert kernels of the forward (gemm.hip) and of the
// backward (backward.hip): the flat list of row tiles over the expert groups, and the
// XOR swizzle of bf16 operand stages in LDS.
#pragma once

#include "moe_internal.h"

namespace moe {

static __device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Row tiles of all experts in one flat list (experts ascending, BM rows each, the last
// tile of an expert possibly partial).  Wave-wide: lane l looks at experts 4l..4l+3; the
// scan gives every lane the number of tiles before its experts and the total.
struct TileScan {
  int tl[4];        // tiles of this lane's experts
  int excl, incl;   // tiles before / up to and including this lane's experts
  int total;        // tiles of all experts
};
template <int BM>
static __device__ __forceinline__ TileScan tile_scan(const int32_t* __restrict__ offsets, int E) {
  const int lane = threadIdx.x & 63;
  TileScan ts;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    const int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    ts.tl[i] = c > 0 ? (c + BM - 1) / BM : 0;
    s += ts.tl[i];
  }
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  ts.incl = incl;
  ts.excl = incl - s;
  ts.total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  return ts;
}
// Expert, first row and row count of tile m; false past the last tile.
template <int BM>
static __device__ __forceinline__ bool tile_lookup(const TileScan& ts, const int32_t* __restrict__ offsets,
                                                   int m, int& e_out, int& row0_out, int& cnt_out) {
  const int lane = threadIdx.x & 63;
  const uint64_t hit = __ballot(m >= ts.excl && m < ts.incl);
  if (hit == 0) return false;
  const int src = __ffsll((long long)hit) - 1;
  int e = -1, r0 = 0, base = ts.excl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e < 0 && m < base + ts.tl[i]) {
      e = lane * 4 + i;
      r0 = (m - base) * BM;
    }
    base += ts.tl[i];
  }
  e_out = __builtin_amdgcn_readfirstlane(__shfl(e, src));   // uniform: kept in scalar registers
  row0_out = __builtin_amdgcn_readfirstlane(__shfl(r0, src));
  cnt_out = __builtin_amdgcn_readfirstlane(offsets[e_out + 1] - offsets[e_out]);
  return true;
}

// LDS layout of a bf16 operand stage: [rows][BK] with the 16-byte chunks of a row
// XOR-swizzled by row bits, which spreads the rows one chunk index touches over the banks.
// Rows of twelve chunks (three 64-byte pieces of 64 elements) XOR the two low chunk bits with
// row bits 2..3, which keeps a chunk inside its aligned group of four: the 16-byte slots
// of sixteen consecutive rows (row stride 192 bytes) then cover all 64 banks once.
// Rows of nine chunks (144 bytes: three fp6 pieces of 64 elements) are not swizzled: at a
// row stride of 36 dwords the 8-byte reads of sixteen consecutive rows already fall on
// distinct banks.
template <int CPR>
static __device__ __forceinline__ int swz_pos(int r, int c) {
  if (CPR == 9) return c;
  if (CPR == 8) return c ^ (r & 7) ^ ((r >> 3) & 1);
  if (CPR == 12) return c ^ ((r >> 2) & 3);
  return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1);
}
template <int CPR>
static __device__ __forceinline__ int swz(int r, int c) { return r * (CPR * 16) + (swz_pos<CPR>(r, c) << 4); }

}  // namespace moe

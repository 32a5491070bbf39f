// Rate calibrations for bench.py (not part of the MoE block).
//
// Matrix cores: the sustained rate of
// v_mfma_f32_32x32x16_bf16 on this GPU when nothing else limits it, for the operand data a
// GEMM really multiplies (random bf16 values) and for constant operands, at one and two waves
// per SIMD.  It is the reference against which the grouped GEMM's matrix-core fraction is read.
//
// Each wave holds four A and two B operand fragments (eight bf16 values per lane each, loaded
// once from `src`, each wave its own) and issues, per iteration, the eight independent
// products of a 128 x 64 output block (the grouped GEMM's wave tile) into eight accumulators,
// so no instruction waits for another's result.  The accumulators are reduced into `sink` at
// the end so that nothing is optimised away; lane 0 of each wave stores its loop's shader
// clock cycles (s_memtime) in `cycles`.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CAL_NA = 4, CAL_NB = 2;

__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(const uint16_t* __restrict__ src, int iters,
                                                        float* __restrict__ sink,
                                                        unsigned long long* __restrict__ cycles) {
  const int lane = threadIdx.x & 63;
  const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  bf16x8 a[CAL_NA], b[CAL_NB];
#pragma unroll
  for (int i = 0; i < CAL_NA; ++i)
    a[i] = *(const bf16x8*)(src + ((w * (CAL_NA + CAL_NB) + i) * 64 + lane) * 8);
#pragma unroll
  for (int j = 0; j < CAL_NB; ++j)
    b[j] = *(const bf16x8*)(src + ((w * (CAL_NA + CAL_NB) + CAL_NA + j) * 64 + lane) * 8);
  f32x16 acc[CAL_NA][CAL_NB];
#pragma unroll
  for (int i = 0; i < CAL_NA; ++i)
#pragma unroll
    for (int j = 0; j < CAL_NB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < CAL_NA; ++i)
#pragma unroll
      for (int j = 0; j < CAL_NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CAL_NA; ++i)
#pragma unroll
    for (int j = 0; j < CAL_NB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) s += acc[i][j][q];
  sink[w * 64 + lane] = s;
  if (lane == 0) cycles[w] = t1 - t0;
}

// blocks of four waves (one per SIMD); waves_per_simd blocks per CU's worth of the grid.
// src: waves * 6 * 64 * 8 bf16; sink: waves * 64 fp32; cycles: waves u64 (waves = 4 * blocks)
extern "C" int moe_calib_mfma(const void* src, int blocks, int iters, float* sink, unsigned long long* cycles,
                              void* stream) {
  if (blocks <= 0 || iters <= 0 || !src || !sink || !cycles) return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint16_t*)src, iters,
                     sink, cycles);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int moe_calib_products_per_iteration(void) { return CAL_NA * CAL_NB; }

// HBM: the sustained read rate of a plain stream of 16-byte loads over a buffer much larger
// than the caches, every byte read once: grid-stride over 16-byte chunks (chunk i = thread +
// j * threads, so each wave's load instruction reads 1 KB contiguous), eight independent loads
// in flight per lane, folded with XOR into one word per thread so nothing is optimised away.
// (Visiting 1 KB blocks in a scattered order instead measured ≈ 4 % slower.)
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t nchunks,
                                                          uint32_t* __restrict__ sink) {
  const int64_t threads = (int64_t)gridDim.x * 256;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 acc = {0u, 0u, 0u, 0u};
  int64_t i = t;
  for (; i + 7 * threads < nchunks; i += 8 * threads) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * threads];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
    }
  }
  for (; i < nchunks; i += threads) {
    const uint4 v = src[i];
    acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
  }
  sink[t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// src: bytes (a multiple of 16) of device memory; sink: blocks * 256 uint32
extern "C" int moe_calib_stream(const void* src, int64_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (blocks <= 0 || bytes < 16 || (bytes & 15) || !src || !sink) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

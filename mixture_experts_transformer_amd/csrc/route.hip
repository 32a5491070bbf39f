// Routing stage of the GPT-OSS MoE block on gfx950: router logits, top-k with softmax
// gates, and the stable grouping of assignments by expert.
//
// Router: a Linear with a bias (torchtitan GPT-OSS guide, section "StateDict adapter").
// The logits decide integer outputs, so they are computed as the exact dot product of
// the bf16 inputs up to float64 rounding, then rounded once to fp32.  The products of
// two bf16 values are exact in fp64, so the only rounding is the fp64 accumulation.
// The dot products run on the fp64 matrix cores (v_mfma_f64_16x16x4f64): a wave owns
// 16 tokens x 16 experts per instruction, converting bf16 operands to fp64 in registers.
// K is split across the grid so small token counts still occupy the chip; the partial
// sums are added in a fixed order by the top-k kernel (deterministic).
//
// Top-k ("gptoss" re-implementation page, basic parameters: top-4 of 32 experts): one
// wave per token, lanes own experts.  Up to 64 experts each lane counts the experts that
// beat its own (value desc, index asc) and the ranks below k are the selection; beyond,
// k rounds of a wave-wide argmax.  Gates: softmax over the k selected logits, in fp64,
// stored as fp32.
//
// Grouping (torchtitan guide, grouped GEMM section: per-expert counts and their int32
// cumulative sum as group offsets): workgroups of 16 waves over chunks of the assignments
// (one workgroup for few assignments; otherwise a per-chunk histogram pass first).  Each
// wave owns a contiguous range, counts it per expert in LDS, and after a scan places each
// assignment at offsets[e] + (earlier assignments of e), computing ranks inside a
// 64-assignment step with ballots over the bits of the expert index.  The result is the
// stable counting sort, independent of any atomic arrival order.
#include "moe_internal.h"

namespace moe {

static __device__ __forceinline__ double bf16_bits_to_f64(uint32_t b) {
  return (double)__uint_as_float(b << 16);
}

// ------------------------------------------------------------------------------ router
constexpr int RT_WAVES = 4;           // waves per workgroup, each owns 16 tokens
constexpr int RT_CHUNK = 32;          // K elements per MFMA group (8 steps of K=4)
constexpr int RT_PD = 4;              // chunks whose loads are in flight (up to 64 experts)

constexpr int64_t RT_TARGET_WAVES = 2048;  // waves the K split aims at (measured choice)
constexpr int64_t RT_MIN_CHUNKS = 3;        // K chunks per split at least (6 measured slower)
int router_ksplit(int64_t T, int64_t D) {
  const int64_t chunks = D / RT_CHUNK;
  const int64_t tiles = (T + 15) / 16;
  // aim at ~2048 waves in flight; keep >= 3 chunks per split so the top-k kernel's
  // sum over splits stays short
  int64_t ks = (RT_TARGET_WAVES + tiles - 1) / tiles;
  int64_t maxks = chunks / RT_MIN_CHUNKS > 0 ? chunks / RT_MIN_CHUNKS : 1;
  if (ks > maxks) ks = maxks;
  if (ks < 1) ks = 1;
  return (int)ks;
}

// v_mfma_f64_16x16x4f64 lane layout (measured on gfx950): A lane l supplies A[l & 15][l >> 4],
// B lane l supplies B[l >> 4][l & 15], and output register r of lane l holds C[m][n] with
// m = (l >> 4) + 4 r, n = l & 15.
//
// One wave's share: the dot products of tokens t0 .. t0 + 15 with experts 0 .. 16 NEB - 1 over
// the 32-element chunks [c_begin, c_end) of D, summed in chunk order.  acc[b][r] of lane l
// is token t0 + (l >> 4) + 4 r, expert 16 b + (l & 15).
template <int NEB>
static __device__ __forceinline__ void router_wave(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                   int T, int D, int E, int t0, int c_begin, int c_end,
                                                   f64x4 (&acc)[NEB]) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 15;   // token (A) / expert-in-block (B)
  const int kg = lane >> 4;    // which 8-element run of the 32-element chunk
  const int t = min(t0 + row, T - 1);
  const uint16_t* xrow = x + (size_t)t * D + kg * 8;
  const uint16_t* wrow[NEB];
#pragma unroll
  for (int b = 0; b < NEB; ++b) {
    const int e = min(b * 16 + row, E - 1);
    wrow[b] = wr + (size_t)e * D + kg * 8;
  }

#pragma unroll
  for (int b = 0; b < NEB; ++b) acc[b] = f64x4{0.0, 0.0, 0.0, 0.0};

  // PD chunks in flight (fewer with many experts, for registers): slot q of the register
  // ring holds chunk c0 + q
  constexpr int PD = NEB >= 16 ? 1 : (NEB >= 8 ? 2 : RT_PD);
  uint4 xa[PD];
  uint4 wa[PD][NEB];
#pragma unroll
  for (int q = 0; q < PD; ++q) {
    xa[q] = uint4{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < NEB; ++b) wa[q][b] = uint4{0, 0, 0, 0};
    if (c_begin + q < c_end) {
      xa[q] = *(const uint4*)(xrow + (c_begin + q) * RT_CHUNK);
#pragma unroll
      for (int b = 0; b < NEB; ++b) wa[q][b] = *(const uint4*)(wrow[b] + (c_begin + q) * RT_CHUNK);
    }
  }
  for (int c0 = c_begin; c0 < c_end; c0 += PD) {
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      const int c = c0 + q;
      if (c >= c_end) break;
      const uint4 xc = xa[q];
      uint4 wc[NEB];
#pragma unroll
      for (int b = 0; b < NEB; ++b) wc[b] = wa[q][b];
      if (c + PD < c_end) {   // refill the slot with the chunk PD ahead
        xa[q] = *(const uint4*)(xrow + (c + PD) * RT_CHUNK);
#pragma unroll
        for (int b = 0; b < NEB; ++b) wa[q][b] = *(const uint4*)(wrow[b] + (c + PD) * RT_CHUNK);
      }
      const uint32_t xw[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t xb = (i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu);
        const double a = bf16_bits_to_f64(xb);
#pragma unroll
        for (int b = 0; b < NEB; ++b) {
          const uint32_t ww[4] = {wc[b].x, wc[b].y, wc[b].z, wc[b].w};
          const uint32_t wb = (i & 1) ? (ww[i >> 1] >> 16) : (ww[i >> 1] & 0xFFFFu);
          acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bf16_bits_to_f64(wb), acc[b], 0, 0, 0);
        }
      }
    }
  }
}

template <int NEB>
__global__ __launch_bounds__(64 * RT_WAVES) void router_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int D, int E,
    int ksplit, double* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * RT_WAVES + wave) * 16;
  if (t0 >= T) return;
  const int s = blockIdx.y;
  const int nchunks = D / RT_CHUNK;
  const int c_begin = (int)((int64_t)nchunks * s / ksplit);
  const int c_end = (int)((int64_t)nchunks * (s + 1) / ksplit);
  f64x4 acc[NEB];
  router_wave<NEB>(x, wr, T, D, E, t0, c_begin, c_end, acc);
  const int row = lane & 15;
  const int kg = lane >> 4;
  // partial[s][t][e]: token t0 + kg + 4r, expert b*16 + row
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tt = t0 + kg + 4 * r;
    if (tt < T) {
      double* dst = partial + ((size_t)s * T + tt) * E;
#pragma unroll
      for (int b = 0; b < NEB; ++b) {
        const int e = b * 16 + row;
        if (e < E) dst[e] = acc[b][r];
      }
    }
  }
}

hipError_t launch_router_partial(const uint16_t* x, const uint16_t* wr, int T, int D, int E,
                                 int ksplit, double* partial, hipStream_t st) {
  const dim3 grid((T + 16 * RT_WAVES - 1) / (16 * RT_WAVES), ksplit);
  const dim3 block(64 * RT_WAVES);
  const int neb = (E + 15) / 16;
  if (neb <= 1)
    hipLaunchKernelGGL(router_partial_kernel<1>, grid, block, 0, st, x, wr, T, D, E, ksplit, partial);
  else if (neb <= 2)
    hipLaunchKernelGGL(router_partial_kernel<2>, grid, block, 0, st, x, wr, T, D, E, ksplit, partial);
  else if (neb <= 4)
    hipLaunchKernelGGL(router_partial_kernel<4>, grid, block, 0, st, x, wr, T, D, E, ksplit, partial);
  else if (neb <= 8)
    hipLaunchKernelGGL(router_partial_kernel<8>, grid, block, 0, st, x, wr, T, D, E, ksplit, partial);
  else
    hipLaunchKernelGGL(router_partial_kernel<16>, grid, block, 0, st, x, wr, T, D, E, ksplit, partial);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ top-k
constexpr int TK_WAVES = 4;

// (v, e) beats (v2, e2): larger value, or equal value and lower index.
static __device__ __forceinline__ bool beats(float v, int e, float v2, int e2) {
  return v > v2 || (v == v2 && e < e2);
}

// Logit of token t and expert e from the split partial sums: added in split order (16
// loads in flight per batch), plus the bias, then rounded once to fp32 (nearest even).
static __device__ __forceinline__ float logit_from_partials(const double* __restrict__ partial, int ksplit,
                                                            const uint16_t* __restrict__ br, int T, int E,
                                                            int t, int e) {
  double s = 0.0;
  for (int q0 = 0; q0 < ksplit; q0 += 16) {
    double pv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
      pv[q] = (q0 + q < ksplit) ? partial[((size_t)(q0 + q) * T + t) * E + e] : 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (q0 + q < ksplit) s += pv[q];
  }
  s += bf16_bits_to_f64(br[e]);
  return (float)s;
}

// Top-k of token t by one wave: lane l holds the selection keys v[i] and the logits lv[i]
// of experts l + 64 i where live[i] (the two are equal without a load-balancing bias).
// Writes idx and gates of the token; sel is k floats of this wave's LDS.
static __device__ __forceinline__ void topk_wave(float (&v)[4], const float (&lv)[4], bool (&live)[4], int k,
                                                 int t, int32_t* __restrict__ idx, float* __restrict__ gates,
                                                 float* sel) {
  constexpr int PER = 4;
  const int lane = threadIdx.x & 63;
  for (int j = 0; j < k; ++j) {
    // lane-local best among live entries; any live entry beats "none" (NONE), so the
    // winner is always a valid expert index even for NaN logits (outside the contract)
    constexpr int NONE = 0x7fffffff;
    float bv = -INFINITY;
    int be = NONE;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (live[i] && (be == NONE || beats(v[i], e, bv, be))) { bv = v[i]; be = e; }
    }
    // wave argmax: the largest value by a butterfly on values alone, then the lowest expert
    // holding it (a lane's own best already has the lowest index among its equal values)
    float mv = (be == NONE) ? -INFINITY : bv;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off));
    // lanes whose best equals the maximum; among them the lowest expert index wins
    const int cand = (be != NONE && bv == mv) ? be : NONE;
    int ce = cand;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ce = min(ce, __shfl_xor(ce, off));
    if (ce == NONE) {
      // every remaining live value is NaN (outside the contract): keep the old rule, the
      // lowest live expert wins, so the index is always valid
      int le = be;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) le = min(le, __shfl_xor(le, off));
      ce = le;
    }
    be = ce;
    // the lane holding the winner retires it and records its logit for the gates
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i == be) {
        live[i] = false;
        sel[j] = lv[i];
      }
    if (lane == 0) idx[(size_t)t * k + j] = be;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // gates: softmax over the k selected logits, in fp64, shifted by their largest (the
  // first slot's unless a bias reordered the selection)
  float tv = -INFINITY;
  for (int j = lane; j < k; j += 64) tv = fmaxf(tv, sel[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tv = fmaxf(tv, __shfl_xor(tv, off));
  const double top = (double)tv;
  double part = 0.0;
  for (int j = lane; j < k; j += 64) part += exp((double)sel[j] - top);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  for (int j = lane; j < k; j += 64)
    gates[(size_t)t * k + j] = (float)(exp((double)sel[j] - top) / part);
}

// Top-k and gates of NT tokens at once by one wave, lane e holding expert e's selection key
// s[i] and logit v[i] (equal without a load-balancing bias; at most 64 experts; live[i]
// false for lanes past E and skipped tokens, t[i] < 0).  The same selection as the top-k
// kernel's, by rank instead of k rounds of wave-wide argmax: each lane counts the experts
// that beat it (larger key, or equal and lower index; -0 equals +0, NaN loses to every
// number), the experts of rank j < k are the token's j-th, and lane j then holds the j-th
// for the gates.  key/sel_v/sel_e: NT x 64 entries of this wave's LDS each.
static __device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);          // -0 -> +0
  if (v != v) return 0u;                                 // NaN: below everything
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);     // monotone in v, >= 0x007FFFFF
}
template <int NT>
static __device__ __forceinline__ void topk_rank_lanes(const float (&s)[NT], const float (&v)[NT],
                                                       const bool (&live)[NT], const int (&t)[NT], int E, int k, int32_t* __restrict__ idx,
                                                       float* __restrict__ gates, uint32_t (*key)[64],
                                                       float (*sel_v)[64], int (*sel_e)[64]) {
  const int lane = threadIdx.x & 63;
  uint32_t my[NT];
  int rank[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    my[i] = live[i] ? order_key(s[i]) : 0u;
    key[i][lane] = my[i];                                // lanes past E: 0, never beat
    rank[i] = 0;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int e0 = 0; e0 < E; e0 += 4) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint4 q = *(const uint4*)&key[i][e0];        // the same address in every lane
      const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) rank[i] += (kk[u] > my[i] || (kk[u] == my[i] && e0 + u < lane)) ? 1 : 0;
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
    if (live[i] && rank[i] < k) {
      sel_v[i][rank[i]] = v[i];
      sel_e[i][rank[i]] = lane;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // gates: softmax over the k selected logits, in fp64 (lane j < k holds the j-th), shifted
  // by their largest (the first slot's unless a bias reordered the selection)
  double ex[NT], sum[NT];
  int my_e[NT];
  float top[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) top[i] = lane < k ? sel_v[i][lane] : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < NT; ++i) top[i] = fmaxf(top[i], __shfl_xor(top[i], off));
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    my_e[i] = lane < k ? sel_e[i][lane] : 0;
    ex[i] = lane < k ? exp((double)sel_v[i][lane] - (double)top[i]) : 0.0;
    sum[i] = ex[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < NT; ++i) sum[i] += __shfl_xor(sum[i], off);
#pragma unroll
  for (int i = 0; i < NT; ++i)
    if (t[i] >= 0 && lane < k) {
      idx[(size_t)t[i] * k + lane] = my_e[i];
      gates[(size_t)t[i] * k + lane] = (float)(ex[i] / sum[i]);
    }
}

__global__ __launch_bounds__(64 * TK_WAVES) void topk_kernel(
    const double* __restrict__ partial, int ksplit, const uint16_t* __restrict__ br,
    const float* __restrict__ ebias, int T, int E, int k, float* __restrict__ logits,
    int32_t* __restrict__ idx, float* __restrict__ gates) {
  __shared__ float sel_v[TK_WAVES][256];
  __shared__ uint32_t rk_key[TK_WAVES][1][64];
  __shared__ float rk_v[TK_WAVES][1][64];
  __shared__ int rk_e[TK_WAVES][1][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * TK_WAVES + wave;
  if (t >= T) return;
  if (E <= 64) {
    // one expert per lane: selection by rank
    const bool live[1] = {lane < E};
    const int tt[1] = {t};
    float v[1] = {-INFINITY};
    if (live[0]) {
      v[0] = logit_from_partials(partial, ksplit, br, T, E, t, lane);
      if (logits) logits[(size_t)t * E + lane] = v[0];
    }
    // the load-balancing bias moves the selection only (one fp32 rounding)
    const float key[1] = {live[0] && ebias ? v[0] + ebias[lane] : v[0]};
    topk_rank_lanes<1>(key, v, live, tt, E, k, idx, gates, rk_key[wave], rk_v[wave], rk_e[wave]);
    return;
  }
  float v[4], key[4];
  bool live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {    // E <= 256 = 4 * 64
    const int e = lane + 64 * i;
    live[i] = e < E;
    v[i] = -INFINITY;
    if (live[i]) {
      v[i] = logit_from_partials(partial, ksplit, br, T, E, t, e);
      if (logits) logits[(size_t)t * E + e] = v[i];
    }
    key[i] = live[i] && ebias ? v[i] + ebias[e] : v[i];
  }
  topk_wave(key, v, live, k, t, idx, gates, sel_v[wave]);
}

hipError_t launch_topk(const double* partial, int ksplit, const uint16_t* br, const float* ebias, int T,
                       int E, int k, float* logits, int32_t* idx, float* gates, hipStream_t st) {
  const dim3 grid((T + TK_WAVES - 1) / TK_WAVES);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(64 * TK_WAVES), 0, st, partial, ksplit, br, ebias, T, E, k,
                     logits, idx, gates);
  return hipGetLastError();
}

// ------------------------------------------------------------- load-balancing bias update
// One step of the per-expert selection bias from the step's assignment counts: an expert
// above the mean count lowers its bias by coeff, one below raises it, one at the mean keeps
// it.  The comparison is exact in integers (sum - E * counts[e] has the sign of
// mean - counts[e]); the update is one fp32 addition.  One workgroup of 256 lanes, E <= 256.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, int E, float coeff,
                                                          float* __restrict__ bias) {
  __shared__ long long part[4];
  const int e = threadIdx.x;
  const long long c = e < E ? (long long)counts[e] : 0;
  long long sum = c;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if ((e & 63) == 0) part[e >> 6] = sum;
  __syncthreads();
  const long long total = part[0] + part[1] + part[2] + part[3];
  if (e < E) {
    const long long d = total - (long long)E * c;
    if (d != 0) bias[e] = bias[e] + (d > 0 ? coeff : -coeff);
  }
}

hipError_t launch_bias_update(const int32_t* counts, int E, float coeff, float* bias, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, st, counts, E, coeff, bias);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ grouping
constexpr int PM_WAVES = 16;
constexpr int PM_CHUNK = 2048;        // assignments per workgroup when the grouping is split

int permute_groups(int64_t A) {
  const int64_t g = (A + PM_CHUNK - 1) / PM_CHUNK;
  return g > 2 ? (int)g : 1;          // up to two chunks one workgroup is as fast
}

// Split grouping, pass 1: hist[g][e] = assignments of chunk g routed to expert e.
__global__ __launch_bounds__(1024) void permute_hist_kernel(const int32_t* __restrict__ idx, int A, int E,
                                                            int32_t* __restrict__ hist) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  if (tid < 256) h[tid] = 0;
  __syncthreads();
  const int lo = blockIdx.x * PM_CHUNK;
  const int hi = min(A, lo + PM_CHUNK);
  for (int a = lo + tid; a < hi; a += blockDim.x) atomicAdd(&h[min(max(idx[a], 0), E - 1)], 1);
  __syncthreads();
  if (tid < E) hist[(size_t)blockIdx.x * E + tid] = h[tid];
}

// Grouping of the assignments [lo, hi) of this workgroup (all of them when hist is null;
// chunk g = blockIdx.x of PM_CHUNK otherwise, placed after the chunks before it using the
// histogram of pass 1).  Each wave owns a contiguous range, counts it per expert in LDS,
// and after a scan places each assignment at its expert's base plus the earlier
// assignments of that expert, ranked inside a 64-assignment step by ballots.
// The body, for a workgroup of NW waves (threads 0 .. 64 NW - 1) and its LDS.
template <int NW>
static __device__ __forceinline__ void group_assignments(
    const int32_t* idx, int A, int E, const int32_t* __restrict__ hist, int G, int g,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int (*cnt)[256], int (*base)[256], int* tot) {
  static_assert(NW * 64 >= 256, "the scan over experts takes 256 threads");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c_lo = hist ? g * PM_CHUNK : 0;
  const int c_hi = hist ? min(A, c_lo + PM_CHUNK) : A;
  for (int i = tid; i < NW * 256; i += NW * 64) (&cnt[0][0])[i] = 0;
  __syncthreads();
  // contiguous range per wave, a multiple of 64 long
  const int per = ((c_hi - c_lo + NW - 1) / NW + 63) & ~63;
  const int lo = min(c_hi, c_lo + wave * per);
  const int hi = min(c_hi, lo + per);
  for (int a = lo + lane; a < hi; a += 64) atomicAdd(&cnt[wave][min(max(idx[a], 0), E - 1)], 1);
  __syncthreads();
  // totals over all assignments and, split, over the chunks before this one; their
  // exclusive scan over experts gives the offsets, and each wave's base per expert follows
  if (E <= 64) {
    // one expert per lane of wave 0: the scan is a wave-wide prefix sum
    if (wave == 0) {
      int s = 0, pre = 0;
      if (lane < E) {
        if (hist) {
          for (int q = 0; q < G; ++q) {
            const int v = hist[(size_t)q * E + lane];
            s += v;
            if (q < g) pre += v;
          }
        } else {
          for (int w = 0; w < NW; ++w) s += cnt[w][lane];
        }
      }
      int inc = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      if (lane < E) {
        if (g == 0) {
          counts[lane] = s;
          offsets[lane] = inc - s;
          if (lane == E - 1) offsets[E] = inc;
        }
        int b = inc - s + pre;
        for (int w = 0; w < NW; ++w) {
          base[w][lane] = b;
          b += cnt[w][lane];
        }
      }
    }
    __syncthreads();
  } else {
    int pre = 0;
    if (tid < 256) {
      int s = 0;
      if (tid < E) {
        if (hist) {
          for (int q = 0; q < G; ++q) {
            const int v = hist[(size_t)q * E + tid];
            s += v;
            if (q < g) pre += v;
          }
        } else {
          for (int w = 0; w < NW; ++w) s += cnt[w][tid];
        }
      }
      tot[tid] = s;
      if (tid < E && g == 0) counts[tid] = s;
    }
    __syncthreads();
    // inclusive scan of the totals over experts (threads 0..255)
    for (int off = 1; off < 256; off <<= 1) {
      int v = 0;
      if (tid < 256 && tid >= off) v = tot[tid - off];
      __syncthreads();
      if (tid < 256) tot[tid] += v;
      __syncthreads();
    }
    if (tid < E) {
      const int first = (tid == 0) ? 0 : tot[tid - 1];   // exclusive prefix
      if (g == 0) {
        offsets[tid] = first;
        if (tid == E - 1) offsets[E] = tot[tid];
      }
      int b = first + pre;
      for (int w = 0; w < NW; ++w) {
        base[w][tid] = b;
        b += cnt[w][tid];
      }
    }
    __syncthreads();
  }
  // place assignments: rank among equal experts inside each 64-wide step by ballots
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int a0 = lo; a0 < hi; a0 += 64) {
    const int a = a0 + lane;
    const bool valid = a < hi;
    const int e = valid ? min(max(idx[a], 0), E - 1) : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t on = __ballot(valid && ((e >> b) & 1));
      match &= ((e >> b) & 1) ? on : ~on;
    }
    if (valid) {
      const uint64_t below = match & ((1ull << lane) - 1ull);
      const int rank = __popcll(below);
      const int pos = base[wave][e] + rank;
      perm[pos] = a;
      const int leader = 63 - __clzll(match);
      // every lane has read base[wave][e] above; the group's highest lane advances it
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) base[wave][e] = pos + 1;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(64 * PM_WAVES) void permute_kernel(
    const int32_t* __restrict__ idx, int A, int E, const int32_t* __restrict__ hist, int G,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  __shared__ int cnt[PM_WAVES][256];
  __shared__ int base[PM_WAVES][256];
  __shared__ int tot[256];
  group_assignments<PM_WAVES>(idx, A, E, hist, G, blockIdx.x, counts, offsets, perm, cnt, base, tot);
}

hipError_t launch_permute(const int32_t* idx, int A, int E, int32_t* hist, int32_t* counts,
                          int32_t* offsets, int32_t* perm, hipStream_t st) {
  const int G = permute_groups(A);
  if (G > 1) {
    hipLaunchKernelGGL(permute_hist_kernel, dim3(G), dim3(1024), 0, st, idx, A, E, hist);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_kernel, dim3(G), dim3(64 * PM_WAVES), 0, st, idx, A, E,
                     G > 1 ? (const int32_t*)hist : nullptr, G, counts, offsets, perm);
  return hipGetLastError();
}

}  // namespace moe

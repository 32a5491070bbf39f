/*
 * moe.h -- C ABI of the GPT-OSS mixture-of-experts feed-forward block for
 * AMD Instinct MI355X (gfx950).
 *
 * What the block computes, per token t with hidden vector x[t] (D values):
 *
 *   1. router logits    l[t,e] = sum_d x[t,d] * Wr[e,d] + br[e]          (E experts)
 *      The router is a Linear layer with a bias (torchtitan GPT-OSS guide,
 *      section "StateDict adapter": router.gate weight and bias).  The sum is
 *      exact up to float64 rounding and is rounded once to fp32.
 *   2. top-k            the k experts with the largest logits; slot j holds the
 *      j-th largest; equal logits go to the lower expert index first
 *      ("gptoss" re-implementation page, section "basic parameters": top-4 of 32).
 *   3. gate weights     g[t,j] = softmax over the k selected logits.
 *   4. grouping         assignment a = t*k + j; counts[e] = #{a : idx[a] = e};
 *      offsets = exclusive prefix sum of counts (offsets[1..E] is the int32
 *      cumulative sum of the torchtitan guide, section "Grouped matrix
 *      multiplication"); perm lists assignments grouped by expert, ascending a
 *      inside each group.
 *   5. mlp1             u = x[t] . W1[e]^T + b1[e], G = 2F outputs; W1 is stored
 *      (experts, out, in) as in the same section; u[0:F] is the gate half and
 *      u[F:2F] the linear half.
 *   6. SwiGLU (GPT-OSS variant, same section): gate clamped from above at LIMIT,
 *      times sigmoid(ALPHA * gate); linear clamped to [-LIMIT, LIMIT], plus 1;
 *      h = gate_c * sigmoid(ALPHA * gate_c) * (lin_c + 1).
 *   7. mlp2 + gate      y[a] = g[a] * (h . W2[e]^T + b2[e]).
 *   8. combine          out[t] = sum_j y[t*k + j]   ("gptoss" page, section
 *      "model run flow": weighted combination of the experts' outputs).
 *
 * Expert weights are bf16 or MXFP4 (GPT-OSS-in-Transformers blog, MXFP4
 * paragraph: 4-bit E2M1 values, 1 sign / 2 exponent / 1 mantissa bit, one scale
 * per 32-element block).  MXFP4 storage used here: one uint8 buffer per matrix,
 * first the codes [E][rows][K/2] (element 2i in the low nibble of byte i, 2i+1
 * in the high nibble), then the E8M0 scale bytes [E][rows][K/32]; scale byte s
 * multiplies its 32 consecutive K elements by 2^(s-127).  K is the reduction
 * dimension: D for W1 (rows = 2F), F for W2 (rows = D).  Scale bytes must lie in
 * [2, 252] so every decoded weight is an exact normal bf16 value; other bytes
 * are outside the contract (not checked on the device).
 *
 * MXFP8 weights (fmt 2: E4M3 elements, 1 sign / 4 exponent bits with bias 7 / 3 mantissa
 * bits, no infinity, 0x7F and 0xFF NaN, one E8M0 scale per 32 elements, OCP Microscaling
 * spec v1.0; the torchtitan guide's grouped GEMM section names MXFP8 converters as the
 * users of its scaled grouped-GEMM seam): one uint8 buffer per matrix, the codes
 * [E][rows][K] (one byte per element) then the scale bytes [E][rows][K/32].  Scale bytes
 * must lie in [10, 246] and codes must not be NaN, so every decoded weight is an exact
 * normal bf16 (not checked on the device).  Decoded to bf16 and multiplied on the bf16
 * matrix instructions at every token count, h carried into mlp2 as a bf16 pair as for
 * MXFP4 at small token counts.
 *
 * Numerics: every product is accumulated in fp32 on the matrix cores except the
 * router (fp64).  The bf16 path rounds h to bf16 once.  With MXFP4 weights, small
 * token counts carry h as a bf16 pair (hi + lo, 16 significant bits) into mlp2;
 * large ones run both GEMMs on the scaled matrix instructions, with x as two fp8
 * (E4M3) pieces times fp4 and h as three fp6 (E2M3) pieces times fp4, the pieces of
 * each 32 elements sharing one power-of-two scale (x exactly but for values far below
 * their block's largest; h to about 12 bits of the block's largest).  The output is fp32
 * and deterministic: no float atomics, fixed summation orders, bitwise equal
 * from run to run.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library keeps
 *     none of them after the call returns.  Every pointer must be 16-byte
 *     aligned and non-null whenever T > 0 (logits may be null).
 *   - Shapes: 1 <= k <= E <= 256; D and F positive multiples of 64 below 2^24;
 *     0 <= T and T*k < 2^31; T*D, T*k*F and D*F below 2^30 (the expert kernels
 *     address activation rows and one expert's weights with 32-bit offsets).
 *     T == 0 returns MOE_OK and launches nothing.
 *   - Calls are asynchronous on the calling thread's stream (moe_set_stream)
 *     and return after enqueueing; device faults surface at the caller's next
 *     synchronisation.  Outputs are fully overwritten and must not alias inputs.
 *   - Return value: MOE_OK (0) or a negative MOE_E* status; on failure nothing
 *     has been launched and moe_last_error() describes the problem.
 *   - Graph capture: a call enqueues kernels only (no allocation, memset, copy or
 *     synchronisation) once the workspace fits its shape, so after one eager call of the
 *     same shape (or with moe_set_workspace) it can be captured into a HIP graph.  A call
 *     on a capturing stream that would have to grow the library-owned workspace fails
 *     with MOE_ENOMEM.  Once a call has been captured, the library-owned buffer it used is
 *     never freed before moe_release: a later, larger call allocates a new one and keeps
 *     the old one, so captured graphs stay valid.  moe_release, and freeing or reusing a
 *     caller workspace (moe_set_workspace), invalidate the graphs captured on it.
 *   - Workspace: a thread that called moe_set_workspace uses its own caller-owned buffer;
 *     every other thread shares the library-owned one, reused from call to call.  Calls
 *     that run concurrently (other threads, other streams) on the same buffer race on it:
 *     serialise them, or give each thread its own buffer with moe_set_workspace.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FMT_BF16 0
#define MOE_FMT_MXFP4 1
#define MOE_FMT_MXFP8 2

/* GPT-OSS SwiGLU constants: the torchtitan guide names alpha and limit but prints no
 * value; these are the published GPT-OSS defaults (alpha = 1.702 is the sigmoid
 * approximation of GELU, Hendrycks & Gimpel 2016). */
#define MOE_SWIGLU_ALPHA 1.702f
#define MOE_SWIGLU_LIMIT 7.0f

#define MOE_OK 0
#define MOE_EINVAL -1   /* bad shape, k, E, null pointer, or T*k overflow */
#define MOE_EFMT -2     /* unknown weight format */
#define MOE_EALIGN -3   /* a pointer is not 16-byte aligned */
#define MOE_ENOMEM -4   /* workspace allocation failed, or the caller's workspace is too small */
#define MOE_EHIP -5     /* a HIP runtime call failed (launch, event, device query) */

/* Whole block (steps 1-8).
 *   x        bf16 [T][D]
 *   router_w bf16 [E][D]             router_b bf16 [E]
 *   w1       fmt 0: bf16 [E][2F][D]; fmt 1: MXFP4 buffer (codes [E][2F][D/2], scales [E][2F][D/32]);
 *            fmt 2: MXFP8 buffer (codes [E][2F][D], scales [E][2F][D/32])
 *   b1       bf16 [E][2F]            ([0,F) gate half, [F,2F) linear half)
 *   w2       fmt 0: bf16 [E][D][F];  fmt 1: MXFP4 buffer (codes [E][D][F/2],  scales [E][D][F/32]);
 *            fmt 2: MXFP8 buffer (codes [E][D][F], scales [E][D][F/32])
 *   b2       bf16 [E][D]
 *   out      fp32 [T][D] (written)
 * Ordering is that of the calling thread's stream.  With MXFP4 weights at many routed rows
 * per expert (the scaled matrix-core engine) and outside graph capture, the split of x into
 * fp8 pieces runs beside the top-k and the grouping on the calling thread's second stream
 * (the one moe_backward uses), which waits for the calling stream's earlier work (through
 * the router) and which the calling stream waits for before mlp1; under capture it runs on
 * the calling stream.
 */
int moe_forward(const void* x, const void* router_w, const void* router_b,
                const void* w1, const void* b1, const void* w2, const void* b2,
                int64_t T, int64_t D, int64_t E, int64_t k, int64_t F,
                int fmt, float* out);

/* moe_forward for callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, same
 * kernels and bitwise the same result as moe_forward, but the intermediates live in a fixed
 * scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends, instead of the workspace: no hipMalloc, hipFree or allocating call
 * is made.  A shape whose intermediates exceed the scratch (moe_workspace_bytes) fails with
 * MOE_ENOMEM before any launch; at the 20B shape (D = F = 2880, 32 experts, top-4) that is
 * above 873 tokens with bf16 weights and above 671 with MXFP4 or MXFP8 ones.  All calls on one GPU share its scratch
 * array: calls that overlap in time on that GPU (other streams, other threads) race on it and
 * must be serialised.  Nothing in the scratch needs to start at zero; it keeps the last call's
 * intermediates.  Not timed by moe_profile_*. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const void* x, const void* router_w, const void* router_b,
                        const void* w1, const void* b1, const void* w2, const void* b2,
                        int64_t T, int64_t D, int64_t E, int64_t k, int64_t F,
                        int fmt, float* out);

/* Steps 1-4 only (routing stage; its integer outputs are exact).
 *   logits   fp32 [T][E] or NULL     topk_idx int32 [T][k]    gates fp32 [T][k]
 *   counts   int32 [E]               offsets  int32 [E+1]     perm  int32 [T*k]
 */
int moe_route(const void* x, const void* router_w, const void* router_b,
              int64_t T, int64_t D, int64_t E, int64_t k,
              float* logits, int32_t* topk_idx, float* gates,
              int32_t* counts, int32_t* offsets, int32_t* perm);

/* The same with a load-balancing expert bias (torchtitan guide, section "StateDict
 * adapter": a per-expert bias buffer kept beside the router during training, rebuilt as
 * zeros when a checkpoint is loaded).  expert_bias is fp32 [E] in device memory.  It moves
 * the selection only: step 2 ranks the fp32 sums l[t,e] + expert_bias[e] (one rounding,
 * ties to the lower index; slot j holds the j-th largest sum), while step 3's gates remain
 * the softmax of the selected unbiased logits, and logits (when not NULL) receives the
 * unbiased l.  An all-zero bias gives exactly the unbiased calls' results.  expert_bias
 * must be non-null and 16-byte aligned whenever T > 0. */
int moe_forward_biased(const void* x, const void* router_w, const void* router_b, const float* expert_bias,
                       const void* w1, const void* b1, const void* w2, const void* b2,
                       int64_t T, int64_t D, int64_t E, int64_t k, int64_t F,
                       int fmt, float* out);
int moe_route_biased(const void* x, const void* router_w, const void* router_b, const float* expert_bias,
                     int64_t T, int64_t D, int64_t E, int64_t k,
                     float* logits, int32_t* topk_idx, float* gates,
                     int32_t* counts, int32_t* offsets, int32_t* perm);

/* One load-balancing step of the expert bias, in place (torchtitan guide, section
 * "StateDict adapter": a hook run after each optimizer step with load_balance_coeff = 1e-3;
 * the rule is the auxiliary-loss-free balancing of the DeepSeek-V3 report).  counts is int32
 * [E] (e.g. moe_route's), expert_bias fp32 [E], both device memory; 1 <= E <= 256, coeff
 * finite.  Expert e's bias becomes expert_bias[e] - coeff if counts[e] exceeds the mean
 * count, + coeff if it falls below it, and is left untouched at the mean (one fp32
 * rounding).  Asynchronous on the calling thread's stream; with profiling on, its time
 * counts under stage 1 (top-k).  Needs no workspace. */
int moe_update_expert_bias(const int32_t* counts, int64_t E, float coeff, float* expert_bias);

/* Steps 5-8 on a given routing (expert stage), e.g. the routing of moe_route or of a
 * reference: the stage isolation of the "gptoss" re-implementation page, section 测试说明
 * (testing notes: each layer can be verified on the reference's inputs rather than on its
 * own upstream output).  gates fp32 [T][k], offsets int32 [E+1] and perm int32 [T*k] must
 * be consistent (as moe_route produces them: perm[offsets[e] .. offsets[e+1]) lists the
 * assignments t*k+j routed to expert e); inconsistent routing is outside the contract, but
 * rows outside [0, T*k) are skipped, never dereferenced.  The expert of a row is the group
 * it sits in and its token and slot come from its assignment id, so the top-k index array
 * would repeat what offsets and perm already say: it is not an argument.  Other arguments
 * as in moe_forward. */
int moe_experts(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
                const float* gates, const int32_t* offsets, const int32_t* perm,
                int64_t T, int64_t D, int64_t E, int64_t k, int64_t F,
                int fmt, float* out);

/* Gradients of the block (bf16 expert weights only), with the routing of the forward held
 * fixed: the torchtitan guide's grouped GEMM section trains this block and unit-tests the
 * gradient of its SwiGLU variant.  The top-k selection is piecewise constant, so gradients
 * reach the router through the softmax gates only, and never the load-balancing bias.
 * Readings: a clamp passes the gradient where its input lies inside the closed interval
 * (gate <= LIMIT; -LIMIT <= linear <= LIMIT); the logits are differentiated as exact reals.
 *   inputs   x, router_w, w1, b1, w2, b2 as in moe_forward (fmt must be MOE_FMT_BF16; the
 *            router bias is not needed); topk_idx int32 [T][k], gates fp32 [T][k], offsets
 *            int32 [E+1], perm int32 [T*k]: the routing of the forward as moe_route returns it;
 *            dout fp32 [T][D], the gradient of the loss with respect to out.
 *   outputs  (fp32, fully overwritten) dx [T][D], d_router_w [E][D], d_router_b [E],
 *            dw1 [E][2F][D], db1 [E][2F], dw2 [E][D][F], db2 [E][D].
 * Per assignment a = t*k + j with expert e and gate g, u = x W1[e]^T + b1[e] is recomputed;
 * dz = g dout[t] gives dW2[e] += dz^T h and db2[e] += dz; du = SwiGLU'(u) (dz W2[e]) gives
 * dW1[e] += du^T x[t], db1[e] += du and dx[t] += du W1[e]; dg = <dout[t], h W2[e]^T + b2[e]>;
 * the softmax over the selected logits gives dl = g (dg - sum_j g_j dg_j), then
 * d_router_w[e] += dl x[t], d_router_b[e] += dl and dx[t] += dl router_w[e].  The matrix
 * products run on the bf16 matrix cores with fp32 accumulation (the products over routed rows
 * on the forward's grouped GEMM kernels, the weights read as stored): dout enters
 * the product with W2 as a bf16 pair (hi + lo, about 16 significant bits), while dz, du and h
 * enter theirs rounded to bf16, which bounds the relative error of each gradient near 2^-9;
 * every sum has a fixed order, so the result is bitwise reproducible.  With
 * T = 0 the parameter gradients are set to zero.  Uses moe_backward_workspace_bytes of
 * workspace (the same workspace rules as the forward).  Timed as stage 7 by moe_profile_*.
 * Ordering is that of the calling thread's stream: at many routed rows per expert and
 * outside graph capture the memory-bound side work runs on a second stream the library keeps
 * per thread (default priority, created on the thread's first such call, destroyed by that
 * thread's moe_release), which waits for the calling stream's earlier work and which the
 * calling stream waits for before the call's last kernel; under capture all of it runs on
 * the calling stream. */
int moe_backward(const void* x, const void* router_w, const void* w1, const void* b1,
                 const void* w2, const void* b2,
                 const int32_t* topk_idx, const float* gates, const int32_t* offsets, const int32_t* perm,
                 const float* dout,
                 int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt,
                 float* dx, float* d_router_w, float* d_router_b,
                 float* dw1, float* db1, float* dw2, float* db2);

/* Device bytes of workspace a moe_backward call of this shape needs (0 for T == 0 or a
 * format the backward does not take). */
size_t moe_backward_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt);

/* Stream for the calling thread's subsequent calls (a hipStream_t; NULL = default stream). */
int moe_set_stream(void* hip_stream);

/* Device bytes of workspace a moe_forward call of this shape needs (0 for T == 0). */
size_t moe_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt);

/* Use caller-owned device memory as the calling thread's workspace (256-byte aligned) for
 * its later calls; other threads are not affected.  Calls whose need exceeds `bytes` fail
 * with MOE_ENOMEM before launching anything.  Passing NULL returns the thread to the shared
 * library-owned workspace, which grows on demand with hipMalloc and is kept until
 * moe_release. */
int moe_set_workspace(void* dev_ptr, size_t bytes);

/* Message for the calling thread's last failing call ("" if none). */
const char* moe_last_error(void);

/* Free the library-owned workspace (with the buffers kept for captured graphs), the
 * profiling events and the calling thread's second stream (forward split, backward side
 * work), and return the calling
 * thread to the library-owned workspace.  Must not run while work that uses the workspace is
 * queued or a captured graph may still replay. */
void moe_release(void);

/* Kernel timing (tracing): while enabled, every launch is bracketed by HIP events on the
 * call's stream, and each kernel's summed device time and launch count accumulate per
 * stage.  Stages: 0 router, 1 top-k, 2 permute, 3 mlp1, 4 mlp2, 5 combine, 6 split (the
 * fp8 pieces of x that the scaled matrix-core engine reads; MXFP4 weights
 * at large token counts only), 7 backward (a whole moe_backward call).  moe_profile_read
 * synchronises on the recorded events; it fills ms[8] and launches[8] (either may be NULL)
 * and resets the counters. */
#define MOE_NUM_STAGES 8
int moe_profile_enable(int on);
int moe_profile_read(double* ms, int64_t* launches);

/* Library build string (architecture and tile configuration). */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

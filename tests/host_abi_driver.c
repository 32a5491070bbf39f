/* Host-side exercise of the C ABI for the sanitizer build (no GPU, no kernel launch).
 *
 * Every entry point is called with the argument errors it must reject (shapes at and far
 * beyond their limits, null and misaligned pointers, unknown formats), the workspace-size
 * queries are swept over many shapes, and the per-thread caller workspace is exercised
 * from several threads.  Under AddressSanitizer and UndefinedBehaviorSanitizer any
 * out-of-bounds access, use after free, signed overflow or misaligned access in the host
 * layer ends the program with a report.  Exit status 0 means every check held. */
#include <inttypes.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

/* fake 16-byte aligned device addresses: only passed to calls that must fail validation */
#define P ((void*)(uintptr_t)0x10000)
#define BAD ((void*)(uintptr_t)0x10008)

static int fwd(void* const p[8], int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt) {
  return moe_forward(p[0], p[1], p[2], p[3], p[4], p[5], p[6], T, D, E, k, F, fmt, (float*)p[7]);
}

static int bwd(void* const p[19], int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt) {
  return moe_backward(p[0], p[1], p[2], p[3], p[4], p[5], (const int32_t*)p[6], (const float*)p[7],
                      (const int32_t*)p[8], (const int32_t*)p[9], (const float*)p[10], T, D, E, k, F, fmt,
                      (float*)p[11], (float*)p[12], (float*)p[13], (float*)p[14], (float*)p[15],
                      (float*)p[16], (float*)p[17]);
}

struct shape { int64_t T, D, E, k, F; int rc; int f_only; }; /* f_only: invalid through F alone */

/* shapes at and beyond every limit the header states, including ones whose products
 * overflow 64-bit integers if they were formed before the bounds were checked */
static const struct shape BAD_SHAPES[] = {
    {-1, 64, 4, 2, 64, MOE_EINVAL},
    {INT64_MIN, 64, 4, 2, 64, MOE_EINVAL},
    {8, 0, 4, 2, 64, MOE_EINVAL},
    {8, -64, 4, 2, 64, MOE_EINVAL},
    {8, 96, 4, 2, 64, MOE_EINVAL},
    {8, 64, 4, 2, 32, MOE_EINVAL, 1},
    {8, 64, 4, 2, 0, MOE_EINVAL, 1},
    {8, 64, 0, 1, 64, MOE_EINVAL},
    {8, 64, 257, 2, 64, MOE_EINVAL},
    {8, 64, INT64_MAX, 2, 64, MOE_EINVAL},
    {8, 64, 4, 0, 64, MOE_EINVAL},
    {8, 64, 4, 5, 64, MOE_EINVAL},
    {(int64_t)1 << 30, 64, 4, 2, 64, MOE_EINVAL},
    {(int64_t)1 << 62, 64, 256, 256, 64, MOE_EINVAL},
    {INT64_MAX, 64, 256, 256, 64, MOE_EINVAL},
    {INT64_MAX, INT64_MAX - 63, 256, 256, INT64_MAX - 63, MOE_EINVAL},
    {1, (int64_t)1 << 40, 4, 2, 64, MOE_EINVAL},
    {1, 64, 4, 2, (int64_t)1 << 40, MOE_EINVAL, 1},
    {1, INT64_MAX - 63, 4, 2, INT64_MAX - 63, MOE_EINVAL},
    {(int64_t)1 << 24, 64, 4, 2, 64, MOE_EINVAL},
    {(int64_t)1 << 22, 64, 4, 4, 64, MOE_EINVAL, 1},
    {1, (int64_t)1 << 15, 4, 2, (int64_t)1 << 15, MOE_EINVAL, 1},
};

static void bad_shapes(void) {
  void* p[19];
  for (int i = 0; i < 19; ++i) p[i] = P;
  for (size_t i = 0; i < sizeof BAD_SHAPES / sizeof BAD_SHAPES[0]; ++i) {
    const struct shape s = BAD_SHAPES[i];
    EXPECT(fwd(p, s.T, s.D, s.E, s.k, s.F, MOE_FMT_BF16) == s.rc);
    EXPECT(strlen(moe_last_error()) > 0);
    EXPECT(moe_forward_noalloc(P, P, P, P, P, P, P, s.T, s.D, s.E, s.k, s.F, MOE_FMT_MXFP4, (float*)P) == s.rc);
    EXPECT(moe_forward_biased(P, P, P, (const float*)P, P, P, P, P, s.T, s.D, s.E, s.k, s.F, MOE_FMT_MXFP8,
                              (float*)P) == s.rc);
    EXPECT(moe_experts(P, P, P, P, P, (const float*)P, (const int32_t*)P, (const int32_t*)P, s.T, s.D, s.E,
                       s.k, s.F, MOE_FMT_BF16, (float*)P) == s.rc);
    EXPECT(bwd(p, s.T, s.D, s.E, s.k, s.F, MOE_FMT_BF16) == s.rc);
    EXPECT(moe_workspace_bytes(s.T, s.D, s.E, s.k, s.F, MOE_FMT_BF16) == 0);
    EXPECT(moe_backward_workspace_bytes(s.T, s.D, s.E, s.k, s.F, MOE_FMT_BF16) == 0);
    if (!s.f_only) { /* the routing calls take no F */
      EXPECT(moe_route(P, P, P, s.T, s.D, s.E, s.k, (float*)P, (int32_t*)P, (float*)P, (int32_t*)P,
                       (int32_t*)P, (int32_t*)P) == s.rc);
      EXPECT(moe_route_biased(P, P, P, (const float*)P, s.T, s.D, s.E, s.k, NULL, (int32_t*)P, (float*)P,
                              (int32_t*)P, (int32_t*)P, (int32_t*)P) == s.rc);
    }
  }
  /* formats */
  EXPECT(fwd(p, 8, 64, 4, 2, 64, 3) == MOE_EFMT);
  EXPECT(fwd(p, 8, 64, 4, 2, 64, -1) == MOE_EFMT);
  EXPECT(bwd(p, 8, 64, 4, 2, 64, MOE_FMT_MXFP4) == MOE_EFMT);
  EXPECT(bwd(p, 8, 64, 4, 2, 64, 7) == MOE_EFMT);
  EXPECT(moe_workspace_bytes(8, 64, 4, 2, 64, 3) == 0);
  EXPECT(moe_backward_workspace_bytes(8, 64, 4, 2, 64, MOE_FMT_MXFP8) == 0);
  /* the bias update */
  EXPECT(moe_update_expert_bias((const int32_t*)P, 0, 1e-3f, (float*)P) == MOE_EINVAL);
  EXPECT(moe_update_expert_bias((const int32_t*)P, 300, 1e-3f, (float*)P) == MOE_EINVAL);
  EXPECT(moe_update_expert_bias((const int32_t*)P, INT64_MIN, 1e-3f, (float*)P) == MOE_EINVAL);
  EXPECT(moe_update_expert_bias((const int32_t*)P, 8, 1.0f / 0.0f, (float*)P) == MOE_EINVAL);
  EXPECT(moe_update_expert_bias(NULL, 8, 1e-3f, (float*)P) == MOE_EINVAL);
  EXPECT(moe_update_expert_bias((const int32_t*)P, 8, 1e-3f, (float*)BAD) == MOE_EALIGN);
}

static void bad_pointers(void) {
  for (int which = 0; which < 8; ++which) {
    void* p[8];
    for (int i = 0; i < 8; ++i) p[i] = P;
    p[which] = NULL;
    EXPECT(fwd(p, 8, 64, 4, 2, 64, MOE_FMT_BF16) == MOE_EINVAL);
    p[which] = BAD;
    EXPECT(fwd(p, 8, 64, 4, 2, 64, MOE_FMT_BF16) == MOE_EALIGN);
    EXPECT(strstr(moe_last_error(), "aligned") != NULL);
  }
  for (int which = 0; which < 18; ++which) { /* moe_backward's 18 pointers */
    void* p[19];
    for (int i = 0; i < 19; ++i) p[i] = P;
    p[which] = NULL;
    EXPECT(bwd(p, 8, 64, 4, 2, 64, MOE_FMT_BF16) == MOE_EINVAL);
    p[which] = BAD;
    EXPECT(bwd(p, 8, 64, 4, 2, 64, MOE_FMT_BF16) == MOE_EALIGN);
  }
  EXPECT(moe_route(P, P, P, 8, 64, 4, 2, (float*)BAD, (int32_t*)P, (float*)P, (int32_t*)P, (int32_t*)P,
                   (int32_t*)P) == MOE_EALIGN);
  EXPECT(moe_route_biased(P, P, P, NULL, 8, 64, 4, 2, NULL, (int32_t*)P, (float*)P, (int32_t*)P, (int32_t*)P,
                          (int32_t*)P) == MOE_EINVAL);
  EXPECT(moe_forward_biased(P, P, P, (const float*)BAD, P, P, P, P, 8, 64, 4, 2, 64, MOE_FMT_BF16,
                            (float*)P) == MOE_EALIGN);
}

static void zero_tokens(void) {
  /* T = 0 launches nothing: pointers may be null */
  EXPECT(moe_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 4, 2, 64, MOE_FMT_MXFP8, NULL) == MOE_OK);
  EXPECT(moe_forward_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 4, 2, 64, MOE_FMT_BF16, NULL) ==
         MOE_OK);
  EXPECT(moe_route(NULL, NULL, NULL, 0, 64, 4, 2, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  EXPECT(moe_experts(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 4, 2, 64, MOE_FMT_MXFP4, NULL) ==
         MOE_OK);
  EXPECT(strcmp(moe_last_error(), "") == 0);
  EXPECT(moe_workspace_bytes(0, 64, 4, 2, 64, MOE_FMT_BF16) == 0);
  EXPECT(moe_backward_workspace_bytes(0, 64, 4, 2, 64, MOE_FMT_BF16) == 0);
}

static void workspace_sizes(void) {
  static const int64_t Ts[] = {1, 2, 63, 64, 65, 255, 256, 1000, 4096, 8192, 16384, 65536, 1 << 20};
  static const int64_t DFs[][2] = {{64, 64}, {64, 128}, {192, 64}, {2880, 2880}, {4096, 1024}};
  static const int64_t Eks[][2] = {{1, 1}, {4, 2}, {8, 8}, {32, 4}, {128, 4}, {256, 8}, {256, 256}};
  for (size_t a = 0; a < sizeof DFs / sizeof DFs[0]; ++a)
    for (size_t b = 0; b < sizeof Eks / sizeof Eks[0]; ++b)
      for (int fmt = 0; fmt < 3; ++fmt)
        for (size_t c = 0; c < sizeof Ts / sizeof Ts[0]; ++c) {
          const int64_t T = Ts[c], D = DFs[a][0], F = DFs[a][1], E = Eks[b][0], k = Eks[b][1];
          const size_t w = moe_workspace_bytes(T, D, E, k, F, fmt);
          const size_t wb = moe_backward_workspace_bytes(T, D, E, k, F, fmt);
          EXPECT(w == moe_workspace_bytes(T, D, E, k, F, fmt));
          if (w == 0) continue; /* beyond a limit */
          /* at least the routing's own outputs (indices, gates, permutation) */
          EXPECT(w >= (size_t)(T * k) * 12);
          EXPECT(w % 256 == 0);
          if (fmt != MOE_FMT_BF16) EXPECT(wb == 0);
          else if (wb) EXPECT(wb % 256 == 0 && wb >= (size_t)(T * k) * (size_t)(2 * F) * 4);
        }
}

struct thread_arg { size_t size; int rc; char msg[256]; };

static void* thread_main(void* v) {
  struct thread_arg* a = (struct thread_arg*)v;
  void* p[8];
  for (int i = 0; i < 8; ++i) p[i] = P;
  if (moe_set_workspace((void*)(uintptr_t)0x200000, a->size) != MOE_OK) {
    a->rc = 1;
    return NULL;
  }
  a->rc = fwd(p, 256, 2880, 32, 4, 2880, MOE_FMT_BF16);
  snprintf(a->msg, sizeof a->msg, "%s", moe_last_error());
  moe_set_workspace(NULL, 0);
  return NULL;
}

static void caller_workspace(void) {
  void* p[8];
  for (int i = 0; i < 8; ++i) p[i] = P;
  EXPECT(moe_set_workspace((void*)(uintptr_t)0x1010, 4096) == MOE_EALIGN);
  EXPECT(moe_set_workspace((void*)(uintptr_t)0x100000, 4096) == MOE_OK);
  EXPECT(fwd(p, 256, 2880, 32, 4, 2880, MOE_FMT_BF16) == MOE_ENOMEM);
  EXPECT(strstr(moe_last_error(), "4096") != NULL);
  EXPECT(moe_experts(P, P, P, P, P, (const float*)P, (const int32_t*)P, (const int32_t*)P, 256, 2880, 32, 4,
                     2880, MOE_FMT_MXFP4, (float*)P) == MOE_ENOMEM);
  EXPECT(bwd((void* [19]){P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P}, 256, 2880, 32, 4, 2880,
             MOE_FMT_BF16) == MOE_ENOMEM);
  struct thread_arg args[4] = {{4096, 0, ""}, {8192, 0, ""}, {12288, 0, ""}, {1u << 20, 0, ""}};
  pthread_t th[4];
  for (int i = 0; i < 4; ++i) EXPECT(pthread_create(&th[i], NULL, thread_main, &args[i]) == 0);
  for (int i = 0; i < 4; ++i) pthread_join(th[i], NULL);
  for (int i = 0; i < 4; ++i) {
    char want[64];
    snprintf(want, sizeof want, "holds %zu bytes", args[i].size);
    EXPECT(args[i].rc == MOE_ENOMEM);
    EXPECT(strstr(args[i].msg, want) != NULL);
  }
  /* this thread kept its own 4096-byte workspace */
  EXPECT(fwd(p, 256, 2880, 32, 4, 2880, MOE_FMT_BF16) == MOE_ENOMEM);
  EXPECT(strstr(moe_last_error(), "holds 4096 bytes") != NULL);
  EXPECT(moe_set_workspace(NULL, 0) == MOE_OK);
  /* beyond the fixed scratch: rejected before any device call */
  EXPECT(moe_forward_noalloc(P, P, P, P, P, P, P, 8192, 2880, 32, 4, 2880, MOE_FMT_BF16, (float*)P) ==
         MOE_ENOMEM);
  EXPECT(strstr(moe_last_error(), "scratch") != NULL);
}

static void profiling_and_misc(void) {
  double ms[MOE_NUM_STAGES];
  int64_t n[MOE_NUM_STAGES];
  EXPECT(moe_profile_enable(1) == MOE_OK);
  EXPECT(moe_profile_read(ms, n) == MOE_OK); /* nothing recorded: all zero */
  for (int s = 0; s < MOE_NUM_STAGES; ++s) EXPECT(ms[s] == 0.0 && n[s] == 0);
  EXPECT(moe_profile_read(NULL, NULL) == MOE_OK);
  EXPECT(moe_profile_enable(0) == MOE_OK);
  EXPECT(moe_set_stream(NULL) == MOE_OK);
  EXPECT(strstr(moe_version(), "gfx950") != NULL);
  moe_release();
  moe_release();
}

int main(void) {
  bad_shapes();
  bad_pointers();
  zero_tokens();
  workspace_sizes();
  caller_workspace();
  profiling_and_misc();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}

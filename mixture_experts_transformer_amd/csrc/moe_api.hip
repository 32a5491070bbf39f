// C ABI of the MoE block: argument validation (host only, before any HIP call),
// workspace management, the calling thread's stream, kernel timing, and the launch
// sequence router -> top-k -> grouping -> mlp1 -> mlp2 -> combine.  Nothing here reads
// device data back: the expert counts stay on the device and the expert stage sizes
// its grid by an upper bound.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;
thread_local hipStream_t g_stream = nullptr;

struct Workspace {
  std::mutex mu;
  void* ptr = nullptr;
  size_t size = 0;
  bool user = false;
};
Workspace g_ws;

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;     // pool
  std::vector<int> stage;                  // stage of each recorded pair
  size_t used = 0;
};
Profiler g_prof;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t partial = 0, hist = 0, idx = 0, gates = 0, counts = 0, offsets = 0, perm = 0;
  size_t h = 0, h_lo = 0, xq = 0, xs = 0, hq = 0, hs = 0, y = 0, total = 0;
};

bool valid_fmt(int fmt) { return fmt == MOE_FMT_BF16 || fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_MXFP8; }

enum Need { NEED_ROUTE = 1, NEED_EXPERTS = 2, NEED_ROUTE_OUTPUTS = 4 };

Layout layout(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt, int need) {
  Layout L;
  const size_t A = (size_t)T * (size_t)k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  if (need & NEED_ROUTE) {
    L.partial = take((size_t)moe::router_ksplit(T, D) * T * E * sizeof(double));
    L.hist = take((size_t)moe::permute_groups(A) * E * 4);
  }
  if (need & NEED_ROUTE_OUTPUTS) {
    L.idx = take(A * 4);
    L.gates = take(A * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.perm = take(A * 4);
  }
  if (need & NEED_EXPERTS) {
    if (moe::mx_engine(fmt, moe::expert_tile_config((int64_t)A, E))) {
      L.xq = take(2 * (size_t)T * D);
      L.xs = take((size_t)T * moe::mx_scale_stride((int)D) * 4);
      L.hq = take(3 * A * (size_t)F);
      L.hs = take(A * (size_t)moe::mx_scale_stride((int)F) * 4);
    } else {
      L.h = take(A * (size_t)F * 2);
      if (fmt != MOE_FMT_BF16) L.h_lo = take(A * (size_t)F * 2);
    }
    L.y = take(A * (size_t)D * 4);
  }
  L.total = off;
  return L;
}

int check_shapes(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, bool with_f) {
  if (T < 0) return fail(MOE_EINVAL, "T = %lld must be >= 0", (long long)T);
  if (D <= 0 || D % 64 != 0) return fail(MOE_EINVAL, "D = %lld must be a positive multiple of 64", (long long)D);
  if (with_f && (F <= 0 || F % 64 != 0))
    return fail(MOE_EINVAL, "F = %lld must be a positive multiple of 64", (long long)F);
  if (E < 1 || E > 256) return fail(MOE_EINVAL, "E = %lld must be in [1, 256]", (long long)E);
  if (k < 1 || k > E) return fail(MOE_EINVAL, "k = %lld must be in [1, E = %lld]", (long long)k, (long long)E);
  if (T * k >= ((int64_t)1 << 31)) return fail(MOE_EINVAL, "T*k = %lld must be < 2^31", (long long)(T * k));
  if (D >= ((int64_t)1 << 24) || (with_f && F >= ((int64_t)1 << 24)))
    return fail(MOE_EINVAL, "D and F must be < 2^24");
  // the expert kernels address rows of x, h and one expert's weights with 32-bit offsets
  if (T * D >= ((int64_t)1 << 30) || (with_f && (T * k * F >= ((int64_t)1 << 30) || D * F >= ((int64_t)1 << 30))))
    return fail(MOE_EINVAL, "T*D, T*k*F and D*F must each be < 2^30");
  return MOE_OK;
}

int check_ptr(const void* p, const char* name, bool nullable = false) {
  if (!p) return nullable ? MOE_OK : fail(MOE_EINVAL, "%s is NULL", name);
  if (((uintptr_t)p) & 15) return fail(MOE_EALIGN, "%s = %p is not 16-byte aligned", name, p);
  return MOE_OK;
}

#define CHECK(expr)              \
  do {                           \
    const int _rc = (expr);      \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

int ensure_workspace(size_t bytes, uint8_t** base) {
  std::lock_guard<std::mutex> lk(g_ws.mu);
  if (g_ws.user) {
    if (g_ws.size < bytes)
      return fail(MOE_ENOMEM, "caller workspace holds %zu bytes, the call needs %zu", g_ws.size, bytes);
    *base = (uint8_t*)g_ws.ptr;
    return MOE_OK;
  }
  if (g_ws.size < bytes) {
    if (g_ws.ptr) {
      hipError_t e = hipFree(g_ws.ptr);   // waits for queued work that may still use it
      g_ws.ptr = nullptr;
      g_ws.size = 0;
      if (e != hipSuccess) return fail(MOE_EHIP, "hipFree(workspace): %s", hipGetErrorString(e));
    }
    const size_t want = align256(bytes + bytes / 4);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, want);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(MOE_ENOMEM, "hipMalloc(%zu) for the workspace failed: %s", want, hipGetErrorString(e));
    }
    g_ws.ptr = p;
    g_ws.size = want;
  }
  *base = (uint8_t*)g_ws.ptr;
  return MOE_OK;
}

// Launch wrapper: optional event bracketing, error translation.
template <class F>
int launch(int stage, const char* name, F&& fn) {
  hipStream_t st = g_stream;
  hipEvent_t a = nullptr, b = nullptr;
  bool prof = false;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.on) {
      if (g_prof.used == g_prof.start.size()) {
        hipEvent_t s0, s1;
        if (hipEventCreate(&s0) != hipSuccess || hipEventCreate(&s1) != hipSuccess)
          return fail(MOE_EHIP, "hipEventCreate failed");
        g_prof.start.push_back(s0);
        g_prof.stop.push_back(s1);
        g_prof.stage.push_back(0);
      }
      a = g_prof.start[g_prof.used];
      b = g_prof.stop[g_prof.used];
      g_prof.stage[g_prof.used] = stage;
      ++g_prof.used;
      prof = true;
    }
  }
  if (prof && hipEventRecord(a, st) != hipSuccess) return fail(MOE_EHIP, "hipEventRecord failed");
  hipError_t e = fn(st);
  if (e != hipSuccess) return fail(MOE_EHIP, "%s launch failed: %s", name, hipGetErrorString(e));
  if (prof && hipEventRecord(b, st) != hipSuccess) return fail(MOE_EHIP, "hipEventRecord failed");
  return MOE_OK;
}

// router -> top-k -> grouping
int run_route(uint8_t* ws, const Layout& L, const void* x, const void* router_w, const void* router_b,
              const float* ebias, int64_t T, int64_t D, int64_t E, int64_t k, float* logits, int32_t* idx,
              float* gates, int32_t* counts, int32_t* offsets, int32_t* perm) {
  double* partial = (double*)(ws + L.partial);
  const int ks = moe::router_ksplit(T, D);
  CHECK(launch(moe::ST_ROUTER, "router", [&](hipStream_t st) {
    return moe::launch_router_partial((const uint16_t*)x, (const uint16_t*)router_w, (int)T, (int)D, (int)E, ks,
                                      partial, st);
  }));
  CHECK(launch(moe::ST_TOPK, "topk", [&](hipStream_t st) {
    return moe::launch_topk(partial, ks, (const uint16_t*)router_b, ebias, (int)T, (int)E, (int)k, logits, idx,
                            gates, st);
  }));
  return launch(moe::ST_PERMUTE, "permute", [&](hipStream_t st) {
    return moe::launch_permute(idx, (int)(T * k), (int)E, (int32_t*)(ws + L.hist), counts, offsets, perm, st);
  });
}

int run_experts(const uint8_t* ws, const Layout& L, const void* x, const void* w1, const void* b1,
                const void* w2, const void* b2, const float* gates, const int32_t* offsets,
                const int32_t* perm, int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt,
                float* out) {
  moe::ExpertArgs ea{};
  ea.x = (const uint16_t*)x;
  ea.w1 = w1;
  ea.b1 = (const uint16_t*)b1;
  ea.w2 = w2;
  ea.b2 = (const uint16_t*)b2;
  ea.gates = gates;
  ea.offsets = offsets;
  ea.perm = perm;
  ea.h = (uint16_t*)(ws + L.h);
  ea.h_lo = fmt != MOE_FMT_BF16 ? (uint16_t*)(ws + L.h_lo) : nullptr;
  ea.y = (float*)(ws + L.y);
  ea.xq = (uint8_t*)(ws + L.xq);
  ea.xs = (uint32_t*)(ws + L.xs);
  ea.hq = (uint8_t*)(ws + L.hq);
  ea.hs = (uint32_t*)(ws + L.hs);
  ea.out = out;
  ea.T = (int)T; ea.D = (int)D; ea.E = (int)E; ea.k = (int)k; ea.F = (int)F; ea.fmt = fmt;
  const int cfg = moe::expert_tile_config(T * k, E);
  if (moe::mx_engine(fmt, cfg))
    CHECK(launch(moe::ST_SPLIT, "split", [&](hipStream_t st) {
      return moe::launch_mx_split(ea.x, T, (int)D, ea.xq, ea.xs, st);
    }));
  CHECK(launch(moe::ST_MLP1, "mlp1", [&](hipStream_t st) { return moe::launch_mlp1(ea, cfg, st); }));
  CHECK(launch(moe::ST_MLP2, "mlp2", [&](hipStream_t st) { return moe::launch_mlp2(ea, cfg, st); }));
  CHECK(launch(moe::ST_COMBINE, "combine",
               [&](hipStream_t st) { return moe::launch_combine(ea.y, ea.T, ea.D, ea.k, out, st); }));
  return MOE_OK;
}

// Whole block; ebias is the load-balancing bias when `biased` (then it must be valid).
int forward_impl(const void* x, const void* router_w, const void* router_b, bool biased, const float* ebias,
                 const void* w1, const void* b1, const void* w2, const void* b2, int64_t T, int64_t D, int64_t E,
                 int64_t k, int64_t F, int fmt, float* out) {
  CHECK(check_shapes(T, D, E, k, F, true));
  if (!valid_fmt(fmt)) return fail(MOE_EFMT, "unknown weight format %d", fmt);
  if (T == 0) return ok();
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(router_w, "router_w"));
  CHECK(check_ptr(router_b, "router_b"));
  if (biased) CHECK(check_ptr(ebias, "expert_bias"));
  CHECK(check_ptr(w1, "w1"));
  CHECK(check_ptr(b1, "b1"));
  CHECK(check_ptr(w2, "w2"));
  CHECK(check_ptr(b2, "b2"));
  CHECK(check_ptr(out, "out"));
  const Layout L = layout(T, D, E, k, F, fmt, NEED_ROUTE | NEED_ROUTE_OUTPUTS | NEED_EXPERTS);
  uint8_t* ws = nullptr;
  CHECK(ensure_workspace(L.total, &ws));
  int32_t* idx = (int32_t*)(ws + L.idx);
  float* gates = (float*)(ws + L.gates);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* perm = (int32_t*)(ws + L.perm);
  CHECK(run_route(ws, L, x, router_w, router_b, ebias, T, D, E, k, nullptr, idx, gates, counts, offsets, perm));
  CHECK(run_experts(ws, L, x, w1, b1, w2, b2, gates, offsets, perm, T, D, E, k, F, fmt, out));
  return ok();
}

int route_impl(const void* x, const void* router_w, const void* router_b, bool biased, const float* ebias,
               int64_t T, int64_t D, int64_t E, int64_t k, float* logits, int32_t* topk_idx, float* gates,
               int32_t* counts, int32_t* offsets, int32_t* perm) {
  CHECK(check_shapes(T, D, E, k, 64, false));
  if (T == 0) return ok();
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(router_w, "router_w"));
  CHECK(check_ptr(router_b, "router_b"));
  if (biased) CHECK(check_ptr(ebias, "expert_bias"));
  CHECK(check_ptr(logits, "logits", true));
  CHECK(check_ptr(topk_idx, "topk_idx"));
  CHECK(check_ptr(gates, "gates"));
  CHECK(check_ptr(counts, "counts"));
  CHECK(check_ptr(offsets, "offsets"));
  CHECK(check_ptr(perm, "perm"));
  const Layout L = layout(T, D, E, k, 64, MOE_FMT_BF16, NEED_ROUTE);
  uint8_t* ws = nullptr;
  CHECK(ensure_workspace(L.total, &ws));
  CHECK(run_route(ws, L, x, router_w, router_b, ebias, T, D, E, k, logits, topk_idx, gates, counts, offsets,
                  perm));
  return ok();
}

}  // namespace

extern "C" {

int moe_forward(const void* x, const void* router_w, const void* router_b, const void* w1,
                const void* b1, const void* w2, const void* b2, int64_t T, int64_t D, int64_t E,
                int64_t k, int64_t F, int fmt, float* out) {
  return forward_impl(x, router_w, router_b, false, nullptr, w1, b1, w2, b2, T, D, E, k, F, fmt, out);
}

int moe_forward_biased(const void* x, const void* router_w, const void* router_b, const float* expert_bias,
                       const void* w1, const void* b1, const void* w2, const void* b2, int64_t T, int64_t D,
                       int64_t E, int64_t k, int64_t F, int fmt, float* out) {
  return forward_impl(x, router_w, router_b, true, expert_bias, w1, b1, w2, b2, T, D, E, k, F, fmt, out);
}

int moe_route(const void* x, const void* router_w, const void* router_b, int64_t T, int64_t D, int64_t E,
              int64_t k, float* logits, int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets,
              int32_t* perm) {
  return route_impl(x, router_w, router_b, false, nullptr, T, D, E, k, logits, topk_idx, gates, counts, offsets, perm);
}

int moe_route_biased(const void* x, const void* router_w, const void* router_b, const float* expert_bias,
                     int64_t T, int64_t D, int64_t E, int64_t k, float* logits, int32_t* topk_idx, float* gates,
                     int32_t* counts, int32_t* offsets, int32_t* perm) {
  return route_impl(x, router_w, router_b, true, expert_bias, T, D, E, k, logits, topk_idx, gates, counts, offsets,
                    perm);
}

int moe_update_expert_bias(const int32_t* counts, int64_t E, float coeff, float* expert_bias) {
  if (E < 1 || E > 256) return fail(MOE_EINVAL, "E = %lld must lie in [1, 256]", (long long)E);
  if (!std::isfinite(coeff)) return fail(MOE_EINVAL, "coeff is not finite");
  CHECK(check_ptr(counts, "counts"));
  CHECK(check_ptr(expert_bias, "expert_bias"));
  CHECK(launch(moe::ST_TOPK, "bias_update", [&](hipStream_t st) {
    return moe::launch_bias_update(counts, (int)E, coeff, expert_bias, st);
  }));
  return ok();
}

int moe_experts(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
                const float* gates, const int32_t* offsets, const int32_t* perm, int64_t T, int64_t D,
                int64_t E, int64_t k, int64_t F, int fmt, float* out) {
  CHECK(check_shapes(T, D, E, k, F, true));
  if (!valid_fmt(fmt)) return fail(MOE_EFMT, "unknown weight format %d", fmt);
  if (T == 0) return ok();
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(w1, "w1"));
  CHECK(check_ptr(b1, "b1"));
  CHECK(check_ptr(w2, "w2"));
  CHECK(check_ptr(b2, "b2"));
  CHECK(check_ptr(gates, "gates"));
  CHECK(check_ptr(offsets, "offsets"));
  CHECK(check_ptr(perm, "perm"));
  CHECK(check_ptr(out, "out"));
  const Layout L = layout(T, D, E, k, F, fmt, NEED_EXPERTS);
  uint8_t* ws = nullptr;
  CHECK(ensure_workspace(L.total, &ws));
  CHECK(run_experts(ws, L, x, w1, b1, w2, b2, gates, offsets, perm, T, D, E, k, F, fmt, out));
  return ok();
}

int moe_set_stream(void* hip_stream) {
  g_stream = (hipStream_t)hip_stream;
  return ok();
}

size_t moe_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt) {
  if (check_shapes(T, D, E, k, F, true) != MOE_OK) return 0;
  if (!valid_fmt(fmt)) return 0;
  if (T == 0) return 0;
  return layout(T, D, E, k, F, fmt, NEED_ROUTE | NEED_ROUTE_OUTPUTS | NEED_EXPERTS).total;
}

int moe_set_workspace(void* dev_ptr, size_t bytes) {
  std::lock_guard<std::mutex> lk(g_ws.mu);
  if (dev_ptr && (((uintptr_t)dev_ptr) & 255))
    return fail(MOE_EALIGN, "workspace %p is not 256-byte aligned", dev_ptr);
  if (!g_ws.user && g_ws.ptr) {
    hipError_t e = hipFree(g_ws.ptr);
    if (e != hipSuccess) return fail(MOE_EHIP, "hipFree(workspace): %s", hipGetErrorString(e));
  }
  g_ws.ptr = dev_ptr;
  g_ws.size = dev_ptr ? bytes : 0;
  g_ws.user = dev_ptr != nullptr;
  return ok();
}

const char* moe_last_error(void) { return g_err.c_str(); }

void moe_release(void) {
  {
    std::lock_guard<std::mutex> lk(g_ws.mu);
    if (!g_ws.user && g_ws.ptr) (void)hipFree(g_ws.ptr);
    g_ws.ptr = nullptr;
    g_ws.size = 0;
    g_ws.user = false;
  }
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (auto e : g_prof.start) (void)hipEventDestroy(e);
  for (auto e : g_prof.stop) (void)hipEventDestroy(e);
  g_prof.start.clear();
  g_prof.stop.clear();
  g_prof.stage.clear();
  g_prof.used = 0;
}

int moe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  return ok();
}

int moe_profile_read(double* ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  double acc[MOE_NUM_STAGES] = {0};
  int64_t cnt[MOE_NUM_STAGES] = {0};
  for (size_t i = 0; i < g_prof.used; ++i) {
    if (hipEventSynchronize(g_prof.stop[i]) != hipSuccess) return fail(MOE_EHIP, "hipEventSynchronize failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof.start[i], g_prof.stop[i]) != hipSuccess)
      return fail(MOE_EHIP, "hipEventElapsedTime failed");
    acc[g_prof.stage[i]] += t;
    cnt[g_prof.stage[i]] += 1;
  }
  g_prof.used = 0;
  for (int s = 0; s < MOE_NUM_STAGES; ++s) {
    if (ms) ms[s] = acc[s];
    if (launches) launches[s] = cnt[s];
  }
  return ok();
}

const char* moe_version(void) {
  return "moe-mi355x gfx950: router fp64-MFMA, top-k wave argmax, grouped GEMM v_mfma_f32_32x32x16_bf16 "
         "(streaming tile 64x128; matrix-core tile 256x256) and, for MXFP4 on matrix-core tiles, "
         "v_mfma_scale_f32_32x32x64_f8f6f4 on fp8 activation pieces; combine fp32";
}

}  // extern "C"

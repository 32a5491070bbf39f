// C ABI of the MoE block: argument validation (host only, before any HIP call),
// workspace management, the calling thread's stream, kernel timing, and the launch
// sequence router -> top-k -> grouping -> mlp1 -> mlp2 -> combine.  Nothing here reads
// device data back: the expert counts stay on the device and the expert stage sizes
// its grid by an upper bound.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;
thread_local hipStream_t g_stream = nullptr;
thread_local bool t_noalloc = false;       // inside moe_forward_noalloc: no event bracketing

// Library-owned workspace, shared by the threads that have not set their own.  Once a call
// has run on a capturing stream, captured graphs may hold its address: from then on a
// larger buffer does not free the old one (it is retired, kept until moe_release), so the
// graphs stay valid.
struct Workspace {
  std::mutex mu;
  void* ptr = nullptr;
  size_t size = 0;
  bool pinned = false;                     // a captured graph may use ptr
  std::vector<void*> retired;              // earlier buffers captured graphs may still use
};
Workspace g_ws;

// Scratch of the allocation-free entry point: a file-scope device array, one copy per GPU
// that loads the library, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is passed to kernels.
__device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

struct ScratchTable {
  std::mutex mu;
  std::vector<uint8_t*> ptr;               // per device ordinal; null until looked up
};
ScratchTable g_scratch;

// A second stream and its join events, per thread (created on first use on the thread's
// current device, default priority, non-blocking; destroyed by moe_release): the backward's
// side products, and the forward's split of x into fp8 pieces beside the routing.
struct SideStream {
  moe::BwdSide side{};
  int device = -1;
  bool made = false;
};
thread_local SideStream t_side;

void drop_side() {
  if (!t_side.made) return;
  (void)hipStreamDestroy(t_side.side.stream);
  for (auto e : t_side.side.ev) (void)hipEventDestroy(e);
  t_side = SideStream{};
}

// Caller-owned workspace of the calling thread (moe_set_workspace).
struct UserWorkspace {
  void* ptr = nullptr;
  size_t size = 0;
};
thread_local UserWorkspace t_user_ws;

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

// Backward workspace (moe_backward), one allocation.
struct BwdLayout {
  size_t poff = 0, padmap = 0, dout_perm = 0, ones = 0, zeros = 0, xT = 0, dzT = 0, u = 0;
  size_t h = 0, du = 0, dgsum = 0, dxs = 0, hT = 0, duT = 0, dl = 0, part_w = 0, part_b2 = 0, part_b1 = 0;
  size_t total = 0;
};

BwdLayout bwd_layout(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F) {
  BwdLayout L;
  const size_t A = (size_t)T * (size_t)k, G = 2 * (size_t)F, DF = (size_t)(D > F ? D : F);
  const size_t ldt = (size_t)moe::bwd_padded_cols((int64_t)A, E);
  const size_t ch = (size_t)moe::bwd_sum_chunks();
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.poff = take((2 * (size_t)E + 1) * 4);
  L.padmap = take(ldt * 4);
  L.dout_perm = take(A * 2 * D * 2);
  L.ones = take(A * 4);
  L.zeros = take((size_t)E * DF * 2);
  L.xT = take((size_t)D * ldt * 2);
  L.dzT = take((size_t)D * ldt * 2);
  L.u = take(A * G * 4);
  L.h = take(A * F * 2);
  L.du = take(A * G * 2);
  L.dgsum = take(A * 4);
  L.dxs = take(A * DF * 4);
  L.hT = take((size_t)F * ldt * 2);
  L.duT = take(G * ldt * 2);
  L.dl = take(A * 4);
  L.part_w = take(ch * E * D * 4);
  L.part_b2 = take(ch * E * D * 4);
  L.part_b1 = take(ch * E * G * 4);
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
  // bound T before forming a product with it (k <= E <= 256, so T*k cannot overflow after this)
  if (T >= ((int64_t)1 << 31) || T * k >= ((int64_t)1 << 31))
    return fail(MOE_EINVAL, "T*k = %lld*%lld must be < 2^31", (long long)T, (long long)k);
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
  if (t_user_ws.ptr) {
    if (t_user_ws.size < bytes)
      return fail(MOE_ENOMEM, "caller workspace holds %zu bytes, the call needs %zu", t_user_ws.size, bytes);
    *base = (uint8_t*)t_user_ws.ptr;
    return MOE_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (g_stream && hipStreamIsCapturing(g_stream, &cs) != hipSuccess)
    return fail(MOE_EHIP, "hipStreamIsCapturing failed");
  const bool capturing = cs != hipStreamCaptureStatusNone;
  std::lock_guard<std::mutex> lk(g_ws.mu);
  if (g_ws.size < bytes) {
    if (capturing)
      return fail(MOE_ENOMEM,
                  "the stream is capturing and the workspace holds %zu bytes, the call needs %zu: run one "
                  "call of this shape eagerly first, or set a workspace with moe_set_workspace",
                  g_ws.size, bytes);
    if (g_ws.ptr) {
      if (g_ws.pinned) {
        g_ws.retired.push_back(g_ws.ptr);  // a captured graph may still replay into it
      } else {
        hipError_t e = hipFree(g_ws.ptr);  // waits for queued work that may still use it
        if (e != hipSuccess) {
          g_ws.ptr = nullptr;
          g_ws.size = 0;
          return fail(MOE_EHIP, "hipFree(workspace): %s", hipGetErrorString(e));
        }
      }
      g_ws.ptr = nullptr;
      g_ws.size = 0;
      g_ws.pinned = false;
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
  if (capturing) g_ws.pinned = true;
  *base = (uint8_t*)g_ws.ptr;
  return MOE_OK;
}

// Launch wrapper: optional event bracketing (on the stream the kernel runs on), error
// translation.
template <class F>
int launch_on(hipStream_t st, int stage, const char* name, F&& fn) {
  hipEvent_t a = nullptr, b = nullptr;
  bool prof = false;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.on && !t_noalloc) {
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
  // a failed launch leaves no pair behind: its stop event would never be recorded
  auto unrecord = [&]() {
    if (!prof) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.used > 0 && g_prof.start[g_prof.used - 1] == a) --g_prof.used;
  };
  if (prof && hipEventRecord(a, st) != hipSuccess) {
    unrecord();
    return fail(MOE_EHIP, "hipEventRecord failed");
  }
  hipError_t e = fn(st);
  if (e != hipSuccess) {
    unrecord();
    return fail(MOE_EHIP, "%s launch failed: %s", name, hipGetErrorString(e));
  }
  if (prof && hipEventRecord(b, st) != hipSuccess) {
    unrecord();
    return fail(MOE_EHIP, "hipEventRecord failed");
  }
  return MOE_OK;
}
template <class F>
int launch(int stage, const char* name, F&& fn) {
  return launch_on(g_stream, stage, name, fn);
}

// The calling thread's side stream on the current device (made on first use), or null when
// the calling stream is capturing a graph: a capture stays on the one stream.
int side_stream(const moe::BwdSide** out) {
  *out = nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (g_stream && hipStreamIsCapturing(g_stream, &cs) != hipSuccess)
    return fail(MOE_EHIP, "hipStreamIsCapturing failed");
  if (cs != hipStreamCaptureStatusNone) return MOE_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_EHIP, "hipGetDevice failed");
  if (t_side.made && t_side.device != dev) drop_side();
  if (!t_side.made) {
    SideStream n;
    bool good = hipStreamCreateWithFlags(&n.side.stream, hipStreamNonBlocking) == hipSuccess;
    int made_ev = 0;
    for (; good && made_ev < 5; ++made_ev)
      good = hipEventCreateWithFlags(&n.side.ev[made_ev], hipEventDisableTiming) == hipSuccess;
    if (!good) {
      (void)hipGetLastError();
      if (n.side.stream) (void)hipStreamDestroy(n.side.stream);
      for (int i = 0; i + 1 < made_ev; ++i) (void)hipEventDestroy(n.side.ev[i]);
      return fail(MOE_EHIP, "creating the side stream failed");
    }
    n.device = dev;
    n.made = true;
    t_side = n;
  }
  *out = &t_side.side;
  return MOE_OK;
}

// router -> top-k -> grouping; after_router (if any) runs once the router is queued
int run_route(uint8_t* ws, const Layout& L, const void* x, const void* router_w, const void* router_b,
              const float* ebias, int64_t T, int64_t D, int64_t E, int64_t k, float* logits, int32_t* idx,
              float* gates, int32_t* counts, int32_t* offsets, int32_t* perm,
              const std::function<int()>& after_router = nullptr) {
  double* partial = (double*)(ws + L.partial);
  const int ks = moe::router_ksplit(T, D);
  CHECK(launch(moe::ST_ROUTER, "router", [&](hipStream_t st) {
    return moe::launch_router_partial((const uint16_t*)x, (const uint16_t*)router_w, (int)T, (int)D, (int)E, ks,
                                      partial, st);
  }));
  if (after_router) CHECK(after_router());
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
                float* out, bool split_done = false) {
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
  if (moe::mx_engine(fmt, cfg) && !split_done)
    CHECK(launch(moe::ST_SPLIT, "split", [&](hipStream_t st) {
      return moe::launch_mx_split(ea.x, T, (int)D, ea.xq, ea.xs, st);
    }));
  CHECK(launch(moe::ST_MLP1, "mlp1", [&](hipStream_t st) { return moe::launch_mlp1(ea, cfg, st); }));
  CHECK(launch(moe::ST_MLP2, "mlp2", [&](hipStream_t st) { return moe::launch_mlp2(ea, cfg, st); }));
  CHECK(launch(moe::ST_COMBINE, "combine",
               [&](hipStream_t st) { return moe::launch_combine(ea.y, ea.T, ea.D, ea.k, out, st); }));
  return MOE_OK;
}

// Device address of the current device's scratch array (looked up on the first call on
// that device).
int scratch_ptr(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  if ((size_t)dev >= g_scratch.ptr.size()) g_scratch.ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch.ptr[dev] = (uint8_t*)p;
  }
  *out = g_scratch.ptr[dev];
  return MOE_OK;
}

// Whole block; ebias is the load-balancing bias when `biased` (then it must be valid).
int forward_impl(const void* x, const void* router_w, const void* router_b, bool biased, const float* ebias,
                 const void* w1, const void* b1, const void* w2, const void* b2, int64_t T, int64_t D, int64_t E,
                 int64_t k, int64_t F, int fmt, float* out, bool noalloc = false) {
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
  if (noalloc) {
    if (L.total > MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ENOMEM,
                  "moe_forward_noalloc: this shape needs %zu bytes of scratch, the fixed scratch holds %zu "
                  "(use moe_forward, or fewer tokens)",
                  L.total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    CHECK(scratch_ptr(&ws));
  } else {
    CHECK(ensure_workspace(L.total, &ws));
  }
  int32_t* idx = (int32_t*)(ws + L.idx);
  float* gates = (float*)(ws + L.gates);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* perm = (int32_t*)(ws + L.perm);
  // On the scaled engine the split of x into fp8 pieces needs only x: it runs on the side
  // stream beside the top-k and the grouping (forked after the router, which fills the GPU;
  // forked before it, the split slowed the router by as much as it slows the top-k here),
  // after everything queued before it, and mlp1 waits for it (not under graph capture, nor
  // in the allocation-free entry point: there one stream).
  const moe::BwdSide* side = nullptr;
  if (!noalloc && moe::mx_engine(fmt, moe::expert_tile_config(T * k, E))) CHECK(side_stream(&side));
  auto fork_split = [&]() -> int {
    if (hipEventRecord(side->ev[0], g_stream) != hipSuccess ||
        hipStreamWaitEvent(side->stream, side->ev[0], 0) != hipSuccess)
      return fail(MOE_EHIP, "forking the split onto the side stream failed");
    CHECK(launch_on(side->stream, moe::ST_SPLIT, "split", [&](hipStream_t st) {
      return moe::launch_mx_split((const uint16_t*)x, (int)T, (int)D, (uint8_t*)(ws + L.xq), (uint32_t*)(ws + L.xs), st);
    }));
    if (hipEventRecord(side->ev[1], side->stream) != hipSuccess)
      return fail(MOE_EHIP, "recording the split's event failed");
    return MOE_OK;
  };
  CHECK(run_route(ws, L, x, router_w, router_b, ebias, T, D, E, k, nullptr, idx, gates, counts, offsets, perm,
                  side ? std::function<int()>(fork_split) : std::function<int()>()));
  if (side && hipStreamWaitEvent(g_stream, side->ev[1], 0) != hipSuccess)
    return fail(MOE_EHIP, "joining the split failed");
  CHECK(run_experts(ws, L, x, w1, b1, w2, b2, gates, offsets, perm, T, D, E, k, F, fmt, out, side != nullptr));
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

int moe_forward_noalloc(const void* x, const void* router_w, const void* router_b, const void* w1,
                        const void* b1, const void* w2, const void* b2, int64_t T, int64_t D, int64_t E,
                        int64_t k, int64_t F, int fmt, float* out) {
  t_noalloc = true;
  const int rc = forward_impl(x, router_w, router_b, false, nullptr, w1, b1, w2, b2, T, D, E, k, F, fmt, out, true);
  t_noalloc = false;
  return rc;
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

int moe_backward(const void* x, const void* router_w, const void* w1, const void* b1, const void* w2,
                 const void* b2, const int32_t* topk_idx, const float* gates, const int32_t* offsets,
                 const int32_t* perm, const float* dout, int64_t T, int64_t D, int64_t E, int64_t k, int64_t F,
                 int fmt, float* dx, float* d_router_w, float* d_router_b, float* dw1, float* db1, float* dw2,
                 float* db2) {
  CHECK(check_shapes(T, D, E, k, F, true));
  if (!valid_fmt(fmt)) return fail(MOE_EFMT, "unknown weight format %d", fmt);
  if (fmt != MOE_FMT_BF16) return fail(MOE_EFMT, "moe_backward takes bf16 expert weights only (fmt %d)", fmt);
  CHECK(check_ptr(d_router_w, "d_router_w"));
  CHECK(check_ptr(d_router_b, "d_router_b"));
  CHECK(check_ptr(dw1, "dw1"));
  CHECK(check_ptr(db1, "db1"));
  CHECK(check_ptr(dw2, "dw2"));
  CHECK(check_ptr(db2, "db2"));
  if (T == 0) {
    // no token: every parameter gradient is zero (dx has no element)
    const int64_t G = 2 * F;
    const struct { float* p; int64_t n; } z[] = {{d_router_w, E * D}, {d_router_b, E}, {dw1, E * G * D},
                                                   {db1, E * G}, {dw2, E * D * F}, {db2, E * D}};
    CHECK(launch(moe::ST_BACKWARD, "backward zero", [&](hipStream_t st) {
      for (const auto& zz : z) {
        const hipError_t e = moe::launch_fill_zero(zz.p, zz.n, st);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }));
    return ok();
  }
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(router_w, "router_w"));
  CHECK(check_ptr(w1, "w1"));
  CHECK(check_ptr(b1, "b1"));
  CHECK(check_ptr(w2, "w2"));
  CHECK(check_ptr(b2, "b2"));
  CHECK(check_ptr(topk_idx, "topk_idx"));
  CHECK(check_ptr(gates, "gates"));
  CHECK(check_ptr(offsets, "offsets"));
  CHECK(check_ptr(perm, "perm"));
  CHECK(check_ptr(dout, "dout"));
  CHECK(check_ptr(dx, "dx"));
  if (T * k + E * 63 + 64 >= ((int64_t)1 << 31))
    return fail(MOE_EINVAL, "T*k = %lld is too large for the backward's padded layout", (long long)(T * k));
  // the grouped GEMMs address a routed row (the backward's have K = 2D and 2F) and one
  // expert's weights (W1: 4 D F bytes) with 32-bit byte offsets; kept with a factor 4 margin
  if (T * k * 2 * (D > F ? D : F) >= ((int64_t)1 << 30) || 4 * D * F >= ((int64_t)1 << 30))
    return fail(MOE_EINVAL, "T*k*2*max(D, F) and 4*D*F must each be < 2^30 for the backward");
  // the weight gradients address rows of the transposed, padded activations ([max(D, 2F)]
  // rows of T*k + 64 E columns) with 32-bit byte offsets
  if ((T * k + 64 * E) * 2 * (D > 2 * F ? D : 2 * F) >= ((int64_t)1 << 31))
    return fail(MOE_EINVAL, "(T*k + 64*E)*2*max(D, 2F) must be < 2^31 for the backward");
  const BwdLayout L = bwd_layout(T, D, E, k, F);
  uint8_t* ws = nullptr;
  CHECK(ensure_workspace(L.total, &ws));
  moe::BwdArgs b{};
  b.x = (const uint16_t*)x; b.wr = (const uint16_t*)router_w;
  b.w1 = (const uint16_t*)w1; b.b1 = (const uint16_t*)b1; b.w2 = (const uint16_t*)w2; b.b2 = (const uint16_t*)b2;
  b.idx = topk_idx; b.gates = gates; b.offsets = offsets; b.perm = perm; b.dout = dout;
  b.dx = dx; b.dwr = d_router_w; b.dbr = d_router_b; b.dw1 = dw1; b.db1 = db1; b.dw2 = dw2; b.db2 = db2;
  b.poff = (int32_t*)(ws + L.poff); b.padmap = (int32_t*)(ws + L.padmap);
  b.dout_perm = (uint16_t*)(ws + L.dout_perm);
  b.ones = (float*)(ws + L.ones); b.zeros = (uint16_t*)(ws + L.zeros);
  b.xT = (uint16_t*)(ws + L.xT); b.dzT = (uint16_t*)(ws + L.dzT); b.u = (float*)(ws + L.u);
  b.h = (uint16_t*)(ws + L.h); b.du = (uint16_t*)(ws + L.du); b.dgsum = (float*)(ws + L.dgsum);
  b.dxs = (float*)(ws + L.dxs); b.hT = (uint16_t*)(ws + L.hT); b.duT = (uint16_t*)(ws + L.duT);
  b.dl = (float*)(ws + L.dl); b.part_w = (float*)(ws + L.part_w); b.part_b2 = (float*)(ws + L.part_b2);
  b.part_b1 = (float*)(ws + L.part_b1);
  b.T = (int)T; b.D = (int)D; b.E = (int)E; b.k = (int)k; b.F = (int)F;
  // the side stream where the grouped products run on matrix-core tiles (many rows per
  // expert: measured at 8192 tokens -2.4 %; at 256 the joins cost more than the overlap
  // gains, +1.8 %), and never under graph capture (there the calling stream runs it all)
  const moe::BwdSide* side = nullptr;
  if (moe::expert_tile_config(T * k, E) != 0) CHECK(side_stream(&side));
  CHECK(launch(moe::ST_BACKWARD, "backward", [&](hipStream_t st) { return moe::launch_backward(b, st, side); }));
  return ok();
}

size_t moe_backward_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k, int64_t F, int fmt) {
  if (check_shapes(T, D, E, k, F, true) != MOE_OK) return 0;
  if (fmt != MOE_FMT_BF16 || T == 0) return 0;
  return bwd_layout(T, D, E, k, F).total;
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
  if (dev_ptr && (((uintptr_t)dev_ptr) & 255))
    return fail(MOE_EALIGN, "workspace %p is not 256-byte aligned", dev_ptr);
  t_user_ws.ptr = dev_ptr;
  t_user_ws.size = dev_ptr ? bytes : 0;
  return ok();
}

const char* moe_last_error(void) { return g_err.c_str(); }

void moe_release(void) {
  {
    std::lock_guard<std::mutex> lk(g_ws.mu);
    if (g_ws.ptr) (void)hipFree(g_ws.ptr);
    for (void* p : g_ws.retired) (void)hipFree(p);
    g_ws.retired.clear();
    g_ws.ptr = nullptr;
    g_ws.size = 0;
    g_ws.pinned = false;
  }
  t_user_ws = UserWorkspace{};
  drop_side();
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
    if (hipEventSynchronize(g_prof.stop[i]) != hipSuccess) {
      g_prof.used = 0;
      return fail(MOE_EHIP, "hipEventSynchronize failed");
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof.start[i], g_prof.stop[i]) != hipSuccess) {
      g_prof.used = 0;
      return fail(MOE_EHIP, "hipEventElapsedTime failed");
    }
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
         "v_mfma_scale_f32_32x32x64_f8f6f4 on fp8 (x) and fp6 (h) activation pieces; combine fp32; backward (bf16) "
         "recomputation and input gradients on the forward's grouped GEMM, weight gradients on 256x256 "
         "v_mfma_f32_32x32x16_bf16 tiles";
}

}  // extern "C"

// C ABI of the MoE hot-path library: argument validation, workspace layout,
// launch sequencing and optional per-kernel event timing.  No compute here.

#include "../../include/moe_dispatch.h"
#include "moe_internal.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_routing(const moe_shape* s) {
  if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->L < 1) return fail(MOE_ERR_INVALID_ARG, "L must be >= 1 (got %lld)", (long long)s->L);
  if (s->E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", s->E);
  if (s->K < 1) return fail(MOE_ERR_INVALID_ARG, "K must be >= 1 (got %d)", s->K);
  if (s->K > s->E) return fail(MOE_ERR_INVALID_ARG, "K (%d) must not exceed E (%d)", s->K, s->E);
  if (s->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024 (got %d)", s->E);
  if (s->K > 255) return fail(MOE_ERR_UNSUPPORTED, "K must be <= 255 (got %d)", s->K);
  if (s->E > 256 && s->K > 8)
    return fail(MOE_ERR_UNSUPPORTED, "K must be <= 8 when E > 256 (got E=%d, K=%d)", s->E, s->K);
  if (s->L > (int64_t)INT32_MAX / s->K)
    return fail(MOE_ERR_UNSUPPORTED, "L*K must be < 2^31 (L=%lld, K=%d)", (long long)s->L, s->K);
  return MOE_OK;
}

int check_ffn_shape(const moe_shape* s) {
  int rc = check_routing(s);
  if (rc != MOE_OK) return rc;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  if (s->act != MOE_SILU && s->act != MOE_SWIGLU)
    return fail(MOE_ERR_INVALID_ARG, "unknown act %d", s->act);
  if ((s->flags & ~MOE_FLAG_RECOMPUTE_G) != 0)
    return fail(MOE_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)s->flags);
  if (s->d < 1 || s->h < 1) return fail(MOE_ERR_INVALID_ARG, "d and h must be >= 1 (d=%d, h=%d)", s->d, s->h);
  if (s->d % 8 != 0 || s->h % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d and h must be multiples of 8 (d=%d, h=%d)", s->d, s->h);
  // The GEMM epilogues form in-tile byte offsets (256 rows of d or h
  // elements) in 32 bits.
  if (s->d > MOE_MAX_WIDTH || s->h > MOE_MAX_WIDTH)
    return fail(MOE_ERR_UNSUPPORTED, "d and h must be <= %d (d=%d, h=%d)", MOE_MAX_WIDTH, s->d,
                s->h);
  // Every launch grid must fit the 32-bit grid size.
  const int64_t cd = ((int64_t)s->d + 255) / 256, ch = ((int64_t)s->h + 127) / 128;
  const int64_t route_tiles = (s->L * s->K + 255) / 256 + s->E;
  const int64_t pass_tiles = (s->L + 255) / 256 + s->E;
  const int64_t weight_tiles = (int64_t)s->E * cd * ch;
  if (route_tiles * ch > INT32_MAX / 2 || pass_tiles * cd > INT32_MAX / 2 ||
      weight_tiles > INT32_MAX / 2)
    return fail(MOE_ERR_UNSUPPORTED, "shape needs more workgroups than one launch holds");
  return MOE_OK;
}

struct PtrCheck {
  const char* name;
  const void* p;
  size_t align;
};

int check_ptrs(const PtrCheck* c, int n) {
  for (int i = 0; i < n; ++i) {
    if (c[i].p == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", c[i].name);
    if (!aligned(c[i].p, c[i].align))
      return fail(MOE_ERR_INVALID_ARG, "%s must be %zu-byte aligned", c[i].name, c[i].align);
  }
  return MOE_OK;
}

int check_ws(void* ws, size_t* ws_bytes, size_t need, bool* query) {
  if (ws_bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "ws_bytes is NULL");
  if (ws == nullptr) {
    *ws_bytes = need;
    *query = true;
    return MOE_OK;
  }
  *query = false;
  if (!aligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  if (*ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", *ws_bytes, need);
  return MOE_OK;
}

moe::FfnDims dims_of(const moe_shape* s) {
  moe::FfnDims d;
  d.L = s->L; d.d = s->d; d.h = s->h; d.E = s->E; d.K = s->K; d.dtype = s->dtype; d.act = s->act;
  d.recompute_g = (s->flags & MOE_FLAG_RECOMPUTE_G) != 0;
  return d;
}

// ------------------------------------------------------------ kernel timing
struct TimedLaunch {
  int name;
  hipEvent_t start, stop;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<std::string> names;
  std::vector<int64_t> launches;
  std::vector<double> total_ms;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> pool;

  int name_id(const char* n) {
    for (size_t i = 0; i < names.size(); ++i)
      if (names[i] == n) return (int)i;
    names.emplace_back(n);
    launches.push_back(0);
    total_ms.push_back(0.0);
    return (int)names.size() - 1;
  }
  hipEvent_t get_event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler& prof() {
  static Profiler p;
  return p;
}

// ------------------------------------------------ allocation-free dispatch
// Workspace of moe_dispatch_build_noalloc.  Every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever handed to a kernel.
static __device__ __align__(256) char scratch[MOE_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_of_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return MOE_OK;
}

}  // namespace

namespace moe {
LaunchTimer::LaunchTimer(const char* name, hipStream_t s) : slot(-1), stream(s) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on) return;
  TimedLaunch tl;
  tl.name = p.name_id(name);
  tl.start = p.get_event();
  tl.stop = p.get_event();
  if (tl.start == nullptr || tl.stop == nullptr) return;
  if (hipEventRecord(tl.start, s) != hipSuccess) {
    p.pool.push_back(tl.start);
    p.pool.push_back(tl.stop);
    return;
  }
  p.pending.push_back(tl);
  slot = (int)p.pending.size() - 1;
}
LaunchTimer::~LaunchTimer() {
  if (slot < 0) return;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (slot < (int)p.pending.size()) (void)hipEventRecord(p.pending[slot].stop, stream);
}
}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_dispatch_build(const moe_shape* s, const float* logits, int32_t* eti, int32_t* offsets,
                       int32_t* tei, int32_t* tim, float* gates, void* ws, size_t* ws_bytes,
                       void* stream) {
  g_err.clear();
  int rc = check_routing(s);
  if (rc != MOE_OK) return rc;
  const PtrCheck pc[] = {{"logits", logits, 4}, {"expert_token_indices", eti, 4},
                         {"expert_token_offsets", offsets, 4}, {"token_expert_indices", tei, 4},
                         {"token_index_map", tim, 4}, {"gates", gates, 4}};
  rc = check_ptrs(pc, 6);
  if (rc != MOE_OK) return rc;
  const moe::DispatchPlan pl = moe::plan_dispatch(s->L, s->E, s->K);
  bool query = false;
  rc = check_ws(ws, ws_bytes, pl.bytes, &query);
  if (rc != MOE_OK || query) return rc;
  hipError_t e = moe::launch_dispatch(pl, s->L, s->E, s->K, logits, eti, offsets, tei, tim, gates,
                                      static_cast<char*>(ws), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_dispatch_build launch");
  return MOE_OK;
}

int moe_dispatch_build_noalloc(const moe_shape* s, const float* logits, int32_t* eti,
                               int32_t* offsets, int32_t* tei, int32_t* tim, float* gates,
                               void* stream) {
  g_err.clear();
  int rc = check_routing(s);
  if (rc != MOE_OK) return rc;
  const PtrCheck pc[] = {{"logits", logits, 4}, {"expert_token_indices", eti, 4},
                         {"expert_token_offsets", offsets, 4}, {"token_expert_indices", tei, 4},
                         {"token_index_map", tim, 4}, {"gates", gates, 4}};
  rc = check_ptrs(pc, 6);
  if (rc != MOE_OK) return rc;
  const moe::DispatchPlan pl = moe::plan_dispatch(s->L, s->E, s->K);
  if (pl.bytes > (size_t)MOE_NOALLOC_WS_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_dispatch_build_noalloc: this shape needs %zu bytes of workspace, more than "
                "the %zu bytes of the library's scratch array (use moe_dispatch_build)",
                pl.bytes, (size_t)MOE_NOALLOC_WS_BYTES);
  char* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != MOE_OK) return rc;
  // The dispatch kernels write every workspace entry they read, so the
  // previous call's contents need no clearing.
  hipError_t e = moe::launch_dispatch(pl, s->L, s->E, s->K, logits, eti, offsets, tei, tim, gates,
                                      ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_dispatch_build_noalloc launch");
  return MOE_OK;
}

int moe_ffn_forward(const moe_shape* s, const void* x, const void* W1, const void* W3,
                    const void* W2, const int32_t* eti, const int32_t* offsets,
                    const int32_t* tei, const int32_t* tim, const float* gates, void* y, void* A,
                    void* B, void* ws, size_t* ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_ffn_shape(s);
  if (rc != MOE_OK) return rc;
  const bool glu = s->act == MOE_SWIGLU;
  const PtrCheck pc[] = {{"x", x, 16}, {"W1", W1, 16}, {"W2", W2, 16},
                         {"expert_token_indices", eti, 4}, {"expert_token_offsets", offsets, 4},
                         {"token_expert_indices", tei, 4}, {"token_index_map", tim, 4},
                         {"gates", gates, 4}, {"y", y, 16}, {"A", A, 16}};
  rc = check_ptrs(pc, 10);
  if (rc != MOE_OK) return rc;
  if (glu) {
    const PtrCheck pg[] = {{"W3", W3, 16}, {"B", B, 16}};
    rc = check_ptrs(pg, 2);
    if (rc != MOE_OK) return rc;
  }
  const moe::FfnDims dm = dims_of(s);
  const moe::FfnPlan pl = moe::plan_ffn(dm, false);
  bool query = false;
  rc = check_ws(ws, ws_bytes, pl.bytes, &query);
  if (rc != MOE_OK || query) return rc;
  hipError_t e = moe::launch_forward(pl, dm, x, W1, glu ? W3 : W1, W2, eti, offsets, tim, gates, y,
                                     A, glu ? B : A, static_cast<char*>(ws),
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_ffn_forward launch");
  return MOE_OK;
}

int moe_ffn_backward(const moe_shape* s, const void* dy, const void* x, const void* W1,
                     const void* W3, const void* W2, const int32_t* eti, const int32_t* offsets,
                     const int32_t* tei, const int32_t* tim, const float* gates, void* A, void* B,
                     void* dx, void* dW1, void* dW3, void* dW2, float* dlogits, void* ws,
                     size_t* ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_ffn_shape(s);
  if (rc != MOE_OK) return rc;
  const bool glu = s->act == MOE_SWIGLU;
  const PtrCheck pc[] = {{"dy", dy, 16}, {"x", x, 16}, {"W1", W1, 16}, {"W2", W2, 16},
                         {"expert_token_indices", eti, 4}, {"expert_token_offsets", offsets, 4},
                         {"token_expert_indices", tei, 4}, {"token_index_map", tim, 4},
                         {"gates", gates, 4}, {"A", A, 16}, {"dx", dx, 16}, {"dW1", dW1, 16},
                         {"dW2", dW2, 16}};
  rc = check_ptrs(pc, 13);
  if (rc != MOE_OK) return rc;
  if (glu) {
    const PtrCheck pg[] = {{"W3", W3, 16}, {"B", B, 16}, {"dW3", dW3, 16}};
    rc = check_ptrs(pg, 3);
    if (rc != MOE_OK) return rc;
  }
  if (dlogits != nullptr && !aligned(dlogits, 4))
    return fail(MOE_ERR_INVALID_ARG, "dlogits must be 4-byte aligned");
  const moe::FfnDims dm = dims_of(s);
  const moe::FfnPlan pl = moe::plan_ffn(dm, true);
  bool query = false;
  rc = check_ws(ws, ws_bytes, pl.bytes, &query);
  if (rc != MOE_OK || query) return rc;
  hipError_t e = moe::launch_backward(pl, dm, dy, x, W1, glu ? W3 : W1, W2, eti, offsets, tim,
                                      gates, A, glu ? B : A, dx, dW1, glu ? dW3 : dW1, dW2, tei,
                                      dlogits, static_cast<char*>(ws),
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_ffn_backward launch");
  return MOE_OK;
}

int moe_profile_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return MOE_OK;
}

int moe_profile_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto& tl : p.pending) {
    (void)hipEventSynchronize(tl.stop);
    p.pool.push_back(tl.start);
    p.pool.push_back(tl.stop);
  }
  p.pending.clear();
  for (size_t i = 0; i < p.names.size(); ++i) {
    p.launches[i] = 0;
    p.total_ms[i] = 0.0;
  }
  return MOE_OK;
}

int moe_profile_read(moe_kernel_stat* stats, int max_stats, int* n_stats) {
  g_err.clear();
  if (n_stats == nullptr) return fail(MOE_ERR_INVALID_ARG, "n_stats is NULL");
  if (max_stats > 0 && stats == nullptr) return fail(MOE_ERR_INVALID_ARG, "stats is NULL");
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto& tl : p.pending) {
    hipError_t e = hipEventSynchronize(tl.stop);
    if (e != hipSuccess) return hip_fail(e, "moe_profile_read");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, tl.start, tl.stop);
    if (e != hipSuccess) return hip_fail(e, "moe_profile_read");
    p.launches[tl.name] += 1;
    p.total_ms[tl.name] += ms;
    p.pool.push_back(tl.start);
    p.pool.push_back(tl.stop);
  }
  p.pending.clear();
  const int n = (int)p.names.size();
  *n_stats = n;
  for (int i = 0; i < n && i < max_stats; ++i) {
    std::memset(stats[i].name, 0, sizeof stats[i].name);
    std::strncpy(stats[i].name, p.names[i].c_str(), sizeof stats[i].name - 1);
    stats[i].launches = p.launches[i];
    stats[i].total_ms = p.total_ms[i];
  }
  return MOE_OK;
}

}  // extern "C"

// mla_host.hip -- host plumbing shared by every entry point: the per-thread
// error message, the compute-unit count used for grid caps, launch status,
// the cache-dtype parser and the library version.
#include <cstdarg>
#include <cstring>

#include "mla_common.hpp"

namespace mla {

namespace {
thread_local char g_error[512] = {0};
thread_local hipEvent_t g_launch_start = nullptr;
thread_local hipEvent_t g_launch_stop = nullptr;
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices] = {0};
}  // namespace

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_error[0] = '\0'; }

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  __atomic_store_n(&g_cu_count[dev], n, __ATOMIC_RELAXED);
  return n;
}

int32_t launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(MLA_ERR_DEVICE, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

bool take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_launch_start || !g_launch_stop) return false;
  *start = g_launch_start;
  *stop = g_launch_stop;
  g_launch_start = g_launch_stop = nullptr;
  return true;
}

int32_t check_cache_dtype(const char* fn, int32_t dt, const float* scales) {
  switch (dt) {
    case MLA_KV_AUTO:
    case MLA_KV_BF16:
      if (scales)
        return fail(MLA_ERR_INVALID_ARGUMENT,
                    "%s: a bf16 cache takes no kv_scales (pass NULL)", fn);
      return MLA_OK;
    case MLA_KV_FP8_E4M3:
    case MLA_KV_FP8_E5M2:
      if (!scales)
        return fail(MLA_ERR_INVALID_ARGUMENT,
                    "%s: an fp8 cache needs kv_scales (one fp32 scale per layer)", fn);
      return MLA_OK;
    default:
      return fail(MLA_ERR_INVALID_ARGUMENT,
                  "%s: unknown KV cache dtype code %d (expected auto, bfloat16, fp8_e4m3 or "
                  "fp8_e5m2)", fn, dt);
  }
}

}  // namespace mla

extern "C" const char* mla_last_error(void) { return mla::g_error; }

extern "C" const char* mla_version(void) { return "mla_kv 0.1.0 gfx950"; }

extern "C" int32_t mla_parse_kv_cache_dtype(const char* s, int32_t* out) {
  mla::clear_error();
  if (!s || !out) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "mla_parse_kv_cache_dtype: null argument");
  if (!strcmp(s, "auto")) { *out = MLA_KV_AUTO; return MLA_OK; }
  if (!strcmp(s, "bfloat16")) { *out = MLA_KV_BF16; return MLA_OK; }
  if (!strcmp(s, "fp8") || !strcmp(s, "fp8_e4m3")) { *out = MLA_KV_FP8_E4M3; return MLA_OK; }
  if (!strcmp(s, "fp8_e5m2")) { *out = MLA_KV_FP8_E5M2; return MLA_OK; }
  return mla::fail(MLA_ERR_INVALID_ARGUMENT,
                   "unknown KV cache dtype '%s' (expected auto, bfloat16, fp8, fp8_e4m3 or "
                   "fp8_e5m2)", s);
}

extern "C" int32_t mla_set_launch_events(void* start_event, void* stop_event) {
  mla::clear_error();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT,
                     "mla_set_launch_events: pass both events or neither");
  mla::g_launch_start = static_cast<hipEvent_t>(start_event);
  mla::g_launch_stop = static_cast<hipEvent_t>(stop_event);
  return MLA_OK;
}

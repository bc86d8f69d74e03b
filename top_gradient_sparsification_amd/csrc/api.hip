// Status codes, error text, options and the device error word.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>

#include "tgs_host.h"

namespace tgs {

static thread_local char t_last_error[512] = "";

tgs_status fail(tgs_status status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_last_error, sizeof t_last_error, fmt, ap);
  va_end(ap);
  return status;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static std::atomic<int64_t> g_opt_path{0};
static std::atomic<int64_t> g_opt_grid{0};

int64_t get_option(int32_t option) {
  switch (option) {
    case TGS_OPT_TOPK_PATH: return g_opt_path.load();
    case TGS_OPT_MAIN_GRID: return g_opt_grid.load();
    default: return 0;
  }
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load();
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cache[dev].store(v);
  return v;
}

// Launch parity per (device, workspace): which of the top-k control block's
// two counter sets the next fast-path launch on that workspace uses.
static std::mutex g_parity_mu;
static std::map<std::pair<int, uintptr_t>, uint32_t> g_parity;

static std::pair<int, uintptr_t> parity_key(const void* workspace) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  return {dev, (uintptr_t)workspace};
}

uint32_t launch_parity(const void* workspace) {
  std::lock_guard<std::mutex> lk(g_parity_mu);
  auto it = g_parity.find(parity_key(workspace));
  return it == g_parity.end() ? 0u : it->second;
}

void advance_parity(const void* workspace) {
  std::lock_guard<std::mutex> lk(g_parity_mu);
  g_parity[parity_key(workspace)] ^= 1u;
}

static std::mutex g_prof_mu;
static hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

void take_profile_events(hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  *start = g_prof_start;
  *stop = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
}

}  // namespace tgs

using namespace tgs;

extern "C" const char* tgs_status_string(tgs_status s) {
  switch (s) {
    case TGS_OK: return "TGS_OK";
    case TGS_EINVAL: return "TGS_EINVAL: invalid argument";
    case TGS_EWORKSPACE: return "TGS_EWORKSPACE: workspace too small";
    case TGS_EHIP: return "TGS_EHIP: HIP runtime error";
    case TGS_EDEVICE: return "TGS_EDEVICE: a kernel flagged invalid input";
    default: return "unknown tgs_status";
  }
}

extern "C" const char* tgs_last_error(void) { return t_last_error; }

extern "C" tgs_status tgs_set_option(int32_t option, int64_t value) {
  switch (option) {
    case TGS_OPT_TOPK_PATH:
      if (value < 0 || value > 9) return fail(TGS_EINVAL, "TGS_OPT_TOPK_PATH takes 0 .. 9");
      g_opt_path.store(value);
      return TGS_OK;
    case TGS_OPT_MAIN_GRID:
      if (value < 0) return fail(TGS_EINVAL, "TGS_OPT_MAIN_GRID must be >= 0");
      g_opt_grid.store(value);
      return TGS_OK;
    default: return fail(TGS_EINVAL, "unknown option %d", (int)option);
  }
}

extern "C" tgs_status tgs_profile_next_call(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return fail(TGS_EINVAL, "profile events: pass both or neither");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_start = start;
  g_prof_stop = stop;
  return TGS_OK;
}

extern "C" tgs_status tgs_profile_elapsed_ms(hipEvent_t start, hipEvent_t stop, float* ms) {
  if (!start || !stop || !ms) return fail(TGS_EINVAL, "profile_elapsed_ms: null argument");
  hipError_t e = hipEventSynchronize(stop);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, start, stop);
  if (e != hipSuccess) return fail(TGS_EHIP, "profile_elapsed_ms: %s", hipGetErrorString(e));
  return TGS_OK;
}

extern "C" tgs_status tgs_check_device_error(const void* workspace, hipStream_t stream) {
  if (!workspace) return fail(TGS_EINVAL, "check_device_error: null workspace");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(TGS_EHIP, "check_device_error: %s", hipGetErrorString(e));
  uint32_t word = 0;
  e = hipMemcpy(&word, workspace, sizeof word, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(TGS_EHIP, "check_device_error: %s", hipGetErrorString(e));
  if (word != 0) return fail(TGS_EDEVICE, "device error word 0x%x (bit0 bad merge input, bit1 grid barrier timeout, bit2 inconsistent counts)", word);
  return TGS_OK;
}

// Status codes, error text, options and the device error word.
#include <atomic>
#include <cstdarg>
#include <cstdio>

#include "tgs_host.h"
#include "tgs_internal.h"

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

// Test and profiling controls: per calling thread, so calls on other threads
// never see them.
static thread_local int64_t t_opt_path = 0;
static thread_local int64_t t_opt_grid = 0;

int64_t get_option(int32_t option) {
  switch (option) {
    case TGS_OPT_TOPK_PATH: return t_opt_path;
    case TGS_OPT_MAIN_GRID: return t_opt_grid;
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

static thread_local hipEvent_t t_prof_start = nullptr, t_prof_stop = nullptr;

void take_profile_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = t_prof_start;
  *stop = t_prof_stop;
  t_prof_start = t_prof_stop = nullptr;
}

// Zero-fills the workspace header (words [0, nwords)).
__global__ void k_workspace_init(u32* ws, u32 nwords) {
  for (u32 i = blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += gridDim.x * blockDim.x) ws[i] = 0u;
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
      if (value < 0 || value > 14) return fail(TGS_EINVAL, "TGS_OPT_TOPK_PATH takes 0 .. 14");
      t_opt_path = value;
      return TGS_OK;
    case TGS_OPT_MAIN_GRID:
      if (value < 0) return fail(TGS_EINVAL, "TGS_OPT_MAIN_GRID must be >= 0");
      t_opt_grid = value;
      return TGS_OK;
    default: return fail(TGS_EINVAL, "unknown option %d", (int)option);
  }
}

extern "C" tgs_status tgs_profile_next_call(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return fail(TGS_EINVAL, "profile events: pass both or neither");
  t_prof_start = start;
  t_prof_stop = stop;
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
  if (word == 0) return TGS_OK;
  // reported once: the word is cleared for the calls that follow
  const uint32_t zero = 0;
  e = hipMemcpy((void*)workspace, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(TGS_EHIP, "check_device_error: %s", hipGetErrorString(e));
  if (word == kErrBadInput)
    return fail(TGS_EINVAL,
                "device error word 0x%x: an input index outside its range (a merge row's index outside [0, n) or "
                "repeated, or a sample position outside [0, n))",
                word);
  return fail(TGS_EDEVICE,
              "device error word 0x%x (bit0 bad input index, bit1 wait timed out: the grid was not all resident, "
              "bit2 inconsistent counts); re-initialise the workspace before its next use",
              word);
}

extern "C" tgs_status tgs_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return fail(TGS_EINVAL, "workspace_init: null workspace");
  if (((uintptr_t)workspace & 3u) != 0) return fail(TGS_EINVAL, "workspace_init: workspace not 4-byte aligned");
  const size_t bytes = workspace_bytes < kWorkspaceHeader ? workspace_bytes : kWorkspaceHeader;
  const u32 nwords = (u32)(bytes / 4);
  if (nwords == 0) return TGS_OK;
  hipLaunchKernelGGL(k_workspace_init, dim3((nwords + 255) / 256), dim3(256), 0, stream, (u32*)workspace, nwords);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "workspace_init: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

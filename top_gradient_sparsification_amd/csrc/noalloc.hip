// The top-k step for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid hipMalloc): its
// workspace is a file-scope device array instead of a caller's buffer.
//
// `scratch` below is the array as the device sees it.  In host code its name
// is only a host-side stand-in, never a device address: every host use goes
// through the pointer hipGetSymbolAddress returns for the current device
// (each GPU holds its own copy at its own address), looked up once per device
// on that device's first call.  The array keeps the last call's contents;
// calls that overlap on one GPU race on it.
#include <mutex>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per GPU

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (null until looked up)

// The current device's copy of `scratch`, ready for the top-k step: on the
// device's first call its address is looked up and its header zero-filled by
// a kernel on `stream` (no allocation, no memset node).
tgs_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TGS_EINVAL, "topk_ef_step_noalloc: device %d not supported", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TGS_EHIP, "topk_ef_step_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const tgs_status st = tgs_workspace_init(p, kScratchBytes, stream);
    if (st != TGS_OK) return st;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TGS_OK;
}

}  // namespace
}  // namespace tgs

using namespace tgs;

extern "C" tgs_status tgs_topk_ef_step_noalloc(const float* grad, float* residual, int64_t n, int64_t k,
                                               int32_t* out_idx, float* out_val, hipStream_t stream) {
  static_assert(kScratchBytes == TGS_NOALLOC_WORKSPACE_BYTES, "the header states the array's size");
  tgs_status st = topk_check_args("topk_ef_step_noalloc", grad, residual, n, k, out_idx, out_val);
  if (st != TGS_OK) return st;
  const size_t need = tgs_topk_workspace_bytes(n, k);
  if (need > kScratchBytes)
    return fail(TGS_EINVAL, "topk_ef_step_noalloc: n=%lld k=%lld needs %zu bytes of workspace, above the %zu-byte "
                "device array", (long long)n, (long long)k, need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(stream, &ws);
  if (st != TGS_OK) return st;
  return tgs_topk_ef_step(grad, residual, n, k, out_idx, out_val, ws, kScratchBytes, stream);
}

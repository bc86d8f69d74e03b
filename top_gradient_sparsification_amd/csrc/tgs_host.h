// Host-side helpers of the sparsifier library: error reporting, argument
// checks, the per-thread test options and the one-shot profiling hook.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tgs.h"
#include "tgs_testing.h"

namespace tgs {

// Records a printf-style message for tgs_last_error() and returns `status`.
tgs_status fail(tgs_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// True when [a, a+na) and [b, b+nb) share a byte (empty ranges never overlap).
bool overlaps(const void* a, size_t na, const void* b, size_t nb);

int64_t get_option(int32_t option);

// The argument checks of the top-k step (sizes, null and misaligned pointers,
// overlapping buffers); `what` names the entry point in the message.
tgs_status topk_check_args(const char* what, const float* grad, const float* residual, int64_t n, int64_t k,
                           const int32_t* out_idx, const float* out_val);

// Compute units of the current device (cached per device; 0 on failure).
int device_cu_count();

// Hands out (and clears) the events set by tgs_profile_next_call; null when
// none are pending.
void take_profile_events(hipEvent_t* start, hipEvent_t* stop);

}  // namespace tgs

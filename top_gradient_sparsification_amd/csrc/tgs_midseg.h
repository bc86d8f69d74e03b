// Host interface of the batched layer-wise path (midseg.hip): the segments
// of one layer-wise call that are at most 2^23 entries long with k <= 4096
// run together, three launches per batch of up to 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tgs.h"

namespace tgs {

constexpr int kMidMaxSeg = 64;                   // segments per batch
constexpr int64_t kMidMaxN = (int64_t)1 << 23;   // entries of a batched segment at most
constexpr int64_t kMidMaxK = 4096;               // its k at most

struct MidSegSpec {
  int64_t start, len, k, out_off;
};

// True when the batched path takes a segment of `len` entries with this k
// (its sampling plan exists); the plan's fields as the kernels use them.
bool mid_plan(int64_t len, int64_t k, uint32_t* nrows, uint32_t* rstride, uint32_t* j);

// Blocks of 1024 entries the pass gives a segment starting at residual + start.
size_t mid_blocks_of(int64_t start, int64_t len, const float* residual);

// Workspace bytes for batches totalling `blocks` blocks.
size_t mid_workspace_bytes(int64_t blocks);

// Enqueues the batched step of nseg segments (each with mid_plan true, grad
// and residual equally aligned modulo 16 bytes) on `stream`.  Device words
// of the workspace: `exact` counts the segments selected exactly from acc
// (never reset), `done` holds kMidMaxSeg arrival counters (zero, and left
// zero); ws_mid is the region of mid_workspace_bytes.
tgs_status mid_launch(const float* grad, float* residual, int32_t* out_idx, float* out_val, int nseg,
                      const MidSegSpec* specs, uint32_t* exact, uint32_t* done, void* ws_mid, hipStream_t stream);

}  // namespace tgs

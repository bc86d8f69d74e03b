// Hard-threshold sparsifier with error feedback on gfx950.
//
// Method (arxivdaily listing for arXiv 2004.05298, entry "Rethinking gradient
// sparsification as total error minimization"): the hard-threshold variant of
// top-k, where the number of entries sent is whatever a constant threshold
// lets through, run with error feedback.
//
// Two launches, no global atomics:
//   k_thr_pass  each workgroup streams its contiguous chunk once (two tiles
//               in flight): acc = residual + grad; qualifying entries
//               (key(acc) >= key(lambda)) are counted and the first
//               `stash_cap` of them are kept, in index order, in the
//               workgroup's stash; residual <- +0 for those, acc for every
//               other entry (non-temporal); the count goes to cnt[wg].
//   k_thr_emit  each workgroup adds up the counts of the workgroups before it
//               (its output offset) and copies its stash to the output while
//               the position is below `capacity`; stashed entries past it get
//               acc back in the residual.  A workgroup whose stash overflowed
//               and whose later entries are still below `capacity` rescans
//               its chunk of acc (in residual) for them.  The last workgroup
//               writes the total count.
// The output is in ascending index order: chunks are contiguous and in
// workgroup order, and inside a chunk entries are ranked by (tile, wave, lane,
// component), which is index order.
#include <algorithm>
#include <climits>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

constexpr int kThrThreads = 1024;
constexpr int kThrWaves = kThrThreads / kWave;
constexpr int kThrMaxBlocks = 2048;

struct ThrArgs {
  const float* grad;
  float* residual;
  int64_t n;
  int64_t head;  // scalar elements before the 16-byte aligned part (vector mode)
  int64_t nv;    // float4 vectors (0 in scalar mode)
  bool vec;
  u32 klam;
  const float* lam_dev;  // when set, the threshold is key(*lam_dev) (read on the device) instead of klam
  u32* cnt;      // [G]
  Pair* stash;   // [G][stash_cap]
  int64_t stash_cap;
  int32_t* out_idx;
  float* out_val;
  int64_t capacity;
  int64_t* d_count;
};

// Walks this workgroup's chunk in index order.  For each tile, `load(i, bits[4],
// idx[4], nval)` fills up to 4 values of thread slot i; qualifying entries get
// consecutive ranks starting at `rank0`, and `put(rank, idx, bits)` is called
// for each.  Returns the number of qualifying entries in the chunk.
template <class Load, class Put>
__device__ int64_t ordered_walk(const ThrArgs& a, Load load, Put put, u32 (*s_wt)[kThrWaves]) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int G = gridDim.x;
  int64_t running = 0;
  int par = 0;
  // chunk in "slots": a slot is one float4 (vector mode) or one float (scalar)
  const int64_t units = a.vec ? a.nv : a.n;
  const int64_t per = (units + G - 1) / G;
  const int64_t ub = std::min<int64_t>(units, (int64_t)blockIdx.x * per);
  const int64_t ue = std::min<int64_t>(units, ub + per);
  // vector mode: head elements belong to workgroup 0 (before its chunk) and the
  // tail to the last workgroup (after its chunk); both run as one extra tile.
  const bool has_head = a.vec && blockIdx.x == 0 && a.head > 0;
  const bool has_tail = a.vec && blockIdx.x == G - 1 && a.head + 4 * a.nv < a.n;
  const int64_t tail0 = a.head + 4 * a.nv;
  const int64_t ntiles_main = (ue - ub + kThrThreads - 1) / kThrThreads;
  const int64_t tail_tiles = has_tail ? (a.n - tail0 + 4 * kThrThreads - 1) / (4 * kThrThreads) : 0;
  const int64_t ntiles = (has_head ? 1 : 0) + ntiles_main + tail_tiles;
  for (int64_t t = 0; t < ntiles; ++t) {
    u32 bits[4] = {0, 0, 0, 0};
    int64_t idx[4] = {0, 0, 0, 0};
    int nval = 0;
    int64_t tt = t;
    int kind = 1;  // 0 head, 1 main, 2 tail
    if (has_head) {
      if (tt == 0) kind = 0;
      else tt -= 1;
    }
    if (kind == 1 && tt >= ntiles_main) {
      kind = 2;
      tt -= ntiles_main;
    }
    if (kind == 0) {
      if (tid < a.head) {
        idx[0] = tid;
        nval = 1;
        load(-1, idx, bits, nval);
      }
    } else if (kind == 1) {
      int64_t i = ub + tt * kThrThreads + tid;
      if (i < ue) {
        if (a.vec) {
          int64_t e = a.head + 4 * i;
          idx[0] = e;
          idx[1] = e + 1;
          idx[2] = e + 2;
          idx[3] = e + 3;
          nval = 4;
        } else {
          idx[0] = i;
          nval = 1;
        }
        load(i, idx, bits, nval);
      }
    } else {
      // tail: up to 4 scalar elements per thread, in index order
      int64_t base = tail0 + tt * 4 * kThrThreads + 4 * (int64_t)tid;
      for (int c = 0; c < 4; ++c)
        if (base + c < a.n) {
          idx[c] = base + c;
          nval = c + 1;
        }
      if (nval) load(-2, idx, bits, nval);
    }
    bool q[4];
    u32 mine = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      q[c] = c < nval && key_of_bits(bits[c]) >= a.klam;
      mine += q[c];
    }
    u32 below = 0, wtot = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u64 m = ballot(q[c]);
      below += lanes_below(m);
      wtot += (u32)__popcll(m);
    }
    if (lane_id() == 0) s_wt[par][w] = wtot;
    __syncthreads();
    u32 woff = 0, ttot = 0;
#pragma unroll
    for (int ww = 0; ww < kThrWaves; ++ww) {
      u32 v = s_wt[par][ww];
      if (ww < w) woff += v;
      ttot += v;
    }
    if (mine) {
      int64_t r = running + woff + below;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (q[c]) put(r++, idx[c], bits[c]);
    }
    running += ttot;
    par ^= 1;
  }
  return running;
}

// Ranks of one tile's qualifying entries (bit c of qmask: component c of
// this thread qualifies), in index order: returns the rank of this thread's
// first one and advances `running` past the tile.  Every thread calls it.
__device__ __forceinline__ u32 tile_rank(u32 qmask, u32& running, u32 (*s_wt)[kThrWaves], int& par) {
  const int w = threadIdx.x / kWave;
  u32 below = 0, wtot = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u64 m = ballot((qmask >> c) & 1u);
    below += lanes_below(m);
    wtot += (u32)__popcll(m);
  }
  if (lane_id() == 0) s_wt[par][w] = wtot;
  __syncthreads();
  u32 woff = 0, ttot = 0;
#pragma unroll
  for (int ww = 0; ww < kThrWaves; ++ww) {
    const u32 v = s_wt[par][ww];
    if (ww < w) woff += v;
    ttot += v;
  }
  const u32 r0 = running + woff + below;
  running += ttot;
  par ^= 1;
  return r0;
}

// The pass writes +0 to the residual of every qualifying entry that goes to
// the stash (rank < stash_cap), acc everywhere else: in the usual case
// (count <= capacity, no overflow) every stashed entry is emitted and the
// emit pass only copies.  Entries the capacity turns away get acc back.
// The arguments with the threshold key in place (read from the device when
// it comes from there).
__device__ __forceinline__ ThrArgs with_key(const ThrArgs& in) {
  ThrArgs a = in;
  if (a.lam_dev) a.klam = __builtin_amdgcn_readfirstlane(__float_as_uint(*a.lam_dev) & 0x7FFFFFFFu);
  return a;
}

__global__ __launch_bounds__(kThrThreads) void k_thr_pass(ThrArgs ain) {
  const ThrArgs a = with_key(ain);
  __shared__ u32 s_wt[2][kThrWaves];
  const float* __restrict__ g = a.grad;
  float* __restrict__ r = a.residual;
  Pair* stash = a.stash + (int64_t)blockIdx.x * a.stash_cap;
  const int64_t cap = a.stash_cap;
  const int tid = threadIdx.x;
  if (!a.vec) {
    auto load = [&](int64_t, const int64_t* idx, u32* bits, int nval) {
      for (int c = 0; c < nval; ++c) {
        float x = r[idx[c]] + g[idx[c]];
        r[idx[c]] = x;
        bits[c] = __float_as_uint(x);
      }
    };
    auto put = [&](int64_t rank, int64_t idx, u32 bits) {
      if (rank < cap) {
        stash[rank] = Pair{(int32_t)idx, bits};
        r[idx] = 0.0f;  // after this thread's own acc store to it
      }
    };
    const int64_t total = ordered_walk(a, load, put, s_wt);
    if (tid == 0) a.cnt[blockIdx.x] = (u32)total;
    return;
  }
  // vector mode: the partition of ordered_walk (which the emit pass's rescan
  // uses): head tile (workgroup 0), main tiles of one float4 per thread with
  // two tiles in flight, tail tile (last workgroup)
  const int G = gridDim.x;
  const int64_t per = (a.nv + G - 1) / G;
  const int64_t ub = std::min<int64_t>(a.nv, (int64_t)blockIdx.x * per);
  const int64_t ue = std::min<int64_t>(a.nv, ub + per);
  const int64_t tail0 = a.head + 4 * a.nv;
  u32 running = 0;
  int par = 0;
  auto scalar_tile = [&](int64_t i0, int64_t cnt) {  // entries i0 + tid for tid < cnt (< 4)
    const bool in = tid < cnt;
    const int64_t i = i0 + tid;
    float x = 0.0f;
    u32 qm = 0;
    if (in) {
      x = r[i] + g[i];
      qm = key_of(x) >= a.klam ? 1u : 0u;
    }
    const u32 rk = tile_rank(qm, running, s_wt, par);
    if (in) {
      if (qm && rk < cap) {
        stash[rk] = Pair{(int32_t)i, __float_as_uint(x)};
        x = 0.0f;
      }
      r[i] = x;
    }
  };
  if (blockIdx.x == 0 && a.head > 0) scalar_tile(0, a.head);
  const v4f* __restrict__ gv = (const v4f*)(g + a.head);
  v4f* __restrict__ rv = (v4f*)(r + a.head);
  const int64_t ntiles = (ue - ub + kThrThreads - 1) / kThrThreads;
  auto load = [&](int64_t t, v4f& gg, v4f& rr) {
    const int64_t i = ub + t * kThrThreads + tid;
    if (t < ntiles && i < ue) {
      gg = __builtin_nontemporal_load(gv + i);
      rr = __builtin_nontemporal_load(rv + i);
    }
  };
  auto step = [&](int64_t t, const v4f& gg, const v4f& rr) {
    const int64_t i = ub + t * kThrThreads + tid;
    const bool in = i < ue;
    v4f acc = rr + gg;
    u32 qm = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) qm |= (in && key_of(acc[c]) >= a.klam ? 1u : 0u) << c;
    u32 rk = tile_rank(qm, running, s_wt, par);
    if (in) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((qm >> c) & 1u) {
          if (rk < cap) {
            stash[rk] = Pair{(int32_t)(a.head + 4 * i + c), __float_as_uint(acc[c])};
            acc[c] = 0.0f;
          }
          ++rk;
        }
      __builtin_nontemporal_store(acc, rv + i);
    }
  };
  v4f ga, ra, gb, rb;
  load(0, ga, ra);
  load(1, gb, rb);
  for (int64_t t = 0; t < ntiles; t += 2) {
    step(t, ga, ra);
    load(t + 2, ga, ra);
    if (t + 1 >= ntiles) break;
    step(t + 1, gb, rb);
    load(t + 3, gb, rb);
  }
  if (blockIdx.x == G - 1 && tail0 < a.n) scalar_tile(tail0, a.n - tail0);
  if (tid == 0) a.cnt[blockIdx.x] = running;
}

__global__ __launch_bounds__(kThrThreads) void k_thr_emit(ThrArgs ain) {
  const ThrArgs a = with_key(ain);
  __shared__ u32 s_wt[2][kThrWaves];
  __shared__ u32 s_scan[kThrWaves + 1];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  u32 before = 0;
  for (int i = tid; i < b; i += kThrThreads) before += a.cnt[i];
  u32 prefix_u;
  block_exclusive_sum<kThrThreads>(before, s_scan, prefix_u);
  const int64_t prefix = prefix_u;
  const int64_t mine = a.cnt[b];
  if (b == gridDim.x - 1 && tid == 0) *a.d_count = prefix + mine;
  if (mine == 0) return;
  const int64_t take = std::max<int64_t>(0, std::min<int64_t>(mine, a.capacity - prefix));
  // stashed entries (ranks below stash_cap; their residual is +0): emitted
  // below `take`, given acc back above it
  const int64_t stashed = std::min<int64_t>(mine, a.stash_cap);
  const Pair* stash = a.stash + (int64_t)b * a.stash_cap;
  float* rw = a.residual;
  for (int64_t j = tid; j < stashed; j += kThrThreads) {
    const Pair e = stash[j];
    if (j < take) {
      a.out_idx[prefix + j] = e.idx;
      a.out_val[prefix + j] = __uint_as_float(e.bits);
    } else {
      rw[e.idx] = __uint_as_float(e.bits);
    }
  }
  if (take <= a.stash_cap) return;
  // the stash overflowed and entries past it are to be emitted: rescan acc
  // (held in residual) in index order.  Stashed entries now hold +0, which
  // qualifies only when lambda is 0: then every entry qualifies and the
  // rescan's ranks are the pass's; otherwise the rescan sees only the
  // entries past the stash, so their ranks start at stash_cap.
  const float* r = a.residual;
  const v4f* rv = (const v4f*)(r + a.head);
  auto load = [&](int64_t i, const int64_t* idx, u32* bits, int nval) {
    if (i >= 0 && a.vec) {
      v4f x = rv[i];
      bits[0] = __float_as_uint(x.x);
      bits[1] = __float_as_uint(x.y);
      bits[2] = __float_as_uint(x.z);
      bits[3] = __float_as_uint(x.w);
    } else {
      for (int c = 0; c < nval; ++c) bits[c] = __float_as_uint(r[idx[c]]);
    }
  };
  const int64_t shift = a.klam == 0u ? 0 : a.stash_cap;
  auto put = [&](int64_t rank0, int64_t idx, u32 bits) {
    const int64_t rank = rank0 + shift;
    if (rank >= a.stash_cap && rank < take) {
      a.out_idx[prefix + rank] = (int32_t)idx;
      a.out_val[prefix + rank] = __uint_as_float(bits);
      rw[idx] = 0.0f;
    }
  };
  ordered_walk(a, load, put, s_wt);
}

__global__ void k_store_zero_count(int64_t* d_count) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *d_count = 0;
}

struct ThrLayout {
  int G;
  int64_t stash_cap;
  size_t cnt, stash, total;
};

static ThrLayout thr_layout(int64_t n) {
  ThrLayout L{};
  int64_t units = (n + 3) / 4;
  int64_t want = (units + kThrThreads - 1) / kThrThreads;
  L.G = (int)std::max<int64_t>(1, std::min<int64_t>(kThrMaxBlocks, want));
  // one workgroup covers at most ceil(n / G) + 3 elements (head/tail shifts);
  // the stash keeps up to 1/64 of them (at least 256)
  int64_t per = (n + L.G - 1) / L.G + 8;
  L.stash_cap = std::max<int64_t>(256, (per + 63) / 64);
  L.cnt = kWorkspaceHeader;  // after the header whose first word is the error word
  size_t cnt_bytes = (((size_t)L.G * 4) + 255) & ~(size_t)255;
  L.stash = L.cnt + cnt_bytes;
  L.total = L.stash + (size_t)L.G * (size_t)L.stash_cap * sizeof(Pair);
  return L;
}

}  // namespace tgs

using namespace tgs;

extern "C" size_t tgs_threshold_workspace_bytes(int64_t n) {
  if (n < 0 || n > INT32_MAX) return 0;
  return thr_layout(n).total;
}

// Validates and launches the threshold step; the threshold is key(lambda),
// or key(*lam_dev) read on the device when lam_dev is set.
static tgs_status threshold_launch(const char* what, const float* grad, float* residual, int64_t n, float lambda,
                                   const float* lam_dev, int32_t* out_idx, float* out_val, int64_t capacity,
                                   int64_t* d_count, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n < 0 || n > INT32_MAX) return fail(TGS_EINVAL, "%s: n=%lld outside [0, 2^31-1]", what, (long long)n);
  if (!lam_dev && !(lambda >= 0.0f)) return fail(TGS_EINVAL, "%s: lambda must be >= 0 and not NaN", what);
  if (capacity < 0) return fail(TGS_EINVAL, "%s: capacity < 0", what);
  if (!d_count || !workspace) return fail(TGS_EINVAL, "%s: null d_count/workspace", what);
  if (n > 0 && (!grad || !residual)) return fail(TGS_EINVAL, "%s: null grad/residual", what);
  if (capacity > 0 && (!out_idx || !out_val)) return fail(TGS_EINVAL, "%s: null outputs", what);
  for (const void* p : {(const void*)grad, (const void*)residual, (const void*)out_idx, (const void*)out_val,
                        (const void*)lam_dev})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "%s: pointer not 4-byte aligned", what);
  if (((uintptr_t)d_count & 7u) != 0) return fail(TGS_EINVAL, "%s: d_count not 8-byte aligned", what);
  const size_t nb4 = (size_t)n * 4, cb4 = (size_t)capacity * 4;
  if (overlaps(grad, nb4, residual, nb4) || overlaps(grad, nb4, out_idx, cb4) || overlaps(grad, nb4, out_val, cb4) ||
      overlaps(residual, nb4, out_idx, cb4) || overlaps(residual, nb4, out_val, cb4) ||
      overlaps(out_idx, cb4, out_val, cb4) || overlaps(d_count, 8, residual, nb4) ||
      overlaps(d_count, 8, out_idx, cb4) || overlaps(d_count, 8, out_val, cb4) || overlaps(d_count, 8, grad, nb4))
    return fail(TGS_EINVAL, "%s: overlapping buffers", what);
  if (lam_dev && (overlaps(lam_dev, 4, residual, nb4) || overlaps(lam_dev, 4, out_idx, cb4) ||
                  overlaps(lam_dev, 4, out_val, cb4) || overlaps(lam_dev, 4, d_count, 8)))
    return fail(TGS_EINVAL, "%s: d_lambda overlaps an output", what);
  const ThrLayout L = thr_layout(n);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "%s: workspace %zu bytes, need %zu", what, workspace_bytes, L.total);
  if (n == 0) {
    hipLaunchKernelGGL(k_store_zero_count, dim3(1), dim3(64), 0, stream, d_count);
  } else {
    char* ws = (char*)workspace;
    ThrArgs a{};
    a.grad = grad;
    a.residual = residual;
    a.n = n;
    a.vec = (((uintptr_t)grad) & 15u) == (((uintptr_t)residual) & 15u);
    if (a.vec) {
      int64_t head = (int64_t)(((16u - (((uintptr_t)residual) & 15u)) & 15u) / 4u);
      a.head = std::min<int64_t>(head, n);
      a.nv = (n - a.head) / 4;
    }
    a.klam = lam_dev ? 0u : (__builtin_bit_cast(uint32_t, lambda) & 0x7FFFFFFFu);
    a.lam_dev = lam_dev;
    a.cnt = (u32*)(ws + L.cnt);
    a.stash = (Pair*)(ws + L.stash);
    a.stash_cap = L.stash_cap;
    a.out_idx = out_idx;
    a.out_val = out_val;
    a.capacity = capacity;
    a.d_count = d_count;
    hipEvent_t ev0, ev1;
    take_profile_events(&ev0, &ev1);
    if (ev0) (void)hipEventRecord(ev0, stream);
    hipLaunchKernelGGL(k_thr_pass, dim3(L.G), dim3(kThrThreads), 0, stream, a);
    if (ev1) (void)hipEventRecord(ev1, stream);
    hipLaunchKernelGGL(k_thr_emit, dim3(L.G), dim3(kThrThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return TGS_OK;
}

extern "C" tgs_status tgs_threshold_ef_step(const float* grad, float* residual, int64_t n, float lambda,
                                            int32_t* out_idx, float* out_val, int64_t capacity,
                                            int64_t* d_count, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  return threshold_launch("threshold_ef_step", grad, residual, n, lambda, nullptr, out_idx, out_val, capacity, d_count,
                          workspace, workspace_bytes, stream);
}

extern "C" tgs_status tgs_threshold_ef_step_dev(const float* grad, float* residual, int64_t n, const float* d_lambda,
                                                int32_t* out_idx, float* out_val, int64_t capacity,
                                                int64_t* d_count, void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
  if (!d_lambda) return fail(TGS_EINVAL, "threshold_ef_step_dev: null d_lambda");
  return threshold_launch("threshold_ef_step_dev", grad, residual, n, 0.0f, d_lambda, out_idx, out_val, capacity,
                          d_count, workspace, workspace_bytes, stream);
}

// Hard-threshold sparsifier with error feedback on gfx950.
//
// Method (arxivdaily listing for arXiv 2004.05298, entry "Rethinking gradient
// sparsification as total error minimization"): the hard-threshold variant of
// top-k, where the number of entries sent is whatever a constant threshold
// lets through, run with error feedback.
//
// Two launches:
//   k_thr_pass  one block of 256 float4 slots (1024 entries) per 256-thread
//               workgroup, a grid of one workgroup per block: the hardware
//               hands blocks out in order, so the stretch of memory the chip
//               streams at any moment stays short (a persistent grid whose
//               workgroups walk their own rows drifts apart over a long
//               vector and streams slower).  acc = residual + grad;
//               qualifying entries (key(acc) >= key(lambda)) are ranked in
//               index order inside the block (ballots and one block scan of
//               the wave counts), the first `cap` go to the block's stash,
//               residual <- +0 for those and acc for every other entry
//               (non-temporal), and the count goes to cnt[block].
//   k_thr_emit  one workgroup per group of 1024 blocks, numbered by a ticket
//               in the order they start.  The group's offset in the output
//               comes from a scan with decoupled look-back (each group
//               publishes its total, then its inclusive prefix, and sums its
//               predecessors' words back to the nearest prefix).  Stashed
//               entries are copied while their position is below `capacity`
//               and get acc back past it.  A block whose entries outran its
//               stash and still have positions below the capacity is scanned
//               again (acc is in residual) by one wave, with the pass's ranks.
//               The last group writes the count.
// The output is in ascending index order: blocks are in index order, and
// inside a block entries are ranked by (wave, lane, component), which is
// index order (the head before the first slot, the tail after the last).
#include <algorithm>
#include <climits>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

constexpr int kPassThreads = 256;               // one float4 slot per thread
constexpr int kPassWaves = kPassThreads / kWave;
constexpr u32 kBlockCap = 32;                    // stash slots per block: 1/32 of its entries
constexpr int kEmitThreads = 1024;               // one block per thread
constexpr int kEmitWaves = kEmitThreads / kWave;
constexpr u64 kFlagTotal = 1ull << 62;   // a group's word: its own total is known
constexpr u64 kFlagPrefix = 2ull << 62;  // a group's word: the total up to and including it is known
constexpr u32 kLookbackSpins = 1u << 22;

struct ThrArgs {
  const float* grad;
  float* residual;
  int64_t n;
  int64_t head;     // entries before the first float4 slot (vector mode; 0 in scalar mode)
  int64_t nv;       // float4 slots (vector mode: 16-byte aligned; scalar mode: floor(n / 4) groups of 4)
  int64_t tail0;    // first entry after the slots: head + 4 nv
  int64_t nblocks;  // blocks of 256 slots (at least 1 when n > 0: block 0 holds the head, the last the tail)
  int64_t ngroups;  // emit groups of kEmitThreads blocks
  u32 klam;
  const float* lam_dev;  // when set, the threshold is key(*lam_dev) (read on the device) instead of klam
  u32* cnt;         // [nblocks]
  Pair* stash;      // [nblocks][kBlockCap]
  u64* status;      // [ngroups] look-back words
  u32* ticket;      // emit groups started
  u32* err;         // device error word
  int32_t* out_idx;
  float* out_val;
  int64_t capacity;
  int64_t* d_count;
  bool wt;          // vector mode, slots on 256-byte boundaries: store them written through at device scope
};

// The arguments with the threshold key in place (read from the device when
// it comes from there).
__device__ __forceinline__ ThrArgs with_key(const ThrArgs& in) {
  ThrArgs a = in;
  if (a.lam_dev) a.klam = __builtin_amdgcn_readfirstlane(__float_as_uint(*a.lam_dev) & 0x7FFFFFFFu);
  return a;
}

// Slot i: 4 consecutive entries, as one float4 (vector mode) or four floats
// (scalar mode, grad and residual not equally aligned).
template <bool VEC>
__device__ __forceinline__ v4f load_slot(const float* p, const ThrArgs& a, int64_t i) {
  if (VEC) return __builtin_nontemporal_load((const v4f*)(p + a.head) + i);
  const float* q = p + 4 * i;
  return v4f{q[0], q[1], q[2], q[3]};
}
// Slot i of a wave whose first slot is i0 (i = i0 + lane).  With `wt` the
// wave's 1 KB goes out as whole lines written through at device scope, which
// leaves the launch's end no dirty lines to write back (on slots that cut
// lines the device-scope stores would cost more than they save).
template <bool VEC>
__device__ __forceinline__ void store_slot(float* p, const ThrArgs& a, int64_t i, int64_t i0, v4f v) {
  if (VEC) {
    if (a.wt) {
      const u64 w0 = (u64)i0;  // the same in every lane: made a scalar for the buffer's base
      const int64_t s0 = (int64_t)((u64)__builtin_amdgcn_readfirstlane((u32)(w0 >> 32)) << 32 | __builtin_amdgcn_readfirstlane((u32)w0));
      st_agent_v4_nt((v4f*)(p + a.head) + s0, (u32)kWave * 16u, (u32)(i - s0) * 16u, v);
    } else {
      __builtin_nontemporal_store(v, (v4f*)(p + a.head) + i);
    }
  } else {
    float* q = p + 4 * i;
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  }
}

// One wave's part of block b, in index order: the head (wave 0 of block 0),
// the wave's 64 slots (this lane's: `slot`, present when `in`), the tail (the
// last wave of the last block).
struct WavePart {
  bool has_head, has_tail;
  int64_t slot;  // this lane's slot
  bool in;       // the slot exists
};

__device__ __forceinline__ WavePart wave_part(const ThrArgs& a, int64_t b, int w) {
  WavePart p;
  p.has_head = b == 0 && w == 0 && a.head > 0;
  p.has_tail = b == a.nblocks - 1 && w == kPassWaves - 1 && a.tail0 < a.n;
  p.slot = b * kPassThreads + w * kWave + lane_id();
  p.in = p.slot < a.nv;
  return p;
}

// The pass.
template <bool VEC>
__global__ __launch_bounds__(kPassThreads) void k_thr_pass(ThrArgs ain) {
  const ThrArgs a = with_key(ain);
  __shared__ u32 s_w[kPassWaves];
  const float* __restrict__ g = a.grad;
  float* __restrict__ r = a.residual;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = lane_id();
  const int64_t b = blockIdx.x;
  // the look-back words and the ticket of the emit launch that follows
  if (tid == 0 && b < a.ngroups) st_agent64(a.status + b, 0ull);
  if (tid == 0 && b == 0) st_agent(a.ticket, 0u);
  const WavePart p = wave_part(a, b, w);
  v4f gg = {0, 0, 0, 0}, rr = gg;
  if (p.in) {
    gg = load_slot<VEC>(g, a, p.slot);
    rr = load_slot<VEC>(r, a, p.slot);
  }
  // head / tail: up to 3 single entries, lane c holding entry i0 + c
  float xh = 0.0f, xt = 0.0f;
  bool qh = false, qt = false;
  if (p.has_head && lane < a.head) {
    xh = r[lane] + g[lane];
    qh = key_of(xh) >= a.klam;
  }
  if (p.has_tail && lane < a.n - a.tail0) {
    xt = r[a.tail0 + lane] + g[a.tail0 + lane];
    qt = key_of(xt) >= a.klam;
  }
  v4f acc = rr + gg;
  u32 qm = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) qm |= (p.in && key_of(acc[c]) >= a.klam ? 1u : 0u) << c;
  const u64 mh = ballot(qh), mt = ballot(qt);
  u32 mtot;
  const u32 mbelow = wave_rank4(qm, mtot);
  const u32 hcnt = (u32)__popcll(mh);
  const u32 wtot = hcnt + mtot + (u32)__popcll(mt);
  if (lane == 0) s_w[w] = wtot;
  __syncthreads();
  u32 woff = 0, btot = 0;
#pragma unroll
  for (int i = 0; i < kPassWaves; ++i) {
    const u32 v = s_w[i];
    woff += i < w ? v : 0u;
    btot += v;
  }
  Pair* __restrict__ stash = a.stash + b * kBlockCap;
  if (qh) {
    const u32 s = woff + lanes_below(mh);
    if (s < kBlockCap) {
      stash[s] = Pair{(int32_t)lane, __float_as_uint(xh)};
      xh = 0.0f;
    }
  }
  if (qm) {
    u32 s = woff + hcnt + mbelow;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if ((qm >> c) & 1u) {
        if (s < kBlockCap) {
          stash[s] = Pair{(int32_t)(a.head + 4 * p.slot + c), __float_as_uint(acc[c])};
          acc[c] = 0.0f;
        }
        ++s;
      }
  }
  if (qt) {
    const u32 s = woff + hcnt + mtot + lanes_below(mt);
    if (s < kBlockCap) {
      stash[s] = Pair{(int32_t)(a.tail0 + lane), __float_as_uint(xt)};
      xt = 0.0f;
    }
  }
  if (p.in) store_slot<VEC>(r, a, p.slot, p.slot - lane, acc);
  if (p.has_head && lane < a.head) r[lane] = xh;
  if (p.has_tail && lane < a.n - a.tail0) r[a.tail0 + lane] = xt;
  if (tid == 0) a.cnt[b] = btot;
}

// Block b scanned again by one wave (every lane calls it), its four wave
// parts in order: its qualifying entries past the first `nst` (the stashed
// ones, whose residual the pass set to +0) go to the output at o + their
// rank in the block while below the capacity, and their residual becomes
// +0.  The stashed entries still qualify when the threshold key is 0
// (key(+0) = 0), so the ranks are the pass's; otherwise the scan sees only
// the others, numbered from nst.
template <bool VEC>
__device__ void rescan_block(const ThrArgs& a, int64_t b, int64_t o, u32 nst) {
  float* r = a.residual;
  const int lane = lane_id();
  const u32 shift = a.klam == 0u ? 0u : nst;
  u32 run = 0;
  auto put = [&](u32 rank, int64_t idx, float x) {
    const int64_t e = (int64_t)rank + shift;
    if (e >= nst && o + e < a.capacity) {
      a.out_idx[o + e] = (int32_t)idx;
      a.out_val[o + e] = x;
      r[idx] = 0.0f;
    }
  };
  auto single = [&](int64_t i0, int64_t cnt) {
    const bool in = lane < cnt;
    const float x = in ? r[i0 + lane] : 0.0f;
    const bool q = in && key_of(x) >= a.klam;
    const u64 m = ballot(q);
    if (q) put(run + lanes_below(m), i0 + lane, x);
    run += (u32)__popcll(m);
  };
  v4f x[kPassWaves];
  WavePart p[kPassWaves];
#pragma unroll
  for (int w = 0; w < kPassWaves; ++w) {
    p[w] = wave_part(a, b, w);
    x[w] = p[w].in ? load_slot<VEC>(r, a, p[w].slot) : v4f{0, 0, 0, 0};
  }
#pragma unroll
  for (int w = 0; w < kPassWaves; ++w) {
    if (p[w].has_head) single(0, a.head);
    u32 qm = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) qm |= (p[w].in && key_of(x[w][c]) >= a.klam ? 1u : 0u) << c;
    u32 tot;
    u32 s = run + wave_rank4(qm, tot);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if ((qm >> c) & 1u) put(s++, a.head + 4 * p[w].slot + c, x[w][c]);
    run += tot;
    if (p[w].has_tail) single(a.tail0, a.n - a.tail0);
  }
}

// Decoupled look-back for group e (wave 0, every lane): the sum of the totals
// of groups 0 .. e-1.  Every group publishes its total before it looks back,
// and a group's ticket is taken after its predecessors', so the waits end;
// the spin is bounded all the same (error bit kErrBarrierTimeout).
__device__ u32 look_back(const ThrArgs& a, int64_t e) {
  const int lane = lane_id();
  u32 sum = 0;
  int64_t k = e - 1;  // the nearest group not yet summed
  while (k >= 0) {
    const int64_t j = k - lane;
    u64 v = j >= 0 ? ld_agent64(a.status + j) : kFlagPrefix;
    u32 spins = 0;
    while (ballot((v >> 62) == 0)) {
      if (++spins > kLookbackSpins) {
        if (lane == 0) or_agent(a.err, kErrBarrierTimeout);
        return sum;
      }
      if ((v >> 62) == 0) v = ld_agent64(a.status + j);
    }
    const u64 pm = ballot((v >> 62) == 2);
    const int stop = pm ? __builtin_ctzll(pm) : kWave - 1;  // lanes 0 .. stop are summed
    sum += wave_sum(lane <= stop ? (u32)v : 0u);
    if (pm) break;
    k -= kWave;
  }
  return sum;
}

template <bool VEC>
__global__ __launch_bounds__(kEmitThreads) void k_thr_emit(ThrArgs ain) {
  const ThrArgs a = with_key(ain);
  __shared__ u32 s_scan[kEmitWaves + 1];
  __shared__ u32 s_off[kEmitThreads];       // a block's first position in the group's output
  __shared__ u32 s_soff[kEmitThreads + 1];  // a block's first stashed entry among the group's
  __shared__ u32 s_e, s_before;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  if (tid == 0) s_e = add_agent_relaxed(a.ticket, 1u);
  __syncthreads();
  const int64_t e = s_e;
  const int64_t x = e * kEmitThreads + tid;  // this thread's block
  const u32 c = x < a.nblocks ? a.cnt[x] : 0u;
  const u32 nst = std::min(c, kBlockCap);
  u32 gtot, stot;
  const u32 off = block_exclusive_sum<kEmitThreads>(c, s_scan, gtot);
  const u32 soff = block_exclusive_sum<kEmitThreads>(nst, s_scan, stot);
  s_off[tid] = off;
  s_soff[tid] = soff;
  if (tid == 0) s_soff[kEmitThreads] = stot;
  if (tid < kWave) {
    if (lane == 0) st_agent64(a.status + e, (e == 0 ? kFlagPrefix : kFlagTotal) | gtot);
    const u32 before = e == 0 ? 0u : look_back(a, e);
    if (lane == 0) {
      if (e > 0) st_agent64(a.status + e, kFlagPrefix | (u64)(before + gtot));
      s_before = before;
      if (e == a.ngroups - 1) *a.d_count = (int64_t)before + gtot;
    }
  }
  __syncthreads();
  const int64_t P = s_before;
  // stashed entries, flattened: entry q of the group is entry q - soff[j] of
  // the group's block j, where soff[j] <= q < soff[j + 1]; four per thread at
  // a time, so that their loads are in flight together
  constexpr int U = 4;
  for (u32 q0 = tid; q0 < stot; q0 += U * kEmitThreads) {
    Pair pr[U];
    int64_t pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32 q = q0 + u * kEmitThreads;
      pos[u] = -1;
      if (q < stot) {
        int lo = 0, hi = kEmitThreads;  // s_soff[lo] <= q < s_soff[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_soff[mid] <= q) lo = mid;
          else hi = mid;
        }
        const u32 j = q - s_soff[lo];
        pr[u] = a.stash[(e * kEmitThreads + lo) * kBlockCap + j];
        pos[u] = P + s_off[lo] + j;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (pos[u] < 0) continue;
      if (pos[u] < a.capacity) {
        a.out_idx[pos[u]] = pr[u].idx;
        a.out_val[pos[u]] = __uint_as_float(pr[u].bits);
      } else {
        a.residual[pr[u].idx] = __uint_as_float(pr[u].bits);
      }
    }
  }
  // blocks whose entries outran the stash with positions still below the
  // capacity: each wave scans its own lanes' blocks in turn
  const int64_t o = P + off;
  u64 m = ballot(c > nst && o + nst < a.capacity);
  while (m) {
    const int L = __builtin_ctzll(m);
    m &= m - 1;
    rescan_block<VEC>(a, __shfl(x, L), __shfl(o, L), __shfl(nst, L));
  }
}

__global__ void k_store_zero_count(int64_t* d_count) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *d_count = 0;
}

struct ThrLayout {
  int64_t nblocks, ngroups;
  size_t ticket, cnt, status, stash, total;
};

// Sized for floor(n / 4) slots, as many as either mode has: a launch's own
// block count is at most L.nblocks.
static ThrLayout thr_layout(int64_t n) {
  ThrLayout L{};
  const int64_t nv = n / 4;
  L.nblocks = std::max<int64_t>(1, (nv + kPassThreads - 1) / kPassThreads);
  L.ngroups = (L.nblocks + kEmitThreads - 1) / kEmitThreads;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  L.ticket = kWorkspaceHeader;  // after the header whose first word is the error word
  L.cnt = L.ticket + 256;
  L.status = L.cnt + up((size_t)L.nblocks * 4);
  L.stash = L.status + up((size_t)L.ngroups * 8);
  L.total = L.stash + (size_t)L.nblocks * kBlockCap * sizeof(Pair);
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
    const bool vec = (((uintptr_t)grad) & 15u) == (((uintptr_t)residual) & 15u);
    if (vec) {
      int64_t head = (int64_t)(((16u - (((uintptr_t)residual) & 15u)) & 15u) / 4u);
      a.head = std::min<int64_t>(head, n);
      a.wt = (((uintptr_t)(residual + a.head)) & 255u) == 0;
    }
    a.nv = (n - a.head) / 4;
    a.tail0 = a.head + 4 * a.nv;
    a.nblocks = std::max<int64_t>(1, (a.nv + kPassThreads - 1) / kPassThreads);
    a.ngroups = (a.nblocks + kEmitThreads - 1) / kEmitThreads;
    a.klam = lam_dev ? 0u : (__builtin_bit_cast(uint32_t, lambda) & 0x7FFFFFFFu);
    a.lam_dev = lam_dev;
    a.cnt = (u32*)(ws + L.cnt);
    a.stash = (Pair*)(ws + L.stash);
    a.status = (u64*)(ws + L.status);
    a.ticket = (u32*)(ws + L.ticket);
    a.err = (u32*)ws;
    a.out_idx = out_idx;
    a.out_val = out_val;
    a.capacity = capacity;
    a.d_count = d_count;
    hipEvent_t ev0, ev1;
    take_profile_events(&ev0, &ev1);
    if (ev0) (void)hipEventRecord(ev0, stream);
    if (vec)
      hipLaunchKernelGGL(k_thr_pass<true>, dim3(a.nblocks), dim3(kPassThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(k_thr_pass<false>, dim3(a.nblocks), dim3(kPassThreads), 0, stream, a);
    if (ev1) (void)hipEventRecord(ev1, stream);
    if (vec)
      hipLaunchKernelGGL(k_thr_emit<true>, dim3(a.ngroups), dim3(kEmitThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(k_thr_emit<false>, dim3(a.ngroups), dim3(kEmitThreads), 0, stream, a);
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

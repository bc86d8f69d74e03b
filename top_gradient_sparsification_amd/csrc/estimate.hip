// Threshold estimate from a sample, on gfx950.
//
// Method (arxivdaily listing for arXiv 2004.05298, entry "Near-Optimal Sparse
// Allreduce for Distributed Deep Learning": top-k picked through an estimated
// threshold instead of a sort; fugumt page for arXiv 2502.07634, related-paper
// entry "An Efficient Statistical-based Gradient Compression Technique for
// Distributed Training Systems": threshold sparsification whose threshold
// estimate matches DGC's, and the Abstract: top-k's sorting costs offset the
// communication it saves): the threshold is the q-th largest |acc| over m
// sampled positions, and the hard threshold keeps every entry that reaches it.
//
// Two launches, no grid-wide wait:
//   k_est_keys    workgroup b takes samples [1024 b, 1024 (b + 1)): the
//                 positions (coalesced), then acc = residual + grad at each
//                 (gathers), its magnitude key to keys[j] and to a 2048-bin LDS
//                 histogram of key >> 20, whose nonzero bins are added into
//                 the header histogram.  A position outside [0, n) sets the
//                 bad-input bit.  The last workgroup to arrive reads (and
//                 zeroes) the histogram and publishes the bin d that holds the
//                 q-th largest key and how many of bin d's keys are still
//                 needed.
//   k_est_select  every workgroup reads its share of keys[] again (one round
//                 trip) and appends the keys of bin d to a list; the last to
//                 arrive finishes the select over the 20 low bits of the list
//                 (two 10-bit digits, in LDS, or over the list in memory when
//                 it is larger than LDS) and writes the key to *d_lambda as
//                 the float of those bits.
#include <algorithm>
#include <climits>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

// k_est_keys: small workgroups, so that the random gathers of even a modest
// sample come from every compute unit at once (they are latency-bound)
constexpr int kKeyThreads = 256;
constexpr int kKeyPer = 4;                          // samples per thread (2: 2 us slower, the
                                                    // workgroups' histogram adds contending more)
constexpr int kKeyChunk = kKeyThreads * kKeyPer;    // samples per workgroup
// k_est_select: coalesced reads of the keys
constexpr int kEstThreads = 1024;
constexpr int kEstPer = 8;                         // keys per thread
constexpr int kEstChunk = kEstThreads * kEstPer;   // keys per workgroup
constexpr int64_t kEstMaxM = (int64_t)1 << 24;     // samples at most
constexpr int kEstList = 16384;                    // keys of the threshold bin held in LDS
static_assert(kEstChunk <= kEstList, "a workgroup's keys of one bin fit its LDS list");
struct EstState;

struct EstArgs {
  const float* grad;
  const float* residual;
  int64_t n;
  const int32_t* sample;  // [m] positions
  u32 m, q;               // 1 <= q <= m
  u32* keys;              // [m] scratch
  u32* list;              // [m] scratch: the keys of the threshold's bin
  HeaderHist* hh;         // zero on entry, left zero
  struct EstState* st;    // zero on entry (listed, done), left zero
  u32* err;
  float* d_lambda;        // out
};

// s_out = {d, above}: the bin d (bins counted from the top, nb <= 2048 of
// them in `cnt`) where the suffix count first reaches `need` (1 <= need <= the
// total), and the count of the bins above it.  Every thread of the block calls
// it; s_out is read after it returns.
template <int NT>
__device__ __forceinline__ void pick_bin(const u32* cnt, int nb, u32 need, u32* s_scan, u32* s_out) {
  const int tid = threadIdx.x;
  if (tid == 0) s_out[0] = s_out[1] = 0;  // (consistent counts always overwrite them)
  constexpr int per = 2048 / NT;  // bins per thread, from the top
  const int hi = nb - per * tid;
  u32 own = 0;
  for (int q = 1; q <= per; ++q)
    if (hi - q >= 0) own += cnt[hi - q];
  u32 tot;
  const u32 above = block_exclusive_sum<NT>(own, s_scan, tot);
  if (above < need && above + own >= need) {
    u32 run = above;
    for (int q = 1; q <= per; ++q) {
      const int d = hi - q;
      if (d < 0) break;
      if (run + cnt[d] >= need) {
        s_out[0] = (u32)d;
        s_out[1] = run;
        break;
      }
      run += cnt[d];
    }
  }
  __syncthreads();
}

// Selection state between the two launches (in the header at
// kEstStateOffset; `listed` and `done` are left zero by the second launch).
struct EstState {
  u32 bin;     // first-level bin d of the q-th largest key
  u32 need;    // keys of bin d still needed (1 <= need <= count of bin d)
  u32 count;   // keys of bin d (the list's length once complete)
  u32 listed;  // list places handed out
  u32 done;    // k_est_select arrivals
  u32 pad[27];
};

static_assert(sizeof(EstState) == 128, "selection state fills its 128 bytes");

__global__ __launch_bounds__(kKeyThreads) void k_est_keys(EstArgs a) {
  constexpr int NT = kKeyThreads, NW = NT / kWave, P = kKeyPer;
  __shared__ u32 s_h[2048];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_out[2];
  __shared__ u32 s_last;
  const int tid = threadIdx.x;
  for (int i = tid; i < 2048; i += NT) s_h[i] = 0;
  __syncthreads();
  const u32 j0 = blockIdx.x * (u32)kKeyChunk;
  int32_t pos[P];
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const u32 j = j0 + (u32)(u * NT + tid);
    pos[u] = j < a.m ? a.sample[j] : 0;
  }
  bool bad = false;
  float gq[P], rq[P];
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const bool in = (int64_t)(u32)pos[u] < a.n;  // negative positions wrap above n
    bad |= j0 + (u32)(u * NT + tid) < a.m && !in;
    const int64_t i = in ? pos[u] : 0;
    gq[u] = a.grad[i];
    rq[u] = a.residual[i];
  }
  if (bad) atomicOr(a.err, kErrBadInput);
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const u32 j = j0 + (u32)(u * NT + tid);
    if (j < a.m) {
      const u32 key = key_of(rq[u] + gq[u]);
      a.keys[j] = key;
      atomicAdd(&s_h[key >> 20], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < 2048; i += NT)
    if (s_h[i]) add_agent_relaxed(&a.hh->hist[i], s_h[i]);
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_acqrel(&a.hh->done, 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  if (tid < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  // the last workgroup: the complete histogram -> bin d
  for (int i = tid; i < 2048; i += NT) {
    s_h[i] = ld_agent(&a.hh->hist[i]);
    st_agent(&a.hh->hist[i], 0u);
  }
  if (tid == 0) st_agent(&a.hh->done, 0u);
  __syncthreads();
  pick_bin<NT>(s_h, 2048, a.q, s_scan, s_out);
  if (tid == 0) {
    a.st->bin = s_out[0];
    a.st->need = a.q - s_out[1];
    a.st->count = s_h[s_out[0]];
  }
}

__global__ __launch_bounds__(kEstThreads) void k_est_select(EstArgs a) {
  constexpr int NT = kEstThreads, NW = NT / kWave;
  __shared__ u32 s_h[1024];
  __shared__ u32 s_list[kEstList];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_out[2];
  __shared__ u32 s_n, s_base, s_last;
  const int tid = threadIdx.x;
  const u32 d = a.st->bin;
  if (tid == 0) s_n = 0;
  __syncthreads();
  // this workgroup's keys of bin d, to LDS, then to the list
  const u32 j0 = blockIdx.x * (u32)kEstChunk;
  u32 kq[kEstPer];
#pragma unroll
  for (int u = 0; u < kEstPer; ++u) {
    const u32 j = j0 + (u32)(u * NT + tid);
    kq[u] = j < a.m ? a.keys[j] : 0xFFFFFFFFu;
  }
#pragma unroll
  for (int u = 0; u < kEstPer; ++u)
    if ((kq[u] >> 20) == d) s_list[atomicAdd(&s_n, 1u)] = kq[u];  // kEstChunk <= kEstList
  __syncthreads();
  const u32 mine = s_n;
  if (tid == 0 && mine) s_base = add_agent_relaxed(&a.st->listed, mine);
  __syncthreads();
  for (u32 i = tid; i < mine; i += NT) st_agent(&a.list[s_base + i], s_list[i]);
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_acqrel(&a.st->done, 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  if (tid < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  // the last workgroup: the list holds every key of bin d
  const u32 cnt = a.st->count;
  u32 need = a.st->need;
  const bool in_lds = cnt <= (u32)kEstList;
  if (in_lds)
    for (u32 i = tid; i < cnt; i += NT) s_list[i] = ld_agent(&a.list[i]);
  u32 prefix = d;
  for (int L = 0; L < 2; ++L) {
    const int sh = 10 - 10 * L;   // digits [19:10], then [9:0]
    const int top = 20 - 10 * L;  // key >> top must equal prefix
    for (int i = tid; i < 1024; i += NT) s_h[i] = 0;
    __syncthreads();
    for (u32 i = tid; i < cnt; i += NT) {
      const u32 key = in_lds ? s_list[i] : ld_agent(&a.list[i]);
      if ((key >> top) == prefix) atomicAdd(&s_h[(key >> sh) & 1023u], 1u);
    }
    __syncthreads();
    pick_bin<NT>(s_h, 1024, need, s_scan, s_out);
    prefix = (prefix << 10) | s_out[0];
    need -= s_out[1];
    __syncthreads();
  }
  if (tid == 0) {
    a.d_lambda[0] = __uint_as_float(prefix);
    st_agent(&a.st->listed, 0u);
    st_agent(&a.st->done, 0u);
  }
}

// ------------------------------------------------------------------ host --
struct EstLayout {
  size_t keys, list, total;
};

static EstLayout est_layout(int64_t m) {
  EstLayout L{};
  const size_t mb = ((size_t)std::max<int64_t>(m, 1) * 4 + 255) & ~(size_t)255;
  L.keys = kWorkspaceHeader;
  L.list = L.keys + mb;
  L.total = L.list + mb;
  return L;
}

}  // namespace tgs

using namespace tgs;

extern "C" size_t tgs_threshold_estimate_workspace_bytes(int64_t m) {
  if (m < 1 || m > kEstMaxM) return 0;
  return est_layout(m).total;
}

extern "C" tgs_status tgs_threshold_estimate(const float* grad, const float* residual, int64_t n,
                                             const int32_t* sample_idx, int64_t m, int64_t q, float* d_lambda,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n < 1 || n > INT32_MAX) return fail(TGS_EINVAL, "threshold_estimate: n=%lld outside [1, 2^31-1]", (long long)n);
  if (m < 1 || m > kEstMaxM) return fail(TGS_EINVAL, "threshold_estimate: m=%lld outside [1, 2^24]", (long long)m);
  if (q < 1 || q > m) return fail(TGS_EINVAL, "threshold_estimate: q=%lld outside [1, m]", (long long)q);
  if (!grad || !residual || !sample_idx || !d_lambda || !workspace)
    return fail(TGS_EINVAL, "threshold_estimate: null pointer");
  for (const void* p : {(const void*)grad, (const void*)residual, (const void*)sample_idx, (const void*)d_lambda})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "threshold_estimate: pointer not 4-byte aligned");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(TGS_EINVAL, "threshold_estimate: workspace not 256-byte aligned");
  const size_t nb4 = (size_t)n * 4;
  if (overlaps(d_lambda, 4, grad, nb4) || overlaps(d_lambda, 4, residual, nb4) ||
      overlaps(d_lambda, 4, sample_idx, (size_t)m * 4))
    return fail(TGS_EINVAL, "threshold_estimate: d_lambda overlaps an input");
  const EstLayout L = est_layout(m);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "threshold_estimate: workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (overlaps(d_lambda, 4, workspace, L.total)) return fail(TGS_EINVAL, "threshold_estimate: d_lambda in workspace");
  EstArgs a{};
  a.grad = grad;
  a.residual = residual;
  a.n = n;
  a.sample = sample_idx;
  a.m = (u32)m;
  a.q = (u32)q;
  a.keys = (u32*)((char*)workspace + L.keys);
  a.list = (u32*)((char*)workspace + L.list);
  a.hh = header_hist(workspace);
  a.st = (EstState*)((char*)workspace + kEstStateOffset);
  a.err = (u32*)workspace;
  a.d_lambda = d_lambda;
  const unsigned G1 = (unsigned)((m + kKeyChunk - 1) / kKeyChunk);
  const unsigned G2 = (unsigned)((m + kEstChunk - 1) / kEstChunk);
  hipLaunchKernelGGL(k_est_keys, dim3(G1), dim3(kKeyThreads), 0, stream, a);
  hipLaunchKernelGGL(k_est_select, dim3(G2), dim3(kEstThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "threshold_estimate: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

// Error-feedback top-k step on gfx950.
//
// Method (arxivdaily listing for arXiv 2004.05298, entries "Sparsified SGD
// with Memory" and "The Convergence of Sparsified Gradient Methods"): add the
// accumulated error to the gradient, send the k entries of largest magnitude,
// keep everything else as the new error.  The listing's entry "Empirical
// Analysis on Top-k Gradient Sparsification ..." names gradient sorting as the
// GPU bottleneck, so nothing here sorts more than the selected entries.
//
// Fast path (three launches, one pass over the data):
//   k_sample    reads ~1% of grad+residual in 64-element chunks, builds a
//               13-bit histogram of key >> 18 and, in its last workgroup, turns
//               it into a plan: a guess T_guess with about 1.4k keys above it
//               and up to 64 key ranges ("buckets") of ~1k expected entries.
//   k_ef_main   the only pass over the data: acc = residual + grad, residual <-
//               acc (non-temporal), and every key >= T_guess is stored as
//               (index, bits) in a fixed slot of (workgroup, bucket): no global
//               atomics, no ordering between workgroups.
//   k_finish    one workgroup per bucket: totals and prefix from the slot
//               counts, a validity verdict, the bucket gathered into LDS and
//               bitonic-sorted by (key desc, index asc); entries whose global
//               rank is below k are written out and their residual zeroed.
//               When the verdict fails, the same 64 workgroups run the exact
//               general path below on acc (now in residual).
// The result never depends on the guess: the fast path's output is used only
// when every candidate was kept, at least k keys reached T_guess and every
// bucket holding a rank below k fit in LDS.  Otherwise the exact path runs.
//
// General path (grid barriers, every workgroup resident): used as the fallback
// inside k_finish, and on its own (k_general) where no fast path applies:
//   radix select of the k-th key over 11/11/9-bit digits, counts per
//   workgroup, ordered compaction of the selected entries in ascending index
//   order (ties at the k-th key resolved by index), a stable LSD radix sort of
//   the k entries by descending key (4 x 8-bit digits), then emit and zero.
#include <algorithm>
#include <climits>
#include <cstring>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

// --------------------------------------------------------------- sizes ----
constexpr int kSampleChunk = 64;           // contiguous elements per sample chunk
constexpr int kHistShift = 18;             // sample histogram bin = key >> 18
constexpr int kHistBins = 1 << (31 - kHistShift);  // 8192
constexpr int kSampleThreads = 1024;
constexpr int kSampleBlocks = 64;
constexpr int kSampleUnroll = 8;          // chunks whose loads one wave issues together
constexpr int kSampleKeyCap = 5120;       // sample keys one workgroup keeps (80 chunks)
constexpr int kListPerBlock = 160;        // top sample keys one workgroup may publish
constexpr int kListCap = kSampleBlocks * kListPerBlock;  // 10240
constexpr int64_t kMaxChunks = (int64_t)kSampleBlocks * (kSampleKeyCap / 64);
constexpr int kRankBinCap = 256;          // bins up to this size are ranked by counting
constexpr int kMaxBuckets = 64;
constexpr int kSlot = 15;                  // entries per (workgroup, bucket); a count >= 16 means overflow
constexpr int kMaxMainBlocks = 2048;
constexpr int kMainThreads = 256;
constexpr int kMainU = 4;                  // float4 per thread per tile
constexpr int kFinishThreads = 1024;
constexpr int kFinishCap = 4096;           // entries one finish workgroup sorts
constexpr int kSubBins = 2048;             // key sub-ranges of a bucket in the finish sort
constexpr int kGenBlocks = 256;
constexpr int kGenThreads = 512;
constexpr int64_t kFastMinN = 1 << 16;
constexpr int64_t kFastMaxK = 48 * 1024;

struct Plan {
  u32 valid;
  u32 t_guess;
  u32 nbuckets;
  u32 pad;
  u32 lo[kMaxBuckets];  // bucket j holds keys in [lo[j], lo[j-1]); lo[-1] = 2^31
};

struct TopkCtl {
  u32 err;        // device error word: offset 0 of every workspace
  u32 ticket;     // k_sample arrivals
  u32 verdict;    // 1 when k_finish produced the whole output
  u32 fallbacks;  // calls whose plan did not hold (never reset by the library)
  u32 why;        // OR of the reasons plans failed: 1 plan, 2 slot overflow,
                  // 4 bucket over capacity, 8 fewer than k candidates
  u32 pad_lc;
  u32 pad0[58];
  Plan plan;
};

// State of the general path; k_ef_main's workgroup 0 clears it every call.
struct GenState {
  u32 hist[3][2048];
  u32 bar_count;
  u32 bar_abort;
  u32 bar_gen;
  u32 pad[61];
};
static_assert(sizeof(TopkCtl) <= 4096, "control block too large");

// Workspace layout (every region 256-byte aligned).
struct TopkLayout {
  size_t ctl, shist, slist, ghist, gcnt, lsd_cnt, lsd_pre, lsd_tot, cnt, slots, bufA, bufB, total;
  bool fast_possible;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool fast_eligible(int64_t n, int64_t k) {
  return k > 0 && n >= kFastMinN && k <= kFastMaxK && k * 8 <= n;
}

static TopkLayout topk_layout(int64_t n, int64_t k) {
  TopkLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.fast_possible = fast_eligible(n, k);
  L.ctl = take(4096);
  L.shist = take(sizeof(u32) * kHistBins);
  L.slist = take(sizeof(u32) * (kListCap + kSampleBlocks));
  L.ghist = take(sizeof(GenState));
  L.gcnt = take(sizeof(u32) * 2 * kGenBlocks);
  L.lsd_cnt = take(sizeof(u32) * 256 * kGenBlocks);
  L.lsd_pre = take(sizeof(u32) * 256 * kGenBlocks);
  L.lsd_tot = take(sizeof(u32) * 256);
  L.cnt = take(L.fast_possible ? (size_t)kMaxMainBlocks * kMaxBuckets : 0);
  L.slots = take(L.fast_possible ? sizeof(Pair) * kMaxMainBlocks * kMaxBuckets * kSlot : 0);
  L.bufA = take(sizeof(Pair) * (size_t)std::max<int64_t>(k, 1));
  L.bufB = take(sizeof(Pair) * (size_t)std::max<int64_t>(k, 1));
  L.total = off;
  return L;
}

// Sampling parameters derived from (n, k) on the host.
struct SampleParams {
  int64_t n;
  int64_t chunks;       // number of 64-element chunks sampled
  int64_t stride;       // chunk c starts at c * stride (stride = n / chunks >= 512)
  u32 c_target;         // sample count that must lie above T_guess
  u32 bucket_samples;   // expected sample count per bucket
  u32 break_plan;       // test hook: publish a plan that cannot hold
};

static SampleParams sample_params(int64_t n, int64_t k) {
  SampleParams sp{};
  sp.n = n;
  double tau = std::max(1.4 * (double)k, (double)k + 8192.0);  // candidates aimed for
  double alpha = tau / (double)k;
  double eps = 1.0 - 1.0 / alpha;                 // relative slack below tau
  double need_stat = 25.0 / (eps * eps);          // ~5 sigma of Poisson noise
  double bucket_elems = std::max(512.0, 1.2 * (double)k / 56.0);
  double nb_needed = std::ceil(1.1 * (double)k / bucket_elems);
  double c = std::max({need_stat, 8.0 * nb_needed, 64.0});
  double m = c * (double)n / tau;                 // sample elements
  int64_t chunks = (int64_t)std::ceil(m / kSampleChunk);
  chunks = std::max<int64_t>(chunks, kSampleBlocks);
  chunks = std::min<int64_t>(chunks, n / (8 * kSampleChunk));
  chunks = std::min<int64_t>(chunks, kMaxChunks);
  sp.chunks = std::max<int64_t>(chunks, 1);
  sp.stride = n / sp.chunks;
  double m_real = (double)sp.chunks * kSampleChunk;
  sp.c_target = (u32)std::max(1.0, std::ceil(tau * m_real / (double)n));
  sp.bucket_samples = (u32)std::max(1.0, std::ceil(bucket_elems * m_real / (double)n));
  return sp;
}

// ----------------------------------------------------------- k_sample ----
// One wave per sampled chunk (64 consecutive elements at c * stride); each
// wave issues the loads of up to kSampleUnroll chunks before using any, and
// the workgroup keeps every sample key in LDS.  Each workgroup publishes the
// top of its 13-bit histogram (bins down to where its own count from the top
// reaches 8x its share of c_target, +32) and the sample keys in those bins.
// Everything published goes through returning device atomics, so no cache
// write-back fences are needed; the last workgroup to arrive (relaxed
// ticket) builds the plan:
//   - T_guess = the c_target-th largest sample key, and bucket boundaries =
//     the (j+1)*bucket_samples-th largest, found exactly: the published keys
//     are grouped by bin (offsets from the histogram's suffix sums) and the
//     keys of each bin that holds a wanted rank are ranked by counting;
//   - where that is not possible (inconsistent counts, a bin larger than
//     kExactBinCap) the key is interpolated inside its bin.
// The plan is only a guess: k_finish checks that it held before using it.
__global__ __launch_bounds__(kSampleThreads) void k_sample(const float* __restrict__ grad,
                                                           const float* __restrict__ residual,
                                                           SampleParams sp, u32* __restrict__ shist,
                                                           u32* __restrict__ slist, TopkCtl* __restrict__ ctl) {
  constexpr int NT = kSampleThreads;
  constexpr int per = kHistBins / NT;  // bins per thread, top first
  constexpr u32 kNoKey = 0xFFFFFFFFu;
  __shared__ u32 s_h[kHistBins];        // 32 KB histogram, then suffix sums
  __shared__ u32 s_keys[kListCap];      // 40 KB sample keys; last workgroup: the published list
  __shared__ u32 s_cur[kHistBins];      // 32 KB last workgroup: group cursors, then bin flags
  __shared__ u32 s_grp[kListCap];       // 40 KB last workgroup: the list grouped by bin
  __shared__ u32 s_scan[NT / kWave + 1];
  __shared__ u32 s_tkey[kMaxBuckets + 1];  // wanted keys: [0] T_guess, [1+j] boundary j
  __shared__ u32 s_last, s_floor, s_bT, s_exact;
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += NT) s_h[i] = 0;
  for (int i = tid; i < kSampleKeyCap; i += NT) s_keys[i] = kNoKey;
  if (tid == 0) s_floor = kHistBins;
  __syncthreads();

  const int lane = lane_id();
  constexpr int waves = NT / kWave;
  const int w = tid / kWave;
  const int64_t wstride = (int64_t)gridDim.x * waves;
  const int64_t first = (int64_t)blockIdx.x * waves + w;
  for (int64_t t0 = 0; first + t0 * wstride < sp.chunks; t0 += kSampleUnroll) {
    float gg[kSampleUnroll], rr[kSampleUnroll];
    bool ok[kSampleUnroll];
#pragma unroll
    for (int j = 0; j < kSampleUnroll; ++j) {
      const int64_t c = first + (t0 + j) * wstride;
      const int64_t i = c * sp.stride + lane;
      ok[j] = c < sp.chunks && i < sp.n;
      gg[j] = ok[j] ? grad[i] : 0.0f;
      rr[j] = ok[j] ? residual[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kSampleUnroll; ++j) {
      if (!ok[j]) continue;
      const u32 key = key_of(rr[j] + gg[j]);
      atomicAdd(&s_h[key >> kHistShift], 1u);
      const int64_t slot = ((t0 + j) * waves + w) * kWave + lane;
      if (slot < kSampleKeyCap) s_keys[slot] = key;
    }
  }
  __syncthreads();
  // Publish the top of this workgroup's histogram -- bins down to where its
  // own count from the top reaches 8x its share of c_target (+32) -- and the
  // sample keys in those bins (at most kListPerBlock, in this workgroup's own
  // region of the list; its count goes to slist[kListCap + block]).  All of it
  // uses returning device atomics, issued together and awaited once.
  {
    const int hi = kHistBins - per * tid;
    u32 own = 0;
#pragma unroll
    for (int q = 1; q <= per; ++q) own += s_h[hi - q];
    u32 total;
    const u32 above = block_exclusive_sum<NT>(own, s_scan, total);
    const u32 want = 8u * ((sp.c_target + gridDim.x - 1) / gridDim.x) + 32u;
    u32 run = above;
    int lowest = kHistBins;
    for (int q = 1; q <= per; ++q) {
      if (run >= want) break;  // bins below this one are not needed
      lowest = hi - q;
      run += s_h[hi - q];
    }
    if (lowest < kHistBins) atomicMin(&s_floor, (u32)lowest);
  }
  __syncthreads();
  {
    const u32 floor_bin = s_floor;
    u32 mine = 0;
    for (int i = tid; i < kSampleKeyCap; i += NT) {
      const u32 key = s_keys[i];
      mine += key != kNoKey && (key >> kHistShift) >= floor_bin;
    }
    u32 count;
    u32 pos = block_exclusive_sum<NT>(mine, s_scan, count);
    u32 sink = 0;
    // histogram bins >= floor_bin
    for (int b = kHistBins - 1 - tid; b >= (int)floor_bin; b -= NT) {
      const u32 v = s_h[b];
      if (v) sink += add_agent_relaxed(&shist[b], v);
    }
    // keys in those bins
    u32* region = slist + (int64_t)blockIdx.x * kListPerBlock;
    for (int i = tid; i < kSampleKeyCap; i += NT) {
      const u32 key = s_keys[i];
      if (key != kNoKey && (key >> kHistShift) >= floor_bin) {
        if (pos < (u32)kListPerBlock)
          sink += __hip_atomic_exchange(&region[pos], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ++pos;
      }
    }
    if (tid == 0) sink += __hip_atomic_exchange(&slist[kListCap + blockIdx.x], count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (sink == 0x12345678u) s_scan[0] = sink;  // keeps the returned values live
  }
  __syncthreads();
  if (tid == 0) s_last = (add_agent_relaxed(&ctl->ticket, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup: histogram + published keys -> plan ----
  {
    u32 v[per];
#pragma unroll
    for (int j = 0; j < per; ++j) v[j] = ld_agent(&shist[tid + j * NT]);
#pragma unroll
    for (int j = 0; j < per; ++j) s_h[tid + j * NT] = v[j];
  }
  // offsets of the published regions (one lane of wave 0 per workgroup);
  // K = all published keys, or ~0 if a workgroup had more than its region holds
  static_assert(kSampleBlocks == kWave, "one lane per sampling workgroup");
  __shared__ u32 s_cnt[kSampleBlocks + 1];
  if (tid < kWave) {
    const u32 c = ld_agent(&slist[kListCap + tid]);
    const u32 cc = std::min(c, (u32)kListPerBlock);
    u32 x = cc;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const u32 y = __shfl_up(x, d, kWave);
      if (tid >= d) x += y;
    }
    s_cnt[tid] = x - cc;
    const bool trunc = ballot(c > (u32)kListPerBlock) != 0;
    if (tid == kWave - 1) s_cnt[kSampleBlocks] = trunc ? 0xFFFFFFFFu : x;
  }
  __syncthreads();
  const u32 K = s_cnt[kSampleBlocks];
  const int hi = kHistBins - per * tid;  // thread t owns bins [hi - per, hi), top first
  u32 own = 0;
#pragma unroll
  for (int q = 1; q <= per; ++q) own += s_h[hi - q];
  u32 total;
  u32 above = block_exclusive_sum<NT>(own, s_scan, total);
  // convert s_h into inclusive suffix sums cum[b] = sum_{b' >= b} h[b']
  {
    u32 run = above;
#pragma unroll
    for (int q = 1; q <= per; ++q) {
      run += s_h[hi - q];
      s_h[hi - q] = run;
    }
  }
  if (tid == 0) {
    s_bT = 0xFFFFFFFFu;
    s_exact = (K == total && K <= (u32)kListCap) ? 1u : 0u;  // K = ~0 if a region was truncated
  }
  __syncthreads();
  // b_T = the largest bin with cum[b_T] >= c_target (cum is non-increasing in b)
  for (int q = 1; q <= per; ++q) {
    if (s_h[hi - q] >= sp.c_target) {
      atomicMax((int*)&s_bT, hi - q);  // s_bT starts at -1 as int
      break;
    }
  }
  __syncthreads();
  const int bT = (int)s_bT;
  Plan* plan = &ctl->plan;
  if (bT < 0 || sp.break_plan) {
    if (tid == 0) {
      plan->valid = 1;
      plan->nbuckets = 1;
      plan->t_guess = sp.break_plan ? 0x7FFFFFFFu : 0xFFFFFFFFu;
      plan->lo[0] = plan->t_guess;
      if (!sp.break_plan) plan->valid = 0;
    }
    return;
  }
  auto bin_of_rank = [&](u32 q) -> int {  // largest b with cum[b] >= q (cum[0] >= q)
    int lo = 0, hi2 = kHistBins - 1;
    while (lo < hi2) {
      int mid = (lo + hi2 + 1) >> 1;
      if (s_h[mid] >= q) lo = mid;
      else hi2 = mid - 1;
    }
    return lo;
  };
  auto cum_above = [&](int b) -> u32 { return b + 1 < kHistBins ? s_h[b + 1] : 0u; };
  // wanted ranks: [0] c_target, [1+j] (j+1)*bucket_samples for j < nb-1
  u32 nb = (sp.c_target + sp.bucket_samples - 1) / sp.bucket_samples;
  nb = std::max(1u, std::min(nb, (u32)kMaxBuckets));
  const int ntarget = (int)nb;  // T_guess + nb-1 boundaries
  // default: interpolation inside the bin (used where no exact key is found)
  if (tid < ntarget) {
    const u32 q = tid == 0 ? sp.c_target : (u32)tid * sp.bucket_samples;
    const int b = bin_of_rank(q);
    const u32 above_b = cum_above(b);
    const u32 h = s_h[b] - above_b;  // >= q - above_b >= 1
    const u32 f = q - above_b;
    const u32 off = (u32)((((u64)f << kHistShift) + h - 1) / h);  // in [1, 2^18]
    s_tkey[tid] = (((u32)b + 1u) << kHistShift) - off;
  }
  for (int i = tid; i < kHistBins; i += NT) s_cur[i] = 0;
  for (int i = tid; i < kListCap; i += NT) s_grp[i] = kNoKey;
  __syncthreads();
  if (s_exact) {
    // flag the bins that hold a wanted rank: 1 = small (rank by counting),
    // 2 = large (second-level histogram)
    if (tid < ntarget) {
      const u32 q = tid == 0 ? sp.c_target : (u32)tid * sp.bucket_samples;
      const int b = bin_of_rank(q);
      atomicMax(&s_cur[b], s_h[b] - cum_above(b) <= (u32)kRankBinCap ? 1u : 2u);
    }
    {  // wave w copies regions w, w + 16, ...: every load issued before any use
      constexpr int kPerWave = kSampleBlocks / (NT / kWave);
      constexpr int kRows = (kListPerBlock + kWave - 1) / kWave;
      u32 v[kPerWave][kRows];
#pragma unroll
      for (int r = 0; r < kPerWave; ++r) {
        const int b2 = w + r * (NT / kWave);
        const u32 c = (b2 + 1 < kSampleBlocks ? s_cnt[b2 + 1] : K) - s_cnt[b2];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
          const u32 i = (u32)(lane + j * kWave);
          v[r][j] = i < c ? ld_agent(&slist[b2 * kListPerBlock + i]) : kNoKey;
        }
      }
#pragma unroll
      for (int r = 0; r < kPerWave; ++r) {
        const int b2 = w + r * (NT / kWave);
        const u32 o = s_cnt[b2];
        const u32 c = (b2 + 1 < kSampleBlocks ? s_cnt[b2 + 1] : K) - o;
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
          const u32 i = (u32)(lane + j * kWave);
          if (i < c) s_keys[o + i] = v[r][j];
        }
      }
    }
    __syncthreads();
    // large flagged bins, listed once each (few: the pile-ups).  Targets in
    // rank order are q_1 < ... < q_{nb-1} <= q_0 = c_target, so their bins do
    // not increase; a target lists its bin when the previous one's differs.
    __shared__ u32 s_fat[kMaxBuckets + 1];
    __shared__ u32 s_nfat;
    if (tid == 0) s_nfat = 0;
    __syncthreads();
    if (tid < ntarget) {
      const int order = tid == 0 ? ntarget - 1 : tid - 1;  // position in rank order
      const u32 q = tid == 0 ? sp.c_target : (u32)tid * sp.bucket_samples;
      const int b = bin_of_rank(q);
      int bprev = -1;
      if (order > 0) {
        const u32 qp = (u32)order * sp.bucket_samples;  // the target just before in rank order
        bprev = bin_of_rank(qp);
      }
      if (s_cur[b] == 2u && b != bprev) s_fat[atomicAdd(&s_nfat, 1u)] = (u32)b;
    }
    __syncthreads();  // s_cur is rewritten below
    // small flagged bins: group their keys (group of bin b starts at cum[b+1])
    for (int i = tid; i < kHistBins; i += NT) s_cur[i] = s_cur[i] == 1u ? (cum_above(i) | 0x80000000u) : 0u;
    __syncthreads();
    for (u32 i = tid; i < K; i += NT) {
      const u32 key = s_keys[i];
      const u32 b = key >> kHistShift;
      if (s_cur[b] & 0x80000000u) {
        const u32 pos = (atomicAdd(&s_cur[b], 1u) & 0x7FFFFFFFu);
        if (pos < (u32)kListCap) s_grp[pos] = key;
      }
    }
    __syncthreads();
    // rank each grouped key inside its bin (ties broken by position); a key of
    // global rank q-1 (0-based, from the top) is the wanted key for rank q
    for (u32 i = tid; i < K; i += NT) {
      const u32 x = s_grp[i];
      if (x == kNoKey) continue;
      const int b = (int)(x >> kHistShift);
      const u32 g0 = cum_above(b), g1 = s_h[b];
      u32 r = 0;
      for (u32 t = g0; t < g1; ++t) {
        const u32 y = s_grp[t];
        r += (y > x) || (y == x && t < i);
      }
      const u32 rank1 = g0 + r + 1;  // 1-based rank of x among all samples
      if (rank1 == sp.c_target) s_tkey[0] = x;
      if (rank1 % sp.bucket_samples == 0) {
        const u32 jj = rank1 / sp.bucket_samples;
        if (jj >= 1 && jj < nb) s_tkey[jj] = x;
      }
    }
    __syncthreads();
    // large bins: histogram of key bits [17:5] (8192 sub-bins of 32 keys) over
    // the bin's keys; a wanted key is the lower edge of the sub-bin where the
    // count from the top reaches its rank (never above the exact key)
    constexpr int kSubShift = 5;
    constexpr int kSubN = 1 << (kHistShift - kSubShift);  // 8192
    u32* sub = s_grp;  // free again
    for (u32 f = 0; f < s_nfat; ++f) {
      const u32 fb = s_fat[f];
      for (int i = tid; i < kSubN; i += NT) sub[i] = 0;
      __syncthreads();
      for (u32 i = tid; i < K; i += NT) {
        const u32 key = s_keys[i];
        if ((key >> kHistShift) == fb) atomicAdd(&sub[(key >> kSubShift) & (kSubN - 1)], 1u);
      }
      __syncthreads();
      const int shi = kSubN - per * tid;  // thread t owns sub-bins [shi - per, shi), top first
      u32 sown = 0;
#pragma unroll
      for (int q2 = 1; q2 <= per; ++q2) sown += sub[shi - q2];
      u32 stot;
      const u32 sabove = block_exclusive_sum<NT>(sown, s_scan, stot);
      {
        u32 run = sabove;
#pragma unroll
        for (int q2 = 1; q2 <= per; ++q2) {
          run += sub[shi - q2];
          sub[shi - q2] = run;  // suffix sums inside the bin
        }
      }
      __syncthreads();
      if (tid < ntarget) {
        const u32 q = tid == 0 ? sp.c_target : (u32)tid * sp.bucket_samples;
        if ((u32)bin_of_rank(q) == fb) {
          const u32 want = q - cum_above((int)fb);  // rank inside the bin, 1-based
          int lo = 0, hi2 = kSubN - 1;              // largest sub-bin with suffix >= want
          while (lo < hi2) {
            int mid = (lo + hi2 + 1) >> 1;
            if (sub[mid] >= want) lo = mid;
            else hi2 = mid - 1;
          }
          s_tkey[tid] = (fb << kHistShift) | ((u32)lo << kSubShift);
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
    const u32 tg = s_tkey[0];
    u32 prev = 0xFFFFFFFFu;
    for (int j = 0; j + 1 < (int)nb; ++j) {
      u32 v = std::max(s_tkey[1 + j], tg);
      v = std::min(v, prev);
      plan->lo[j] = v;
      prev = v;
    }
    plan->lo[nb - 1] = tg;
    plan->t_guess = tg;
    plan->nbuckets = nb;
    plan->valid = 1;
  }
}

// --------------------------------------------------------- k_ef_main ----
struct MainArgs {
  const float* grad;
  float* residual;
  int64_t n;
  int64_t head;  // scalar elements before the 16-byte aligned part
  int64_t nv;    // float4 vectors in the aligned part (0 = scalar mode)
  const Plan* plan;
  unsigned char* cnt;  // [G][kMaxBuckets]
  Pair* slots;         // [G][kMaxBuckets][kSlot]
  u32* zero_ptr;       // general-path state cleared by workgroup 0
  int zero_words;
  u32* err;            // device error word, cleared by workgroup 0
};

template <bool SPEC>
__device__ __forceinline__ void main_emit(int64_t idx, u32 bits, u32 tg, int nb, const u32* s_lo,
                                          u32* s_cnt, Pair* slots) {
  if (!SPEC) return;
  u32 key = key_of_bits(bits);
  if (key < tg) return;
  int lo = 0, hi = nb;  // bucket = #{i < nb : lo[i] > key}
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (s_lo[mid] > key) lo = mid + 1;
    else hi = mid;
  }
  int j = lo < nb ? lo : nb - 1;
  u32 pos = atomicAdd(&s_cnt[j], 1u);
  if (pos < (u32)kSlot) slots[((int64_t)blockIdx.x * kMaxBuckets + j) * kSlot + pos] = Pair{(int32_t)idx, bits};
}

template <bool SPEC, bool VEC>
__global__ __launch_bounds__(kMainThreads) void k_ef_main(MainArgs a) {
  __shared__ u32 s_lo[kMaxBuckets];
  __shared__ u32 s_cnt[kMaxBuckets];
  __shared__ u32 s_meta[2];
  const int tid = threadIdx.x;
  u32 tg = 0xFFFFFFFFu;
  int nb = 1;
  if (SPEC) {
    if (tid < kMaxBuckets) {
      s_cnt[tid] = 0;
      s_lo[tid] = a.plan->lo[tid];
    }
    if (tid == 0) {
      u32 v = a.plan->valid, b = a.plan->nbuckets;
      bool ok = (v == 1) && b >= 1 && b <= (u32)kMaxBuckets;
      s_meta[0] = ok ? a.plan->t_guess : 0xFFFFFFFFu;
      s_meta[1] = ok ? b : 1u;
    }
    __syncthreads();
    tg = s_meta[0];
    nb = (int)s_meta[1];
  }
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.zero_words; i += kMainThreads) a.zero_ptr[i] = 0u;
    if (tid == 0) *a.err = 0u;
  }

  const float* __restrict__ g = a.grad;
  float* __restrict__ r = a.residual;
  if (VEC) {
    // scalar head (workgroup 0), then this workgroup's contiguous vector range
    if (blockIdx.x == 0 && tid < a.head) {
      float acc = r[tid] + g[tid];
      r[tid] = acc;
      main_emit<SPEC>(tid, __float_as_uint(acc), tg, nb, s_lo, s_cnt, a.slots);
    }
    const v4f* __restrict__ gv = (const v4f*)(g + a.head);
    v4f* __restrict__ rv = (v4f*)(r + a.head);
    // tiles of kMainThreads * kMainU vectors, dealt round-robin to the
    // workgroups so that the whole grid sweeps the arrays front to back
    constexpr int64_t tile = (int64_t)kMainThreads * kMainU;
    const int64_t ve = a.nv;
    for (int64_t base = (int64_t)blockIdx.x * tile; base < ve; base += (int64_t)gridDim.x * tile) {
      v4f gg[kMainU], rr[kMainU];
#pragma unroll
      for (int u = 0; u < kMainU; ++u) {
        int64_t i = base + u * kMainThreads + tid;
        if (i < ve) {
          gg[u] = __builtin_nontemporal_load(gv + i);
          rr[u] = __builtin_nontemporal_load(rv + i);
        }
      }
#pragma unroll
      for (int u = 0; u < kMainU; ++u) {
        int64_t i = base + u * kMainThreads + tid;
        if (i < ve) {
          v4f acc = rr[u] + gg[u];
          __builtin_nontemporal_store(acc, rv + i);
          if (SPEC) {
            u32 b0 = __float_as_uint(acc.x), b1 = __float_as_uint(acc.y);
            u32 b2 = __float_as_uint(acc.z), b3 = __float_as_uint(acc.w);
            u32 kmax = std::max(std::max(key_of_bits(b0), key_of_bits(b1)),
                                std::max(key_of_bits(b2), key_of_bits(b3)));
            if (kmax >= tg) {
              int64_t e = a.head + 4 * i;
              main_emit<SPEC>(e + 0, b0, tg, nb, s_lo, s_cnt, a.slots);
              main_emit<SPEC>(e + 1, b1, tg, nb, s_lo, s_cnt, a.slots);
              main_emit<SPEC>(e + 2, b2, tg, nb, s_lo, s_cnt, a.slots);
              main_emit<SPEC>(e + 3, b3, tg, nb, s_lo, s_cnt, a.slots);
            }
          }
        }
      }
    }
    // scalar tail (last workgroup)
    if (blockIdx.x == gridDim.x - 1) {
      for (int64_t i = a.head + 4 * a.nv + tid; i < a.n; i += kMainThreads) {
        float acc = r[i] + g[i];
        r[i] = acc;
        main_emit<SPEC>(i, __float_as_uint(acc), tg, nb, s_lo, s_cnt, a.slots);
      }
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kMainThreads + tid; i < a.n; i += (int64_t)gridDim.x * kMainThreads) {
      float acc = r[i] + g[i];
      r[i] = acc;
      main_emit<SPEC>(i, __float_as_uint(acc), tg, nb, s_lo, s_cnt, a.slots);
    }
  }
  if (SPEC) {
    __syncthreads();
    if (tid < kMaxBuckets)
      a.cnt[(int64_t)blockIdx.x * kMaxBuckets + tid] = (unsigned char)std::min(s_cnt[tid], 255u);
  }
}

// --------------------------------------------------------- k_general ----
struct GenArgs {
  const float* acc;  // == residual; holds acc when this kernel runs
  float* residual;
  int64_t n, k;
  int32_t* out_idx;
  float* out_val;
  u32* ghist;    // 3 x 2048, zero on entry
  u32* gcnt;     // [G][2]
  u32* lsd_cnt;  // [G][256]
  u32* lsd_pre;  // [G][256]
  u32* lsd_tot;  // [256]
  Pair* bufA;
  Pair* bufB;
  GridBar bar;
};

// Sum over the block of one value per thread.
template <int NT>
__device__ __forceinline__ u32 block_sum(u32 v, u32* lds) {
  u32 total;
  block_exclusive_sum<NT>(v, lds, total);
  return total;
}

// The exact general path.  Every workgroup of the grid must be resident at
// once (grid barriers); NT is the workgroup size.
template <int NT>
__device__ void general_path(const GenArgs& a) {
  constexpr int NW = NT / kWave;
  __shared__ u32 s_hist[2048];
  __shared__ u32 s_wcnt[NW][256];
  __shared__ u32 s_base[256];
  __shared__ u32 s_run[256];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_found[4];
  const int tid = threadIdx.x;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int64_t per = (a.n + G - 1) / G;
  const int64_t cb = std::min<int64_t>(a.n, (int64_t)b * per);
  const int64_t ce = std::min<int64_t>(a.n, cb + per);
  const u32* accb = (const u32*)a.acc;

  // ---------------- radix select of the k-th largest key ----------------
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  u32 prefix = 0;      // digits chosen so far (the key's top bits)
  int64_t need = a.k;  // entries still to take among keys matching prefix
  int64_t t_strict = -1;  // select every key > t_strict ...
  u32 t_eq = 0;           // ... and the first r keys equal to t_eq
  int64_t r = 0;
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L], wd = widths[L];
    const u32 nbins = 1u << wd;
    for (int i = tid; i < 2048; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (int64_t i = cb + tid; i < ce; i += NT) {
      u32 key = key_of_bits(accb[i]);
      if ((key >> (sh + wd)) == prefix) atomicAdd(&s_hist[(key >> sh) & (nbins - 1)], 1u);
    }
    __syncthreads();
    for (int i = tid; i < (int)nbins; i += NT) {
      u32 v = s_hist[i];
      if (v) add_agent_relaxed(&a.ghist[L * 2048 + i], v);
    }
    if (!grid_sync(a.bar)) return;
    for (int i = tid; i < (int)nbins; i += NT) s_hist[i] = a.ghist[L * 2048 + i];
    __syncthreads();
    // thread t owns bins [nbins - cpt(t+1), nbins - cpt*t), scanning from the top
    const int cpt = (int)nbins / NT > 0 ? (int)nbins / NT : 1;
    const int top = (int)nbins - cpt * tid;  // exclusive
    u32 own = 0;
    if (top > 0)
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) own += s_hist[d];
    u32 tot;
    u32 above = block_exclusive_sum<NT>(own, s_scan, tot);
    if (tid == 0) s_found[0] = 0xFFFFFFFFu;
    __syncthreads();
    if (top > 0 && (int64_t)above < need && (int64_t)(above + own) >= need) {
      u32 run = above;
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) {
        u32 h = s_hist[d];
        if ((int64_t)(run + h) >= need) {
          s_found[0] = (u32)d;
          s_found[1] = run;
          s_found[2] = h;
          break;
        }
        run += h;
      }
    }
    __syncthreads();
    const u32 d = s_found[0];
    if (d == 0xFFFFFFFFu) {  // cannot happen for consistent counts
      if (tid == 0) atomicOr(a.bar.err, 1u << 2);
      return;
    }
    need -= (int64_t)s_found[1];
    const int64_t h = s_found[2];
    prefix = (prefix << wd) | d;
    if (need == h) {  // the whole digit range is taken: select key >= prefix << sh
      t_strict = (int64_t)((u64)prefix << sh) - 1;
      r = 0;
      break;
    }
    if (L == 2) {
      t_strict = prefix;
      t_eq = prefix;
      r = need;
    }
    __syncthreads();
  }

  // ---------------- per-workgroup counts ----------------
  u32 c_gt = 0, c_eq = 0;
  for (int64_t i = cb + tid; i < ce; i += NT) {
    u32 key = key_of_bits(accb[i]);
    c_gt += (int64_t)key > t_strict;
    c_eq += (r > 0) && key == t_eq;
  }
  c_gt = block_sum<NT>(c_gt, s_scan);
  c_eq = block_sum<NT>(c_eq, s_scan);
  if (tid == 0) {
    a.gcnt[2 * b] = c_gt;
    a.gcnt[2 * b + 1] = c_eq;
  }
  if (!grid_sync(a.bar)) return;

  // ---------------- ordered compaction (ascending index) ----------------
  {
    u32 pg = 0, pe = 0;
    for (int i = tid; i < b; i += NT) {
      pg += a.gcnt[2 * i];
      pe += a.gcnt[2 * i + 1];
    }
    pg = block_sum<NT>(pg, s_scan);
    pe = block_sum<NT>(pe, s_scan);
    int64_t out = (int64_t)pg + std::min<int64_t>((int64_t)pe, r);
    int64_t eq_seen = pe;
    for (int64_t base = cb; base < ce; base += NT) {
      int64_t i = base + tid;
      bool valid = i < ce;
      u32 bits = valid ? accb[i] : 0u;
      u32 key = key_of_bits(bits);
      bool gt = valid && (int64_t)key > t_strict;
      bool eq = valid && r > 0 && key == t_eq;
      u32 eq_tot;
      u32 eq_ex = block_exclusive_sum<NT>(eq ? 1u : 0u, s_scan, eq_tot);
      bool sel = gt || (eq && eq_seen + (int64_t)eq_ex < r);
      u32 sel_tot;
      u32 sel_ex = block_exclusive_sum<NT>(sel ? 1u : 0u, s_scan, sel_tot);
      if (sel && out + sel_ex < a.k) a.bufA[out + sel_ex] = Pair{(int32_t)i, bits};
      out += sel_tot;
      eq_seen += eq_tot;
    }
  }
  if (!grid_sync(a.bar)) return;

  // ---------------- stable LSD radix sort by descending key ----------------
  const int64_t per2 = (a.k + G - 1) / G;
  const int64_t sb = std::min<int64_t>(a.k, (int64_t)b * per2);
  const int64_t se = std::min<int64_t>(a.k, sb + per2);
  Pair* src = a.bufA;
  Pair* dst = a.bufB;
  const int w = tid / kWave;
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 8 * pass;
    for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (int64_t i = sb + tid; i < se; i += NT) {
      u32 inv = 0x7FFFFFFFu - key_of_bits(src[i].bits);
      atomicAdd(&s_hist[(inv >> sh) & 0xFFu], 1u);
    }
    __syncthreads();
    for (int i = tid; i < 256; i += NT) a.lsd_cnt[b * 256 + i] = s_hist[i];
    if (!grid_sync(a.bar)) return;
    // column scans: digit d handled by workgroup d % G
    for (int d = b; d < 256; d += G) {  // G <= NT: one column entry per thread
      u32 c = tid < G ? a.lsd_cnt[tid * 256 + d] : 0u;
      u32 colsum;
      u32 ex = block_exclusive_sum<NT>(c, s_scan, colsum);
      if (tid < G) a.lsd_pre[tid * 256 + d] = ex;
      if (tid == 0) a.lsd_tot[d] = colsum;
    }
    if (!grid_sync(a.bar)) return;
    for (int i = tid; i < 256; i += NT) s_hist[i] = a.lsd_tot[i];
    __syncthreads();
    bool identity = false;
    for (int i = 0; i < 256; ++i) identity = identity || ((int64_t)s_hist[i] == a.k);
    // every wave must finish reading s_hist before the next pass clears it
    __syncthreads();
    if (identity) continue;  // every key shares this digit: the pass is a no-op
    {
      u32 v = tid < 256 ? s_hist[tid] : 0u;
      u32 t;
      u32 ex = block_exclusive_sum<NT>(v, s_scan, t);
      if (tid < 256) {
        s_base[tid] = ex + a.lsd_pre[b * 256 + tid];
        s_run[tid] = 0;
      }
    }
    for (int i = tid; i < NW * 256; i += NT) (&s_wcnt[0][0])[i] = 0;
    __syncthreads();
    for (int64_t base = sb; base < se; base += NT) {
      int64_t i = base + tid;
      bool valid = i < se;
      Pair e = valid ? src[i] : pair_sentinel();
      u32 d = valid ? (((0x7FFFFFFFu - key_of_bits(e.bits)) >> sh) & 0xFFu) : 0u;
      u64 peers = ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        bool on = (d >> bit) & 1u;
        u64 m = ballot(valid && on);
        peers &= on ? m : ~m;
      }
      u32 rank = lanes_below(peers);
      if (valid && rank == 0) s_wcnt[w][d] = (u32)__popcll(peers);
      __syncthreads();
      if (valid) {
        u32 off = 0;
        for (int ww = 0; ww < w; ++ww) off += s_wcnt[ww][d];
        u32 pos = s_base[d] + s_run[d] + off + rank;
        if ((int64_t)pos < a.k) dst[pos] = e;
      }
      __syncthreads();
      if (tid < 256) {
        u32 s = 0;
        for (int ww = 0; ww < NW; ++ww) {
          s += s_wcnt[ww][tid];
          s_wcnt[ww][tid] = 0;
        }
        s_run[tid] += s;
      }
      __syncthreads();
    }
    if (!grid_sync(a.bar)) return;
    Pair* t = src;
    src = dst;
    dst = t;
  }

  // ---------------- emit and zero ----------------
  for (int64_t i = sb + tid; i < se; i += NT) {
    Pair e = src[i];
    a.out_idx[i] = e.idx;
    a.out_val[i] = __uint_as_float(e.bits);
    if (e.idx >= 0 && (int64_t)e.idx < a.n) a.residual[e.idx] = 0.0f;
  }
}

__global__ __launch_bounds__(kGenThreads) void k_general(GenArgs a) { general_path<kGenThreads>(a); }

// ---------------------------------------------------------- k_finish ----
struct FinishArgs {
  const Plan* plan;
  const unsigned char* cnt;
  const Pair* slots;
  int G1;
  int64_t n;
  int64_t k;
  int32_t* out_idx;
  float* out_val;
  float* residual;
  TopkCtl* ctl;
  u32* shist;
  GenArgs gen;  // fallback: the exact general path on this kernel's grid
};

__global__ __launch_bounds__(kFinishThreads) void k_finish(FinishArgs a) {
  constexpr int NT = kFinishThreads;
  constexpr int NW = NT / kWave;
  __shared__ Pair s_a[kFinishCap];         // 32 KB: the bucket as gathered
  __shared__ Pair s_b[kFinishCap];         // 32 KB: grouped by key sub-range
  __shared__ u32 s_sub_cnt[kSubBins];      // 8 KB
  __shared__ u32 s_sub_off[kSubBins];      // 8 KB
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_rows[kMaxMainBlocks];   // (row << 8) | count for this bucket
  __shared__ u32 s_part[NW][kMaxBuckets];  // per-wave bucket totals
  __shared__ u32 s_lo[kMaxBuckets];
  __shared__ u32 s_nrows, s_ovf, s_pos, s_kmin, s_kmax;
  __shared__ u32 s_ok;
  __shared__ int64_t s_start, s_mytot;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int j = blockIdx.x;
  if (tid < kMaxBuckets) s_lo[tid] = a.plan->lo[tid];
  if (tid == 0) {
    s_nrows = 0;
    s_ovf = 0;
    s_pos = 0;
    s_kmin = 0xFFFFFFFFu;
    s_kmax = 0;
  }
  // Slot counts: G1 rows of 64 bytes (one per bucket), read as 16 words per
  // row.  Thread t always sees word q = t % 16 of a row (buckets 4q .. 4q+3)
  // and adds the four byte counts as two pairs of 16-bit lanes.
  const u32* cw = (const u32*)a.cnt;
  const int q = tid & 15;
  constexpr int kWordsPerThread = kMaxMainBlocks * kMaxBuckets / 4 / NT;
  const int nwords = a.G1 * (kMaxBuckets / 4);
  u32 xw[kWordsPerThread];
#pragma unroll
  for (int i = 0; i < kWordsPerThread; ++i) {  // all loads in flight at once
    const int wd = tid + i * NT;
    xw[i] = wd < nwords ? cw[wd] : 0u;
  }
  __syncthreads();
  u32 even = 0, odd = 0, ovf = 0;
  const bool mine = q == (j >> 2);
  const int myb = j & 3;
#pragma unroll
  for (int i = 0; i < kWordsPerThread; ++i) {
    const u32 x = xw[i];
    even += x & 0x00FF00FFu;
    odd += (x >> 8) & 0x00FF00FFu;
    ovf |= x & 0xF0F0F0F0u;  // a count >= 16 = kSlot + 1: the slot overflowed
    if (mine) {
      const u32 v = (x >> (8 * myb)) & 0xFFu;
      if (v) {
        u32 p = atomicAdd(&s_nrows, 1u);
        s_rows[p] = ((u32)((tid + i * NT) >> 4) << 8) | v;
      }
    }
  }
  // reduce over the lanes of a wave that share q (q, q+16, q+32, q+48)
  even += __shfl_xor(even, 16, kWave);
  even += __shfl_xor(even, 32, kWave);
  odd += __shfl_xor(odd, 16, kWave);
  odd += __shfl_xor(odd, 32, kWave);
  if (lane < 16) {
    s_part[w][4 * q + 0] = even & 0xFFFFu;
    s_part[w][4 * q + 1] = odd & 0xFFFFu;
    s_part[w][4 * q + 2] = even >> 16;
    s_part[w][4 * q + 3] = odd >> 16;
  }
  if (ovf) atomicOr(&s_ovf, 1u);
  __syncthreads();
  // Verdict and bucket offsets, in wave 0 (lane i = bucket i).
  if (w == 0) {
    u32 t = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) t += s_part[ww][lane];
    const u32 nb = a.plan->nbuckets;
    bool plan_ok = a.plan->valid == 1 && nb >= 1 && nb <= (u32)kMaxBuckets;
    if (plan_ok) {
      const u32 lo_i = s_lo[lane];
      const u32 lo_prev = lane > 0 ? s_lo[lane - 1] : 0xFFFFFFFFu;
      const bool mono = (u32)lane >= nb || (u32)lane == 0 || lo_i <= lo_prev;
      plan_ok = ballot(!mono) == 0 && s_lo[nb - 1] == a.plan->t_guess;
    }
    u32 x = t;  // inclusive scan of the totals over buckets 0..63
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      u32 y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    const int64_t start = (int64_t)(x - t), all = __shfl(x, kWave - 1, kWave);
    const bool live = (u32)lane < nb;
    const bool bad = (!live && t != 0) || (live && start < a.k && t > (u32)kFinishCap);
    const bool valid = plan_ok && !s_ovf && ballot(bad) == 0 && all >= a.k;
    const u32 why = (plan_ok ? 0u : 1u) | (s_ovf ? 2u : 0u) | (ballot(bad) != 0 ? 4u : 0u) | (all >= a.k ? 0u : 8u);
    if (lane == j) {
      s_start = start;
      s_mytot = live ? t : 0;
    }
    if (lane == 0) {
      s_ok = valid;
      if (j == 0) {
        a.ctl->verdict = valid ? 1u : 0u;
        if (!valid) {
          a.ctl->fallbacks += 1u;
          a.ctl->why |= why;
        }
      }
    }
  }
  __syncthreads();
  if (!s_ok) {
    // the plan did not hold: every workgroup of this grid runs the exact path
    // (they all computed the same verdict from the same counts)
    general_path<NT>(a.gen);
    if (j == 0) {
      for (int i = tid; i < kHistBins; i += NT) a.shist[i] = 0u;
      if (tid == 0) {
        a.ctl->ticket = 0u;
      }
    }
    return;
  }
  const int64_t mystart = s_start, mytot = s_mytot;
  if (mytot > 0 && mystart < a.k) {
    const int m = (int)mytot;
    for (int i = tid; i < kSubBins; i += NT) s_sub_cnt[i] = 0;
    for (u32 rI = tid; rI < s_nrows; rI += NT) {
      u32 rc = s_rows[rI];
      u32 row = rc >> 8, c = rc & 0xFFu;
      u32 base = atomicAdd(&s_pos, c);
      const Pair* src = a.slots + ((int64_t)row * kMaxBuckets + j) * kSlot;
      Pair e8[kSlot];
#pragma unroll
      for (int e = 0; e < kSlot; ++e) e8[e] = (u32)e < c ? src[e] : pair_sentinel();
      u32 kmin = 0xFFFFFFFFu, kmax = 0;
#pragma unroll
      for (int e = 0; e < kSlot; ++e)
        if ((u32)e < c && base + e < (u32)kFinishCap) {
          s_a[base + e] = e8[e];
          const u32 kk = key_of_bits(e8[e].bits);
          kmin = std::min(kmin, kk);
          kmax = std::max(kmax, kk);
        }
      if (c) {
        atomicMin(&s_kmin, kmin);
        atomicMax(&s_kmax, kmax);
      }
    }
    __syncthreads();
    // Split [kmin, kmax] into kSubBins equal key sub-ranges, numbered from the
    // top (descending key), and group the entries by sub-range (counting
    // sort).  Inside a sub-range an entry's place is the number of entries of
    // that sub-range that rank before it; ranks are unique (indices differ).
    const u32 kmin = s_kmin;
    const u32 span = s_kmax - kmin + 1u;  // >= 1
    const int bits = span <= 1 ? 0 : 32 - __clz(span - 1);
    const int sh = bits > 11 ? bits - 11 : 0;  // kSubBins = 2^11
    auto sub_of = [&](const Pair& e) -> u32 {
      const u32 d = (key_of_bits(e.bits) - kmin) >> sh;
      return (u32)(kSubBins - 1) - (d < (u32)kSubBins ? d : (u32)(kSubBins - 1));
    };
    for (int i = tid; i < m; i += NT) atomicAdd(&s_sub_cnt[sub_of(s_a[i])], 1u);
    __syncthreads();
    {
      constexpr int per = kSubBins / NT;  // 2 consecutive sub-ranges per thread
      u32 v[per], own = 0;
#pragma unroll
      for (int q2 = 0; q2 < per; ++q2) {
        v[q2] = s_sub_cnt[tid * per + q2];
        own += v[q2];
      }
      u32 tot;
      u32 ex = block_exclusive_sum<NT>(own, s_scan, tot);
#pragma unroll
      for (int q2 = 0; q2 < per; ++q2) {
        s_sub_off[tid * per + q2] = ex;
        s_sub_cnt[tid * per + q2] = ex;  // becomes the fill cursor
        ex += v[q2];
      }
    }
    __syncthreads();
    for (int i = tid; i < m; i += NT) {
      Pair e = s_a[i];
      s_b[atomicAdd(&s_sub_cnt[sub_of(e)], 1u)] = e;
    }
    __syncthreads();
    const int64_t take = std::min<int64_t>(mytot, a.k - mystart);
    for (int i = tid; i < m; i += NT) {
      const Pair e = s_b[i];
      const u32 sb = sub_of(e);
      const u32 s0 = s_sub_off[sb], s1 = s_sub_cnt[sb];  // the cursor ended at the range's end
      const u64 re = pair_rank(e);
      u32 r = 0;
      for (u32 t = s0; t < s1; ++t) r += pair_rank(s_b[t]) < re;
      const int64_t p = (int64_t)(s0 + r);
      if (p < take) {
        a.out_idx[mystart + p] = e.idx;
        a.out_val[mystart + p] = __uint_as_float(e.bits);
        if (e.idx >= 0 && (int64_t)e.idx < a.n) a.residual[e.idx] = 0.0f;
      }
    }
  }
  if (j == 0) {
    for (int i = tid; i < kHistBins; i += NT) a.shist[i] = 0u;
    if (tid == 0) {
      a.ctl->ticket = 0u;
    }
  }
}

}  // namespace tgs

// ==================================================================== host ==
using namespace tgs;

extern "C" size_t tgs_topk_workspace_bytes(int64_t n, int64_t k) {
  if (n < 0 || n > INT32_MAX || k < 0 || k > n) return 0;
  return topk_layout(n, k).total;
}

extern "C" tgs_status tgs_topk_ef_step(const float* grad, float* residual, int64_t n, int64_t k,
                                       int32_t* out_idx, float* out_val, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (n < 0 || n > INT32_MAX) return fail(TGS_EINVAL, "topk_ef_step: n=%lld outside [0, 2^31-1]", (long long)n);
  if (k < 0 || k > n) return fail(TGS_EINVAL, "topk_ef_step: k=%lld outside [0, n=%lld]", (long long)k, (long long)n);
  if (n > 0 && (!grad || !residual)) return fail(TGS_EINVAL, "topk_ef_step: null grad/residual");
  if (k > 0 && (!out_idx || !out_val)) return fail(TGS_EINVAL, "topk_ef_step: null output pointer");
  if (!workspace) return fail(TGS_EINVAL, "topk_ef_step: null workspace");
  for (const void* p : {(const void*)grad, (const void*)residual, (const void*)out_idx, (const void*)out_val})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "topk_ef_step: pointer not 4-byte aligned");
  const size_t nb4 = (size_t)n * 4, kb4 = (size_t)k * 4;
  if (overlaps(grad, nb4, residual, nb4) || overlaps(grad, nb4, out_idx, kb4) ||
      overlaps(grad, nb4, out_val, kb4) || overlaps(residual, nb4, out_idx, kb4) ||
      overlaps(residual, nb4, out_val, kb4) || overlaps(out_idx, kb4, out_val, kb4))
    return fail(TGS_EINVAL, "topk_ef_step: overlapping buffers");
  const TopkLayout L = topk_layout(n, k);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "topk_ef_step: workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (n == 0) return TGS_OK;
  char* ws = (char*)workspace;
  TopkCtl* ctl = (TopkCtl*)(ws + L.ctl);

  const int path = (int)get_option(TGS_OPT_TOPK_PATH);
  const bool fast = path != 1 && L.fast_possible;

  MainArgs ma{};
  ma.grad = grad;
  ma.residual = residual;
  ma.n = n;
  const bool vec = (((uintptr_t)grad) & 15u) == (((uintptr_t)residual) & 15u);
  if (vec) {
    int64_t head = (int64_t)(((16u - (((uintptr_t)residual) & 15u)) & 15u) / 4u);
    head = std::min<int64_t>(head, n);
    ma.head = head;
    ma.nv = (n - head) / 4;
  }
  ma.plan = &ctl->plan;
  ma.cnt = (unsigned char*)(ws + L.cnt);
  ma.slots = (Pair*)(ws + L.slots);
  // general-path state: its histograms and the grid-barrier words
  GenState* gs = (GenState*)(ws + L.ghist);
  ma.zero_ptr = (u32*)gs;
  ma.zero_words = (int)(sizeof(GenState) / sizeof(u32));
  ma.err = &ctl->err;
  int64_t units = vec ? ma.nv : n;
  int64_t want = (units + kMainThreads * kMainU * (vec ? 1 : 4) - 1) / (kMainThreads * kMainU * (vec ? 1 : 4));
  int G1 = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxMainBlocks, want));
  int64_t gopt = get_option(TGS_OPT_MAIN_GRID);
  if (gopt > 0) G1 = (int)std::min<int64_t>(gopt, kMaxMainBlocks);

  hipEvent_t ev0, ev1;
  take_profile_events(&ev0, &ev1);

  if (fast) {
    SampleParams sp = sample_params(n, k);
    sp.break_plan = path == 2 ? 1u : 0u;
    hipLaunchKernelGGL(k_sample, dim3(kSampleBlocks), dim3(kSampleThreads), 0, stream, grad, residual, sp,
                       (u32*)(ws + L.shist), (u32*)(ws + L.slist), ctl);
  }
  if (ev0) (void)hipEventRecord(ev0, stream);
  if (fast) {
    if (vec) hipLaunchKernelGGL((k_ef_main<true, true>), dim3(G1), dim3(kMainThreads), 0, stream, ma);
    else hipLaunchKernelGGL((k_ef_main<true, false>), dim3(G1), dim3(kMainThreads), 0, stream, ma);
  } else {
    if (vec) hipLaunchKernelGGL((k_ef_main<false, true>), dim3(G1), dim3(kMainThreads), 0, stream, ma);
    else hipLaunchKernelGGL((k_ef_main<false, false>), dim3(G1), dim3(kMainThreads), 0, stream, ma);
  }
  if (ev1) (void)hipEventRecord(ev1, stream);

  if (k > 0) {
    GenArgs ga{};
    ga.acc = residual;
    ga.residual = residual;
    ga.n = n;
    ga.k = k;
    ga.out_idx = out_idx;
    ga.out_val = out_val;
    ga.ghist = &gs->hist[0][0];
    ga.gcnt = (u32*)(ws + L.gcnt);
    ga.lsd_cnt = (u32*)(ws + L.lsd_cnt);
    ga.lsd_pre = (u32*)(ws + L.lsd_pre);
    ga.lsd_tot = (u32*)(ws + L.lsd_tot);
    ga.bufA = (Pair*)(ws + L.bufA);
    ga.bufB = (Pair*)(ws + L.bufB);
    ga.bar.count = &gs->bar_count;
    ga.bar.gen = &gs->bar_gen;
    ga.bar.abort = &gs->bar_abort;
    ga.bar.err = &ctl->err;
    if (fast) {
      FinishArgs fa{};
      fa.plan = &ctl->plan;
      fa.cnt = ma.cnt;
      fa.slots = ma.slots;
      fa.G1 = G1;
      fa.n = n;
      fa.k = k;
      fa.out_idx = out_idx;
      fa.out_val = out_val;
      fa.residual = residual;
      fa.ctl = ctl;
      fa.shist = (u32*)(ws + L.shist);
      fa.gen = ga;
      // kMaxBuckets workgroups of kFinishThreads: far below one per compute
      // unit, so all are resident for the fallback's grid barriers
      hipLaunchKernelGGL(k_finish, dim3(kMaxBuckets), dim3(kFinishThreads), 0, stream, fa);
    } else {
      // every workgroup of k_general must be resident at once (grid barriers):
      // at most one per compute unit per occupancy slot, and never above kGenBlocks
      static int occ = 0;
      if (occ == 0) {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_general, kGenThreads, 0) != hipSuccess || o < 1) o = 1;
        occ = o;
      }
      const int cus = device_cu_count();
      if (cus <= 0) return fail(TGS_EHIP, "topk_ef_step: cannot read the compute-unit count");
      const int G = std::max(1, std::min(kGenBlocks, cus * occ));
      hipLaunchKernelGGL(k_general, dim3(G), dim3(kGenThreads), 0, stream, ga);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

// The layer-wise top-k step for the mid-size and small segments of one call,
// batched on gfx950.
//
// Method (fugumt page for arXiv 2502.07634, related-paper entry "L-GreCo:
// Layerwise-Adaptive Gradient Compression for Efficient and Accurate Deep
// Learning": compression layer by layer, each layer with its own degree; the
// step itself from the arxivdaily listing for arXiv 2004.05298, entries
// "Sparsified SGD with Memory" and "The Convergence of Sparsified Gradient
// Methods"): every segment gets the error-feedback top-k step with its own k.
//
// Segments of at most 2^23 entries with k <= 4096 run together, up to 64 per
// batch, in three launches whatever their number:
//   k_mid_guess   for each segment longer than 8192 entries: whole rows of
//                 4096 entries spread evenly over the segment are sampled,
//                 four rows per workgroup, into a 4096-bin histogram of
//                 key >> 19 (LDS, then added into the segment's histogram in
//                 memory); the segment's last workgroup to arrive takes the
//                 guess T, the lower edge of the bin that holds the j-th
//                 largest sampled key, and leaves the histogram zero.  j is
//                 set on the host: as few entries of the segment at or above
//                 T as keep at least k there by six standard deviations of
//                 the sample, and at most 8192.  The guess decides only how
//                 much work follows, never the result.
//   k_mid_pass    one block of 256 float4 (1024 entries) per 256-thread
//                 workgroup, in order over all the segments: acc = residual +
//                 grad written back; the entries with key >= T are ranked in
//                 index order inside the block and the first 64 stashed; the
//                 block's count.
//   k_mid_select  one workgroup per segment: its candidates into LDS in index
//                 order (the stashes, block after block; a segment of at most
//                 8192 entries is read whole from acc), then ordered by (key
//                 desc, index asc) with a counting sort over 2048 sub-ranges
//                 of their key span and a count of the entries ahead inside
//                 each sub-range; the first k emitted, their residual +0.
//                 When the guess did not hold (fewer than k candidates, more
//                 than 8192, or a stash that overflowed) the workgroup selects
//                 exactly from acc instead: three streaming radix levels over
//                 the segment and an ordered compaction in index order give
//                 the k entries, ordered the same way.  Every entry at or
//                 above the k-th key is a candidate whenever the guess holds,
//                 so both routes give the same set.
#include <algorithm>
#include <climits>
#include <cmath>

#include "tgs_host.h"
#include "tgs_internal.h"
#include "tgs_midseg.h"
#include "tgs_rank.h"

namespace tgs {

constexpr int kMidThreads = 1024;   // guess and select workgroups
constexpr int kMidWaves = kMidThreads / kWave;
constexpr int kMidRow = 4 * kMidThreads;  // a sampled row: 4096 entries
constexpr int kMidMaxRows = 64;     // sampled rows per segment at most
constexpr u32 kGuessRows = 4;       // sampled rows per workgroup of k_mid_guess
constexpr int kMidPassThreads = 256;
constexpr int kMidPassWaves = kMidPassThreads / kWave;
constexpr u32 kMidBlockCap = 64;    // stash places per block
constexpr int kMidList = 8192;  // candidates one select workgroup holds (LDS)
static_assert(kMidList <= kRankList, "the ranking's list holds them");
constexpr u32 kMidDirect = kMidList;  // segments read whole by the select workgroup
constexpr int kMidHistBins = 4096;  // sample histogram: key >> 19
constexpr u32 kMidNoGuess = 0xFFFFFFFFu;  // no stashing (the whole segment is read, or k = 0)
constexpr int kMidStream = 16;      // loads in flight per thread in the exact route

struct MidSeg {
  int64_t start;     // first entry (from grad / residual)
  u32 len, k;
  u32 out_off;       // its pairs start at out_idx + out_off; indices relative to `start`
  u32 nv;            // float4 slots after the head
  u32 blk0;          // its first block of the pass
  u32 rstride;       // sampled rows are rows 0, rstride, 2 rstride, ...
  u32 j;             // rank of the guess among the sampled keys
  u16 head;          // entries before the first 256-byte aligned one (< 64)
  u16 nrows;         // sampled rows (0: no guess)
  u32 gwg0;          // its first workgroup of k_mid_guess
  u32 pad;
};
static_assert(sizeof(MidSeg) == 48, "segment table entry");

struct MidArgs {
  const float* grad;
  float* residual;
  int32_t* out_idx;
  float* out_val;
  u32* T;            // [kMidMaxSeg] the guesses
  u32* H;            // [kMidMaxSeg][kMidHistBins] sample histograms (left zero)
  u32* cnt;          // [blocks] entries at or above T per block
  Pair* stash;       // [blocks][kMidBlockCap]
  u32* exact;        // segments selected exactly from acc (never reset)
  u32* done;         // [kMidMaxSeg] arrivals of k_mid_guess (left zero)
  u32 force_exact;   // test hook: every segment takes the exact route
  int nseg;
  MidSeg seg[kMidMaxSeg];
};

__host__ __device__ inline u32 mid_blocks(const MidSeg& s) {
  return std::max<u32>(1u, (s.nv + kMidPassThreads - 1) / kMidPassThreads);
}
// Workgroups of k_mid_guess for a segment (one that only writes the "no
// guess" mark when it samples nothing).
__host__ __device__ inline u32 guess_wgs(const MidSeg& s) {
  return std::max<u32>(1u, (s.nrows + kGuessRows - 1) / kGuessRows);
}
// The last segment of the table whose first unit (of `field`) is <= b.
template <class F>
__device__ __forceinline__ int seg_of(const MidArgs& a, u32 b, F field) {
  int lo = 0;
  for (int hi = a.nseg; hi - lo > 1;) {
    const int mid = (lo + hi) >> 1;
    if (field(a.seg[mid]) <= b) lo = mid;
    else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------ k_mid_guess ----
__global__ __launch_bounds__(kMidThreads) void k_mid_guess(MidArgs a) {
  __shared__ u32 s_h[kMidHistBins];
  __shared__ u32 s_scan[kMidWaves + 1];
  __shared__ u32 s_pick, s_last;
  const int tid = threadIdx.x;
  const int sg = seg_of(a, blockIdx.x, [](const MidSeg& m) { return m.gwg0; });
  const MidSeg S = a.seg[sg];
  if (S.nrows == 0 || S.k == 0) {
    if (tid == 0) a.T[sg] = kMidNoGuess;
    return;
  }
  const u32 w = blockIdx.x - S.gwg0, nw = guess_wgs(S);
  const u32 q0 = w * kGuessRows, q1 = std::min<u32>(S.nrows, q0 + kGuessRows);
  for (int i = tid; i < kMidHistBins; i += kMidThreads) s_h[i] = 0u;
  __syncthreads();
  // rows of the aligned body (after the head): one float4 per thread and row
  {
    const v4f* g = (const v4f*)(a.grad + S.start + S.head);
    const v4f* r = (const v4f*)(a.residual + S.start + S.head);
    v4f x[kGuessRows];
#pragma unroll
    for (u32 u = 0; u < kGuessRows; ++u) {
      const int64_t e = (int64_t)(q0 + u < q1 ? q0 + u : q0) * S.rstride * kMidThreads + tid;
      x[u] = __builtin_nontemporal_load(r + e) + __builtin_nontemporal_load(g + e);
    }
#pragma unroll
    for (u32 u = 0; u < kGuessRows; ++u)
      if (q0 + u < q1)
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&s_h[key_of(x[u][c]) >> 19], 1u);
  }
  __syncthreads();
  u32* H = a.H + (size_t)sg * kMidHistBins;
  for (int i = tid; i < kMidHistBins; i += kMidThreads)
    if (s_h[i]) (void)add_agent_relaxed(&H[i], s_h[i]);
  // the segment's last workgroup to arrive picks the guess: the adds are
  // complete before each workgroup arrives
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_relaxed(a.done + sg, 1u) == nw - 1u ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  for (int i = tid; i < kMidHistBins; i += kMidThreads) {
    s_h[i] = ld_agent(&H[i]);
    st_agent(&H[i], 0u);
  }
  if (tid == 0) s_pick = 0u;  // (unreached: the sample holds j keys)
  __syncthreads();
  constexpr int per = kMidHistBins / kMidThreads;
  const int top = kMidHistBins - per * tid;  // exclusive
  u32 c[per], own = 0;
#pragma unroll
  for (int u = 0; u < per; ++u) {
    c[u] = s_h[top - 1 - u];
    own += c[u];
  }
  u32 tot;
  const u32 above = block_exclusive_sum<kMidThreads>(own, s_scan, tot);
  if (above < S.j && above + own >= S.j) {
    u32 run = above;
#pragma unroll
    for (int u = 0; u < per; ++u) {
      if (run < S.j && run + c[u] >= S.j) s_pick = (u32)(top - 1 - u);
      run += c[u];
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.T[sg] = s_pick << 19;
    st_agent(a.done + sg, 0u);
  }
}

// ------------------------------------------------------------- k_mid_pass ----
__global__ __launch_bounds__(kMidPassThreads) void k_mid_pass(MidArgs a) {
  __shared__ u32 s_w[kMidPassWaves];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const u32 b = blockIdx.x;
  const int sg = seg_of(a, b, [](const MidSeg& m) { return m.blk0; });
  const MidSeg S = a.seg[sg];
  const u32 bl = b - S.blk0;
  const u32 nblk = mid_blocks(S);
  const u32 T = a.force_exact ? kMidNoGuess : a.T[sg];
  const float* __restrict__ g = a.grad + S.start;
  float* __restrict__ r = a.residual + S.start;
  const int64_t slot = (int64_t)bl * kMidPassThreads + w * kWave + lane;
  const bool in = slot < S.nv;
  const bool has_head = bl == 0 && w == 0 && S.head > 0;
  const u32 tail0 = S.head + 4 * S.nv;
  const bool has_tail = bl == nblk - 1 && w == kMidPassWaves - 1 && tail0 < S.len;
  v4f gg = {0, 0, 0, 0}, rr = gg;
  if (in) {
    gg = __builtin_nontemporal_load((const v4f*)(g + S.head) + slot);
    rr = __builtin_nontemporal_load((const v4f*)(r + S.head) + slot);
  }
  float xh = 0.0f, xt = 0.0f;
  bool qh = false, qt = false;
  if (has_head && (u32)lane < S.head) {
    xh = r[lane] + g[lane];
    qh = key_of(xh) >= T;
  }
  if (has_tail && (u32)lane < S.len - tail0) {
    xt = r[tail0 + lane] + g[tail0 + lane];
    qt = key_of(xt) >= T;
  }
  const v4f acc = rr + gg;
  u32 qm = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) qm |= (in && key_of(acc[c]) >= T ? 1u : 0u) << c;
  const u64 mh = ballot(qh), mt = ballot(qt);
  u32 mtot;
  const u32 mbelow = wave_rank4(qm, mtot);
  const u32 hcnt = (u32)__popcll(mh);
  if (lane == 0) s_w[w] = hcnt + mtot + (u32)__popcll(mt);
  __syncthreads();
  u32 woff = 0, btot = 0;
#pragma unroll
  for (int i = 0; i < kMidPassWaves; ++i) {
    const u32 v = s_w[i];
    woff += i < w ? v : 0u;
    btot += v;
  }
  Pair* __restrict__ stash = a.stash + (size_t)b * kMidBlockCap;
  if (qh) {
    const u32 s = woff + lanes_below(mh);
    if (s < kMidBlockCap) stash[s] = Pair{lane, __float_as_uint(xh)};
  }
  if (qm) {
    u32 s = woff + hcnt + mbelow;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if ((qm >> c) & 1u) {
        if (s < kMidBlockCap) stash[s] = Pair{(int32_t)(S.head + 4 * slot + c), __float_as_uint(acc[c])};
        ++s;
      }
  }
  if (qt) {
    const u32 s = woff + hcnt + mtot + lanes_below(mt);
    if (s < kMidBlockCap) stash[s] = Pair{(int32_t)(tail0 + lane), __float_as_uint(xt)};
  }
  if (in) {
    // the wave's 1 KB as whole lines (the body starts on a 256-byte
    // boundary), written through at device scope: the launch's end then has
    // no dirty lines of it to write back
    const u64 w0 = (u64)(slot - lane);  // the same in every lane: a scalar for the buffer's base
    const int64_t s0 = (int64_t)((u64)__builtin_amdgcn_readfirstlane((u32)(w0 >> 32)) << 32 | __builtin_amdgcn_readfirstlane((u32)w0));
    st_agent_v4_nt((v4f*)(r + S.head) + s0, (u32)kWave * 16u, (u32)(slot - s0) * 16u, acc);
  }
  if (has_head && (u32)lane < S.head) r[lane] = xh;
  if (has_tail && (u32)lane < S.len - tail0) r[tail0 + lane] = xt;
  if (tid == 0) a.cnt[b] = btot;
}

// ----------------------------------------------------------- k_mid_select ----
// Shared memory of the select workgroup: RankLds (list, sorting scratch).
using SelLds = RankLds;

// Exact route, streaming acc (len entries at r) from memory: the rule that
// selects the top `need` (every key >= t_lo, plus the first rr keys equal to
// t_eq), by three radix levels of 11, 11 and 9 bits.
__device__ void stream_select(const float* r, u32 len, u32 need, SelLds& s, u32& t_lo, u32& t_eq, u32& rr) {
  constexpr int NT = kMidThreads, B = kMidStream;
  const int tid = threadIdx.x;
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  u32 prefix = 0;
  t_lo = 0;
  t_eq = 0;
  rr = 0;
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L], wd = widths[L];
    const int nbins = 1 << wd;
    for (int i = tid; i < 2048; i += NT) s.cnt[i] = 0u;
    __syncthreads();
    for (u32 i0 = 0; i0 < len; i0 += (u32)B * NT) {
      u32 key[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const u32 i = i0 + (u32)u * NT + tid;
        key[u] = i < len ? key_of(r[i]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const u32 i = i0 + (u32)u * NT + tid;
        if (i < len && (key[u] >> (sh + wd)) == prefix) atomicAdd(&s.cnt[(key[u] >> sh) & (u32)(nbins - 1)], 1u);
      }
    }
    __syncthreads();
    const int cpt = nbins / NT > 0 ? nbins / NT : 1;
    const int top = nbins - cpt * tid;
    u32 own = 0;
    if (top > 0)
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) own += s.cnt[d];
    u32 tot;
    const u32 above = block_exclusive_sum<NT>(own, s.scan, tot);
    if (top > 0 && above < need && above + own >= need) {
      u32 run = above;
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) {
        const u32 h = s.cnt[d];
        if (run + h >= need) {
          s.found[0] = (u32)d;
          s.found[1] = run;
          s.found[2] = h;
          break;
        }
        run += h;
      }
    }
    __syncthreads();
    const u32 d = s.found[0];
    need -= s.found[1];
    const u32 h = s.found[2];
    prefix = (prefix << wd) | d;
    __syncthreads();
    if (need == h) {  // the whole digit range is taken
      t_lo = prefix << sh;
      return;
    }
    if (L == 2) {
      t_lo = prefix + 1;
      t_eq = prefix;
      rr = need;
    }
  }
}

// Exact route: the selected entries of acc (rule of stream_select) to
// s.list[0 ..) in index order; rows of kMidThreads entries, kMidStream rows
// in flight.
__device__ void stream_compact(const float* r, u32 len, u32 t_lo, u32 t_eq, u32 rr, SelLds& s) {
  constexpr int NT = kMidThreads, NW = kMidWaves, B = kMidStream;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  u32 gt_seen = 0, eq_seen = 0;
  int par = 0;
  for (u32 i0 = 0; i0 < len; i0 += (u32)B * NT) {
    u32 bits[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const u32 i = i0 + (u32)u * NT + tid;
      bits[u] = i < len ? __float_as_uint(r[i]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const u32 i = i0 + (u32)u * NT + tid;
      const bool inr = i < len;
      const u32 key = key_of_bits(bits[u]);
      const bool gsel = inr && key >= t_lo, esel = inr && rr > 0 && key == t_eq;
      const u64 bg = ballot(gsel), be = ballot(esel);
      if (lane == 0) {
        s.wc[par][w][0] = (u32)__popcll(bg);
        s.wc[par][w][1] = (u32)__popcll(be);
      }
      __syncthreads();
      u32 og = 0, oe = 0, tg = 0, te = 0;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const u32 cg = s.wc[par][q][0], ce = s.wc[par][q][1];
        og += q < w ? cg : 0u;
        oe += q < w ? ce : 0u;
        tg += cg;
        te += ce;
      }
      const u32 gb = gt_seen + og + lanes_below(bg), eb = eq_seen + oe + lanes_below(be);
      if (gsel || (esel && eb < rr)) s.list[gb + std::min(eb, rr)] = pack_pair(Pair{(int32_t)i, bits[u]});
      gt_seen += tg;
      eq_seen += te;
      par ^= 1;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kMidThreads) void k_mid_select(MidArgs a) {
  constexpr int NT = kMidThreads;
  __shared__ SelLds s;
  const int tid = threadIdx.x;
  const MidSeg S = a.seg[blockIdx.x];
  if (S.k == 0) return;
  const u32 k = S.k;
  float* r = a.residual + S.start;
  const u32 T = a.force_exact ? kMidNoGuess : a.T[blockIdx.x];
  // the candidates, in index order
  bool exact = false;
  u32 total = 0;
  if (T == kMidNoGuess && S.len <= kMidDirect && !a.force_exact) {
    total = S.len;  // the whole segment
    for (u32 i0 = 0; i0 < S.len; i0 += (u32)kMidStream * NT) {
      u32 bits[kMidStream];
#pragma unroll
      for (int u = 0; u < kMidStream; ++u) {
        const u32 i = i0 + (u32)u * NT + tid;
        bits[u] = i < S.len ? __float_as_uint(r[i]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kMidStream; ++u) {
        const u32 i = i0 + (u32)u * NT + tid;
        if (i < S.len) s.list[i] = pack_pair(Pair{(int32_t)i, bits[u]});
      }
    }
  } else if (T != kMidNoGuess) {
    // thread t owns blocks [t per, (t + 1) per) of the segment
    const u32 nblk = mid_blocks(S);
    const u32 per = (nblk + NT - 1) / NT;  // <= 8 (2^23 entries)
    const u32 q0 = std::min<u32>(nblk, (u32)tid * per), q1 = std::min<u32>(nblk, q0 + per);
    u32 c[8], own = 0, bad = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[u] = q0 + (u32)u < q1 ? a.cnt[S.blk0 + q0 + u] : 0u;
      own += c[u];
      bad |= c[u] > kMidBlockCap ? 1u : 0u;
    }
    if (tid == 0) s.flag = 0u;
    u32 tot;
    const u32 pre = block_exclusive_sum<NT>(own, s.scan, tot);
    if (bad) atomicOr(&s.flag, 1u);
    __syncthreads();
    total = tot;
    exact = s.flag != 0u || tot < k || tot > (u32)kMidList;
    if (!exact) {
      u32 at = pre;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const Pair* st = a.stash + (size_t)(S.blk0 + q0 + u) * kMidBlockCap;
        for (u32 e0 = 0; e0 < c[u]; e0 += 8) {
          Pair e[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) e[v] = e0 + v < c[u] ? st[e0 + v] : pair_sentinel();
#pragma unroll
          for (int v = 0; v < 8; ++v)
            if (e0 + v < c[u]) s.list[at + e0 + v] = pack_pair(e[v]);
        }
        at += c[u];
      }
    }
  } else {
    exact = true;  // (test hook)
  }
  __syncthreads();
  if (exact) {
    if (tid == 0) (void)add_agent_relaxed(a.exact, 1u);
    u32 t_lo, t_eq, rr;
    stream_select(r, S.len, k, s, t_lo, t_eq, rr);
    stream_compact(r, S.len, t_lo, t_eq, rr, s);
    total = k;
  }
  rank_emit(s, total, k, r, a.out_idx + S.out_off, a.out_val + S.out_off);
}

// ------------------------------------------------------------------ host ----
// The sampling plan of a segment, or false when the batched path should not
// take it (too long, k too large, or no sample size that keeps the expected
// candidate count in [k, kMidList] by a wide margin).
bool mid_plan(int64_t len, int64_t k, u32* nrows, u32* rstride, u32* j) {
  if (len <= 0 || len > kMidMaxN || k < 0 || k > kMidMaxK) return false;
  *nrows = 0;
  *rstride = 0;
  *j = 0;
  if (k == 0 || len <= kMidDirect) return true;  // no guess: acc only, or the whole segment
  const int64_t R = (len - 63) / kMidRow;  // whole rows of the aligned body, whatever the head
  // rows for about 1024 sampled keys at or above the guess when t = 1.3 k
  const double want = std::ceil(1024.0 / (1.3 * (double)k) * (double)len / kMidRow);
  const int64_t rows = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(R, kMidMaxRows), (int64_t)want));
  const double f = (double)rows * kMidRow / (double)len;
  // the smallest expected candidate count t whose guess holds by six
  // standard deviations: the j-th sampled key (j = f t) has t (1 -+ 6 /
  // sqrt(j)) entries of the segment at or above it (and at least j); the bin
  // below it adds at most a quarter
  for (double t = 1.1 * (double)k; t <= (double)kMidList; t *= 1.05) {
    const double jj = std::floor(f * t);
    if (jj < 1.0) continue;
    const double sd = 6.0 / std::sqrt(jj);
    if (!(jj >= (double)k || t * (1.0 - sd) >= 1.05 * (double)k)) continue;
    if (t * (1.0 + sd) * 1.25 > (double)kMidList) return false;
    *nrows = (u32)rows;
    *rstride = (u32)std::max<int64_t>(1, R / rows);
    *j = (u32)jj;
    return true;
  }
  return false;
}

size_t mid_blocks_of(int64_t start, int64_t len, const float* residual) {
  MidSeg s{};
  const uintptr_t p = (uintptr_t)(residual + start);
  s.len = (u32)len;
  s.head = (u16)std::min<int64_t>(len, (int64_t)(((256u - (p & 255u)) & 255u) / 4u));
  s.nv = (u32)((len - s.head) / 4);
  return mid_blocks(s);
}

size_t mid_workspace_bytes(int64_t blocks) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(4 * (size_t)kMidMaxSeg) + al(4 * (size_t)kMidMaxSeg * kMidHistBins) + al(4 * (size_t)blocks) +
         al(sizeof(Pair) * kMidBlockCap * (size_t)blocks);
}

tgs_status mid_launch(const float* grad, float* residual, int32_t* out_idx, float* out_val, int nseg,
                      const MidSegSpec* specs, u32* exact, u32* done, void* ws_mid, hipStream_t stream) {
  MidArgs m{};
  m.grad = grad;
  m.residual = residual;
  m.out_idx = out_idx;
  m.out_val = out_val;
  m.exact = exact;
  m.done = done;
  m.force_exact = get_option(TGS_OPT_TOPK_PATH) == 10 ? 1u : 0u;
  int64_t blocks = 0;
  for (int s = 0; s < nseg; ++s) blocks += (int64_t)mid_blocks_of(specs[s].start, specs[s].len, residual);
  char* w = (char*)ws_mid;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  m.T = (u32*)w;
  w += al(4 * (size_t)kMidMaxSeg);
  m.H = (u32*)w;
  w += al(4 * (size_t)kMidMaxSeg * kMidHistBins);
  m.cnt = (u32*)w;
  w += al(4 * (size_t)blocks);
  m.stash = (Pair*)w;
  int first = 0;
  while (first < nseg) {
    const int nb = std::min(kMidMaxSeg, nseg - first);
    m.nseg = nb;
    u32 blk = 0, gwg = 0;
    for (int q = 0; q < nb; ++q) {
      const MidSegSpec& sp = specs[first + q];
      MidSeg& s = m.seg[q];
      s = MidSeg{};
      s.start = sp.start;
      s.len = (u32)sp.len;
      s.k = (u32)sp.k;
      s.out_off = (u32)sp.out_off;
      const uintptr_t p = (uintptr_t)(residual + sp.start);
      s.head = (u16)std::min<int64_t>(sp.len, (int64_t)(((256u - (p & 255u)) & 255u) / 4u));
      s.nv = (u32)((sp.len - s.head) / 4);
      s.blk0 = blk;
      u32 nrows = 0;
      if (!mid_plan(sp.len, sp.k, &nrows, &s.rstride, &s.j))
        return fail(TGS_EINVAL, "topk_ef_step_segmented: segment of %lld entries, k=%lld, outside the batched path",
                    (long long)sp.len, (long long)sp.k);
      s.nrows = (u16)nrows;
      s.gwg0 = gwg;
      blk += mid_blocks(s);
      gwg += guess_wgs(s);
    }
    hipLaunchKernelGGL(k_mid_guess, dim3(gwg), dim3(kMidThreads), 0, stream, m);
    hipLaunchKernelGGL(k_mid_pass, dim3(blk), dim3(kMidPassThreads), 0, stream, m);
    hipLaunchKernelGGL(k_mid_select, dim3((unsigned)nb), dim3(kMidThreads), 0, stream, m);
    first += nb;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step_segmented: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

}  // namespace tgs

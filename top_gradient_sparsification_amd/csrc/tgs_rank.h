// Ordering of up to 8192 (index, value) pairs by one workgroup of 1024
// threads: (key desc, index asc), the first k emitted.  Used by the batched
// layer-wise path and by the bucketed ranking of the top-k step.
#pragma once

#include "tgs_internal.h"

namespace tgs {

constexpr int kRankThreads = 1024;
constexpr int kRankList = 12288;  // entries one workgroup orders (LDS)
constexpr int kRankBins = 2048;   // sub-ranges of the key span

__device__ __forceinline__ u32 umin(u32 x, u32 y) { return x < y ? x : y; }

static_assert(kRankList <= 65536, "places fit 16 bits");

// Shared memory of a ranking workgroup.
struct RankLds {
  u64 list[kRankList];  // the entries: packed pairs
  u16 tmp[kRankList];   // their places in list, grouped by sub-range of the key span
                        // (places, not copies: the room goes to a longer list)
  u32 cnt[kRankBins];  // entries per sub-range (and the radix histogram of the exact route)
  u32 start[kRankBins];
  u32 cur[kRankBins];
  u32 scan[kRankThreads / kWave + 1];
  u32 found[4];
  u32 wc[2][kRankThreads / kWave][2];
  u64 kmin, kmax;  // rank keys' span
  u32 flag;
};

// Orders the n entries of s.list (k <= n <= kRankList) by (key desc, index
// asc) and emits the first k: a counting sort over kRankBins equal
// sub-ranges of the span of the rank keys ((0x7FFFFFFF - key) << 32 |
// index), which keeps only the sub-ranges that start below rank k, then each
// entry's rank inside its sub-range by counting the entries of the sub-range
// before it; the emitted entries' residual becomes +0.  With np > 1 only the
// entries of sub-ranges [part kRankBins / np, (part + 1) kRankBins / np) are
// emitted (np workgroups that order the same entries then emit them all
// between them).  Entries whose key is at or above `sure` keep the residual
// they have (+0 already).  Every thread calls it.
__device__ inline void rank_emit(RankLds& s, u32 n, u32 k, float* r, int32_t* oi, float* ov, u32 part = 0,
                                 u32 np = 1) {
  constexpr int NT = kRankThreads;
  const int tid = threadIdx.x;
  // the rank order of an entry: (key desc, index asc), unique
  auto rkey = [](u64 pv) {
    return ((u64)(0x7FFFFFFFu - key_of_bits((u32)(pv >> 32))) << 32) | (u64)(u32)pv;
  };
  u64 mn = ~0ull, mx = 0ull;
  for (u32 i = tid; i < n; i += NT) {
    const u64 c = rkey(s.list[i]);
    mn = c < mn ? c : mn;
    mx = c > mx ? c : mx;
  }
  mn = wave_min64(mn);
  mx = wave_max64(mx);
  if (tid == 0) {
    s.kmin = ~0ull;
    s.kmax = 0ull;
  }
  for (int i = tid; i < kRankBins; i += NT) {
    s.cnt[i] = 0u;
    s.cur[i] = 0u;
  }
  __syncthreads();
  if (lane_id() == 0) {
    atomicMin(&s.kmin, mn);
    atomicMax(&s.kmax, mx);
  }
  __syncthreads();
  // sub-range of a rank key: monotone in it, so that the sub-ranges are
  // consecutive stretches of the order (and equal keys spread by index)
  const u64 cmin = s.kmin, span = s.kmax - s.kmin;
  const double scale = span ? (double)(kRankBins - 1) / (double)span : 0.0;
  auto sub = [&](u64 c) { return std::min<u32>((u32)((double)(c - cmin) * scale), (u32)(kRankBins - 1)); };
  for (u32 i = tid; i < n; i += NT) atomicAdd(&s.cnt[sub(rkey(s.list[i]))], 1u);
  __syncthreads();
  static_assert(kRankBins == 2 * NT, "two sub-ranges per thread");
  const u32 c0 = s.cnt[2 * tid], c1 = s.cnt[2 * tid + 1];
  u32 tot;
  const u32 b0 = block_exclusive_sum<NT>(c0 + c1, s.scan, tot);
  s.start[2 * tid] = b0;
  s.start[2 * tid + 1] = b0 + c0;
  // the sub-ranges that start below k hold the first E entries
  u32 E;
  (void)block_exclusive_sum<NT>((b0 < k ? c0 : 0u) + (b0 + c0 < k ? c1 : 0u), s.scan, E);
  for (u32 i = tid; i < n; i += NT) {
    const u64 pv = s.list[i];
    const u32 sb = sub(rkey(pv));
    const u32 a = s.start[sb];
    if (a < k) s.tmp[a + atomicAdd(&s.cur[sb], 1u)] = (u16)i;
  }
  __syncthreads();
  // this workgroup's share of the places [0, E): whole sub-ranges (minima
  // taken by value: std::min's references to E and to an LDS word would keep
  // E in scratch memory, which every launch then has to set up)
  const u32 lo = part == 0 ? 0u : umin(E, (u32)s.start[part * kRankBins / np]);
  const u32 hi = part + 1 >= np ? E : umin(E, (u32)s.start[(part + 1) * kRankBins / np]);
  for (u32 p = lo + tid; p < hi; p += NT) {
    const u64 pv = s.list[s.tmp[p]];
    const u64 me = rkey(pv);
    const u32 sb = sub(me);
    const u32 a = s.start[sb], c = s.cnt[sb];
    u32 rank = a;
    for (u32 q = a; q < a + c; ++q) rank += rkey(s.list[s.tmp[q]]) < me ? 1u : 0u;
    if (rank < k) {
      const Pair e = unpack_pair(pv);
      oi[rank] = e.idx;
      ov[rank] = __uint_as_float(e.bits);
      r[e.idx] = 0.0f;
    }
  }
}

}  // namespace tgs

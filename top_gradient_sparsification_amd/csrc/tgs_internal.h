// Internal helpers shared by the gfx950 kernels of the sparsifier library.
//
// Magnitude key (all kernels): key(x) = bits(x) & 0x7FFFFFFF, compared as an
// unsigned integer.  For every non-NaN float this orders like |x|; NaN ranks
// above infinity; -0 and +0 are equal.  Ties go to the lower index, so the
// rank order of (index, value) pairs is the ascending order of
//     rank_key = (0x7FFFFFFF - key) << 32 | index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tgs.h"

namespace tgs {

typedef uint32_t u32;
typedef uint64_t u64;
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Every workspace starts with this header; its first word is the device error
// word.  The top-k step keeps its control block (two sets of counters used by
// alternate calls) here; the other operations touch only the error word, so a
// workspace can move between operations without clearing it.
constexpr size_t kWorkspaceHeader = 32768;

// The end of every header: a 2048-bin histogram and an arrival counter that a
// launch's workgroups add into and its last arrival reads and leaves zero
// (the top-k guess, the threshold estimate).  Calls on one workspace are
// ordered, so they can share it.
struct HeaderHist {
  u32 hist[2048];
  u32 done;
  u32 pad[63];
};
constexpr size_t kHeaderHistOffset = kWorkspaceHeader - sizeof(HeaderHist);
// The 128 bytes before it: the threshold estimate's selection state.
constexpr size_t kEstStateOffset = kHeaderHistOffset - 128;
__host__ __device__ inline HeaderHist* header_hist(void* workspace) {
  return (HeaderHist*)((char*)workspace + kHeaderHistOffset);
}

// Device error word bits.
constexpr u32 kErrBadInput = 1u << 0;  // an index outside its range, or a repeated merge index

// ---------------------------------------------------------------- keys ----
__device__ __forceinline__ u32 key_of_bits(u32 b) { return b & 0x7FFFFFFFu; }
__device__ __forceinline__ u32 key_of(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }
__device__ __forceinline__ u64 rank_key(u32 bits, u32 idx) {
  return ((u64)(0x7FFFFFFFu - key_of_bits(bits)) << 32) | (u64)idx;
}

// A selected entry: index and the raw bits of its value.
struct Pair {
  int32_t idx;
  u32 bits;
};
// Sorts after every real entry (real indices are below 2^31).
__device__ __forceinline__ Pair pair_sentinel() { return Pair{-1, 0u}; }
__device__ __forceinline__ u64 pair_rank(const Pair& p) { return rank_key(p.bits, (u32)p.idx); }
__device__ __forceinline__ u64 pack_pair(const Pair& p) { return (u64)(u32)p.idx | ((u64)p.bits << 32); }
__device__ __forceinline__ Pair unpack_pair(u64 v) { return Pair{(int32_t)(u32)v, (u32)(v >> 32)}; }

// -------------------------------------------------------- wave helpers ----
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ u64 ballot(bool p) { return __ballot(p); }
// number of set bits of `mask` in lanes below this one
__device__ __forceinline__ u32 lanes_below(u64 mask) {
  return __builtin_amdgcn_mbcnt_hi((u32)(mask >> 32), __builtin_amdgcn_mbcnt_lo((u32)mask, 0u));
}

// ------------------------------------------------ device-scope atomics ----
__device__ __forceinline__ u32 ld_agent(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(u32* p, u32 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 add_agent_acqrel(u32* p, u32 v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 add_agent_relaxed(u32* p, u32 v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 xchg_agent(u32* p, u32 v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_agent64(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 add_agent64(u64* p, u64 v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 xchg_agent64(u64* p, u64 v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 or_agent(u32* p, u32 v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent64(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
typedef uint16_t u16;
__device__ __forceinline__ void st_agent_u16(u16* p, u16 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 ld_agent_u16(const u16* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A float4 store made at device scope (written through to where every XCD
// sees it, as the device-scope atomics are), with the streaming hint: a raw
// buffer store with the sc1 and nt cache-policy bits.  `base` must be the same
// in every lane of the wave; lanes whose byte offset lies at or beyond
// `nbytes` store nothing.  Once a wave has waited for its stores to complete
// (s_waitcnt vmcnt(0)), a store another workgroup makes to the same address
// after hearing from it through a device-scope atomic lands later.
constexpr int kPolicyNtSc1 = 2 | 16;  // cache-policy bits: nt = 2, sc1 = 16
__device__ __forceinline__ void st_agent_v4_nt(v4f* base, u32 nbytes, u32 off, v4f v) {
  typedef u32 v4u __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)nbytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rs, (int)off, 0, kPolicyNtSc1);
}
// The same uniform value in a scalar register the compiler cannot trace back
// to where it came from.  Kernel arguments are loaded as wide scalar blocks
// that stay one register tuple; under register pressure a spilled tuple is
// reloaded whole (16 registers) wherever any one of its fields is used.
__device__ __forceinline__ u32 opaque_u32(u32 v) {
  asm volatile("" : "+s"(v));
  return v;
}
template <class T>
__device__ __forceinline__ T* opaque_ptr(T* p) {
  u64 v = (u64)p;
  asm volatile("" : "+s"(v));
  return (T*)v;
}
// Waits until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// ------------------------------------------------- wave scans (DPP) ----
// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS traffic).  Every lane of the wave must be active.
__device__ __forceinline__ u32 wave_inclusive_sum(u32 x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
// Inclusive prefix minimum over the 64 lanes (same pattern, identity ~0).
__device__ __forceinline__ u32 wave_inclusive_min(u32 x) {
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x111, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x112, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x114, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x118, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x142, 0xa, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x143, 0xc, 0xf, false));
  return x;
}
// Sum, maximum and minimum over the wave, returned to every lane.
__device__ __forceinline__ u32 wave_sum(u32 x) { return __builtin_amdgcn_readlane(wave_inclusive_sum(x), 63); }
__device__ __forceinline__ u32 wave_max(u32 x) {
  x = max(x, (u32)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false));
  x = max(x, (u32)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false));
  x = max(x, (u32)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false));
  x = max(x, (u32)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false));
  x = max(x, (u32)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false));
  x = max(x, (u32)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ u32 wave_min(u32 x) {
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x111, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x112, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x114, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x118, 0xf, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x142, 0xa, 0xf, false));
  x = min(x, (u32)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// -------------------------------------------------- block-wide scans ----
// Exclusive prefix sum of one u32 per thread over the block; `total` gets the
// block sum.  `lds` needs one u32 per wave (+1).  Every thread must call it.
template <int NT>
__device__ __forceinline__ u32 block_exclusive_sum(u32 v, u32* lds, u32& total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const u32 x = wave_inclusive_sum(v);
  if (lane == kWave - 1) lds[w] = x;
  __syncthreads();
  u32 wave_off = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const u32 t = lds[i];
    if (i < w) wave_off += t;
    sum += t;
  }
  __syncthreads();
  total = sum;
  return wave_off + x - v;
}

// ---------------------------------------------------- grid barrier ----
// For the `nwg` workgroups 0 .. nwg-1 of a kernel whose whole grid is resident
// at once.  Every counter only grows (all are zero when the kernel starts).
// Workgroup b arrives at the counter of its group (b % 8).  No workgroup can
// arrive at barrier e+1 before every workgroup has arrived at barrier e, so
// the value an arrival returns tells which barrier it is (e = old / per + 1
// for a group of `per` workgroups) and whether it completes its group.  The
// last arrival of a group adds one to each of 8 copies of the all-counter
// (one cache line each, so that each group of pollers has its own), and
// barrier e is complete once a copy reaches 8 e (or nwg e below 8
// workgroups).  No reset or generation word sits on the critical path.  A
// bounded spin turns a missing workgroup into an error (flag bit in *err,
// `abort` set) instead of a hang; after an abort every barrier returns at once.
//
// Writes: every wave waits for its own memory operations to complete before
// its workgroup arrives, and data that crosses workgroups is stored at device
// scope (sc1 stores, atomics), which no L2 holds back, so no write-back is
// needed.  Reads: after the barrier the workgroup drops its cached lines
// (an agent-scope acquire: L1 and L2 invalidate, no write-back), so plain
// loads then see what the others wrote.
struct GridBar {
  u32* cnt;    // [9][32]: the 8 group counters, one cache line each; zero at start
  u32* gen;    // [8][32]: the 8 copies of the all-counter, one per line; zero at start
  u32* abort;  // zero at start
  u32* err;    // device error word
  u32 nwg;     // participating workgroups
};

constexpr u32 kErrBarrierTimeout = 1u << 1;

__device__ __forceinline__ bool grid_sync(const GridBar& gb) {
  __shared__ u32 s_ok;
  wait_all_memory();  // every wave: its own stores have completed at device scope
  __syncthreads();
  if (threadIdx.x == 0) {
    u32 ok = 1;
    if (ld_agent(gb.abort) != 0) {
      ok = 0;
    } else {
      const u32 ng = gb.nwg < 8u ? gb.nwg : 8u;
      const u32 x = blockIdx.x % ng;
      const u32 per = (gb.nwg - 1u - x) / ng + 1u;
      const u32 old = add_agent_relaxed(gb.cnt + 32 * x, 1u);
      const u32 e = old / per + 1u;
      if (old + 1u == e * per) {  // last of its group
#pragma unroll
        for (int i = 0; i < 8; ++i) (void)add_agent_relaxed(gb.gen + 32 * i, 1u);
      }
      const u32* mine = gb.gen + 32 * (blockIdx.x & 7u);
      const u32 target = e * ng;
      u32 spins = 0;
      while ((int)(ld_agent(mine) - target) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 23)) {
          atomicOr(gb.err, kErrBarrierTimeout);
          st_agent(gb.abort, 1u);
          ok = 0;
          break;
        }
        if ((spins & 1023u) == 0 && ld_agent(gb.abort) != 0) {
          ok = 0;
          break;
        }
      }
    }
    s_ok = ok;
  }
  if (threadIdx.x < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  return s_ok != 0;
}

// Rank inside the wave of this lane's first qualifying component (bit c of
// qm: component c qualifies), lanes in order and components in order inside
// a lane; `tot` gets the wave's count.  Every lane of the wave calls it.
__device__ __forceinline__ u32 wave_rank4(u32 qm, u32& tot) {
  u32 below = 0;
  tot = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u64 m = ballot((qm >> c) & 1u);
    below += lanes_below(m);
    tot += (u32)__popcll(m);
  }
  return below;
}

// ------------------------------------------------ LDS select / sort ----
// Radix select in LDS of the need-th largest key among `len` entries, whose
// key is key_at(i) (i < len, 8 per thread at i = tid + j NT).  Returns the
// selection rule: every key >= t_lo, plus the first r keys equal to t_eq.
template <int NT, class KeyAt>
__device__ __forceinline__ void lds_select(KeyAt key_at, u32 len, u32 need, u32* s_hist, u32* s_scan, u32* s_found,
                                           u32& t_lo, u32& t_eq, u32& r) {
  const int tid = threadIdx.x;
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  u32 prefix = 0;
  t_lo = 0;
  t_eq = 0;
  r = 0;
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L], wd = widths[L];
    const int nbins = 1 << wd;
    for (int i = tid; i < 2048; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (u32 i = tid; i < len; i += NT) {
      const u32 key = key_at(i);
      if ((key >> (sh + wd)) == prefix) atomicAdd(&s_hist[(key >> sh) & (u32)(nbins - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins [nbins - cpt (t+1), nbins - cpt t), from the top
    const int cpt = nbins / NT > 0 ? nbins / NT : 1;
    const int top = nbins - cpt * tid;
    u32 own = 0;
    if (top > 0)
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) own += s_hist[d];
    u32 tot;
    const u32 above = block_exclusive_sum<NT>(own, s_scan, tot);
    if (top > 0 && above < need && above + own >= need) {
      u32 run = above;
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) {
        const u32 h = s_hist[d];
        if (run + h >= need) {
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
    need -= s_found[1];
    const u32 h = s_found[2];
    prefix = (prefix << wd) | d;
    __syncthreads();  // s_found is rewritten by the next level
    if (need == h) {  // the whole digit range is taken
      t_lo = prefix << sh;
      return;
    }
    if (L == 2) {
      t_lo = prefix + 1;
      t_eq = prefix;
      r = need;
    }
  }
}

// Ordered compaction: entries i < len (pair_at(i), key of its bits) in index
// order i = j NT + tid; the selected ones (key >= t_lo, or among the first r
// equal to t_eq) go to place(pos, pair) with pos their rank among them.
template <int NT, int ROWS, class PairAt, class Place>
__device__ __forceinline__ void lds_compact(PairAt pair_at, u32 len, u32 t_lo, u32 t_eq, u32 r, u32 (*s_wc)[NT / kWave][2],
                                            Place place) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  u32 gt_seen = 0, eq_seen = 0;
  for (int j = 0; j < ROWS; ++j) {
    const u32 i = (u32)(j * NT + tid);
    const bool in = i < len;
    const u64 pv = in ? pair_at(i) : 0ull;
    const u32 key = key_of_bits((u32)(pv >> 32));
    const bool g = in && key >= t_lo, e = in && r > 0 && key == t_eq;
    const u64 bg = ballot(g), be = ballot(e);
    const int par = j & 1;
    if (lane == 0) {
      s_wc[par][w][0] = (u32)__popcll(bg);
      s_wc[par][w][1] = (u32)__popcll(be);
    }
    __syncthreads();
    u32 og = 0, oe = 0, tg = 0, te = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const u32 cg = s_wc[par][q][0], ce = s_wc[par][q][1];
      og += q < w ? cg : 0u;
      oe += q < w ? ce : 0u;
      tg += cg;
      te += ce;
    }
    const u32 gb = gt_seen + og + lanes_below(bg), eb = eq_seen + oe + lanes_below(be);
    if (g || (e && eb < r)) place(gb + std::min(eb, r), pv);
    gt_seen += tg;
    eq_seen += te;
  }
}

// Sorted runs of 64-bit keys by one workgroup of kSortThreads; merges of
// them kSortTile outputs to a workgroup.
constexpr int kSortTile = 4096;
constexpr int kSortThreads = 1024;
constexpr int kSortPer = kSortTile / kSortThreads;
// Rank key of a pair: ascending order is (key desc, index asc); the sign
// rides in bit 0 (never decides: (key, index) is unique).
__device__ __forceinline__ u64 rank64(const Pair& e) {
  const u32 key = key_of_bits(e.bits);
  return ((u64)(0x7FFFFFFFu - key) << 32) | ((u64)((u32)e.idx & 0x7FFFFFFFu) << 1) | (u64)(e.bits >> 31);
}
__device__ __forceinline__ Pair unrank64(u64 r) {
  const u32 key = 0x7FFFFFFFu - (u32)(r >> 32);
  return Pair{(int32_t)(((u32)r >> 1) & 0x7FFFFFFFu), key | (((u32)r & 1u) << 31)};
}

// 64-bit minimum and maximum over the wave (every lane gets them).
__device__ __forceinline__ u64 wave_min64(u64 v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const u64 o = ((u64)(u32)__shfl_xor((int)(u32)(v >> 32), m) << 32) | (u64)(u32)__shfl_xor((int)(u32)v, m);
    v = o < v ? o : v;
  }
  return v;
}
__device__ __forceinline__ u64 wave_max64(u64 v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const u64 o = ((u64)(u32)__shfl_xor((int)(u32)(v >> 32), m) << 32) | (u64)(u32)__shfl_xor((int)(u32)v, m);
    v = o > v ? o : v;
  }
  return v;
}

// LDS of block_sort<PER, BINS>, in u64 words: the keys grouped by
// sub-range, then two tables of BINS counters.
constexpr int block_sort_lds(int per, int bins) { return per * kSortThreads + bins; }

// Sorts PER * kSortThreads keys ascending; thread t holds elements PER t ..
// PER t + PER - 1 in x, and the sorted ones there after the call.  Keys equal
// to ~0 (padding) must sit at the tail and stay there.  A counting sort of
// the other keys over BINS equal sub-ranges of their span, then each key's
// place inside its sub-range by counting the keys there below it (a few to
// a sub-range, where a bitonic network over 4096 keys takes 78
// compare-and-exchange stages; equal keys keep the order in which they were
// grouped).  Every thread calls it.
template <int PER, int BINS>
__device__ inline void block_sort(u64 (&x)[PER], u64* lds) {
  constexpr int NT = kSortThreads, B = BINS, TILE = PER * NT, BPT = B / NT;
  static_assert(BPT * NT == B && (BPT == 1 || BPT == 2), "one or two sub-ranges per thread");
  __shared__ u64 s_lo, s_hi;
  __shared__ u32 s_scan[NT / kWave + 1];
  u64* keys = lds;                     // [TILE]
  u32* cnt = (u32*)(lds + TILE);       // [B]: counts, then fill cursors (sub-range ends)
  u32* start = cnt + B;                // [B]
  const int tid = threadIdx.x;
  u64 lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int c = 0; c < PER; ++c)
    if (x[c] != ~0ull) {
      lo = x[c] < lo ? x[c] : lo;
      hi = x[c] > hi ? x[c] : hi;
    }
  lo = wave_min64(lo);
  hi = wave_max64(hi);
  if (tid == 0) {
    s_lo = ~0ull;
    s_hi = 0ull;
  }
  for (int i = tid; i < B; i += NT) cnt[i] = 0u;
  __syncthreads();
  if (lane_id() == 0) {
    atomicMin(&s_lo, lo);
    atomicMax(&s_hi, hi);
  }
  __syncthreads();
  const u64 base = s_lo;
  const double scale = s_hi > s_lo ? (double)(B - 1) / (double)(s_hi - s_lo) : 0.0;
  u32 sb[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    sb[c] = std::min<u32>((u32)((double)(x[c] - base) * scale), (u32)(B - 1));  // monotone in the key
    if (x[c] != ~0ull) atomicAdd(&cnt[sb[c]], 1u);
  }
  __syncthreads();
  const u32 c0 = cnt[BPT * tid], c1 = BPT == 2 ? cnt[BPT * tid + 1] : 0u;
  u32 all;
  const u32 b0 = block_exclusive_sum<NT>(c0 + c1, s_scan, all);
  start[BPT * tid] = b0;
  cnt[BPT * tid] = b0;
  if (BPT == 2) {
    start[BPT * tid + 1] = b0 + c0;
    cnt[BPT * tid + 1] = b0 + c0;
  }
  __syncthreads();
  u32 at[PER];  // each key's slot in its sub-range's group
#pragma unroll
  for (int c = 0; c < PER; ++c)
    if (x[c] != ~0ull) {
      at[c] = atomicAdd(&cnt[sb[c]], 1u);
      keys[at[c]] = x[c];
    }
  __syncthreads();
  u32 place[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    place[c] = (u32)(PER * tid + c);  // padding keeps its place
    if (x[c] == ~0ull) continue;
    const u32 a = start[sb[c]], e = cnt[sb[c]];
    u32 r = a;
    for (u32 q = a; q < e; ++q) r += (keys[q] < x[c] || (keys[q] == x[c] && q < at[c])) ? 1u : 0u;
    place[c] = r;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < PER; ++c) keys[place[c]] = x[c];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < PER; ++c) x[c] = keys[PER * tid + c];
  __syncthreads();  // (the caller may reuse lds)
}

}  // namespace tgs

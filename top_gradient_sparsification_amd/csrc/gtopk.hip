// gTop-k tournament of P workers' sparse sets on one gfx950 GPU.
//
// Method (nubint review "A Distributed Synchronous SGD Algorithm with Global
// Top-k Sparsification for Low Bandwidth Networks", ABSTRACT and Method): the
// global top-k largest |values| over P workers, found by a tournament of
// O(log P) pairwise rounds; only the indices that survive keep their index
// information, and each worker learns which of its own entries survived.
//
// A merge needs the union by index of two k-sets and the k best of it.  The
// union is a hash join in LDS: the indices are hashed into NP parts, and one
// workgroup per (merge, part) builds a table of the A side's entries of its
// part and looks the B side's entries of its part up in it.  Every set is
// kept grouped by part (a directory gives each part's place and length), so a
// workgroup reads its own part and nothing else.  No set is ever sorted by
// index and no table lives in memory:
//   k_gt_rcount    counts each row's entries per part, per chunk of 4096 (and
//                  zero-fills the call's histograms and counters);
//   k_gt_rscatter  copies each row grouped by part, every entry with its
//                  place in the row, and writes the rows' directories.
//   round r, for every merge m (slot s = m 2^(r+1) absorbs s + 2^r):
//     k_gt_join   workgroup (m, part): the A entries of its part into an LDS
//                 table; each B entry of its part found there adds its value
//                 to that entry (one binary32 add), the others go to the
//                 part's region of the merge's union W; then the A entries.
//                 The union's keys are counted into the merge's histogram of
//                 key >> 20, and the last workgroup of the merge to arrive
//                 finds the bin b1 that holds the k-th key.
//     k_gt_keep   workgroup (m, part): every entry of its part of W above bin
//                 b1 goes to the same part of slot s's output, the entries of
//                 bin b1 are listed as candidates, and the last workgroup of
//                 the merge to arrive finds the k-th key T and the largest
//                 index I kept at T among them, places the candidates with
//                 key > T, or key = T and index <= I (ties keep the lowest
//                 indices), each in its part, and writes the directory.
//   k_gt_final  the mask, as a join of each row's part against the final
//               set's (and the rows' precondition check: a repeated index
//               within a row, or one outside [0, n), sets the error word),
//               and runs of 4096 of the final set sorted by (key desc, index
//               asc) with a counting sort in LDS;
//   k_gt_merge  passes merge the runs; the last one writes the outputs.
// Slots without a partner keep their data where it is until they are merged:
// a slot's data is its grouped row until it has been a merge's destination,
// then its output region, which each later merge into it rewrites.
#include <algorithm>
#include <climits>
#include <vector>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

constexpr int kGtThreads = 1024;
constexpr int kGtWaves = kGtThreads / kWave;
constexpr int kGtBins = 2048;      // first-level bins: key >> 20
constexpr int kSelList = 8192;     // candidates the select holds in LDS
constexpr int kGtBatch = 16;       // loads in flight per thread in the scans
constexpr u32 kLogSlots = 13;      // places of one part's LDS table
constexpr u32 kSlots = 1u << kLogSlots;
constexpr int64_t kPartLoad = 2048;  // entries of one set a part holds on average at most
constexpr int64_t kGtMaxK = (int64_t)1 << 20;
constexpr u32 kMaxParts = 512;     // parts at k = kGtMaxK
// The final set is sorted in runs of kRunTile (one workgroup each, a counting
// sort over kRunBins sub-ranges in LDS), which merge passes then join.  (Runs
// of 8192 over 1024 sub-ranges, one merge pass fewer, were slower: the
// final set's keys crowd just above its least, and the count inside a
// sub-range grows with the square of its size.)
constexpr int kRunPer = 4;
constexpr int kRunTile = kRunPer * kSortThreads;
constexpr int kRunBins = 2048;
constexpr int kRowPer = 4;
constexpr int kRowChunk = kRowPer * kGtThreads;  // row entries per workgroup of the row kernels
constexpr int kJoinPer = 8;        // part entries per thread in flight in k_gt_join

typedef u32 v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32 gt_bin(u32 bits) { return key_of_bits(bits) >> 20; }

// Multiplicative (Fibonacci) hashing of an index: the top logNP bits pick
// the part, the next kLogSlots bits the first place of the probe sequence
// inside the part's table (which wraps around).
struct HashPart {
  u32 part, slot;
};
__device__ __forceinline__ HashPart gt_hash(int32_t idx, u32 logNP) {
  const u32 h = (u32)idx * 0x9E3779B1u;
  return HashPart{logNP ? h >> (32u - logNP) : 0u, (h >> (32u - logNP - kLogSlots)) & (kSlots - 1u)};
}

// Where one part of a set lies (entries [start, start + count) of the set's
// region) and how many entries it has.
struct PartDir {
  u32 start, count;
};

// An LDS table of one part: key[h] = index + 1 (0: empty), val[h] = the
// entry's value bits.
// Inserts (idx, bits); false if idx is there already or the table is full.
__device__ bool lds_insert(u32* key, u32* val, u32 h, int32_t idx, u32 bits) {
  const u32 want = (u32)idx + 1u;
  u32 old = 0u, probe = 0u;
  do {  // one exit: an empty place taken, the index found, or every place tried
    old = atomicCAS(&key[h], 0u, want);
    if (old != 0u && old != want) h = (h + 1u) & (kSlots - 1u);
  } while (old != 0u && old != want && ++probe < kSlots);
  if (old != 0u) return false;
  if (val) val[h] = bits;
  return true;
}
// The place of idx, or -1.
__device__ int lds_find(const u32* key, u32 h, int32_t idx) {
  const u32 want = (u32)idx + 1u;
  u32 kk = 0u, probe = 0u;
  do {
    kk = key[h];
    if (kk != 0u && kk != want) h = (h + 1u) & (kSlots - 1u);
  } while (kk != 0u && kk != want && ++probe < kSlots);
  return kk == want ? (int)h : -1;
}

// Adds the workgroup's LDS histogram to a merge's histogram in memory.
__device__ __forceinline__ void flush_hist(const u32* s_h, u32* H) {
  for (int i = threadIdx.x; i < kGtBins; i += blockDim.x)
    if (s_h[i]) (void)add_agent_relaxed(&H[i], s_h[i]);
}

// Appends cnt entries of each thread at places a counter in memory hands out
// (one device add per workgroup): returns the place of this thread's first.
// s_scan holds kGtWaves + 1 words.  Every thread calls it.
__device__ int64_t wg_append_n(u32 cnt, u32* counter, u32* s_scan, u32* s_base) {
  u32 tot;
  const u32 before = block_exclusive_sum<kGtThreads>(cnt, s_scan, tot);
  if (threadIdx.x == 0) *s_base = tot ? add_agent_relaxed(counter, tot) : 0u;
  __syncthreads();
  const int64_t pos = (int64_t)*s_base + before;
  __syncthreads();
  return pos;
}

// The wave's lanes with `keep` set take the next places of an LDS counter (one
// LDS add per wave): returns this lane's place (meaningless without keep).
// Every lane of the wave calls it.
__device__ __forceinline__ u32 wave_take(bool keep, u32* s_n) {
  const u64 bal = ballot(keep);
  u32 base = 0;
  if (bal) {
    if (lane_id() == 0) base = atomicAdd(s_n, (u32)__popcll(bal));
    base = __builtin_amdgcn_readfirstlane(base);
  }
  return base + lanes_below(bal);
}

// ---------------------------------------------------------- the rows ----
struct RowArgs {
  const int32_t* idx;  // the rows [P][k]
  const float* val;
  int64_t k, cpr;      // chunks of kRowChunk per row
  u32 logNP;
  u32* rcnt;           // [P][cpr][NP] entries per (row, chunk, part)
  PartDir* rdir;       // [P][NP] each row's parts in its grouped copy
  Pair* prow;          // [P][k] the rows grouped by part
  u32* ppos;           // [P][k] each grouped entry's place in its row
  v4u* clear;          // zero-filled by k_gt_rcount: the call's counters
  int64_t nclear;      // (16-byte words)
};

// Workgroup (p, c) counts chunk c of row p per part; the grid also
// zero-fills the histograms and counters of the rounds.
__global__ __launch_bounds__(kGtThreads) void k_gt_rcount(RowArgs a) {
  __shared__ u32 s_c[kMaxParts];
  const int tid = threadIdx.x;
  for (int64_t i = (int64_t)blockIdx.x * kGtThreads + tid; i < a.nclear; i += (int64_t)gridDim.x * kGtThreads)
    a.clear[i] = v4u{0u, 0u, 0u, 0u};
  const u32 NP = 1u << a.logNP;
  const int64_t p = blockIdx.x / a.cpr, c = blockIdx.x % a.cpr;
  const int32_t* row = a.idx + p * a.k;
  int32_t ix[kRowPer];
#pragma unroll
  for (int u = 0; u < kRowPer; ++u) {
    const int64_t j = c * kRowChunk + u * kGtThreads + tid;
    ix[u] = j < a.k ? row[j] : 0;
  }
  for (u32 i = tid; i < NP; i += kGtThreads) s_c[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kRowPer; ++u) {
    const int64_t j = c * kRowChunk + u * kGtThreads + tid;
    if (j < a.k) atomicAdd(&s_c[gt_hash(ix[u], a.logNP).part], 1u);
  }
  __syncthreads();
  for (u32 i = tid; i < NP; i += kGtThreads) a.rcnt[(p * a.cpr + c) * NP + i] = s_c[i];
}

// Workgroup (p, c) places chunk c of row p: part g of the row starts after
// the row's entries of parts below g, and the chunk's entries of part g after
// those of the chunks before it.  Inside a chunk's share of a part the order
// is whatever the LDS adds give (no result depends on it).
__global__ __launch_bounds__(kGtThreads) void k_gt_rscatter(RowArgs a) {
  __shared__ u32 s_c[kMaxParts], s_off[kMaxParts];
  __shared__ u32 s_scan[kGtWaves + 1];
  const int tid = threadIdx.x;
  const u32 NP = 1u << a.logNP;
  const int64_t p = blockIdx.x / a.cpr, c = blockIdx.x % a.cpr;
  const int32_t* row = a.idx + p * a.k;
  const float* vrow = a.val + p * a.k;
  int32_t ix[kRowPer];
  u32 vb[kRowPer];
#pragma unroll
  for (int u = 0; u < kRowPer; ++u) {
    const int64_t j = c * kRowChunk + u * kGtThreads + tid;
    ix[u] = j < a.k ? row[j] : 0;
    vb[u] = j < a.k ? __float_as_uint(vrow[j]) : 0u;
  }
  // the row's counts, every (chunk, part) word loaded by its own thread:
  // per part the row's total and the earlier chunks' sum
  for (u32 g = tid; g < NP; g += kGtThreads) {
    s_c[g] = 0u;
    s_off[g] = 0u;
  }
  __syncthreads();
  {
    const u32* rc = a.rcnt + p * a.cpr * NP;
    const int64_t nw = a.cpr * NP;
    for (int64_t i0 = 0; i0 < nw; i0 += (int64_t)kGtBatch * kGtThreads) {
      u32 v[kGtBatch];
#pragma unroll
      for (int u = 0; u < kGtBatch; ++u) {
        const int64_t i = i0 + (int64_t)u * kGtThreads + tid;
        v[u] = i < nw ? rc[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kGtBatch; ++u) {
        const int64_t i = i0 + (int64_t)u * kGtThreads + tid;
        if (v[u]) {
          atomicAdd(&s_c[i % NP], v[u]);
          if (i / NP < c) atomicAdd(&s_off[i % NP], v[u]);
        }
      }
    }
  }
  __syncthreads();
  const u32 tot = (u32)tid < NP ? s_c[tid] : 0u, below = (u32)tid < NP ? s_off[tid] : 0u;
  u32 all;
  const u32 start = block_exclusive_sum<kGtThreads>(tot, s_scan, all);
  if ((u32)tid < NP) {
    s_off[tid] = start + below;
    s_c[tid] = 0u;
    if (c == 0) a.rdir[p * NP + tid] = PartDir{start, tot};
  }
  __syncthreads();
  Pair* prow = a.prow + p * a.k;
  u32* ppos = a.ppos + p * a.k;
#pragma unroll
  for (int u = 0; u < kRowPer; ++u) {
    const int64_t j = c * kRowChunk + u * kGtThreads + tid;
    if (j < a.k) {
      const u32 g = gt_hash(ix[u], a.logNP).part;
      const u32 pos = s_off[g] + atomicAdd(&s_c[g], 1u);
      prow[pos] = Pair{ix[u], vb[u]};
      ppos[pos] = (u32)j;
    }
  }
}

// Merges of round r: slot s = m 2^(r+1) absorbs s + 2^r while that slot exists.
__host__ __device__ inline int64_t gt_merges(int64_t P, int r) {
  const int64_t half = (int64_t)1 << r;
  return P > half ? (P - half + 2 * half - 1) / (2 * half) : 0;
}

// Where slot s's data is before round r: its output region if it was a
// merge's destination in a round before r, else its grouped row.
struct SlotData {
  const Pair* pairs;
  const PartDir* dir;
};
__device__ SlotData slot_data(int64_t P, int64_t k, u32 NP, int r, int64_t s, const Pair* out, const PartDir* odir,
                              const Pair* prow, const PartDir* rdir) {
  for (int q = r - 1; q >= 0; --q)
    if (s % ((int64_t)2 << q) == 0 && s + ((int64_t)1 << q) < P)
      return SlotData{out + (s >> 1) * 2 * k, odir + (s >> 1) * NP};
  return SlotData{prow + s * k, rdir + s * NP};
}

// --------------------------------------------------------------- selection ----
// The k-th best live entry of a merge by (key desc, index asc) is found in
// two steps.  From the merge's histogram of key >> 20 (complete once every
// probing workgroup has added to it), the bin b1 that holds it and `need`,
// its rank inside the bin.  Then, among the bin's entries (the candidates,
// which k_gt_keep lists), radix levels over the rest of the key and, among
// the entries whose key is T, the k-th key, over the index: T and I, the
// largest index kept at T (ties keep the lowest indices).
struct BinShared {  // the histogram levels
  u32 h[kGtBins];
  u32 scan[kGtWaves + 1];
  u32 pick, before, count;
};
struct SelShared : BinShared {  // and the candidates
  Pair list[kSelList];
};

// Bins 0..nb-1 (nb = 1024 or 2048) in s.h; the bin where the count from the
// top (desc) or the bottom (asc) reaches `need`, the count before it and the
// bin's own count land in s.pick, s.before, s.count.  Every thread calls it.
__device__ void pick_level(BinShared& s, int nb, u32 need, bool desc) {
  const int tid = threadIdx.x;
  const int per = nb / kGtThreads;  // 1 or 2
  u32 c[2] = {0u, 0u};
  int bin[2] = {0, 0};
  u32 own = 0;
  for (int u = 0; u < per; ++u) {
    const int o = tid * per + u;  // order position
    bin[u] = desc ? nb - 1 - o : o;
    c[u] = s.h[bin[u]];
    own += c[u];
  }
  u32 tot;
  const u32 before = block_exclusive_sum<kGtThreads>(own, s.scan, tot);
  if (tid == 0) {
    s.pick = 0xFFFFFFFFu;
    s.before = 0;
    s.count = 0;
  }
  __syncthreads();
  if (before < need && before + own >= need) {
    u32 run = before;
    for (int u = 0; u < per; ++u) {
      if (run + c[u] >= need) {
        s.pick = (u32)bin[u];
        s.before = run;
        s.count = c[u];
        break;
      }
      run += c[u];
    }
  }
  __syncthreads();
}

// First step, one workgroup: b1 and need into sel[0], sel[1] (b1 = 2^32 - 1
// when the merge has fewer than k live entries, which only rows that break
// the preconditions can cause).  Leaves H zero.
__device__ void select_bin(BinShared& s, int64_t k, u32* H, u32* sel, u32* err) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kGtBins; i += kGtThreads) {
    s.h[i] = ld_agent(&H[i]);
    st_agent(&H[i], 0u);
  }
  __syncthreads();
  pick_level(s, kGtBins, (u32)k, true);
  if (tid == 0) {
    if (s.pick == 0xFFFFFFFFu) atomicOr(err, kErrBadInput);
    st_agent(&sel[0], s.pick);
    st_agent(&sel[1], (u32)k - s.before);
  }
}

// Second step, one workgroup, over the nc candidates of clist (read with
// device-scope loads): T and I with the rank `need` inside bin b1.
__device__ void select_in_bin(SelShared& s, const Pair* clist, u32 nc, u32 b1, u32 need, u32& T, u32& I) {
  const int tid = threadIdx.x;
  const bool in_lds = nc <= (u32)kSelList;
  if (in_lds) {
    for (u32 i0 = tid; i0 < nc; i0 += (u32)kGtBatch * kGtThreads) {
      Pair e[kGtBatch];
#pragma unroll
      for (int u = 0; u < kGtBatch; ++u) {
        const u32 i = i0 + (u32)u * kGtThreads;
        if (i < nc) e[u] = unpack_pair(ld_agent64((const u64*)(clist + i)));
      }
#pragma unroll
      for (int u = 0; u < kGtBatch; ++u) {
        const u32 i = i0 + (u32)u * kGtThreads;
        if (i < nc) s.list[i] = e[u];
      }
    }
    __syncthreads();
  }
  // calls f(e) for every candidate that passes pred(e); every thread calls it
  auto for_cands = [&](auto pred, auto f) {
    if (in_lds) {
      for (u32 i = tid; i < nc; i += kGtThreads) {
        const Pair e = s.list[i];
        if (pred(e)) f(e);
      }
    } else {
      for (u32 i = tid; i < nc; i += kGtThreads) {
        const Pair e = unpack_pair(ld_agent64((const u64*)(clist + i)));
        if (pred(e)) f(e);
      }
    }
  };
  auto level = [&](int nb, u32 nd, bool desc, auto pred, auto digit) {
    for (int i = tid; i < nb; i += kGtThreads) s.h[i] = 0;
    __syncthreads();
    for_cands(pred, [&](const Pair& e) { atomicAdd(&s.h[digit(e)], 1u); });
    __syncthreads();
    pick_level(s, nb, nd, desc);
  };
  // key bits 19..10, then 9..0 (from the top)
  level(1024, need, true, [](const Pair&) { return true; },
        [](const Pair& e) { return (key_of_bits(e.bits) >> 10) & 1023u; });
  const u32 d1 = s.pick;
  need -= s.before;
  const u32 p2 = (b1 << 10) | (d1 & 1023u);
  level(1024, need, true, [p2](const Pair& e) { return (key_of_bits(e.bits) >> 10) == p2; },
        [](const Pair& e) { return key_of_bits(e.bits) & 1023u; });
  T = (p2 << 10) | (s.pick & 1023u);
  need -= s.before;
  I = 0x7FFFFFFFu;
  if (need < s.count) {
    // ties at T: the need lowest indices, over index bits 30..20, 19..10, 9..0
    const u32 t = T;
    level(2048, need, false, [t](const Pair& e) { return key_of_bits(e.bits) == t; },
          [](const Pair& e) { return ((u32)e.idx >> 20) & 2047u; });
    const u32 i1 = s.pick & 2047u;
    need -= s.before;
    level(1024, need, false, [t, i1](const Pair& e) { return key_of_bits(e.bits) == t && ((u32)e.idx >> 20) == i1; },
          [](const Pair& e) { return ((u32)e.idx >> 10) & 1023u; });
    const u32 i2 = (i1 << 10) | (s.pick & 1023u);
    need -= s.before;
    level(1024, need, false, [t, i2](const Pair& e) { return key_of_bits(e.bits) == t && ((u32)e.idx >> 10) == i2; },
          [](const Pair& e) { return (u32)e.idx & 1023u; });
    I = (i2 << 10) | (s.pick & 1023u);
  }
}

// --------------------------------------------------------------- k_gt_join ----
struct JoinArgs {
  int32_t P;
  int r;
  int64_t k;
  u32 logNP;
  const Pair* prow;    // the grouped rows and their directories
  const PartDir* rdir;
  const Pair* out;     // the slots' output regions (2k places each) and directories
  const PartDir* odir;
  Pair* W;             // the round's unions, 2k places per merge
  PartDir* wdir;       // [merge][NP] each part's place and length in W
  u32* hist;           // histograms, kGtBins per merge
  u32* arrive;         // arrival counters (32 words apart)
  u32* sel;            // [2] per merge: b1, need
  u32* err;
};

__global__ __launch_bounds__(kGtThreads) void k_gt_join(JoinArgs a) {
  __shared__ u32 s_key[kSlots];
  __shared__ u32 s_val[kSlots];
  __shared__ BinShared s;
  __shared__ PartDir s_da, s_db;
  __shared__ u32 s_ws, s_n, s_last;
  const int tid = threadIdx.x;
  const u32 NP = 1u << a.logNP;
  const int64_t m = blockIdx.x / NP;
  const u32 g = blockIdx.x % NP;
  const int64_t half = (int64_t)1 << a.r;
  const int64_t sa = m * 2 * half;  // A slot; B is sa + half
  const SlotData A = slot_data(a.P, a.k, NP, a.r, sa, a.out, a.odir, a.prow, a.rdir);
  const SlotData B = slot_data(a.P, a.k, NP, a.r, sa + half, a.out, a.odir, a.prow, a.rdir);
  // this part's region of W: after those of the parts below it, each as
  // large as the two sides' entries of its part
  {
    u32 cap = 0;
    PartDir da{0u, 0u}, db{0u, 0u};
    if ((u32)tid < NP) {
      da = A.dir[tid];
      db = B.dir[tid];
      cap = da.count + db.count;
    }
    u32 all;
    const u32 ws = block_exclusive_sum<kGtThreads>(cap, s.scan, all);
    if ((u32)tid == g) {
      s_da = da;
      s_db = db;
      s_ws = ws;
      s_n = 0u;
    }
  }
  for (u32 i = tid; i < kSlots; i += kGtThreads) s_key[i] = 0u;
  for (int i = tid; i < kGtBins; i += kGtThreads) s.h[i] = 0u;
  __syncthreads();
  const PartDir da = s_da, db = s_db;
  // the first batch of B entries is loaded with the A entries, so that its
  // loads are in flight while the table is built
  Pair eb[kJoinPer];
#pragma unroll
  for (int u = 0; u < kJoinPer; ++u) {
    const u32 i = (u32)u * kGtThreads + tid;
    eb[u] = i < db.count ? B.pairs[db.start + i] : pair_sentinel();
  }
  // the A entries of this part into the table (a repeated index is the
  // rows' fault, a full table a part far above its expected load: both are
  // reported as bad input)
  for (u32 i0 = 0; i0 < da.count; i0 += (u32)kJoinPer * kGtThreads) {
    Pair e[kJoinPer];
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      e[u] = i < da.count ? A.pairs[da.start + i] : pair_sentinel();
    }
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      if (i < da.count && !lds_insert(s_key, s_val, gt_hash(e[u].idx, a.logNP).slot, e[u].idx, e[u].bits))
        atomicOr(a.err, kErrBadInput);
    }
  }
  __syncthreads();
  Pair* W = a.W + m * 2 * a.k + s_ws;
  // the B entries of this part: found, added to the A entry; else to W
  for (u32 i0 = 0; i0 < db.count; i0 += (u32)kJoinPer * kGtThreads) {
    Pair e[kJoinPer];
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      e[u] = i0 == 0 ? eb[u] : i < db.count ? B.pairs[db.start + i] : pair_sentinel();
    }
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      bool app = false;
      if (i < db.count) {
        const int h = lds_find(s_key, gt_hash(e[u].idx, a.logNP).slot, e[u].idx);
        if (h >= 0) {
          s_val[h] = __float_as_uint(__uint_as_float(s_val[h]) + __uint_as_float(e[u].bits));
        } else {
          app = true;
          atomicAdd(&s.h[gt_bin(e[u].bits)], 1u);
        }
      }
      const u32 pos = wave_take(app, &s_n);
      if (app) W[pos] = e[u];
    }
  }
  __syncthreads();
  // the A entries of this part (every B entry has been looked up): slots
  // tid + i 1024
  {
    constexpr int kPer = kSlots / kGtThreads;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const u32 h = i * kGtThreads + tid;
      const u32 kk = s_key[h];
      const Pair e{(int32_t)(kk - 1u), s_val[h]};
      if (kk) atomicAdd(&s.h[gt_bin(e.bits)], 1u);
      const u32 pos = wave_take(kk != 0u, &s_n);
      if (kk) W[pos] = e;
    }
  }
  __syncthreads();
  if (tid == 0) a.wdir[m * NP + g] = PartDir{s_ws, s_n};
  flush_hist(s.h, a.hist + m * kGtBins);
  // the last workgroup of the merge to arrive picks the first-level bin: it
  // needs only the histogram, whose adds are complete before each workgroup
  // arrives
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_relaxed(&a.arrive[m * 32], 1u) == NP - 1u ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  select_bin(s, a.k, a.hist + m * kGtBins, a.sel + 2 * m, a.err);
  if (tid == 0) st_agent(&a.arrive[m * 32], 0u);
}

// --------------------------------------------------------------- k_gt_keep ----
struct KeepArgs {
  int r;
  int64_t k;
  u32 logNP;
  const Pair* W;       // the round's unions
  const PartDir* wdir;
  const u32* sel;      // b1, need
  u32* ccnt;           // candidate counters (32 words apart)
  u32* karrive;        // arrival counters (32 words apart)
  u32* kabove;         // [merge][NP] entries above b1 each part keeps
  Pair* cand;          // candidate lists, 2k per merge
  Pair* out;           // the slots' output regions, 2k places each
  PartDir* odir;       // and their directories
  u32* err;
};

constexpr int kKeepPer = 2;  // union places per thread and pass of k_gt_keep
constexpr int kKeepSpan = kKeepPer * kGtThreads;

__global__ __launch_bounds__(kGtThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_gt_keep(KeepArgs a) {
  __shared__ SelShared s;
  __shared__ u32 s_at[kMaxParts], s_kc[kMaxParts], s_ab[kMaxParts];
  __shared__ u32 s_base, s_last, s_n, s_placed, s_above;
  const int tid = threadIdx.x;
  const u32 NP = 1u << a.logNP;
  const int64_t m = blockIdx.x / NP;
  const u32 g = blockIdx.x % NP;
  const int64_t len = 2 * a.k;
  const int64_t slot = m << (a.r + 1);
  Pair* O = a.out + (slot >> 1) * len;
  const PartDir wd = a.wdir[m * NP + g];
  const u32 b1 = a.sel[2 * m];
  const bool b1ok = b1 != 0xFFFFFFFFu;
  Pair* clist = a.cand + m * len;
  const Pair* W = a.W + m * len + wd.start;
  if (tid == 0) s_n = 0u;
  __syncthreads();
  for (u32 i0 = 0; i0 < wd.count; i0 += (u32)kKeepSpan) {
    Pair e[kKeepPer];
#pragma unroll
    for (int u = 0; u < kKeepPer; ++u) {
      const u32 q = i0 + (u32)u * kGtThreads + tid;
      e[u] = q < wd.count ? W[q] : pair_sentinel();
    }
    u32 cd = 0, nc0 = 0;  // bit u: e[u] is a candidate
#pragma unroll
    for (int u = 0; u < kKeepPer; ++u) {
      const bool live = i0 + (u32)u * kGtThreads + tid < wd.count;
      const u32 bin = gt_bin(e[u].bits);
      const bool keep = live && b1ok && bin > b1;
      if (live && !keep && (bin == b1 || !b1ok)) {
        cd |= 1u << u;
        ++nc0;
      }
      const u32 pos = wave_take(keep, &s_n);
      if (keep) O[wd.start + pos] = e[u];
    }
    // candidates: stored at device scope for the selecting workgroup
    int64_t cp = wg_append_n(nc0, a.ccnt + m * 32, s.scan, &s_base);
#pragma unroll
    for (int u = 0; u < kKeepPer; ++u)
      if ((cd >> u) & 1u) st_agent64((u64*)(clist + cp++), pack_pair(e[u]));
  }
  __syncthreads();
  if (tid == 0) st_agent(&a.kabove[m * NP + g], s_n);
  // the last workgroup of the merge to arrive resolves the candidates
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_relaxed(&a.karrive[m * 32], 1u) == NP - 1u ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  const u32 nc = ld_agent(&a.ccnt[m * 32]);
  u32 T = 0u, I = 0x7FFFFFFFu;  // (no b1: every candidate is kept as far as room allows)
  if (b1ok) select_in_bin(s, clist, nc, b1, a.sel[2 * m + 1], T, I);
  // each part's candidates go after its entries above b1
  u32 ab = 0;
  if ((u32)tid < NP) {
    ab = ld_agent(&a.kabove[m * NP + tid]);
    s_ab[tid] = ab;
    s_at[tid] = a.wdir[m * NP + tid].start + ab;
    s_kc[tid] = 0u;
  }
  {
    u32 all;
    (void)block_exclusive_sum<kGtThreads>(ab, s.scan, all);
    if (tid == 0) {
      s_above = all;
      s_placed = 0u;
    }
  }
  __syncthreads();
  const bool lds = b1ok && nc <= (u32)kSelList;
  const int64_t room = a.k - (int64_t)s_above;  // (k entries at most, whatever the input)
  for (u32 i0 = 0; i0 < nc; i0 += kGtThreads) {
    const u32 i = i0 + tid;
    Pair ce = pair_sentinel();
    if (i < nc) ce = lds ? s.list[i] : unpack_pair(ld_agent64((const u64*)(clist + i)));
    const u32 key = key_of_bits(ce.bits);
    const bool pass = i < nc && (key > T || (key == T && (u32)ce.idx <= I));
    const u32 q = wave_take(pass, &s_placed);
    if (pass && (int64_t)q < room) {
      const u32 gp = gt_hash(ce.idx, a.logNP).part;
      O[s_at[gp] + atomicAdd(&s_kc[gp], 1u)] = ce;
    }
  }
  __syncthreads();
  if ((u32)tid < NP)
    a.odir[(slot >> 1) * NP + tid] = PartDir{s_at[tid] - s_ab[tid], s_ab[tid] + s_kc[tid]};
  if (tid == 0) {
    st_agent(&a.karrive[m * 32], 0u);
    st_agent(&a.ccnt[m * 32], 0u);
  }
}


// -------------------------------------------------------------- final ----
struct FinalArgs {
  int32_t P;
  int64_t k, n;
  u32 logNP;
  uint8_t* mask;
  const Pair* F;       // the final set, grouped by part
  const PartDir* fdir;
  const Pair* prow;    // the grouped rows, their places in the rows and directories
  const u32* ppos;
  const PartDir* rdir;
  int64_t nruns;       // workgroups that sort runs; the others make the mask
  u64* runs;           // sorted runs (more than one run)
  int32_t* out_idx;    // (one run)
  float* out_val;
  u32* err;
};

// Workgroups 0 .. nruns-1 sort runs of the final set; workgroup (p, part)
// after them joins row p's entries of its part against the final set's (the
// mask) and checks them: in [0, n), and no index twice in the row.
__global__ __launch_bounds__(kGtThreads) void k_gt_final(FinalArgs a) {
  constexpr int kLds = block_sort_lds(kRunPer, kRunBins);
  static_assert(kLds <= (int)kSlots, "the sort fits in the two tables' LDS");
  __shared__ u64 s_lds[kSlots];  // the two tables, or the sort's LDS
  __shared__ u32 s_pre[kMaxParts], s_fst[kMaxParts];
  __shared__ u32 s_scan[kGtWaves + 1];
  u32* s_key = (u32*)s_lds;      // the final set's part
  u32* s_row = s_key + kSlots;   // the row's part (the repeat check)
  u64* s = s_lds;
  const int tid = threadIdx.x;
  const u32 NP = 1u << a.logNP;
  if ((int64_t)blockIdx.x < a.nruns) {
    // entry i of the final set, counted part after part
    u32 cnt = 0;
    if ((u32)tid < NP) {
      const PartDir d = a.fdir[tid];
      cnt = d.count;
      s_fst[tid] = d.start;
    }
    u32 total;
    const u32 pre = block_exclusive_sum<kGtThreads>(cnt, s_scan, total);
    if ((u32)tid < NP) s_pre[tid] = pre;
    __syncthreads();
    const int64_t have = std::min<int64_t>(a.k, total);  // (k, unless the rows broke the preconditions)
    const int64_t base = (int64_t)blockIdx.x * kRunTile;
    u64 x[kRunPer];
#pragma unroll
    for (int c = 0; c < kRunPer; ++c) {
      const int64_t i = base + kRunPer * tid + c;
      x[c] = ~0ull;
      if (i < have) {
        u32 lo = 0, hi = NP;  // the last part whose first entry is at or below i
        while (hi - lo > 1) {
          const u32 mid = (lo + hi) >> 1;
          if ((int64_t)s_pre[mid] <= i) lo = mid;
          else hi = mid;
        }
        x[c] = rank64(a.F[s_fst[lo] + (u32)(i - s_pre[lo])]);
      }
    }
    block_sort<kRunPer, kRunBins>(x, s);
    const bool one = a.k <= kRunTile;
#pragma unroll
    for (int c = 0; c < kRunPer; ++c) {
      const int64_t i = base + kRunPer * tid + c;
      if (i >= a.k) continue;
      if (one) {
        const Pair e = unrank64(x[c]);
        a.out_idx[i] = e.idx;
        a.out_val[i] = __uint_as_float(e.bits);
      } else {
        a.runs[i] = x[c];
      }
    }
    return;
  }
  const int64_t b = (int64_t)blockIdx.x - a.nruns;
  const int64_t p = b / NP;
  const u32 g = (u32)(b % NP);
  const PartDir fd = a.fdir[g];
  const PartDir rd = a.rdir[p * NP + g];
  for (u32 i = tid; i < kSlots; i += kGtThreads) {
    s_key[i] = 0u;
    s_row[i] = 0u;
  }
  __syncthreads();
  // the final set's indices of this part (a table that cannot hold them all:
  // a part far above its expected load, reported as bad input)
  for (u32 i0 = 0; i0 < fd.count; i0 += (u32)kJoinPer * kGtThreads) {
    int32_t x[kJoinPer];
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      x[u] = i < fd.count ? a.F[fd.start + i].idx : 0;
    }
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      if (i < fd.count && !lds_insert(s_key, nullptr, gt_hash(x[u], a.logNP).slot, x[u], 0u) &&
          lds_find(s_key, gt_hash(x[u], a.logNP).slot, x[u]) < 0)
        atomicOr(a.err, kErrBadInput);
    }
  }
  __syncthreads();
  // row p's entries of this part, with their places in the row
  const Pair* prow = a.prow + p * a.k + rd.start;
  const u32* ppos = a.ppos + p * a.k + rd.start;
  uint8_t* mrow = a.mask + p * a.k;
  for (u32 i0 = 0; i0 < rd.count; i0 += (u32)kJoinPer * kGtThreads) {
    int32_t x[kJoinPer];
    u32 j[kJoinPer];
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      x[u] = i < rd.count ? prow[i].idx : 0;
      j[u] = i < rd.count ? ppos[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kJoinPer; ++u) {
      const u32 i = i0 + (u32)u * kGtThreads + tid;
      if (i >= rd.count) continue;
      const u32 h = gt_hash(x[u], a.logNP).slot;
      const bool bad = x[u] < 0 || (int64_t)x[u] >= a.n || !lds_insert(s_row, nullptr, h, x[u], 0u);
      if (bad) atomicOr(a.err, kErrBadInput);
      mrow[j[u]] = (x[u] >= 0 && lds_find(s_key, h, x[u]) >= 0) ? 1 : 0;
    }
  }
}

// Number of A entries among the first o outputs of the merge of sorted
// A[0, la) and B[0, lb) (A first on equal keys); one wave, every lane.
__device__ int64_t wave_merge_split(const u64* A, int64_t la, const u64* B, int64_t lb, int64_t o) {
  const int lane = lane_id();
  int64_t lo = std::max<int64_t>(0, o - lb), hi = std::min<int64_t>(o, la);
  // the answer is lo + #{i in [lo, hi) : A[i] <= B[o - i - 1]} (true for a prefix)
  while (hi > lo) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int64_t i = lo + step * lane;
    const bool t = i < hi && A[i] <= B[o - i - 1];
    const u32 cnt = (u32)__popcll(ballot(t));
    if (step == 1) return lo + cnt;
    if (cnt == 0) return lo;
    const int64_t nlo = lo + step * (cnt - 1) + 1;
    hi = std::min<int64_t>(hi, lo + step * cnt);
    lo = nlo;
  }
  return lo;
}

struct MergeArgs {
  const u64* src;
  u64* dst;            // (not the last pass)
  int64_t k, L;        // runs of L become runs of 2L
  bool last;           // write the outputs
  int32_t* out_idx;
  float* out_val;
};

__global__ __launch_bounds__(kGtThreads) void k_gt_merge(MergeArgs a) {
  __shared__ u64 s[kSortTile];
  __shared__ int64_t s_cut[2];
  const int tid = threadIdx.x, w = tid / kWave;
  const int64_t t0 = (int64_t)blockIdx.x * kSortTile;  // first output
  const int64_t pb = (t0 / (2 * a.L)) * (2 * a.L);     // the pair of runs
  const int64_t la = std::min<int64_t>(a.L, a.k - pb);
  const int64_t lb = std::max<int64_t>(0, std::min<int64_t>(a.L, a.k - pb - a.L));
  const u64* A = a.src + pb;
  const u64* B = A + la;
  const int64_t o0 = t0 - pb, o1 = std::min<int64_t>(o0 + kSortTile, la + lb);
  if (w < 2) {
    const int64_t cut = wave_merge_split(A, la, B, lb, w == 0 ? o0 : o1);
    if (lane_id() == 0) s_cut[w] = cut;
  }
  __syncthreads();
  const int64_t i0 = s_cut[0], i1 = s_cut[1];
  const int64_t j0 = o0 - i0, j1 = o1 - i1;
  const int na = (int)(i1 - i0), nb = (int)(j1 - j0);
  for (int i = tid; i < na; i += kGtThreads) s[i] = A[i0 + i];
  for (int i = tid; i < nb; i += kGtThreads) s[na + i] = B[j0 + i];
  __syncthreads();
  const u64* sA = s;
  const u64* sB = s + na;
  const int d = kSortPer * tid;
  const int nout = na + nb;
  if (d >= nout) return;
  int lo = std::max(0, d - nb), hi = std::min(d, na);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sA[mid] <= sB[d - mid - 1]) lo = mid + 1;
    else hi = mid;
  }
  int i = lo, j = d - lo;
  for (int u = 0; u < kSortPer && d + u < nout; ++u) {
    const bool takeA = j >= nb || (i < na && sA[i] <= sB[j]);
    const u64 v = takeA ? sA[i++] : sB[j++];
    const int64_t o = pb + o0 + d + u;
    if (a.last) {
      const Pair e = unrank64(v);
      a.out_idx[o] = e.idx;
      a.out_val[o] = __uint_as_float(e.bits);
    } else {
      a.dst[o] = v;
    }
  }
}

// ------------------------------------------------------------------ layout ----
static int gt_rounds(int64_t P) {
  int R = 0;
  while (((int64_t)1 << R) < P) ++R;
  return R;
}

struct GtLayout {
  int R;
  int64_t nmax;  // merges of round 0 (the most of any round; also the output regions), at least 1
  u32 logNP;     // hash parts: 2^logNP
  int64_t cpr;   // row chunks of the row kernels
  size_t hist, arrive, ccnt, karrive, clear_end;  // zero-filled at the start of a call
  size_t sel, rcnt, rdir, prow, ppos, wdir, kabove, odir, W, cand, out, runs[2], total;
};

static GtLayout gt_layout(int64_t P, int64_t k) {
  GtLayout L{};
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t kk = std::max<int64_t>(k, 1);
  L.R = gt_rounds(P);
  L.nmax = std::max<int64_t>(1, gt_merges(P, 0));
  u32 lp = 0;
  while (((int64_t)kPartLoad << lp) < kk) ++lp;
  L.logNP = lp;
  const size_t NP = (size_t)1 << lp;
  L.cpr = (kk + kRowChunk - 1) / kRowChunk;
  size_t o = kWorkspaceHeader;  // after the header whose first word is the error word
  L.hist = o;
  o += al(4 * (size_t)kGtBins * (size_t)L.nmax);
  for (size_t* f : {&L.arrive, &L.ccnt, &L.karrive}) {
    *f = o;
    o += al(128 * (size_t)L.nmax);
  }
  L.clear_end = o;
  auto take = [&](size_t& f, size_t bytes) {
    f = o;
    o += al(bytes);
  };
  take(L.sel, 8 * (size_t)L.nmax);
  take(L.rcnt, 4 * (size_t)P * (size_t)L.cpr * NP);
  take(L.rdir, sizeof(PartDir) * (size_t)P * NP);
  take(L.prow, sizeof(Pair) * (size_t)P * (size_t)kk);
  take(L.ppos, 4 * (size_t)P * (size_t)kk);
  take(L.wdir, sizeof(PartDir) * (size_t)L.nmax * NP);
  take(L.kabove, 4 * (size_t)L.nmax * NP);
  take(L.odir, sizeof(PartDir) * (size_t)L.nmax * NP);
  take(L.W, sizeof(Pair) * 2 * (size_t)kk * (size_t)L.nmax);
  take(L.cand, sizeof(Pair) * 2 * (size_t)kk * (size_t)L.nmax);
  take(L.out, sizeof(Pair) * 2 * (size_t)kk * (size_t)L.nmax);
  take(L.runs[0], 8 * (size_t)kk);
  take(L.runs[1], 8 * (size_t)kk);
  L.total = o;
  return L;
}

}  // namespace tgs

using namespace tgs;

extern "C" size_t tgs_gtopk_workspace_bytes(int32_t P, int64_t k, int64_t n) {
  if (P < 1 || k < 0 || n < 0 || n > INT32_MAX || k > n || k > kGtMaxK || (int64_t)P * k > INT32_MAX) return 0;
  return gt_layout(P, k).total;
}

extern "C" tgs_status tgs_gtopk_merge(const int32_t* idx, const float* val, int32_t P, int64_t k, int64_t n,
                                      int32_t* out_idx, float* out_val, uint8_t* out_mask, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (P < 1) return fail(TGS_EINVAL, "gtopk_merge: P=%d < 1", (int)P);
  if (n < 0 || n > INT32_MAX) return fail(TGS_EINVAL, "gtopk_merge: n=%lld outside [0, 2^31-1]", (long long)n);
  if (k < 0 || k > n) return fail(TGS_EINVAL, "gtopk_merge: k=%lld outside [0, n]", (long long)k);
  if (k > kGtMaxK) return fail(TGS_EINVAL, "gtopk_merge: k=%lld above 2^20", (long long)k);
  if ((int64_t)P * k > INT32_MAX) return fail(TGS_EINVAL, "gtopk_merge: P*k too large");
  if (!workspace) return fail(TGS_EINVAL, "gtopk_merge: null workspace");
  if (k > 0 && (!idx || !val || !out_idx || !out_val || !out_mask))
    return fail(TGS_EINVAL, "gtopk_merge: null array pointer");
  for (const void* p : {(const void*)idx, (const void*)val, (const void*)out_idx, (const void*)out_val})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "gtopk_merge: pointer not 4-byte aligned");
  if (((uintptr_t)workspace & 15u) != 0) return fail(TGS_EINVAL, "gtopk_merge: workspace not 16-byte aligned");
  const size_t pk4 = (size_t)P * (size_t)k * 4, k4 = (size_t)k * 4, pk1 = (size_t)P * (size_t)k;
  if (overlaps(out_idx, k4, out_val, k4) || overlaps(out_idx, k4, out_mask, pk1) || overlaps(out_val, k4, out_mask, pk1) ||
      overlaps(idx, pk4, out_idx, k4) || overlaps(idx, pk4, out_val, k4) || overlaps(idx, pk4, out_mask, pk1) ||
      overlaps(val, pk4, out_idx, k4) || overlaps(val, pk4, out_val, k4) || overlaps(val, pk4, out_mask, pk1))
    return fail(TGS_EINVAL, "gtopk_merge: overlapping buffers");
  const GtLayout L = gt_layout(P, k);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "gtopk_merge: workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (k == 0) return TGS_OK;
  char* ws = (char*)workspace;
  u32* err = (u32*)ws;
  const int R = L.R;
  const int64_t NP = (int64_t)1 << L.logNP;
  const Pair* prow = (const Pair*)(ws + L.prow);
  const PartDir* rdir = (const PartDir*)(ws + L.rdir);
  Pair* outs = (Pair*)(ws + L.out);
  PartDir* odir = (PartDir*)(ws + L.odir);
  {
    RowArgs ra{};
    ra.idx = idx;
    ra.val = val;
    ra.k = k;
    ra.cpr = L.cpr;
    ra.logNP = L.logNP;
    ra.rcnt = (u32*)(ws + L.rcnt);
    ra.rdir = (PartDir*)(ws + L.rdir);
    ra.prow = (Pair*)(ws + L.prow);
    ra.ppos = (u32*)(ws + L.ppos);
    ra.clear = (v4u*)(ws + L.hist);
    ra.nclear = (int64_t)(L.clear_end - L.hist) / 16;
    const unsigned grid = (unsigned)((int64_t)P * L.cpr);
    hipLaunchKernelGGL(k_gt_rcount, dim3(grid), dim3(kGtThreads), 0, stream, ra);
    hipLaunchKernelGGL(k_gt_rscatter, dim3(grid), dim3(kGtThreads), 0, stream, ra);
  }
  for (int r = 0; r < R; ++r) {
    const int64_t nm = gt_merges(P, r);
    JoinArgs ja{};
    ja.P = P;
    ja.r = r;
    ja.k = k;
    ja.logNP = L.logNP;
    ja.prow = prow;
    ja.rdir = rdir;
    ja.out = outs;
    ja.odir = odir;
    ja.W = (Pair*)(ws + L.W);
    ja.wdir = (PartDir*)(ws + L.wdir);
    ja.hist = (u32*)(ws + L.hist);
    ja.arrive = (u32*)(ws + L.arrive);
    ja.sel = (u32*)(ws + L.sel);
    ja.err = err;
    hipLaunchKernelGGL(k_gt_join, dim3((unsigned)(nm * NP)), dim3(kGtThreads), 0, stream, ja);
    KeepArgs ka{};
    ka.r = r;
    ka.k = k;
    ka.logNP = L.logNP;
    ka.W = ja.W;
    ka.wdir = ja.wdir;
    ka.sel = ja.sel;
    ka.ccnt = (u32*)(ws + L.ccnt);
    ka.karrive = (u32*)(ws + L.karrive);
    ka.kabove = (u32*)(ws + L.kabove);
    ka.cand = (Pair*)(ws + L.cand);
    ka.out = outs;
    ka.odir = odir;
    ka.err = err;
    hipLaunchKernelGGL(k_gt_keep, dim3((unsigned)(nm * NP)), dim3(kGtThreads), 0, stream, ka);
  }
  {
    const int64_t nruns = (k + kRunTile - 1) / kRunTile;      // sorted runs
    const int64_t ntiles = (k + kSortTile - 1) / kSortTile;   // merge workgroups
    FinalArgs fa{};
    fa.P = P;
    fa.k = k;
    fa.n = n;
    fa.logNP = L.logNP;
    fa.mask = out_mask;
    // the final set: slot 0's output region, or (P = 1) its grouped row
    fa.F = R > 0 ? outs : prow;
    fa.fdir = R > 0 ? odir : rdir;
    fa.prow = prow;
    fa.ppos = (const u32*)(ws + L.ppos);
    fa.rdir = rdir;
    fa.nruns = nruns;
    fa.runs = (u64*)(ws + L.runs[0]);
    fa.out_idx = out_idx;
    fa.out_val = out_val;
    fa.err = err;
    hipLaunchKernelGGL(k_gt_final, dim3((unsigned)(nruns + (int64_t)P * NP)), dim3(kGtThreads), 0, stream, fa);
    int cur = 0;
    for (int64_t Lr = kRunTile; Lr < k; Lr *= 2) {
      MergeArgs ma{};
      ma.src = (const u64*)(ws + L.runs[cur]);
      ma.dst = (u64*)(ws + L.runs[1 - cur]);
      ma.k = k;
      ma.L = Lr;
      ma.last = 2 * Lr >= k;
      ma.out_idx = out_idx;
      ma.out_val = out_val;
      hipLaunchKernelGGL(k_gt_merge, dim3((unsigned)ntiles), dim3(kGtThreads), 0, stream, ma);
      cur = 1 - cur;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "gtopk_merge: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

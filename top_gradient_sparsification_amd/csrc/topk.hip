// Error-feedback top-k step on gfx950.
//
// Method (arxivdaily listing for arXiv 2004.05298, entries "Sparsified SGD
// with Memory" and "The Convergence of Sparsified Gradient Methods"): add the
// accumulated error to the gradient, send the k entries of largest magnitude,
// keep everything else as the new error.  The listing's entry "Empirical
// Analysis on Top-k Gradient Sparsification ..." names gradient sorting as the
// GPU bottleneck, so nothing here sorts more than the candidates.
//
// Fast path: ONE launch, k_step, one workgroup of 1024 threads per compute
// unit, every workgroup resident.  Workgroup 0 plans; workgroups 1..G-1 each
// stream their share of the vector; workgroups 0..63 finish.
//   sample   every workgroup reads ~1/G of a ~1% sample (64-element chunks
//            spread over the whole vector) into a 12-bit LDS histogram of
//            key >> 19.  It publishes its top sample keys (device atomics) and
//            derives its own local threshold T_loc, a sample quantile several
//            times below the k-th key.
//   plan     workgroup 0 gathers the published keys and ranks them exactly:
//            T_guess (about 1.4k entries expected above it) and up to 64
//            bucket boundaries between T_guess and the top.  It publishes
//            the plan while the others stream.
//   stream   acc = residual + grad, one pass over rows of 1024 float4, dealt
//            round-robin (streaming workgroup m takes rows m, m + M, ...),
//            two rows in flight per workgroup.  Every acc goes back to
//            residual as a whole float4 (non-temporal; partial lines would
//            cost far more), and entries with key >= T_loc are also appended
//            to an LDS list.  Nothing waits for the plan here: wave 0 polls
//            its flag once per row and loads it into LDS once published.
//   publish  at the end of its share a workgroup reads the plan, keeps the
//            list entries with key >= T_guess (the candidates), groups them
//            by bucket and publishes them and their per-bucket counts with
//            device atomics.  A workgroup whose list overflowed, or whose
//            T_loc lay above T_guess, first re-reads its own rows of residual.
//   finish   finisher f waits for every workgroup, adds up the bucket counts,
//            checks that the plan held (at least k candidates, every bucket
//            that holds a rank below k fits in LDS, nothing overflowed),
//            gathers bucket f, orders it by (key desc, index asc), writes the
//            entries of rank < k to the output and stores +0 to their
//            residual.  Every acc store of every streaming workgroup completed
//            at device scope before that workgroup arrived, so the zero lands
//            after the acc it replaces.
// Everything one workgroup reads from another is written with device-scope
// stores or atomics and read with device-scope loads, so the fast path needs
// no cache write-back fences.
//
// State between launches: the control block holds two counter sets and a
// parity word saying which one the next launch uses.  Every workgroup reads
// the parity when it starts; workgroup 0 clears the other set, and once every
// workgroup has arrived at the sample phase (so has read the parity) it flips
// the word.  A launch therefore finds its set clean whatever launched before
// it, on the host or replayed from a graph, and nothing is kept on the host.
//
// When the plan did not hold, residual already holds acc everywhere: the
// grid fences, meets at a barrier and runs the exact general path below.
//
// General path (grid barriers; the fallback of the fast path and of the
// bucketed ranking, inside their launches, and a launch of its own,
// k_general, where neither applies):
//   radix select of the k-th key over 11/11/9-bit digits, counts per
//   workgroup, ordered compaction of the selected entries in ascending index
//   order (ties at the k-th key resolved by index), a stable LSD radix sort of
//   the k entries by descending key (4 x 8-bit digits), then emit and zero.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstddef>
#include <cstring>
#include <type_traits>
#include <vector>

#include "tgs_host.h"
#include "tgs_internal.h"
#include "tgs_midseg.h"
#include "tgs_rank.h"

namespace tgs {

// --------------------------------------------------------------- sizes ----
constexpr int kStepThreads = 1024;
constexpr int kStepWaves = kStepThreads / kWave;    // 16
constexpr int kMaxStepBlocks = 256;
constexpr int kMaxBuckets = 64;                     // also the number of finishers
constexpr int kHistShift = 19;                      // sample histogram bin = key >> 19
constexpr int kHistBins = 1 << (31 - kHistShift);   // 4096
constexpr int kSampleChunk = 64;                    // contiguous elements per sample chunk
constexpr int kSampleRounds = 2;                    // chunks per wave at most
constexpr int kSampleKeyCap = kSampleRounds * kStepThreads;  // sample keys per workgroup
constexpr int kPubCap = 40;                         // sample keys one workgroup may publish
constexpr int kPlanCap = kPubCap * kMaxStepBlocks;  // 10240
constexpr int kListCap = 8192;                      // local list of one workgroup (LDS)
constexpr int kSlotTotal = 4096;                    // slots of one bucket over all workgroups (G * S)
constexpr int kOvfCap = 4096;                       // candidates one workgroup may put past its slots
constexpr int kFinishCap = 4096;                    // bucket entries a finisher orders in LDS
constexpr int kSubBins = 2048;
constexpr int kRawWords = 28672;                    // 112 KB of LDS shared by the phases
constexpr int64_t kFastMinN = (int64_t)kMaxStepBlocks * kStepWaves * kSampleRounds * kSampleChunk;  // 2^19
constexpr u32 kSpinLimit = 1u << 18;
// plain pass + standalone general path
constexpr int kAccThreads = 1024;
constexpr int kMaxAccBlocks = 256;  // one first-level histogram row each
constexpr int kGenThreads = 512;
constexpr int kGenBlocks = 256;
constexpr int kMaxGenWG = 256;  // workgroups of either general-path launch
constexpr int kLsdDigits = 512;  // digits of an LSD pass at most (9 bits)

// reasons a plan did not hold (StepCtl::why)
constexpr int kSmallThreads = 1024;
constexpr int kSmallPer = 8192;            // entries per workgroup of k_small (8 per thread)
constexpr int64_t kSmallMaxN = 1 << 18;    // k_small: n <= this (at most 32 workgroups) ...
constexpr int64_t kSmallMaxK = 256;        // ... and k <= this
constexpr int kSmallMaxSeg = 64;           // segments one k_small launch takes
constexpr u32 kNoGuide = 0xFFFFFFFFu;  // guided accumulate pass: keep no candidates
constexpr u32 kBktMax = 8192;     // buckets of the guided ranking at most
constexpr u32 kBktCap = 1024;     // entries one bucket may hold
constexpr u32 kBktBatch = 4096;   // entries a workgroup sorts at once (LDS)
constexpr u32 kBktRanges = 2048;  // ranges of buckets sorted by one workgroup each, at most
constexpr int kGuessThreads = 1024;
constexpr int kGuessBlocks = 64;
constexpr int kGuessUnroll = 8;  // sample chunks per wave, all loads in flight at once
constexpr int kGuessChunk = 4 * kWave;  // entries per sample chunk: one float4 per lane
constexpr int64_t kGuessMaxChunks = (int64_t)kGuessBlocks * (kGuessThreads / kWave) * kGuessUnroll;
constexpr int64_t kGuideMinN = (int64_t)1 << 18;  // smaller vectors take the plain accumulate pass
constexpr int kRkBuckets = 1024;   // buckets of the bucketed ranking at most (one ranking workgroup each)
constexpr int64_t kRkMinK = 32768; // the bucketed ranking serves k from this on
constexpr int kRkStage = 12288;    // candidates one accumulate workgroup stages in LDS (its region)
constexpr u32 kRkPart = 3072;      // a bucket above this many entries is shared by several ranking workgroups
constexpr u32 kRkMaxParts = 4;     // ... at most this many
static_assert(kRkBuckets <= kRankThreads, "one bucket total per ranking thread");
constexpr u32 kWhyPlan = 1u, kWhyBucket = 4u, kWhyFew = 8u, kWhyRegion = 16u, kWhyList = 32u, kWhyWait = 64u;

// ------------------------------------------------------------- state ----
struct Plan {
  u32 valid;     // 1 when the plan below was built
  u32 t_guess;   // candidates are the keys >= t_guess
  u32 nbuckets;  // 1..kMaxBuckets
  u32 pad;
  u32 lo[kMaxBuckets];  // bucket j holds keys in [lo[j], lo[j-1]); lo[nbuckets-1] == t_guess
};

struct alignas(128) Counter {  // one cache line each
  u64 v;
  u64 pad[15];
};

// The counters one k_step launch synchronises with; zero when it starts.
// Flags many workgroups wait on are written to 8 lines and each workgroup
// polls the one of its group (blockIdx % 8): same-address accesses serialise
// at the memory, and a few hundred pollers on one line would slow down
// everything else that goes there.
struct StepSet {
  Counter samp_grp[8], samp_all;  // sample phase arrivals (workgroup 0 polls samp_all)
  Counter main_grp[8], main_all;  // streaming workgroups published (the finishers poll main_all)
  Counter plan_flag[8];           // 1 once the plan is published
  Counter verdict_flag[8];        // 1 = the plan held, 2 = run the exact path
  Counter bad;                    // low word: OR of kWhy* failures seen by the streaming workgroups
  alignas(128) u32 tot[kMaxBuckets];  // candidates per bucket over all workgroups (device adds)
};
constexpr int kSetCounters = (int)(offsetof(StepSet, tot) / sizeof(Counter));

// Thread 0 only: sets all 8 copies of a replicated flag (no wait).
__device__ __forceinline__ void flag_set(Counter* f, u64 v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) xchg_agent64(&f[i].v, v);
}

// Start of every top-k workspace.  Launches alternate between the two
// counter sets (the parity word says which); workgroup 0 of each launch
// clears the set the next launch uses, which no one else touches meanwhile.
struct StepCtl {
  u32 err;        // device error word (offset 0 of every workspace)
  u32 pad0;
  u32 verdict;    // 1 when the last fast-path call's plan held
  u32 fallbacks;  // fast-path calls whose plan did not hold (never reset)
  u32 why;        // OR of kWhy* reasons over those calls (never reset)
  u32 rescans;    // workgroup shares re-read because their list was incomplete (never reset)
  u32 guided_used;    // guided general-path calls that selected from the copied candidates (never reset)
  u32 guided_missed;  // guided calls whose guess or regions did not hold: acc read again (never reset)
  u32 parity;         // counter set the next k_step launch uses (flipped by each launch)
  u32 mid_exact;      // batched layer-wise segments selected exactly from acc (never reset)
  u32 rk_count;       // bucketed ranking: buckets of this call (0: none), set by k_guess
  u32 rk_ok;          // 1 once the bucketed ranking has emitted the step
  u32 rk_ovf;         // set when an accumulate workgroup's stage of candidates overflowed
  u32 rk_used;        // calls whose bucketed ranking held (never reset)
  u32 rk_missed;      // calls whose bucketed ranking did not hold: the general path ran (never reset)
  u32 pad1[49];
  StepSet set[2];
  Plan plan;
  u32 seg_done[64];  // arrivals per segment of a k_small or k_mid_guess launch; each segment's last workgroup leaves it zero
  // guided accumulate pass (standalone general path): k_guess adds its sample
  // histogram into the header histogram; its last workgroup picks guide_bin
  // and leaves the histogram, its counter and guide_ovf zero
  u32 guide_bin;   // candidates are the entries of first-level bins >= guide_bin (kNoGuide: none)
  u32 guide_ovf;   // set by the accumulate pass when a workgroup's region overflowed
  u32 acc_ticket;  // row pairs handed out by the accumulate pass (k_guess sets it to zero)
};
static_assert(sizeof(StepCtl) <= kEstStateOffset, "control block overlaps the header's shared state");
static_assert(offsetof(StepCtl, mid_exact) == 36 && offsetof(StepCtl, rk_used) == 52,
              "the tests read the route counters at fixed offsets");
static_assert(kMaxAccBlocks <= kMaxGenWG, "guided regions are the general path's");

// State of the general path (zero when it starts).
struct GenState {
  u32 hist[3][2048];
  u32 bar_cnt[9][32];  // grid barrier group counters, one cache line each
  u32 bar_gen[8][32];  // grid barrier all-counter, 8 copies
  u32 bar_abort;
  u32 cand_ovf;
};

struct TopkLayout {
  size_t ctl, gstate, gcnt, lsd_cnt, lsd_pre, lsd_tot, bufA, bufB, cand, hist_rows, guide_cnt, bkt_cnt, bkt_cur, bkt_buf,
      small, pub, rcnt, slots, ovf, rk_tab, rk_tot, rk_cnt, rk_slots, total;
  u32 cand_cap;
  int64_t rk_entries;  // candidate places of the bucketed ranking (0: not provided)
  u32 rk_target;       // entries per bucket the bucketed ranking aims at
};

// The bucketed ranking's sizes for (n, k): the accumulate workgroups (as
// the host launches them) and the entries per bucket aimed at: about 240
// buckets for the ~1.5 k candidates, so that the ranking workgroups (one per
// compute unit: each holds 152 KB of LDS) run in one wave, 256 to 3000 each.
struct RkSizes {
  int G1;
  u32 target;
};
static RkSizes rk_sizes(int64_t n, int64_t k) {
  RkSizes z{};
  const int64_t units = n / 4, per = (int64_t)kAccThreads * 2;
  z.G1 = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxAccBlocks, (units + per - 1) / per));
  z.target = (u32)std::min<int64_t>(3000, std::max<int64_t>(256, (3 * k + 479) / 480));
  return z;
}

// Pairs one candidate region (one wave of the standalone general path) holds:
// room for 4 k spread evenly, plus slack.  The guided accumulate pass fills
// the regions of one workgroup's waves as a single region.
static u32 cand_region_cap(int64_t k) {
  const int64_t regions = (int64_t)kMaxGenWG * (kGenThreads / kWave);
  const int64_t c = (4 * k + regions - 1) / regions + 64;
  return (u32)((c + 63) / 64 * 64);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static TopkLayout topk_layout(int64_t n, int64_t k) {
  TopkLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.ctl = take(kWorkspaceHeader);
  L.gstate = take(sizeof(GenState));
  L.gcnt = take(sizeof(u32) * 2 * kMaxGenWG * (kStepThreads / kWave));  // per (workgroup, wave)
  L.lsd_cnt = take(sizeof(u32) * kLsdDigits * kMaxGenWG);
  L.lsd_pre = take(sizeof(u32) * kLsdDigits * kMaxGenWG);
  L.lsd_tot = take(sizeof(u32) * kLsdDigits);
  L.bufA = take(sizeof(Pair) * (size_t)std::max<int64_t>(k, 1));
  L.bufB = take(sizeof(Pair) * (size_t)std::max<int64_t>(k, 1));
  L.cand_cap = cand_region_cap(k);
  L.cand = take(sizeof(u64) * (size_t)kMaxGenWG * (kGenThreads / kWave) * L.cand_cap);
  L.hist_rows = take(sizeof(u32) * 2048 * (size_t)kMaxAccBlocks);
  L.guide_cnt = take(sizeof(u32) * (size_t)kMaxGenWG);
  L.bkt_cnt = take(sizeof(u32) * kBktMax);
  L.bkt_cur = take(sizeof(u32) * kBktMax);
  L.bkt_buf = take(sizeof(u64) * (size_t)kMaxGenWG * (kGenThreads / kWave) * L.cand_cap);
  L.small = take(sizeof(u64) * (size_t)(kSmallMaxN / kSmallPer) * kSmallMaxK);
  L.pub = take(sizeof(u32) * ((size_t)kPlanCap + kMaxStepBlocks));
  L.rcnt = take(sizeof(u16) * (size_t)kMaxStepBlocks * kMaxBuckets);
  L.slots = take(sizeof(Pair) * (size_t)kMaxBuckets * kSlotTotal);
  L.ovf = take(sizeof(Pair) * (size_t)kMaxStepBlocks * kOvfCap);
  if (k >= kRkMinK && n >= kGuideMinN) {
    const RkSizes z = rk_sizes(n, k);
    L.rk_target = z.target;
    L.rk_entries = (int64_t)z.G1 * kRkStage;
    L.rk_tab = take(sizeof(u32) * 2048);
    L.rk_tot = take(sizeof(u32) * kRkBuckets);
    L.rk_cnt = take(sizeof(u32) * (size_t)kRkBuckets * kMaxAccBlocks);
    L.rk_slots = take(sizeof(u64) * (size_t)L.rk_entries);
  }
  L.total = off;
  return L;
}

// ------------------------------------------------------ phase counters ----
// A phase completes when every workgroup of the grid has arrived.  Arrivals
// are counted per group of workgroups (blockIdx % 8, each counter on its own
// cache line) and the last arrival of a group bumps the phase counter, so
// no single address takes more than G/8 + 8 atomics.  Counters start at zero.
__device__ __forceinline__ int phase_groups(int G) { return G < 8 ? G : 8; }

// Thread 0 only.  True when this arrival completed the phase.
__device__ __forceinline__ bool phase_arrive(Counter* grp, Counter* all, int G) {
  const int ng = phase_groups(G);
  const int x = (int)blockIdx.x % ng;
  const u64 per = (u64)((G - 1 - x) / ng + 1);
  if (add_agent64(&grp[x].v, 1) + 1 != per) return false;
  return add_agent64(&all->v, 1) + 1 == (u64)ng;
}

// Thread 0 only.  Bounded wait for the phase; a timeout sets an error bit.
__device__ __forceinline__ bool phase_wait(const Counter* all, int G, u32* err) {
  const u64 target = (u64)phase_groups(G);
  u32 spins = 0;
  while (ld_agent64(&all->v) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      atomicOr(err, kErrBarrierTimeout);
      return false;
    }
  }
  return true;
}

// Thread 0 only.  Bounded wait for a nonzero flag; 0 on timeout.
__device__ __forceinline__ u32 flag_wait(const Counter* flag, u32* err) {
  u32 spins = 0;
  for (;;) {
    const u64 v = ld_agent64(&flag->v);
    if (v != 0) return (u32)v;
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      atomicOr(err, kErrBarrierTimeout);
      return 0;
    }
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
  u32* gcnt;     // [G][waves][2]
  u32* lsd_cnt;  // [G][digits]
  u32* lsd_pre;  // [G][digits]
  u32* lsd_tot;  // [digits]
  Pair* bufA;
  Pair* bufB;
  GridBar bar;
  u64* cand;      // candidate regions, cand_cap pairs per (workgroup, wave)
  u32* cand_ovf;  // set when a region overflows (zero on entry)
  u32 cand_cap;
  u32 acc_rows;          // rows of acc_hist (standalone path)
  const u32* acc_hist;   // [acc_rows][2048] first-level histograms from the accumulate pass
  // guided accumulate pass (guided != 0; then acc_rows <= the grid): the
  // entries of first-level bins >= *guide_bin streamed by its workgroup b, in
  // no particular order, fill the regions of this kernel's workgroup b's
  // waves as one region of guide_cnt[b] pairs
  u32 guided;
  u32 guide_stride;  // pairs between consecutive workgroups' regions
  const u32* guide_bin;
  const u32* guide_ovf;
  const u32* guide_cnt;
  u32* guide_stats;  // [2]: guided_used, guided_missed
  // bucket ranking of the guided candidates
  u32* bkt_cnt;  // [kBktMax] entries per bucket (cleared by this kernel)
  u32* bkt_cur;  // [kBktMax] places handed out per range of buckets (cleared by this kernel)
  u64* bkt_buf;  // the candidates, grouped by bucket in bucket order
};

// LDS words the general path's tables take when the caller lends them.
template <int NT, int DB>
constexpr int general_lds_words() {
  return 2048 + (NT / kWave) * (1 << DB) + 2 * (1 << DB);
}

// Sum over the block of one value per thread.
template <int NT>
__device__ __forceinline__ u32 block_sum(u32 v, u32* lds) {
  u32 total;
  block_exclusive_sum<NT>(v, lds, total);
  return total;
}

// The exact general path, run by workgroups 0 .. a.bar.nwg-1, which must all
// be resident at once (grid barriers); NT is the workgroup size and V the
// rows of NT entries each pass keeps in flight per tile (kPipe: the next
// tile's loads go out before a tile is processed).  acc is read from
// residual, which every participant must be able to see.
template <int NT, int V, bool kPipe, int DB, bool kCand, bool kExt = false>
__device__ __forceinline__ void general_path(const GenArgs& a, u32* ext = nullptr) {
  constexpr int NW = NT / kWave;
  constexpr int ND = 1 << DB;  // digits of one LSD pass
  static_assert(ND <= kLsdDigits && ND <= 2048, "LSD digit tables");
  // the tables in LDS of their own, or (kExt) in the caller's LDS from `ext`
  // on (general_lds_words<NT, DB>() words the caller does not use meanwhile)
  __shared__ u32 own_hist[kExt ? 1 : 2048];
  __shared__ u32 own_wcnt[kExt ? 1 : NW][kExt ? 1 : ND];
  __shared__ u32 own_base[kExt ? 1 : ND];
  __shared__ u32 own_run[kExt ? 1 : ND];
  u32* const s_hist = kExt ? ext : own_hist;
  u32 (*const s_wcnt)[ND] = reinterpret_cast<u32 (*)[ND]>(kExt ? ext + 2048 : &own_wcnt[0][0]);
  u32* const s_base = kExt ? ext + 2048 + NW * ND : own_base;
  u32* const s_run = kExt ? ext + 2048 + NW * ND + ND : own_run;
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_found[4];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int G = (int)a.bar.nwg;
  const int b = blockIdx.x;
  const int64_t per = (a.n + G - 1) / G;
  if constexpr (kCand) {
    if (a.guided)  // zero before the first barrier, used after it
      for (u32 i = (u32)b * NT + tid; i < kBktMax; i += (u32)G * NT) {
        st_agent(&a.bkt_cnt[i], 0u);
        st_agent(&a.bkt_cur[i], 0u);
      }
  }
  const int64_t cb = std::min<int64_t>(a.n, (int64_t)b * per);
  const int64_t ce = std::min<int64_t>(a.n, cb + per);
  const u32* accb = (const u32*)a.acc;
  // Entry base + j NT + tid of a tile (j < V); bit j of the returned mask
  // says whether it lies before ce.  The loads are unconditional (an index
  // past the end reads entry cb instead), so all V are in flight before any
  // is used: a load under a branch would be waited for on its own.  Per-entry
  // flags live in bit masks: bool arrays become wave masks in scalar
  // registers, which spill.
  // Offsets are 32-bit and relative to cb (a chunk is below 2^31 entries).
  const u32* accc = opaque_ptr(accb + cb);
  const u32 clen = opaque_u32((u32)(ce - cb));
  auto load_tile = [&](int64_t base, u32* bits) -> u32 {
    const u32 o0 = (u32)(base - cb) + (u32)tid;
    u32 vm = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const u32 o = o0 + (u32)(j * NT);
      const bool in = o < clen;
      vm |= (u32)in << j;
      bits[j] = accc[in ? o : 0u];
    }
    return vm;
  };
  // body(base, bits, valid) on every tile of [cb, ce) in order; the next
  // tile's loads are in flight while one is processed (one workgroup per
  // compute unit needs two tiles in flight to keep HBM busy).
  auto for_each_tile = [&](auto&& body) {
    constexpr int64_t TS = (int64_t)V * NT;
    u32 b0[V], b1[V];
    if constexpr (kPipe) {
      u32 v0 = cb < ce ? load_tile(cb, b0) : 0u, v1;
      for (int64_t base = cb; base < ce; base += 2 * TS) {
        v1 = load_tile(base + TS, b1);
        body(base, b0, v0);
        if (base + TS >= ce) break;
        v0 = load_tile(base + 2 * TS, b0);
        body(base + TS, b1, v1);
      }
    } else {
      for (int64_t base = cb; base < ce; base += TS) body(base, b0, load_tile(base, b0));
    }
  };

  // Wave w owns the contiguous slice [wb, we) of the workgroup's chunk; the
  // candidate pass, the counts and the ordered compaction walk it in rows of
  // 64 entries, V rows per tile, with no barrier and no LDS.  Counts, places
  // and indices fit in 32 bits (n < 2^31).
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // the same in every lane
  const u32 wlen = (clen + NW - 1) / NW;
  const u32 wb = std::min<u32>(clen, (u32)w * wlen), we = std::min<u32>(clen, wb + wlen);
  auto load_wave_tile = [&](u32 o, u32* bits) -> u32 {
    u32 vm = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const u32 q = o + (u32)(j * kWave + lane);
      const bool in = q < we;
      vm |= (u32)in << j;
      bits[j] = accc[in ? q : 0u];
    }
    return vm;
  };
  auto for_each_wave_tile = [&](auto&& body) {
    constexpr u32 TS = (u32)(V * kWave);
    u32 b0[V], b1[V];
    if constexpr (kPipe) {
      u32 v0 = wb < we ? load_wave_tile(wb, b0) : 0u, v1;
      for (u32 o = wb; o < we; o += 2 * TS) {
        v1 = load_wave_tile(o + TS, b1);
        body(o, b0, v0);
        if (o + TS >= we) break;
        v0 = load_wave_tile(o + 2 * TS, b0);
        body(o + TS, b1, v1);
      }
    } else {
      for (u32 o = wb; o < we; o += TS) body(o, b0, load_wave_tile(o, b0));
    }
  };
  // Candidates (standalone path): this wave's entries of the first-level bins
  // at and above the threshold bin, in index order, in its own region of
  // cand_cap pairs.  ccount is the wave's count; use_cand is the same in
  // every workgroup.
  bool use_cand = false;
  u32 ccount = 0;
  const u64* creg = kCand ? opaque_ptr(a.cand + (size_t)(b * NW + w) * a.cand_cap) : nullptr;
  auto load_cand_tile = [&](u32 o, u64* pv) -> u32 {
    u32 vm = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const u32 q = o + (u32)(j * kWave + lane);
      const bool in = q < ccount;
      vm |= (u32)in << j;
      pv[j] = creg[in ? q : 0u];
    }
    return vm;
  };
  auto for_each_cand_tile = [&](auto&& body) {
    constexpr u32 TS = (u32)(V * kWave);
    u64 p0[V], p1[V];
    u32 v0 = ccount > 0 ? load_cand_tile(0, p0) : 0u, v1;
    for (u32 o = 0; o < ccount; o += 2 * TS) {
      v1 = load_cand_tile(o + TS, p1);
      body(p0, v0);
      if (o + TS >= ccount) break;
      v0 = load_cand_tile(o + 2 * TS, p0);
      body(p1, v1);
    }
  };

  // Guided candidates (any order in the regions): sort every entry of the
  // first-level bins >= d -- all C of them, the k-th key's bin included --
  // by (key desc, index asc) and emit the first k.  Each bin's key range is
  // cut into ceil(count / target) equal buckets, numbered from the top, so
  // the buckets split the C entries in descending key order:
  //   1. bucket counts (LDS, then device-scope adds)                | barrier
  //   2. bucket starts (scan of the counts); the buckets grouped into
  //      ranges of fewer than kBktBatch entries; places reserved per
  //      (workgroup, range) and the entries scattered to bkt_buf    | barrier
  //   3. workgroup b loads ranges b, b + G, ... into LDS; each wave ranks
  //      whole buckets by counting and writes the entries of place < k.
  // Returns 1 when done, 0 when a bucket is too large (nothing written; the
  // caller goes on with the radix select over copies from acc), -1 if a
  // barrier failed.
  auto bucket_rank = [&](auto d, auto C) -> int {  // generic: instantiated only where called
    __shared__ u32 s_bkt[kBktMax];  // counts, then starts
    __shared__ u64 s_ent[kBktBatch];  // step 3: one range's entries
    __shared__ u32 s_bbase[2048];   // first bucket of bin j (j >= d)
    __shared__ u32 s_bnum[2048];    // buckets of bin j
    __shared__ u32 s_misc[4];
    __shared__ u32 s_rbeg[kBktRanges];  // first entry of range r
    __shared__ u32 s_rcnt[kBktRanges];  // this workgroup's entries of range r, then its next place there
    const u32 target = std::max(32u, (C + (kBktMax - 2048u) - 1u) / (kBktMax - 2048u));
    // thread t owns bins [2048 - 4 (t + 1), 2048 - 4 t), scanned from the top
    static_assert(2048 % NT == 0, "bins per thread");
    constexpr int BPT = 2048 / NT;
    const int top = 2048 - BPT * tid;
    u32 own = 0;
    for (int j = top - 1; j >= top - BPT; --j) {
      const u32 nb = (u32)j >= d ? (s_hist[j] + target - 1) / target : 0u;
      s_bnum[j] = nb;
      own += nb;
    }
    u32 nbk;
    u32 run = block_exclusive_sum<NT>(own, s_scan, nbk);
    for (int j = top - 1; j >= top - BPT; --j) {
      s_bbase[j] = run;
      run += s_bnum[j];
    }
    if (nbk > kBktMax) return 0;  // cannot happen: C / target + 2048 bins <= kBktMax
    for (u32 i = tid; i < nbk; i += NT) s_bkt[i] = 0u;
    __syncthreads();
    auto bucket_of_key = [&](u32 key) -> u32 {
      const u32 j = key >> 20, nb = s_bnum[j];
      return s_bbase[j] + nb - 1u - (u32)(((u64)(key & 0xFFFFFu) * nb) >> 20);
    };
    // 1. counts
    for_each_cand_tile([&](const u64* pv, u32 vm) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const u32 key = key_of_bits((u32)(pv[j] >> 32));
        if (((vm >> j) & 1u) && (key >> 20) >= d) atomicAdd(&s_bkt[bucket_of_key(key)], 1u);
      }
    });
    __syncthreads();
    for (u32 i = tid; i < nbk; i += NT)
      if (s_bkt[i]) add_agent_relaxed(&a.bkt_cnt[i], s_bkt[i]);
    if (!grid_sync(a.bar)) return -1;
    // 2. bucket starts (exclusive scan of the counts; thread t holds buckets
    // [q0, q1)) into s_bkt; the largest bucket
    const u32 per_t = (nbk + NT - 1) / NT;
    const u32 q0 = std::min(nbk, (u32)tid * per_t), q1 = std::min(nbk, q0 + per_t);
    u32 sum = 0, mx = 0;
    for (u32 q = q0; q < q1; ++q) {
      const u32 c = a.bkt_cnt[q];
      sum += c;
      mx = std::max(mx, c);
    }
    u32 total;
    const u32 start0 = block_exclusive_sum<NT>(sum, s_scan, total);
    mx = wave_max(mx);
    if (tid == 0) s_misc[0] = 0u;
    __syncthreads();
    if (lane == 0) atomicMax(&s_misc[0], mx);
    // Range r holds the buckets that start in [r S, (r+1) S): whole buckets,
    // fewer than S + kBktCap <= kBktBatch entries, sorted by one workgroup.
    // Buckets start at most kBktCap apart, so every range holds one.
    constexpr u32 S = kBktBatch - kBktCap;
    const u32 D = (C + S - 1) / S;
    __syncthreads();
    if (s_misc[0] > kBktCap || total != C || D > kBktRanges) return 0;  // the same in every workgroup
    for (u32 r = tid; r < D; r += NT) {
      s_rbeg[r] = C;
      s_rcnt[r] = 0u;
    }
    __syncthreads();
    {
      u32 st = start0;
      for (u32 q = q0; q < q1; ++q) {
        const u32 c = a.bkt_cnt[q];
        s_bkt[q] = st;
        if (st < C) atomicMin(&s_rbeg[st / S], st);  // a range begins at its first bucket
        st += c;
      }
    }
    __syncthreads();
    // this workgroup's entries per range, then places reserved per range
    for_each_cand_tile([&](const u64* pv, u32 vm) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const u32 key = key_of_bits((u32)(pv[j] >> 32));
        if (((vm >> j) & 1u) && (key >> 20) >= d) atomicAdd(&s_rcnt[s_bkt[bucket_of_key(key)] / S], 1u);
      }
    });
    __syncthreads();
    for (u32 r = tid; r < D; r += NT) {
      const u32 c = s_rcnt[r];
      if (c) s_rcnt[r] = s_rbeg[r] + add_agent_relaxed(&a.bkt_cur[r], c);
    }
    __syncthreads();
    u64* const bout = opaque_ptr(a.bkt_buf);
    for_each_cand_tile([&](const u64* pv, u32 vm) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const u32 key = key_of_bits((u32)(pv[j] >> 32));
        if (((vm >> j) & 1u) && (key >> 20) >= d)
          st_agent64(bout + atomicAdd(&s_rcnt[s_bkt[bucket_of_key(key)] / S], 1u), pv[j]);
      }
    });
    if (!grid_sync(a.bar)) return -1;
    // 3. workgroup b ranks ranges b, b + G, ...: the entries of range r,
    // [s_rbeg[r], s_rbeg[r+1]) in bkt_buf, are grouped by bucket into LDS
    // (counting sort over the range's buckets u0..u1; s_bkt then holds each
    // bucket's end), and wave w ranks buckets u0 + w, u0 + w + 8, ... by
    // counting, inside the bucket, the entries with a smaller
    // (0x7FFFFFFF - key, index).  An entry's place is the range's start plus
    // its bucket's start in the range plus that count; places below k are
    // written.
    static_assert(kBktCap < kBktBatch, "a range holds whole buckets");
    const u32 kk = (u32)a.k;
    auto ck = [](u64 p) { return rank_key((u32)(p >> 32), (u32)p); };
    for (u32 r = (u32)b; r < D; r += (u32)G) {  // the same in every thread
      const u32 x = s_rbeg[r], y = r + 1 < D ? s_rbeg[r + 1] : C;
      if (x >= kk) break;
      if (x >= y) continue;  // cannot happen: every range holds a bucket
      const u32 m = y - x;
      // the range's entries in registers (every load in flight at once)
      constexpr int EPT = kBktBatch / NT;
      u64 pv[EPT];
      u32 uq[EPT];
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const u32 i = (u32)tid + (u32)j * NT;
        pv[j] = a.bkt_buf[x + (i < m ? i : 0u)];
      }
      u32 umin = 0xFFFFFFFFu, umax = 0u;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        uq[j] = bucket_of_key(key_of_bits((u32)(pv[j] >> 32)));
        if ((u32)tid + (u32)j * NT < m) {
          umin = std::min(umin, uq[j]);
          umax = std::max(umax, uq[j]);
        }
      }
      umin = wave_min(umin);
      umax = wave_max(umax);
      if (tid == 0) {
        s_misc[1] = 0xFFFFFFFFu;
        s_misc[2] = 0u;
      }
      __syncthreads();
      if (lane == 0) {
        atomicMin(&s_misc[1], umin);
        atomicMax(&s_misc[2], umax);
      }
      __syncthreads();
      const u32 u0 = s_misc[1], span = s_misc[2] - u0 + 1;  // span <= nbk <= kBktMax
      for (u32 i = tid; i < span; i += NT) s_bkt[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if ((u32)tid + (u32)j * NT < m) atomicAdd(&s_bkt[uq[j] - u0], 1u);
      __syncthreads();
      {  // exclusive scan of the span's counts, kBktMax / NT per thread
        constexpr u32 PT = kBktMax / NT;
        const u32 i0 = (u32)tid * PT;
        u32 own_sum = 0;
        for (u32 i = i0; i < i0 + PT && i < span; ++i) own_sum += s_bkt[i];
        u32 tot_unused;
        u32 run2 = block_exclusive_sum<NT>(own_sum, s_scan, tot_unused);
        for (u32 i = i0; i < i0 + PT && i < span; ++i) {
          const u32 c = s_bkt[i];
          s_bkt[i] = run2;
          run2 += c;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if ((u32)tid + (u32)j * NT < m) s_ent[atomicAdd(&s_bkt[uq[j] - u0], 1u)] = pv[j];
      __syncthreads();  // s_bkt[u - u0] is now the end of bucket u in s_ent
      // Lane l holds entries bs + l + 64 e (e < NE) of a bucket of at most
      // 64 NE and counts, for all of them at once, the smaller ones among
      // the bucket's entries, read one at a time (the same LDS address in
      // every lane).
      auto rank_bucket = [&](u32 bs, u32 be, auto ne_c) {
        constexpr int NE = decltype(ne_c)::value;
        u64 ci[NE];
        u32 rk[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const u32 i = bs + (u32)lane + (u32)(e * kWave);
          ci[e] = i < be ? ck(s_ent[i]) : ~0ull;
          rk[e] = 0;
        }
#pragma unroll 4
        for (u32 j = bs; j < be; ++j) {
          const u64 cj = ck(s_ent[j]);
#pragma unroll
          for (int e = 0; e < NE; ++e) rk[e] += cj < ci[e];
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const u32 i = bs + (u32)lane + (u32)(e * kWave), pos = x + bs + rk[e];
          if (i < be && pos < kk) {
            const Pair p = unpack_pair(s_ent[i]);
            a.out_idx[pos] = p.idx;
            a.out_val[pos] = __uint_as_float(p.bits);
            st_agent_f32(a.residual + p.idx, 0.0f);
          }
        }
      };
      static_assert(kBktCap <= 16 * kWave, "a bucket fits 16 entries per lane");
      for (u32 v = (u32)w; v < span; v += NW) {  // the same in every lane
        const u32 bs = v == 0 ? 0u : s_bkt[v - 1], be = s_bkt[v];
        if (bs >= be || x + bs >= kk) continue;
        const u32 mb = be - bs;
        if (mb <= kWave) rank_bucket(bs, be, std::integral_constant<int, 1>{});
        else if (mb <= 2 * kWave) rank_bucket(bs, be, std::integral_constant<int, 2>{});
        else if (mb <= 4 * kWave) rank_bucket(bs, be, std::integral_constant<int, 4>{});
        else if (mb <= 8 * kWave) rank_bucket(bs, be, std::integral_constant<int, 8>{});
        else rank_bucket(bs, be, std::integral_constant<int, 16>{});
      }
      __syncthreads();
    }
    return 1;
  };

  // ---------------- radix select of the k-th largest key ----------------
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  u32 prefix = 0;      // digits chosen so far (the key's top bits)
  int64_t need = a.k;  // entries still to take among keys matching prefix
  int64_t t_strict = -1;  // select every key > t_strict ...
  u32 t_eq = 0;           // ... and the first r keys equal to t_eq
  int64_t r = 0;
  u32 kmax = 0x7FFFFFFFu;  // at least the largest key (top of its level-0 bin)
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L], wd = widths[L];
    const u32 nbins = 1u << wd;
    for (int i = tid; i < 2048; i += NT) s_hist[i] = 0;
    __syncthreads();
    if (kCand && L == 0) {
      // the accumulate pass left one histogram row per workgroup: this
      // workgroup sums the columns of its share of the bins
      const int per_wg = (2048 + G - 1) / G;
      const int bin0 = std::min(2048, b * per_wg), nbin = std::min(2048, bin0 + per_wg) - bin0;
      const int rows = (int)a.acc_rows;
      for (int q = tid; q < nbin * rows; q += NT) {
        const u32 v = a.acc_hist[(size_t)(q / nbin) * 2048 + bin0 + q % nbin];
        if (v) atomicAdd(&s_hist[q % nbin], v);
      }
      __syncthreads();
      for (int i = tid; i < nbin; i += NT) st_agent(&a.ghist[bin0 + i], s_hist[i]);
    } else {
    auto hist_key = [&](u32 key) {
      if ((key >> (sh + wd)) == prefix) atomicAdd(&s_hist[(key >> sh) & (nbins - 1)], 1u);
    };
    if (kCand && use_cand) {
      for_each_cand_tile([&](const u64* pv, u32 vm) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          if ((vm >> j) & 1u) hist_key(key_of_bits((u32)(pv[j] >> 32)));
      });
    } else {
      for_each_tile([&](int64_t, const u32* bits, u32 vm) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          if ((vm >> j) & 1u) hist_key(key_of_bits(bits[j]));
      });
    }
    __syncthreads();
    for (int i = tid; i < (int)nbins; i += NT) {
      u32 v = s_hist[i];
      if (v) add_agent_relaxed(&a.ghist[L * 2048 + i], v);
    }
    }
    if (!grid_sync(a.bar)) return;
    for (int i = tid; i < (int)nbins; i += NT) s_hist[i] = a.ghist[L * 2048 + i];
    if (L == 0 && tid == 0) s_found[3] = 0;
    __syncthreads();
    if (L == 0) {
      for (int i = tid; i < (int)nbins; i += NT)
        if (s_hist[i] != 0) atomicMax(&s_found[3], (u32)i);
      __syncthreads();
      kmax = (s_found[3] << sh) | ((1u << sh) - 1u);
    }
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
    const int64_t n_above = s_found[1];
    need -= n_above;
    const int64_t h = s_found[2];
    prefix = (prefix << wd) | d;
    if constexpr (kCand) {
      // The guided accumulate pass already copied out every entry of the bins
      // >= its guessed bin, wave by wave into the regions this kernel's waves
      // read: when that bin is at or below d and no region overflowed, those
      // copies hold every entry still in play.  Every workgroup reads the
      // same words, so all decide alike.
      if (L == 0 && a.guided) {
        const u32 gb = *a.guide_bin;
        bool ranked = false;
        if (gb != kNoGuide && gb <= d && *a.guide_ovf == 0u) {
          const u32 cntb = (u32)b < a.acc_rows ? a.guide_cnt[b] : 0u;  // the accumulate pass may have fewer workgroups
          const u32 part = (cntb + NW - 1) / NW;
          const u32 lo = std::min(cntb, (u32)w * part), hi = std::min(cntb, lo + part);
          const u64* const wave_reg = creg;
          creg = opaque_ptr(a.cand + (size_t)b * a.guide_stride + lo);
          ccount = hi - lo;
          const int st = bucket_rank(d, (u32)(n_above + h));
          if (st < 0) return;
          ranked = st > 0;
          creg = wave_reg;  // not ranked: the regions are refilled from acc below
          ccount = 0;
        }
        if (b == 0 && tid == 0) atomicAdd(&a.guide_stats[ranked ? 0 : 1], 1u);
        if (ranked) return;
      }
    }
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
    if constexpr (kCand) {
      // After the first level: copy the entries of bins >= d (n_above + h of
      // them) out of acc once, and run the rest on the copies -- unless they
      // would crowd the regions, or one wave's share does not fit.
      if (L == 0 && !use_cand && (u64)(n_above + h) <= (u64)a.bar.nwg * NW * a.cand_cap * 3 / 4) {
        const u32 lo = d << sh;
        u64* const out = (u64*)creg;
        const u32 i0 = (u32)cb + (u32)lane;
        u32 cnt = 0;
        for_each_wave_tile([&](u32 o, const u32* bits, u32 vm) {
#pragma unroll
          for (int j = 0; j < V; ++j) {
            const bool keep = ((vm >> j) & 1u) && key_of_bits(bits[j]) >= lo;
            const u64 m = ballot(keep);
            const u32 pos = cnt + lanes_below(m);
            if (keep && pos < a.cand_cap) out[pos] = pack_pair(Pair{(int32_t)(i0 + o + (u32)(j * kWave)), bits[j]});
            cnt += (u32)__popcll(m);
          }
        });
        if (cnt > a.cand_cap && lane == 0) st_agent(a.cand_ovf, 1u);
        ccount = cnt;
        if (!grid_sync(a.bar)) return;
        use_cand = ld_agent(a.cand_ovf) == 0u;
      }
    }
    __syncthreads();
  }

  // ---------------- per-wave counts ----------------
  const u32 t_lo = (u32)(t_strict + 1), r32 = (u32)r, k32 = opaque_u32((u32)a.k);
  {
    u32 c_gt = 0, c_eq = 0;
    auto count_key = [&](u32 key) {
      c_gt += key >= t_lo;
      c_eq += r32 > 0 && key == t_eq;
    };
    if (kCand && use_cand) {
      for_each_cand_tile([&](const u64* pv, u32 vm) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          if ((vm >> j) & 1u) count_key(key_of_bits((u32)(pv[j] >> 32)));
      });
    } else {
      for_each_wave_tile([&](u32, const u32* bits, u32 vm) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          if ((vm >> j) & 1u) count_key(key_of_bits(bits[j]));
      });
    }
    c_gt = wave_sum(c_gt);
    c_eq = wave_sum(c_eq);
    if (lane == 0) {
      st_agent(&a.gcnt[2 * (b * NW + w)], c_gt);
      st_agent(&a.gcnt[2 * (b * NW + w) + 1], c_eq);
    }
  }
  if (!grid_sync(a.bar)) return;

  // ---------------- ordered compaction (ascending index) ----------------
  {
    // greater / equal keys in every slice before this wave's, in index order
    u32 pg = 0, pe = 0;
    for (int i = tid; i < b * NW; i += NT) {
      pg += a.gcnt[2 * i];
      pe += a.gcnt[2 * i + 1];
    }
    pg = block_sum<NT>(pg, s_scan);
    pe = block_sum<NT>(pe, s_scan);
    for (int q = 0; q < w; ++q) {
      pg += a.gcnt[2 * (b * NW + q)];
      pe += a.gcnt[2 * (b * NW + q) + 1];
    }
    // An entry's place: (greater keys before it) + min(equal keys before it,
    // r); it is selected if its key is greater, or equal with fewer than r
    // equal keys before it.
    u32 gt_seen = pg, eq_seen = pe;
    u64* const outA = opaque_ptr((u64*)a.bufA);
    auto place = [&](bool in, u32 key, u64 pair) {
      const bool g = in && key >= t_lo, e = in && r32 > 0 && key == t_eq;
      const u64 bg = ballot(g), be = ballot(e);
      const u32 gb = gt_seen + lanes_below(bg), eb = eq_seen + lanes_below(be);
      const bool sel = g || (e && eb < r32);
      const u32 pos = gb + std::min(eb, r32);
      if (sel && pos < k32) st_agent64(outA + pos, pair);
      gt_seen += (u32)__popcll(bg);
      eq_seen += (u32)__popcll(be);
    };
    if (kCand && use_cand) {
      for_each_cand_tile([&](const u64* pv, u32 vm) {
#pragma unroll
        for (int j = 0; j < V; ++j) place((vm >> j) & 1u, key_of_bits((u32)(pv[j] >> 32)), pv[j]);
      });
    } else {
      const u32 i0 = (u32)cb + (u32)lane;
      for_each_wave_tile([&](u32 o, const u32* bits, u32 vm) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          place((vm >> j) & 1u, key_of_bits(bits[j]), pack_pair(Pair{(int32_t)(i0 + o + (u32)(j * kWave)), bits[j]}));
      });
    }
  }
  if (!grid_sync(a.bar)) return;

  // ---------------- stable LSD radix sort by descending key ----------------
  // Every selected key lies in [kmin, kmax], so all of them agree above the
  // highest bit where kmin and kmax differ: only the bits below it are
  // sorted, DB per pass (the inverse key's bits are the key's complemented).
  const u32 kmin = r > 0 ? t_eq : (u32)(t_strict + 1);
  const int nbits = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);
  const int npass = (nbits + DB - 1) / DB;
  const int64_t per2 = (a.k + G - 1) / G;
  const int64_t sb = std::min<int64_t>(a.k, (int64_t)b * per2);
  const int64_t se = std::min<int64_t>(a.k, sb + per2);
  Pair* src = a.bufA;
  Pair* dst = a.bufB;
  for (int pass = 0; pass < npass; ++pass) {
    const int sh = DB * pass;
    for (int i = tid; i < ND; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (int64_t base = sb; base < se; base += (int64_t)V * NT) {
      u64 pv[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {  // unconditional loads (see load_tile)
        const int64_t i = base + (int64_t)j * NT + tid;
        pv[j] = ((const u64*)src)[i < se ? i : sb];
      }
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const u32 inv = 0x7FFFFFFFu - key_of_bits(unpack_pair(pv[j]).bits);
        if (base + (int64_t)j * NT + tid < se) atomicAdd(&s_hist[(inv >> sh) & (ND - 1)], 1u);
      }
    }
    __syncthreads();
    for (int i = tid; i < ND; i += NT) st_agent(&a.lsd_cnt[b * ND + i], s_hist[i]);
    if (!grid_sync(a.bar)) return;
    // column scans: digit d handled by workgroup d % G
    for (int d = b; d < ND; d += G) {  // G <= NT: one column entry per thread
      u32 c = tid < G ? a.lsd_cnt[tid * ND + d] : 0u;
      u32 colsum;
      u32 ex = block_exclusive_sum<NT>(c, s_scan, colsum);
      if (tid < G) st_agent(&a.lsd_pre[tid * ND + d], ex);
      if (tid == 0) st_agent(&a.lsd_tot[d], colsum);
    }
    if (!grid_sync(a.bar)) return;
    for (int i = tid; i < ND; i += NT) s_hist[i] = a.lsd_tot[i];
    if (tid == 0) s_found[3] = 0;
    __syncthreads();
    for (int i = tid; i < ND; i += NT)
      if ((int64_t)s_hist[i] == a.k) s_found[3] = 1;
    __syncthreads();
    if (s_found[3] != 0) continue;  // every key shares this digit: the pass is a no-op
    static_assert(ND <= NT, "one digit per thread in the base scan");
    {
      u32 v = tid < ND ? s_hist[tid] : 0u;
      u32 t;
      u32 ex = block_exclusive_sum<NT>(v, s_scan, t);
      if (tid < ND) {
        s_base[tid] = ex + a.lsd_pre[b * ND + tid];
        s_run[tid] = 0;
      }
    }
    for (int i = tid; i < NW * ND; i += NT) (&s_wcnt[0][0])[i] = 0;
    __syncthreads();
    // rows of NT entries, V rows' loads in flight at a time
    u64 pv[V];
    for (int64_t base = sb; base < se; base += NT) {
      const int64_t row = (base - sb) / NT;
      if (row % V == 0) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int64_t i = base + (int64_t)j * NT + tid;
          pv[j] = ((const u64*)src)[i < se ? i : sb];
        }
      }
      int64_t i = base + tid;
      bool valid = i < se;
      u64 cur = pv[0];
#pragma unroll
      for (int j = 1; j < V; ++j) cur = (row % V == j) ? pv[j] : cur;
      Pair e = valid ? unpack_pair(cur) : pair_sentinel();
      u32 d = valid ? (((0x7FFFFFFFu - key_of_bits(e.bits)) >> sh) & (ND - 1)) : 0u;
      u64 peers = ballot(valid);
#pragma unroll
      for (int bit = 0; bit < DB; ++bit) {
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
        if ((int64_t)pos < a.k) st_agent64((u64*)dst + pos, pack_pair(e));
      }
      __syncthreads();
      if (tid < ND) {
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
  for (int64_t base = sb; base < se; base += (int64_t)V * NT) {
    u64 pv[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      pv[j] = ((const u64*)src)[i < se ? i : sb];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      if (i >= se) continue;
      const Pair e = unpack_pair(pv[j]);
      a.out_idx[i] = e.idx;
      a.out_val[i] = __uint_as_float(e.bits);
      if (e.idx >= 0 && (int64_t)e.idx < a.n) st_agent_f32(a.residual + e.idx, 0.0f);
    }
  }
}


// ---------------------------------------------------------- k_acc_pass ----
// acc = residual + grad written back to residual; the general path then runs
// on it.  Workgroup 0 clears the general-path state.
struct AccArgs {
  const float* grad;
  float* residual;
  int64_t n;
  int64_t head;  // scalar elements before the aligned part (< 64)
  int64_t nv;    // float4 vectors in the aligned part
  u32* zero_ptr;
  int zero_words;
  u32* hist_rows;  // [gridDim.x][2048]: each workgroup's first-level histogram
};

template <bool VEC>
__global__ __launch_bounds__(kAccThreads) void k_acc_pass(AccArgs a) {
  constexpr int NT = kAccThreads;
  __shared__ u32 s_h[2048];  // first-level histogram of this workgroup's keys (key >> 20)
  const int tid = threadIdx.x;
  for (int i = tid; i < 2048; i += NT) s_h[i] = 0;
  if (blockIdx.x == 0)
    for (int i = tid; i < a.zero_words; i += NT) a.zero_ptr[i] = 0u;
  __syncthreads();
  const float* __restrict__ g = a.grad;
  float* __restrict__ r = a.residual;
  auto add = [&](int64_t i) {
    const float acc = r[i] + g[i];
    r[i] = acc;
    atomicAdd(&s_h[key_of_bits(__float_as_uint(acc)) >> 20], 1u);
  };
  if (VEC) {
    if (blockIdx.x == 0 && tid < a.head) add(tid);
    const v4f* __restrict__ gv = (const v4f*)(g + a.head);
    v4f* __restrict__ rv = (v4f*)(r + a.head);
    // rows of NT float4: row t, then t + G, ...; the next row's loads go out
    // before a row is processed (two rows of a workgroup in flight)
    const int64_t nrows = (a.nv + NT - 1) / NT, G = gridDim.x;
    auto load = [&](int64_t t, v4f& gg, v4f& rr) {
      const int64_t i = t * NT + tid;
      if (t < nrows && i < a.nv) {
        gg = __builtin_nontemporal_load(gv + i);
        rr = __builtin_nontemporal_load(rv + i);
      }
    };
    auto process = [&](int64_t t, const v4f& gg, const v4f& rr) {
      const int64_t i = t * NT + tid;
      if (i < a.nv) {
        const v4f acc = rr + gg;
        __builtin_nontemporal_store(acc, rv + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) atomicAdd(&s_h[key_of_bits(__float_as_uint(acc[q])) >> 20], 1u);
      }
    };
    v4f ga, ra, gb, rb;
    int64_t t = blockIdx.x;
    load(t, ga, ra);
    load(t + G, gb, rb);
    for (; t < nrows; t += 2 * G) {
      process(t, ga, ra);
      load(t + 2 * G, ga, ra);
      if (t + G >= nrows) break;
      process(t + G, gb, rb);
      load(t + 3 * G, gb, rb);
    }
    if (blockIdx.x == gridDim.x - 1)
      for (int64_t i = a.head + 4 * a.nv + tid; i < a.n; i += NT) add(i);
  } else {
    for (int64_t i = (int64_t)blockIdx.x * NT + tid; i < a.n; i += (int64_t)gridDim.x * NT) add(i);
  }
  __syncthreads();
  for (int i = tid; i < 2048; i += NT) a.hist_rows[(size_t)blockIdx.x * 2048 + i] = s_h[i];
}

// ------------------------------------------------------------- k_guess ----
// Guess of the first-level bin that holds the k-th key, from a sample of
// chunks of 256 consecutive entries (one float4 per lane) spread over the
// 16-byte aligned part of the vector.  The guessed bin is the highest one
// whose bins and those above it hold at least c_req sample entries, c_req
// being the expected sample count above the k-th key plus six standard
// deviations of its Poisson noise: the whole vector then holds at least k
// entries in those bins except with negligible probability.  A guess whose
// bins would hold more than s_max sample entries (more candidates than the
// regions can take) is dropped.  For the bucketed ranking (rk_tab set) the
// last workgroup also builds the bucket table.  The guess shapes only how
// much work the later passes do; whether it held is checked against exact
// counts.
struct GuessArgs {
  const v4f* grad;      // the aligned parts (grad + head, residual + head)
  const v4f* residual;
  int64_t chunks, stride;  // chunk c covers float4 [c * stride, c * stride + 64); stride >= 64
  u32 c_req, s_max;
  StepCtl* ctl;
  HeaderHist* hh;
  // bucketed ranking (rk_tab set): the bucket table, the bucket totals (left
  // zero here) and the sample entries one bucket should hold
  u32* rk_tab;
  u32* rk_tot;
  float rk_samples;
};

__global__ __launch_bounds__(kGuessThreads) void k_guess(GuessArgs a) {
  constexpr int NT = kGuessThreads, NW = NT / kWave;
  __shared__ u32 s_h[2048];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_last, s_pick, s_kept;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  for (int i = tid; i < 2048; i += NT) s_h[i] = 0;
  __syncthreads();
  const int64_t W = (int64_t)gridDim.x * NW;
  const int64_t c0 = (int64_t)blockIdx.x * NW + w;
  v4f gq[kGuessUnroll], rq[kGuessUnroll];
#pragma unroll
  for (int u = 0; u < kGuessUnroll; ++u) {
    const int64_t c = c0 + u * W;
    if (c < a.chunks) {
      const int64_t i = c * a.stride + lane;
      gq[u] = __builtin_nontemporal_load(a.grad + i);
      rq[u] = __builtin_nontemporal_load(a.residual + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kGuessUnroll; ++u)
    if (c0 + u * W < a.chunks) {
      const v4f acc = rq[u] + gq[u];
#pragma unroll
      for (int q = 0; q < 4; ++q) atomicAdd(&s_h[key_of(acc[q]) >> 20], 1u);
    }
  __syncthreads();
  StepCtl* ctl = a.ctl;
  for (int i = tid; i < 2048; i += NT)
    if (s_h[i]) add_agent_relaxed(&a.hh->hist[i], s_h[i]);
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_acqrel(&a.hh->done, 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  // last workgroup: every other one has added its histogram (read coalesced
  // into LDS: strided device-scope loads would each fetch a line for a few
  // words)
  static_assert(NT * 2 == 2048, "two bins per thread");
  for (int i = tid; i < 2048; i += NT) s_h[i] = ld_agent(&a.hh->hist[i]);
  if (tid == 0) {
    s_pick = 0u;           // no bin reaches c_req: every bin ...
    s_kept = 0xFFFFFFFFu;  // ... and every sample entry kept
  }
  __syncthreads();
  const int hi = 2047 - 2 * tid;  // this thread's bins, from the top: hi, hi - 1
  const u32 h1 = s_h[hi], h0 = s_h[hi - 1];
  u32 tot;
  const u32 above = block_exclusive_sum<NT>(h1 + h0, s_scan, tot);
  if (above < a.c_req && above + h1 + h0 >= a.c_req) {
    // the pick, and the sample entries in the bins at or above it
    const bool top = above + h1 >= a.c_req;
    s_pick = top ? (u32)hi : (u32)(hi - 1);
    s_kept = top ? above + h1 : above + h1 + h0;
  }
  __syncthreads();
  const u32 pick = s_pick, kept = s_kept == 0xFFFFFFFFu ? tot : s_kept;
  if (a.rk_tab) {
    // The bucketed ranking's buckets, numbered from the top: bin j >= pick is
    // cut into s_j equal sub-ranges of its 2^20 keys, s_j the sample entries
    // of the bin over those one bucket should hold, rounded up; a bin without
    // sample entries joins the bucket just above it (bucket 0 for the top
    // bins).  rk_tab[j] = first bucket of bin j << 16 | s_j.  More than
    // kRkBuckets buckets: twice the entries per bucket, again.
    float per = a.rk_samples;
    auto cut = [&](u32& s1, u32& s0) {
      s1 = (u32)hi >= pick && h1 ? (u32)ceilf((float)h1 / per) : 0u;
      s0 = (u32)(hi - 1) >= pick && h0 ? (u32)ceilf((float)h0 / per) : 0u;
    };
    u32 s1, s0, nb;
    cut(s1, s0);
    u32 base = block_exclusive_sum<NT>(s1 + s0, s_scan, nb);
    if (nb > (u32)kRkBuckets) {  // (the same in every thread)
      for (int tries = 1; tries < 12 && nb > (u32)kRkBuckets; ++tries) {
        per *= 2.0f;
        cut(s1, s0);
        nb = block_sum<NT>(s1 + s0, s_scan);
      }
      base = block_exclusive_sum<NT>(s1 + s0, s_scan, nb);
    }
    a.rk_tab[hi] = base << 16 | s1;
    a.rk_tab[hi - 1] = (base + s1) << 16 | s0;
    for (int i = tid; i < kRkBuckets; i += NT) a.rk_tot[i] = 0u;
    if (tid == 0) {
      ctl->rk_count = nb <= (u32)kRkBuckets ? std::max(nb, 1u) : 0u;
      ctl->rk_ok = 0u;
      ctl->rk_ovf = 0u;
    }
  }
  // the histogram left zero (coalesced, after the workgroup's last barrier)
  for (int i = tid; i < 2048; i += NT) st_agent(&a.hh->hist[i], 0u);
  if (tid == 0) {
    st_agent(&ctl->guide_bin, kept <= a.s_max ? pick : kNoGuide);
    st_agent(&ctl->guide_ovf, 0u);
    st_agent(&ctl->acc_ticket, 0u);
    st_agent(&a.hh->done, 0u);
  }
}

// ------------------------------------------------------- k_acc_guided ----
// The accumulate pass of the standalone general path, given the guessed bin:
// acc = residual + grad written back to residual and the first-level
// histogram of each workgroup, as k_acc_pass does (rows of NT float4, two in
// flight), and the candidates -- every entry of the bins >= the guessed bin
// -- copied into one region per workgroup, in no particular order: a wave
// reserves room for a row's candidates with one LDS atomic and places them by
// a DPP scan over its lanes, so waves never wait for each other.  k_general
// ranks them by (key desc, index asc) itself.
//
// Rows go out in pairs.  With DYN true (long vectors) workgroup b takes
// pair b and then the pairs a ticket hands out (G + the ticket's count), one
// pair ahead: the workgroups then stay on one short stretch of memory however
// their speeds differ, where a fixed deal lets the slower ones fall behind and
// finish last.  With DYN false the first nstatic pairs of each workgroup are
// dealt (b, b + G, ...) and only the last few come from the ticket, which
// then evens out the workgroups' finish (the dies' speeds differ by several
// percent) without queueing on its atomic.
//
// With BKT (the bucketed ranking) the candidates are staged in LDS instead
// (the same wave-wise placement) and, at the end, written to the
// workgroup's own region grouped by bucket (k_guess's table: a bin's entries
// split into equal key sub-ranges), with each bucket's place and count in
// the region; the counts are added into the buckets' totals.  More
// candidates than the stage holds flag the overflow.
struct GuidedArgs {
  const float* grad;
  float* residual;
  int64_t n;
  int64_t head;  // scalar entries before the aligned part (< 64)
  int64_t nv;    // float4 vectors in the aligned part
  u32* zero_ptr;
  int zero_words;
  u32* hist_rows;      // [gridDim.x][2048]
  const StepCtl* ctl;  // guide_bin
  u32* guide_ovf;      // set when a region overflowed
  u32* guide_cnt;      // [gridDim.x] candidates each workgroup found (above cap: its region overflowed)
  u64* cand;           // workgroup b's region: cand + b * cap
  u32 cap;
  u32* ticket;         // zero at the start
  int64_t nstatic;     // row pairs each workgroup is dealt before it takes them from the ticket (>= 1)
  // BKT
  const u32* rk_tab;   // [2048] first bucket of bin j << 16 | its buckets
  const u32* rk_count; // buckets
  u32* rk_cnt;         // [bucket][gridDim.x] place in the region << 16 | entries
  u32* rk_tot;         // [bucket] entries over all workgroups (zero on entry)
  u64* rk_reg;         // [gridDim.x][kRkStage] packed pairs, grouped by bucket
  u32* rk_ovf;
  u32 rk_cap;          // candidates staged at most (kRkStage; less to test)
};

// Bucket of a candidate key under the bucketed ranking's table (k_guess).
__device__ __forceinline__ u32 rk_bucket(const u32* tab, u32 key) {
  const u32 t = tab[key >> 20], base = t >> 16, sj = t & 0xFFFFu;
  return sj ? base + (u32)(((u64)(0xFFFFFu - (key & 0xFFFFFu)) * sj) >> 20) : (base ? base - 1u : 0u);
}

template <bool DYN, bool BKT>
__global__ __launch_bounds__(kAccThreads) void k_acc_guided(GuidedArgs a) {
  constexpr int NT = kAccThreads;
  __shared__ u32 s_h[2048];
  __shared__ u32 s_tab[BKT ? 2048 : 1];
  __shared__ u32 s_bc[BKT ? kRkBuckets : 1];
  __shared__ u64 s_stage[BKT ? kRkStage : 1];
  __shared__ u32 s_scan[BKT ? kAccThreads / kWave + 1 : 1];
  __shared__ u32 s_cnt;
  __shared__ int64_t s_next;
  const int tid = threadIdx.x, lane = lane_id();
  for (int i = tid; i < 2048; i += NT) s_h[i] = 0;
  if (tid == 0) s_cnt = 0;
  if (blockIdx.x == 0)
    for (int i = tid; i < a.zero_words; i += NT) a.zero_ptr[i] = 0u;
  const u32 gbin = a.ctl->guide_bin;
  const u32 nbk = BKT ? *a.rk_count : 0u;
  const bool guide = gbin != kNoGuide && (!BKT || nbk > 0);  // the same in every thread
  if (BKT) {
    for (int i = tid; i < 2048; i += NT) s_tab[i] = a.rk_tab[i];
    for (int i = tid; i < kRkBuckets; i += NT) s_bc[i] = 0u;
  }
  const int64_t nrows = (a.nv + NT - 1) / NT, npairs = (nrows + 1) / 2, G = gridDim.x;
  // Row pair j of this workgroup: b + j G while j < nstatic, then the next
  // one the ticket hands out (pairs nstatic G, nstatic G + 1, ...), so the
  // workgroups that stream faster take more of the last pairs.  Thread 0
  // fetches one pair ahead.
  const int64_t S = a.nstatic;
  int64_t jn = 1, nn = 0;  // thread 0: the next pair's number j, and the pair after the next one
  auto fetch = [&]() -> int64_t {
    const int64_t j = jn++;
    return j < S ? (int64_t)blockIdx.x + j * G : S * G + (int64_t)add_agent_relaxed(a.ticket, 1u);
  };
  if (tid == 0) {
    s_next = fetch();
    nn = fetch();
  }
  __syncthreads();
  u64* const reg = a.cand + (size_t)blockIdx.x * a.cap;
  // this lane's kept entries i0 + j (bit j of m4) go to the region (BKT: to
  // their bucket's slots); every lane of the wave calls it
  auto place = [&](u32 m4, int64_t i0, const u32* bq) {
    const u32 c = (u32)__popc(m4);
    if (ballot(c != 0u) == 0u) return;
    const u32 incl = wave_inclusive_sum(c);
    u32 base = 0;
    if (lane == kWave - 1) base = atomicAdd(&s_cnt, incl);
    u32 pos = __builtin_amdgcn_readlane(base, kWave - 1) + incl - c;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((m4 >> j) & 1u) {
        const u64 pv = pack_pair(Pair{(int32_t)(i0 + j), bq[j]});
        if (BKT) {
          if (pos < a.rk_cap) s_stage[pos] = pv;
        } else if (pos < a.cap) {
          reg[pos] = pv;
        }
        ++pos;
      }
  };
  float* __restrict__ r = a.residual;
  const float* __restrict__ g = a.grad;
  auto scalar = [&](int64_t i, bool in) {  // entry i if `in`; every lane of the wave calls it
    u32 m = 0, bq[4] = {0u, 0u, 0u, 0u};
    if (in) {
      const float acc = r[i] + g[i];
      r[i] = acc;
      bq[0] = __float_as_uint(acc);
      const u32 bin = key_of_bits(bq[0]) >> 20;
      if (!BKT) atomicAdd(&s_h[bin], 1u);
      m = guide && bin >= gbin ? 1u : 0u;
    }
    if (guide) place(m, i, bq);
  };
  if (blockIdx.x == 0 && tid < kWave) scalar(tid, tid < a.head);
  const v4f* __restrict__ gv = (const v4f*)(g + a.head);
  v4f* __restrict__ rv = (v4f*)(r + a.head);
  auto load = [&](int64_t t, v4f& gg, v4f& rr) {
    const int64_t i = t * NT + tid;
    if (t < nrows && i < a.nv) {
      gg = __builtin_nontemporal_load(gv + i);
      rr = __builtin_nontemporal_load(rv + i);
    }
  };
  // a row's candidates are placed after the loads of the row two ahead
  // are out, so the LDS atomic of the placement does not hold them back
  auto process = [&](int64_t t, const v4f& gg, const v4f& rr, u32& m4, u32* bq) {
    const int64_t i = t * NT + tid;
    m4 = 0;
    if (t < nrows && i < a.nv) {
      const v4f acc = rr + gg;
      // (written through at device scope with the streaming hint: stores
      // that allocate in the caches leave the next call a residual's worth
      // of dirty lines to write back, which costs more than the ranking's
      // scattered +0 stores gain from them, and the write-through ones also
      // leave this launch's end less to write back than the hint alone;
      // the aligned part starts on a 256-byte boundary, so a wave's stores
      // cover whole lines)
      st_agent_v4_nt(rv + t * NT, (u32)NT * 16u, (u32)tid * 16u, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bq[e] = __float_as_uint(acc[e]);
        const u32 bin = key_of_bits(bq[e]) >> 20;
        if (!BKT) atomicAdd(&s_h[bin], 1u);
        m4 |= (guide && bin >= gbin ? 1u : 0u) << e;
      }
    }
  };
  // unit u: rows 2u and 2u + 1
  auto row0 = [&](int64_t u) { return 2 * u; };
  auto row1 = [&](int64_t u) { return 2 * u + 1; };
  const int64_t nunits = npairs;
  v4f ga, ra, gb, rb;
  u32 m4, bq[4] = {0u, 0u, 0u, 0u};
  int64_t u = blockIdx.x;  // this unit
  int64_t un = s_next;     // the next one
  load(row0(u), ga, ra);
  load(row1(u), gb, rb);
  while (u < nunits) {
    process(row0(u), ga, ra, m4, bq);
    load(row0(un), ga, ra);
    if (guide) place(m4, a.head + 4 * (row0(u) * NT + tid), bq);
    process(row1(u), gb, rb, m4, bq);
    load(row1(un), gb, rb);
    if (guide) place(m4, a.head + 4 * (row1(u) * NT + tid), bq);
    u = un;
    __syncthreads();  // every thread has read s_next
    if (tid == 0) {
      s_next = nn;
      if (nn < npairs) nn = fetch();
    }
    __syncthreads();
    un = s_next;
  }
  if (blockIdx.x == gridDim.x - 1 && tid < kWave) {
    const int64_t i = a.head + 4 * a.nv + tid;
    scalar(i, i < a.n);
  }
  __syncthreads();
  // (the first-level histogram rows are k_general's; the bucketed ranking's
  // fallback reads acc itself)
  if (!BKT)
    for (int i = tid; i < 2048; i += NT) a.hist_rows[(size_t)blockIdx.x * 2048 + i] = s_h[i];
  if (BKT) {
    // the staged candidates to the region, grouped by bucket
    const u32 ns = s_cnt;
    if (ns > a.rk_cap) {
      if (tid == 0) atomicOr(a.rk_ovf, 1u);
    } else if (guide) {
      for (u32 i = tid; i < ns; i += NT) atomicAdd(&s_bc[rk_bucket(s_tab, key_of_bits((u32)(s_stage[i] >> 32)))], 1u);
      __syncthreads();
      static_assert(kRkBuckets == NT, "one bucket per thread");
      const u32 c = (u32)tid < nbk ? s_bc[tid] : 0u;
      u32 all;
      const u32 off = block_exclusive_sum<NT>(c, s_scan, all);
      if ((u32)tid < nbk) {
        a.rk_cnt[(size_t)tid * gridDim.x + blockIdx.x] = off << 16 | c;
        if (c) (void)add_agent_relaxed(&a.rk_tot[tid], c);
        s_bc[tid] = off;  // now the bucket's next place
      }
      __syncthreads();
      u64* const rg = a.rk_reg + (size_t)blockIdx.x * kRkStage;
      for (u32 i = tid; i < ns; i += NT) {
        const u64 pv = s_stage[i];
        rg[atomicAdd(&s_bc[rk_bucket(s_tab, key_of_bits((u32)(pv >> 32)))], 1u)] = pv;
      }
    }
  } else if (tid == 0) {
    const u32 cnt = s_cnt;
    a.guide_cnt[blockIdx.x] = cnt;
    if (cnt > a.cap) atomicOr(a.guide_ovf, 1u);
  }
}

// ------------------------------------------------------------- k_rank ----
// The bucketed ranking: workgroup w orders buckets w, w + G, ...  Every
// workgroup reads the bucket totals and decides alike whether the route
// held: no accumulate workgroup's stage overflowed, the buckets hold at least
// k entries (then every entry at or above the k-th key is among them, the
// guessed bin being at or below the k-th key's bin) and none holds more than
// one workgroup orders.  Then bucket b's entries take the places after those
// of the buckets above it: the workgroup gathers them from every accumulate
// workgroup's region, orders them by (key desc, index asc) and emits the
// ones whose place is below k, setting their residual to +0.  When the route
// did not hold, the general path selects from acc in the same launch (every
// workgroup of the grid is resident; the ranking's LDS holds its tables).
struct RankArgs {
  StepCtl* ctl;        // rk_count, rk_ovf; rk_ok is set when the route held
  const u32* tot;      // [bucket]
  const u32* cnt;      // [bucket][G1] place << 16 | entries
  const u64* reg;      // [G1][kRkStage]
  u32 G1;
  int64_t k;
  int32_t* out_idx;
  float* out_val;
  float* residual;
  GenArgs gen;         // the general path's (bar.nwg: this grid, at most kMaxGenWG)
};

__global__ __launch_bounds__(kRankThreads) void k_rank(RankArgs a) {
  __shared__ RankLds s;
  __shared__ u32 s_pre[kRkBuckets];
  __shared__ u32 s_max, s_item;
  const int tid = threadIdx.x;
  const u32 B = a.ctl->rk_count;
  const u32 v = (u32)tid < B ? a.tot[tid] : 0u;
  if (tid == 0) s_max = 0u;
  u32 sum;
  s_pre[tid] = block_exclusive_sum<kRankThreads>(v, s.scan, sum);
  const u32 mx = wave_max(v);
  if (lane_id() == 0) atomicMax(&s_max, mx);
  __syncthreads();
  const bool ok = B > 0 && a.ctl->rk_ovf == 0u && (int64_t)sum >= a.k && s_max <= (u32)kRankList;
  if (blockIdx.x == 0 && tid == 0) {
    if (ok) a.ctl->rk_ok = 1u;
    atomicAdd(ok ? &a.ctl->rk_used : &a.ctl->rk_missed, 1u);
  }
  if (!ok) {
    // (the same verdict in every workgroup, so all of them take part)
    static_assert(general_lds_words<kRankThreads, 8>() * sizeof(u32) <= sizeof(s.list), "the tables fit the list");
    general_path<kRankThreads, 4, true, 8, false, true>(a.gen, (u32*)s.list);
    return;
  }
  // Work items, bucket after bucket: a bucket of more than kRkPart entries
  // is shared by several workgroups (at most kRkMaxParts), each of which
  // gathers and orders the whole bucket but emits only its share of it, so
  // that one large bucket does not leave its workgroup storing long after
  // the others.  Thread b holds bucket b's items [ip, ip + parts).  Items
  // it = blockIdx.x, + gridDim.x, ...
  const u32 parts = (u32)tid < B ? std::min<u32>(kRkMaxParts, std::max<u32>(1u, (v + kRkPart - 1) / kRkPart)) : 0u;
  u32 nitems;
  const u32 ip = block_exclusive_sum<kRankThreads>(parts, s.scan, nitems);
  for (u32 it = blockIdx.x; it < nitems; it += gridDim.x) {
    if (ip <= it && it < ip + parts) s_item = (u32)tid << 8 | (it - ip) << 4 | parts;
    __syncthreads();
    const u32 b = s_item >> 8, part = (s_item >> 4) & 15u, np = s_item & 15u;
    const u32 start = s_pre[b];
    if ((int64_t)start >= a.k) break;  // (so does every later item)
    const u32 nb = a.tot[b];
    const u32 kk = (u32)std::min<int64_t>(nb, a.k - start);
    // bucket b's entries from the accumulate workgroups' regions (thread w:
    // those of workgroup w), in any order: the ordering needs none
    const u32 oc = (u32)tid < a.G1 ? a.cnt[(size_t)b * a.G1 + tid] : 0u;
    const u32 c = oc & 0xFFFFu;
    u32 tot;
    const u32 at = block_exclusive_sum<kRankThreads>(c, s.scan, tot);
    const u64* sl = a.reg + (size_t)tid * kRkStage + (oc >> 16);
    for (u32 e0 = 0; e0 < c; e0 += 8) {
      u64 e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = e0 + j < c ? sl[e0 + j] : 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (e0 + j < c) s.list[at + e0 + j] = e[j];
    }
    __syncthreads();
    rank_emit(s, nb, kk, a.residual, a.out_idx + start, a.out_val + start, part, np);
    __syncthreads();  // s and s_item are reused by the next item
  }
}

__global__ __launch_bounds__(kGenThreads) void k_general(GenArgs a) { general_path<kGenThreads, 16, true, 9, true>(a); }

// ------------------------------------------------------------- k_small ----
// Small vectors (n <= 2^18, k <= 256) in one launch with no grid barrier,
// up to 64 of them (the segments of one vector, layer by layer) per launch.
// Workgroup b belongs to the last segment whose first workgroup is <= b and
// takes that segment's entries [8192 b', 8192 (b'+1)) (b' = b minus the
// segment's first workgroup): acc = residual + grad, written back at device
// scope, keys kept in LDS; it selects its own top min(k, len) by a
// three-level radix select in LDS and writes them, in index order, to its
// candidate list.  The segment's last workgroup to arrive selects the top k
// of its lists (in workgroup order, so in index order: ties go to the lower
// index as everywhere), sorts them by (key desc, index asc) and emits them.
// Any entry of the segment's top k is in its own workgroup's top k.  With
// k = 0 a segment only writes acc.
struct SmallSeg {
  int64_t start;  // first entry (from grad / residual)
  u32 len;        // entries, <= kSmallMaxN
  u32 k;          // <= min(kSmallMaxK, len)
  u32 out_off;    // its pairs start at out_idx + out_off; indices relative to `start`
  u32 wg0;        // its first workgroup
};
struct SmallArgs {
  const float* grad;
  float* residual;
  int32_t* out_idx;
  float* out_val;
  u32* done;  // [nseg] arrival counters, zero on entry, left zero
  u64* cand;  // [gridDim.x][kSmallMaxK]
  int nseg;
  SmallSeg seg[kSmallMaxSeg];
};

__global__ __launch_bounds__(kSmallThreads) void k_small(SmallArgs a) {
  constexpr int NT = kSmallThreads, NW = NT / kWave, EPT = kSmallPer / NT;
  constexpr int MAXC = (int)(kSmallMaxN / kSmallPer * kSmallMaxK);  // candidates at most
  __shared__ u32 s_bits[kSmallPer];
  __shared__ u64 s_cand[MAXC];
  __shared__ u64 s_sel[kSmallMaxK];
  __shared__ u32 s_hist[2048];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_found[4];
  __shared__ u32 s_wc[2][NW][2];
  __shared__ u32 s_last;
  const int tid = threadIdx.x;
  const u32 b = blockIdx.x;
  int sg = 0;  // this workgroup's segment (the same in every thread)
  for (int q = 1; q < a.nseg; ++q)
    if (a.seg[q].wg0 <= b) sg = q;
  const SmallSeg S = a.seg[sg];
  const u32 bl = b - S.wg0;                          // workgroup within the segment
  const u32 G = (S.len + kSmallPer - 1) / kSmallPer;  // the segment's workgroups
  const u32 cb = bl * kSmallPer;                     // relative to the segment
  const u32 len = std::min<u32>(kSmallPer, S.len - cb);
  const u32 kk = std::min<u32>(S.k, len);
  const float* __restrict__ g = a.grad + S.start;
  float* __restrict__ res = a.residual + S.start;
  {
    float gq[EPT], rq[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const u32 i = (u32)(j * NT + tid);
      const u32 e = cb + (i < len ? i : 0u);
      gq[j] = g[e];
      rq[j] = res[e];
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const u32 i = (u32)(j * NT + tid);
      if (i < len) {
        const float acc = rq[j] + gq[j];
        st_agent_f32(res + cb + i, acc);
        s_bits[i] = __float_as_uint(acc);
      }
    }
  }
  if (S.k == 0) return;
  __syncthreads();
  u32 t_lo, t_eq, r;
  lds_select<NT>([&](u32 i) { return key_of_bits(s_bits[i]); }, len, kk, s_hist, s_scan, s_found, t_lo, t_eq, r);
  u64* const mine = a.cand + (size_t)b * kSmallMaxK;
  lds_compact<NT, EPT>([&](u32 i) { return pack_pair(Pair{(int32_t)(cb + i), s_bits[i]}); }, len, t_lo, t_eq, r, s_wc,
                       [&](u32 pos, u64 pv) { st_agent64(mine + pos, pv); });
  wait_all_memory();  // acc and the list have completed at device scope
  __syncthreads();
  if (tid == 0) s_last = add_agent_acqrel(&a.done[sg], 1u) == G - 1u ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  if (tid < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  // every list of the segment but its last holds k entries
  const u32 k = S.k;
  const u32 M = (G - 1) * k + std::min<u32>(k, S.len - (G - 1) * kSmallPer);
  const u64* const lists = a.cand + (size_t)S.wg0 * kSmallMaxK;
  for (u32 q = tid; q < M; q += NT) s_cand[q] = ld_agent64(lists + (size_t)(q / k) * kSmallMaxK + q % k);
  __syncthreads();
  lds_select<NT>([&](u32 i) { return key_of_bits((u32)(s_cand[i] >> 32)); }, M, k, s_hist, s_scan, s_found, t_lo, t_eq,
                 r);
  for (int i = tid; i < kSmallMaxK; i += NT) s_sel[i] = pack_pair(pair_sentinel());
  __syncthreads();
  lds_compact<NT, MAXC / NT>([&](u32 i) { return s_cand[i]; }, M, t_lo, t_eq, r, s_wc,
                             [&](u32 pos, u64 pv) { s_sel[pos] = pv; });
  __syncthreads();
  // bitonic sort of the (at most 256) selected by (key desc, index asc);
  // the padding sorts last
  for (u32 k2 = 2; k2 <= (u32)kSmallMaxK; k2 <<= 1)
    for (u32 jj = k2 >> 1; jj > 0; jj >>= 1) {
      if (tid < kSmallMaxK / 2) {
        const u32 t2 = (u32)tid, i = 2 * t2 - (t2 & (jj - 1)), l = i + jj;
        const u64 pi = s_sel[i], pl = s_sel[l];
        const bool up = (i & k2) == 0;
        if ((pair_rank(unpack_pair(pi)) > pair_rank(unpack_pair(pl))) == up) {
          s_sel[i] = pl;
          s_sel[l] = pi;
        }
      }
      __syncthreads();
    }
  int32_t* const oi = a.out_idx + S.out_off;
  float* const ov = a.out_val + S.out_off;
  for (u32 i = tid; i < k; i += NT) {
    const Pair e = unpack_pair(s_sel[i]);
    oi[i] = e.idx;
    ov[i] = __uint_as_float(e.bits);
    st_agent_f32(res + e.idx, 0.0f);
  }
  if (tid == 0) st_agent(&a.done[sg], 0u);
}

// ------------------------------------------------------------- k_step ----
struct StepArgs {
  const float* grad;
  float* residual;
  int64_t n, k;
  int64_t head, nv;  // aligned mode: head scalars, then nv float4 (from residual + head)
  int vec;           // 0: scalar mode (grad and residual differ in 16-byte alignment)
  int32_t* out_idx;
  float* out_val;
  int64_t chunks, stride;        // sample chunk c covers [c * stride, c * stride + 64)
  u32 c_target, bucket_samples;  // plan: sample ranks of T_guess and of the bucket edges
  u32 pub_want;                  // sample keys each workgroup publishes at least
  u32 loc_q16;                   // T_loc: rank fraction of the local sample, in 1/65536
  u32 break_plan;                // test hook: publish a plan that cannot hold
  u32 loc_mode;                  // test hook: 1 = T_loc above every key, 2 = T_loc = 0
  u32 region_cap;                // candidates one workgroup may publish (no limit; less to test)
  u32 slot_log;                  // each workgroup has S = 2^slot_log slots per bucket
  StepCtl* ctl;
  u32* pub;      // [kMaxStepBlocks][kPubCap] keys, then [kMaxStepBlocks] count | floor << 16
  u16* cnt_t;    // [kMaxBuckets][kMaxStepBlocks] workgroup b's candidates of bucket j at j * 256 + b
  u64* slots;    // [kMaxBuckets][G][S] candidates (packed pairs): bucket j's first S of workgroup b
  u64* ovf;      // [kMaxStepBlocks][kOvfCap] the rest of workgroup b's candidates, by bucket
  u32* gstate;   // the general path's state, cleared by workgroup 0
  int gstate_words;
  GenArgs gen;   // the exact path on this grid
};


// bucket of a candidate key: #{j < nb : lo[j] > key}, at most nb - 1
__device__ __forceinline__ int bucket_of(u32 key, const u32* lo, int nb) {
  int l = 0, h = nb;
  while (l < h) {
    const int mid = (l + h) >> 1;
    if (lo[mid] > key) l = mid + 1;
    else h = mid;
  }
  return l < nb ? l : nb - 1;
}

// Keeps (idx, bits) in the workgroup's list (its acc is in residual
// already); a full list is marked incomplete.
__device__ __forceinline__ void list_keep(Pair* s_list, u32* s_nlist, u32* s_ovf, int64_t idx, u32 bits) {
  const u32 pos = atomicAdd(s_nlist, 1u);
  if (pos < (u32)kListCap) s_list[pos] = Pair{(int32_t)idx, bits};
  else *s_ovf = 1u;
}

// Publishes a plan (all threads of workgroup 0): the words with device-scope
// stores, then the flag once they have all completed (a streaming workgroup
// that sees the flag must read this plan and no older one).
__device__ __forceinline__ void publish_plan(StepCtl* ctl, StepSet* cs, u32 valid, u32 tg, u32 nb, const u32* lo) {
  const int tid = threadIdx.x;
  if (tid < kMaxBuckets) st_agent(&ctl->plan.lo[tid], lo[tid]);
  if (tid == kMaxBuckets) st_agent(&ctl->plan.t_guess, tg);
  if (tid == kMaxBuckets + 1) st_agent(&ctl->plan.nbuckets, nb);
  if (tid == kMaxBuckets + 2) st_agent(&ctl->plan.valid, valid);
  wait_all_memory();
  __syncthreads();
  if (tid == 0) flag_set(cs->plan_flag, 1u);
}

// Workgroup 0: the published sample keys -> plan.
//   T_guess = the c_target-th largest sample key; bucket edge j = the
//   (j+1)*bucket_samples-th largest.  A 12-bit histogram of the keys gives
//   b_T, the bin of the c_target-th key, and a radix select inside that bin
//   (10 + 9 more bits) gives T_guess itself.  The keys >= T_guess -- about
//   c_target of them; error feedback piles entries up just below the last
//   threshold, so the bin b_T itself can be large -- are then ranked exactly
//   (a counting sort by sub-range of the key, then counting inside each).  This
//   is exact when b_T lies at or above every workgroup's floor (all bins
//   from the highest floor up were published in full); otherwise the keys
//   are interpolated inside their bins.  The plan is a guess either way.
__device__ __forceinline__ void step_plan(const StepArgs& a, u32 par, u32* s_raw, u32* s_scan) {
  constexpr int NT = kStepThreads;
  constexpr int NW = kStepWaves;
  constexpr int per = kHistBins / NT;  // 4 bins per thread, top first
  constexpr int kTopCap = 4096;        // keys of bins >= b_T ranked exactly
  constexpr u32 kNoKey = 0xFFFFFFFFu;
  u32* s_h = s_raw;                    // [kHistBins] histogram, then suffix sums
  u32* s_keys = s_raw + kHistBins;     // [kPlanCap] the published keys
  u32* s_top = s_keys + kPlanCap;      // [kTopCap] keys of bins >= b_T
  static_assert(kHistBins + kPlanCap + kTopCap <= kRawWords, "LDS");
  __shared__ u32 s_off[kMaxStepBlocks + 1];
  __shared__ u32 s_tkey[kMaxBuckets + 1];  // [0] T_guess, [1+j] edge j
  __shared__ u32 s_lo[kMaxBuckets];
  __shared__ u32 s_maxfloor, s_bT, s_ok, s_ntop, s_kmax;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int G = gridDim.x;
  StepCtl* ctl = a.ctl;
  StepSet* cs = &ctl->set[par];
  if (tid == 0) {
    s_ok = phase_wait(&cs->samp_all, G, &ctl->err) ? 1u : 0u;
    // every workgroup has read the parity (its arrival used it): the next
    // launch takes the other set, cleared at this launch's start
    st_agent(&ctl->parity, par ^ 1u);
    s_maxfloor = 0;
    s_kmax = 0;
    s_bT = 0xFFFFFFFFu;
    s_ntop = 0;
  }
  for (int i = tid; i < kHistBins; i += NT) s_h[i] = 0;
  __syncthreads();
  u32 c = 0;
  if (tid < G) {  // a workgroup that left keys out is complete from floor + 1 up
    const u32 v = ld_agent(&a.pub[kPlanCap + tid]);
    c = v & 0xFFFFu;
    atomicMax(&s_maxfloor, (v >> 16) + (c > (u32)kPubCap ? 1u : 0u));
  }
  u32 K;
  const u32 off = block_exclusive_sum<NT>(std::min(c, (u32)kPubCap), s_scan, K);
  if (tid < G) s_off[tid] = off;
  if (tid == 0) s_off[G] = K;
  __syncthreads();
  {  // wave w loads workgroups w, w + 16, ...: all its loads in flight at once
    constexpr int kPerWave = kMaxStepBlocks / NW;
    u32 v[kPerWave];
#pragma unroll
    for (int r = 0; r < kPerWave; ++r) {
      const int wg = w + r * NW;
      const u32 cnt = wg < G ? s_off[wg + 1] - s_off[wg] : 0u;
      v[r] = (u32)lane < cnt ? ld_agent(&a.pub[wg * kPubCap + lane]) : kNoKey;
    }
#pragma unroll
    for (int r = 0; r < kPerWave; ++r) {
      const int wg = w + r * NW;
      const u32 cnt = wg < G ? s_off[wg + 1] - s_off[wg] : 0u;
      if ((u32)lane < cnt) {
        s_keys[s_off[wg] + lane] = v[r];
        atomicAdd(&s_h[v[r] >> kHistShift], 1u);
      }
    }
  }
  __syncthreads();
  const int hi = kHistBins - per * tid;  // thread t owns bins [hi - per, hi)
  {
    u32 own = 0;
#pragma unroll
    for (int q = 1; q <= per; ++q) own += s_h[hi - q];
    u32 total;
    u32 run = block_exclusive_sum<NT>(own, s_scan, total);
#pragma unroll
    for (int q = 1; q <= per; ++q) {  // inclusive suffix sums cum[b] = sum_{b' >= b} h[b']
      const u32 h = s_h[hi - q];
      if (run < a.c_target && run + h >= a.c_target) s_bT = (u32)(hi - q);  // b_T: where cum reaches c_target
      run += h;
      s_h[hi - q] = run;
    }
  }
  __syncthreads();
  const int bT = (int)s_bT;
  u32 nb = (a.c_target + a.bucket_samples - 1) / a.bucket_samples;
  nb = std::max(1u, std::min(nb, (u32)kMaxBuckets));
  if (bT < 0 || !s_ok || a.break_plan) {
    // no plan (T_guess above every key), or the test hook's plan: a
    // threshold no finite key reaches
    const u32 tg = a.break_plan ? 0x7FFFFFFFu : 0xFFFFFFFFu;
    if (tid < kMaxBuckets) s_lo[tid] = tid == 0 ? tg : 0u;
    __syncthreads();
    publish_plan(ctl, cs, a.break_plan ? 1u : 0u, tg, 1u, s_lo);
    return;
  }
  const int ntarget = (int)nb;  // wanted ranks: [0] c_target, [j] j * bucket_samples for 1 <= j < nb
  auto rank_of = [&](int t) -> u32 { return t == 0 ? a.c_target : (u32)t * a.bucket_samples; };
  if (tid < ntarget) {  // default: interpolation inside the bin of each wanted rank
    const u32 q = rank_of(tid);
    int lo = 0, hi2 = kHistBins - 1;  // largest b with cum[b] >= q
    while (lo < hi2) {
      const int mid = (lo + hi2 + 1) >> 1;
      if (s_h[mid] >= q) lo = mid;
      else hi2 = mid - 1;
    }
    const u32 above_b = lo + 1 < kHistBins ? s_h[lo + 1] : 0u;
    const u32 h = s_h[lo] - above_b;  // >= q - above_b >= 1
    const u32 f = q - above_b;
    const u32 offk = (u32)((((u64)f << kHistShift) + h - 1) / h);  // in [1, 2^19]
    s_tkey[tid] = (((u32)lo + 1u) << kHistShift) - offk;
  }
  const bool exact = bT >= (int)s_maxfloor;
  if (exact) {
    // T_guess exactly: radix select of the c_target-th key inside bin b_T
    // over key bits [18:9] then [8:0] (their histograms go in s_top).
    const u32 cum_above_bT = bT + 1 < kHistBins ? s_h[bT + 1] : 0u;
    u32 need = a.c_target - cum_above_bT;  // 1-based rank inside bin b_T
    u32 prefix = (u32)bT;                    // the key's bits chosen so far
    int shift = kHistShift;
    const int widths[2] = {10, 9};
    for (int L = 0; L < 2; ++L) {
      const int wd = widths[L];
      const int nbins = 1 << wd;
      shift -= wd;
      __syncthreads();  // s_h (or the last level's histogram) is still being read
      for (int i = tid; i < nbins; i += NT) s_top[i] = 0;
      __syncthreads();
      for (u32 i = tid; i < K; i += NT) {
        const u32 key = s_keys[i];
        if ((key >> (shift + wd)) == prefix) atomicAdd(&s_top[(key >> shift) & (nbins - 1)], 1u);
      }
      __syncthreads();
      // suffix counts from the top bin down; thread t owns bin nbins - 1 - t
      const u32 hcount = tid < nbins ? s_top[nbins - 1 - tid] : 0u;
      u32 tot;
      const u32 above = block_exclusive_sum<NT>(hcount, s_scan, tot);
      if (tid < nbins && above < need && above + hcount >= need) {
        s_bT = (u32)(nbins - 1 - tid);  // the digit (s_bT is free again)
        s_ntop = above;
      }
      __syncthreads();
      prefix = (prefix << wd) | s_bT;
      need -= s_ntop;
    }
    const u32 tg = prefix;  // the c_target-th largest sample key
    __syncthreads();
    // the keys >= T_guess (c_target of them, more with ties), ranked exactly
    if (tid == 0) {
      s_tkey[0] = tg;
      s_ntop = 0;
    }
    __syncthreads();
    for (u32 i = tid; i < K; i += NT) {
      const u32 key = s_keys[i];
      if (key >= tg) {
        const u32 pos = atomicAdd(&s_ntop, 1u);
        if (pos < (u32)kTopCap) s_top[pos] = key;
      }
    }
    __syncthreads();
    // Rank them: counting sort by 2048 sub-ranges of key - T_guess from the
    // top (the key bits are close to log2 |value|, so the sub-ranges stay
    // small even for a long tail), then each key's place inside its sub-range
    // by counting.  The key of 1-based rank q lands in s_final[q - 1].
    const u32 ntop = std::min(s_ntop, (u32)kTopCap);
    u32* s_sub = s_h;                  // [kSubBins] counts, then fill cursors
    u32* s_subo = s_h + kSubBins;      // [kSubBins] starts
    u32* s_sorted = s_keys;            // [ntop] grouped by sub-range
    u32* s_final = s_keys + kTopCap;   // [ntop] in rank order
    static_assert(2 * kSubBins <= kHistBins && 2 * kTopCap <= kPlanCap, "LDS");
    {
      u32 km = 0;
      for (u32 i = tid; i < ntop; i += NT) km = std::max(km, s_top[i]);
      km = wave_max(km);
      if (lane == 0) atomicMax(&s_kmax, km);
      for (int i = tid; i < kSubBins; i += NT) s_sub[i] = 0;
    }
    __syncthreads();
    const u32 span = s_kmax - tg + 1u;  // >= 1
    const int sbits = span <= 1 ? 0 : 32 - __clz(span - 1);
    const int ssh = sbits > 11 ? sbits - 11 : 0;  // kSubBins = 2^11
    auto sub_of = [&](u32 x) -> u32 {
      const u32 d = (x - tg) >> ssh;
      return (u32)(kSubBins - 1) - (d < (u32)kSubBins ? d : (u32)(kSubBins - 1));
    };
    for (u32 i = tid; i < ntop; i += NT) atomicAdd(&s_sub[sub_of(s_top[i])], 1u);
    __syncthreads();
    {
      constexpr int sper = kSubBins / NT;
      u32 v[sper], own = 0;
#pragma unroll
      for (int q2 = 0; q2 < sper; ++q2) {
        v[q2] = s_sub[tid * sper + q2];
        own += v[q2];
      }
      u32 tot;
      u32 ex = block_exclusive_sum<NT>(own, s_scan, tot);
#pragma unroll
      for (int q2 = 0; q2 < sper; ++q2) {
        s_subo[tid * sper + q2] = ex;
        s_sub[tid * sper + q2] = ex;  // becomes the fill cursor
        ex += v[q2];
      }
    }
    __syncthreads();
    for (u32 i = tid; i < ntop; i += NT) {
      const u32 x = s_top[i];
      s_sorted[atomicAdd(&s_sub[sub_of(x)], 1u)] = x;
    }
    __syncthreads();
    for (u32 i = tid; i < ntop; i += NT) {
      const u32 x = s_sorted[i];
      const u32 sb = sub_of(x);
      const u32 s0 = s_subo[sb], s1 = s_sub[sb];  // the cursor ended at the range's end
      u32 r = 0;
      for (u32 t = s0; t < s1; ++t) {
        const u32 y = s_sorted[t];
        r += (y > x) | ((y == x) & (t < i));
      }
      s_final[s0 + r] = x;
    }
    __syncthreads();
    if (tid >= 1 && tid < (int)nb) {
      const u32 q = (u32)tid * a.bucket_samples;  // 1-based rank of edge tid - 1
      if (q <= ntop) s_tkey[tid] = s_final[q - 1];
    }
  }
  __syncthreads();  // every wanted key is in s_tkey
  if (w == 0) {  // monotone edges, each at least T_guess (a prefix minimum over lanes)
    const u32 tg = s_tkey[0];
    const u32 j = (u32)lane;
    const u32 x = j + 1 < nb ? std::max(s_tkey[1 + j], tg) : 0xFFFFFFFFu;
    const u32 v = wave_inclusive_min(x);  // every lane takes part
    s_lo[j] = j + 1 < nb ? v : (j + 1 == nb ? tg : 0u);
  }
  __syncthreads();
  publish_plan(ctl, cs, 1u, s_lo[nb - 1], nb, s_lo);
}

// Finisher f (workgroups 0..63), once every workgroup has published: the
// verdict, then bucket f.  Returns false when the plan did not hold.
__device__ __forceinline__ bool step_finish(const StepArgs& a, u32 par, u32* s_raw, u32* s_scan) {
  constexpr int NT = kStepThreads;
  constexpr int kSlotIters = kSlotTotal / NT;            // slots per thread
  Pair* s_a = (Pair*)s_raw;                      // [kFinishCap] the bucket, as gathered
  Pair* s_b = (Pair*)(s_raw + 2 * kFinishCap);   // [kFinishCap] grouped by key sub-range
  u32* s_sub_cnt = s_raw + 4 * kFinishCap;       // [kSubBins]
  u32* s_sub_off = s_sub_cnt + kSubBins;         // [kSubBins]
  static_assert(4 * kFinishCap + 2 * kSubBins <= kRawWords, "LDS");
  __shared__ u32 s_plo[kMaxBuckets];
  __shared__ u32 s_phdr[3];
  __shared__ u32 s_kmin, s_kmax, s_ok, s_wait, s_seen, s_n;
  __shared__ int64_t s_start, s_mytot;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int f = blockIdx.x;
  const int G = gridDim.x;
  const u32 slog = a.slot_log, S = 1u << slog;
  StepCtl* ctl = a.ctl;
  StepSet* cs = &ctl->set[par];
  __syncthreads();  // s_raw changes role
  // The plan is final before any workgroup publishes (every streaming
  // workgroup waited for it), so it is read while waiting for the others.
  if (tid < kMaxBuckets) s_plo[tid] = ld_agent(&ctl->plan.lo[tid]);
  if (tid == kMaxBuckets) s_phdr[0] = ld_agent(&ctl->plan.t_guess);
  if (tid == kMaxBuckets + 1) s_phdr[1] = ld_agent(&ctl->plan.nbuckets);
  if (tid == kMaxBuckets + 2) s_phdr[2] = ld_agent(&ctl->plan.valid);
  for (int i = tid; i < kSubBins; i += NT) s_sub_cnt[i] = 0;
  if (tid == 0) {
    s_wait = phase_wait(&cs->main_all, G, &ctl->err) ? 1u : 0u;  // every streaming workgroup published
    s_kmin = 0xFFFFFFFFu;
    s_kmax = 0;
    s_n = 0;
  }
  __syncthreads();
  // One round trip: bucket f's slots and the count of each slot's workgroup
  // (the bucket's column of the count table), the bucket totals (wave 0,
  // lane j = bucket j) and the failure word.
  const int nslots = G << slog;  // <= kSlotTotal
  u64 sv[kSlotIters];
  u32 cw[kSlotIters];
  u32 tj = 0;
  {
    const u64* mine = a.slots + ((int64_t)f << slog) * G;
    const u16* col = a.cnt_t + f * kMaxStepBlocks;
    // Unconditional loads (an index out of range reads row 1's first slot
    // instead), so all of them are in flight at once: a load under a branch
    // would be waited for on its own.
#pragma unroll
    for (int q = 0; q < kSlotIters; ++q) {
      const int i = tid + q * NT;
      const int ic = i < nslots && (i >> slog) >= 1 ? i : (int)S;  // row 0 (the planner) publishes nothing
      sv[q] = ld_agent64(mine + ic);
      cw[q] = ld_agent_u16(col + (ic >> slog));
    }
#pragma unroll
    for (int q = 0; q < kSlotIters; ++q) {
      const int i = tid + q * NT;
      if (!(i < nslots && (i >> slog) >= 1)) cw[q] = 0u;
    }
    if (w == 0) tj = ld_agent(&cs->tot[lane]);
    if (tid == 0) s_seen = ld_agent((const u32*)&cs->bad.v);
  }
  // Gather the slots below their workgroup's count into s_a, in any order
  // (the sort below ranks by key and index): one LDS append per wave and
  // slot round.  Entries past a workgroup's S slots (rare) come from its
  // overflow area, which holds its candidates past S grouped by bucket.
  u32 gmin = 0xFFFFFFFFu, gmax = 0;
  auto take_entry = [&](const Pair& p, u32 at) {
    if (at < (u32)kFinishCap) s_a[at] = p;
    const u32 kk = key_of_bits(p.bits);
    gmin = std::min(gmin, kk);
    gmax = std::max(gmax, kk);
  };
#pragma unroll
  for (int q = 0; q < kSlotIters; ++q) {
    const int i = tid + q * NT;
    const bool keep = ((u32)i & (S - 1u)) < cw[q];
    const u64 bm = ballot(keep);
    if (bm == 0) continue;  // wave-uniform
    u32 base = 0;
    if (lane == 0) base = atomicAdd(&s_n, (u32)__popcll(bm));
    base = __builtin_amdgcn_readfirstlane(base);
    if (keep) take_entry(unpack_pair(sv[q]), base + lanes_below(bm));
  }
#pragma unroll
  for (int q = 0; q < kSlotIters; ++q) {
    const int i = tid + q * NT;
    if (((u32)i & (S - 1u)) == 0u && cw[q] > S) {  // workgroup i >> slog overflowed in bucket f
      const int row = i >> slog;
      u32 off = 0;  // its overflow entries of buckets 0..f-1
      for (int j = 0; j < f; ++j) {
        const u32 cj = ld_agent_u16(a.cnt_t + j * kMaxStepBlocks + row);
        off += cj > S ? cj - S : 0u;
      }
      const u64* src = a.ovf + (int64_t)row * kOvfCap + off;
      const u32 extra = cw[q] - S;
      const u32 at = atomicAdd(&s_n, extra);
      for (u32 e = 0; e < extra; ++e) take_entry(unpack_pair(ld_agent64(src + e)), at + e);
    }
  }
  gmin = wave_min(gmin);
  gmax = wave_max(gmax);
  if (lane == 0) {
    atomicMin(&s_kmin, gmin);
    atomicMax(&s_kmax, gmax);
  }
  // verdict and bucket offsets in wave 0 (lane j = bucket j)
  if (w == 0) {
    const u32 t = tj;
    const u32 nb = s_phdr[1];
    bool plan_ok = s_wait && s_phdr[2] == 1u && nb >= 1 && nb <= (u32)kMaxBuckets;
    if (plan_ok) {
      const u32 lo_i = s_plo[lane];
      const u32 lo_prev = lane > 0 ? s_plo[lane - 1] : 0xFFFFFFFFu;
      const bool mono = (u32)lane >= nb || lane == 0 || lo_i <= lo_prev;
      plan_ok = ballot(!mono) == 0 && s_plo[nb - 1] == s_phdr[0];
    }
    const u32 x = wave_inclusive_sum(t);  // over buckets 0..63
    const int64_t start = (int64_t)(x - t), all = __builtin_amdgcn_readlane(x, kWave - 1);
    const bool live = (u32)lane < nb;
    const bool bad = (!live && t != 0) || (live && start < a.k && t > (u32)kFinishCap);
    const u32 seen = s_seen;
    const bool any_bad = ballot(bad) != 0;
    const bool valid = plan_ok && seen == 0 && !any_bad && all >= a.k;
    if (lane == f) {
      s_start = start;
      s_mytot = live ? t : 0;
    }
    if (lane == 0) {
      s_ok = valid ? 1u : 0u;
      if (f == 0) {
        ctl->verdict = valid ? 1u : 0u;
        if (!valid) {
          ctl->fallbacks += 1u;
          ctl->why |= (plan_ok ? 0u : kWhyPlan) | seen | (any_bad ? kWhyBucket : 0u) | (all >= a.k ? 0u : kWhyFew);
        }
        flag_set(cs->verdict_flag, valid ? 1u : 2u);
      }
    }
  }
  __syncthreads();
  if (!s_ok) return false;
  const int64_t mystart = s_start, mytot = s_mytot;
  if (mytot == 0 || mystart >= a.k) return true;  // no rank below k here
  if ((int64_t)s_n != mytot) {  // the column and the total disagree: cannot happen
    if (tid == 0) atomicOr(&ctl->err, 1u << 2);
    return true;
  }
  const int m = (int)mytot;  // <= kFinishCap (verdict)
  // Split [kmin, kmax] into kSubBins equal key sub-ranges numbered from the
  // top and group the entries by sub-range (counting sort); inside a
  // sub-range an entry's place is the number of its entries that rank before
  // it (ranks are unique: indices differ).
  const u32 kmin = s_kmin;
  const u32 span = s_kmax - kmin + 1u;
  const int bits = span <= 1 ? 0 : 32 - __clz(span - 1);
  const int sh = bits > 11 ? bits - 11 : 0;  // kSubBins = 2^11
  auto sub_of = [&](const Pair& e) -> u32 {
    const u32 d = (key_of_bits(e.bits) - kmin) >> sh;
    return (u32)(kSubBins - 1) - (d < (u32)kSubBins ? d : (u32)(kSubBins - 1));
  };
  for (int i = tid; i < m; i += NT) atomicAdd(&s_sub_cnt[sub_of(s_a[i])], 1u);
  __syncthreads();
  {
    constexpr int per = kSubBins / NT;
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
    const Pair e = s_a[i];
    s_b[atomicAdd(&s_sub_cnt[sub_of(e)], 1u)] = e;
  }
  __syncthreads();
  // Entries of rank < k: to the output, and their residual to +0.  Every
  // streaming workgroup's acc stores completed at device scope before it
  // arrived, so these stores land after them.  The +0 stores carry only the
  // non-temporal hint, not device scope: nothing in this launch reads these
  // entries again (a failed verdict never gets here), the launch's end makes
  // them visible, and one partial line each need not go through to memory
  // at once (0.8 us a step at n = 25.6M, k = 25,600).
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
      __builtin_nontemporal_store(0.0f, a.residual + e.idx);
    }
  }
  return true;
}

__global__ __launch_bounds__(kStepThreads) void k_step(StepArgs a) {
  constexpr int NT = kStepThreads;
  constexpr int NW = kStepWaves;
  constexpr int per = kHistBins / NT;
  constexpr u32 kNoKey = 0xFFFFFFFFu;
  __shared__ __align__(16) u32 s_raw[kRawWords];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_lo[kMaxBuckets];
  __shared__ u32 s_bcnt[kMaxBuckets];
  __shared__ u32 s_boff[kMaxBuckets];
  __shared__ u32 s_hdr[3];
  __shared__ u32 s_nlist, s_ovf, s_npub, s_novf, s_flag, s_floor, s_tlocbin;
  __shared__ bool s_plan_in_lds;
  __shared__ u32 s_par;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int M = G - 1, m = b - 1;  // streaming workgroups and this one's rank among them
  StepCtl* ctl = a.ctl;
  // the counter set of this launch: issued first, so waiting for it does not
  // wait for the data loads behind it
  u32 par_ld = 0;
  if (tid == 0) par_ld = ld_agent(&ctl->parity);
  float* __restrict__ r = a.residual;
  const float* __restrict__ g = a.grad;
  const v4f* __restrict__ gv = (const v4f*)(g + a.head);
  v4f* __restrict__ rv = (v4f*)(r + a.head);
  // Aligned mode streams rows of NT float4: streaming workgroup m takes rows
  // m, m + M, ... (measured against run-time hand-out of the last quarter of
  // the rows in pairs: 66.1 against 66.4 us at n = 25.6M; the hand-out's
  // barrier per pair costs more than the balance gains).  Scalar mode streams
  // tiles of NT * 8 elements, tile t to workgroup t % M.
  constexpr int64_t TE = (int64_t)NT * 8;
  const int64_t nrows = a.vec ? (a.nv + NT - 1) / NT : (a.n + TE - 1) / TE;

  // sample loads first, then the first two rows, all in flight together
  float sg[kSampleRounds], sr[kSampleRounds];
  bool sok[kSampleRounds];
#pragma unroll
  for (int j = 0; j < kSampleRounds; ++j) {  // chunk c belongs to workgroup c % G
    const int64_t c = b + (int64_t)G * (w + NW * j);
    const int64_t i = c * a.stride + lane;
    sok[j] = c < a.chunks && i < a.n;
    sg[j] = sok[j] ? g[i] : 0.0f;
    sr[j] = sok[j] ? r[i] : 0.0f;
  }
  // two row buffers: A = row m, B = row m + M (loads issued now)
  v4f ag, ar, bg, br;
  auto load_row = [&](int64_t t, v4f& gg, v4f& rr) {
    const int64_t i = t * NT + tid;
    if (i < a.nv) {
      gg = __builtin_nontemporal_load(gv + i);
      rr = __builtin_nontemporal_load(rv + i);
    }
  };
  if (b > 0 && a.vec) {
    if ((int64_t)m < nrows) load_row(m, ag, ar);
    if ((int64_t)m + M < nrows) load_row((int64_t)m + M, bg, br);
  }

  // ---------------- sample ----------------
  // The sample keys stay past the list and staging areas (the list fills
  // while they are published); the histogram is done with before streaming.
  u32* s_keys = s_raw + 2 * kListCap + 2 * kOvfCap;  // [kSampleKeyCap]
  static_assert(2 * kListCap + 2 * kOvfCap + kSampleKeyCap <= kRawWords, "LDS");
  {
    u32* s_h = s_raw;  // [kHistBins]
    for (int i = tid; i < kHistBins; i += NT) s_h[i] = 0;
    for (int i = tid; i < kSampleKeyCap; i += NT) s_keys[i] = kNoKey;
    if (tid < kMaxBuckets) s_bcnt[tid] = 0;
    if (tid == 0) {
      s_floor = 0;
      s_tlocbin = 0;
      s_nlist = 0;
      s_ovf = 0;
      s_npub = 0;
      s_novf = 0;
      s_plan_in_lds = false;
    }
    if (b == 0)  // the exact path's state starts at zero
      for (int i = tid; i < a.gstate_words; i += NT) st_agent(&a.gstate[i], 0u);
    if (tid == 0) s_par = par_ld & 1u;
    __syncthreads();
    if (b == 0) {  // the other counter set is cleared for the next launch
      StepSet* other = &ctl->set[s_par ^ 1u];
      if (tid < kSetCounters) st_agent64(&((Counter*)other)[tid].v, 0u);
      if (tid >= 128 && tid < 128 + kMaxBuckets) st_agent(&other->tot[tid - 128], 0u);
    }
#pragma unroll
    for (int j = 0; j < kSampleRounds; ++j) {
      if (!sok[j]) continue;
      const u32 key = key_of(sr[j] + sg[j]);
      atomicAdd(&s_h[key >> kHistShift], 1u);
      s_keys[(j * NW + w) * kWave + lane] = key;
    }
    __syncthreads();
    {  // floor bin (at least pub_want keys at or above it) and T_loc's bin
      const int hi = kHistBins - per * tid;
      u32 own = 0;
#pragma unroll
      for (int q = 1; q <= per; ++q) own += s_h[hi - q];
      u32 total;
      u32 run = block_exclusive_sum<NT>(own, s_scan, total);
      const u32 rl = std::max(1u, (u32)(((u64)total * a.loc_q16) >> 16));
#pragma unroll
      for (int q = 1; q <= per; ++q) {
        const u32 h = s_h[hi - q];
        if (run < a.pub_want && run + h >= a.pub_want) s_floor = (u32)(hi - q);
        if (run < rl && run + h >= rl) s_tlocbin = (u32)(hi - q);
        run += h;
      }
    }
    __syncthreads();
  }
  const u32 par = s_par;
  StepSet* const cs = &ctl->set[par];
  // Publishes the sample keys of bins >= floor and their count: first those
  // of bins above the floor bin (fewer than pub_want, so they always fit),
  // then those of the floor bin while kPubCap allows.  A workgroup that had
  // to leave some out is complete from floor + 1 up.  Nothing waits for
  // these stores: workgroup 0 reads them only after every workgroup has
  // arrived, microseconds later, and the keys only shape the plan, which is a
  // guess -- whatever it holds, the verdict makes the result exact.
  auto sample_publish = [&]() {
    const u32 floor_bin = s_floor;
    u32 mine = 0;  // keys above the floor bin (low half) and in it (high half)
    for (int i = tid; i < kSampleKeyCap; i += NT) {
      const u32 key = s_keys[i];
      if (key != kNoKey) {
        const u32 bin = key >> kHistShift;
        mine += bin > floor_bin ? 1u : bin == floor_bin ? 0x10000u : 0u;
      }
    }
    u32 count;
    const u32 pos = block_exclusive_sum<NT>(mine, s_scan, count);
    const u32 above = count & 0xFFFFu;
    u32 pos_hi = pos & 0xFFFFu, pos_eq = above + (pos >> 16);
    u32* mine_pub = a.pub + (int64_t)b * kPubCap;
    for (int i = tid; i < kSampleKeyCap; i += NT) {
      const u32 key = s_keys[i];
      if (key == kNoKey) continue;
      const u32 bin = key >> kHistShift;
      if (bin > floor_bin) {
        st_agent(&mine_pub[pos_hi++], key);
      } else if (bin == floor_bin) {
        if (pos_eq < (u32)kPubCap) st_agent(&mine_pub[pos_eq], key);
        ++pos_eq;
      }
    }
    const u32 total = above + (count >> 16);
    if (tid == 0) st_agent(&a.pub[kPlanCap + b], std::min(total, 0xFFFFu) | (floor_bin << 16));
  };
  // Arrival at the sample phase, once this workgroup's published values are
  // all in (waiting for the atomics' returned values).
  auto sample_arrive = [&]() {
    __syncthreads();
    if (tid == 0) phase_arrive(cs->samp_grp, &cs->samp_all, G);
  };

  if (b == 0) {
    // ---------------- plan ----------------
    sample_publish();
    sample_arrive();
    step_plan(a, par, s_raw, s_scan);
    __syncthreads();
    if (tid == 0) phase_arrive(cs->main_grp, &cs->main_all, G);
  } else {
    // ---------------- stream ----------------
    const u32 tloc = a.loc_mode == 1u ? 0x7FFFFFFFu : a.loc_mode == 2u ? 0u : s_tlocbin << kHistShift;
    Pair* s_list = (Pair*)s_raw;                      // [kListCap]
    Pair* s_ovl = (Pair*)(s_raw + 2 * kListCap);     // [kOvfCap] candidates past their nslot slots
    u32* s_ovt = s_raw + 2 * kListCap + 2 * kOvfCap;  // [kOvfCap] bucket << 16 | place past nslot
    static_assert(2 * kListCap + 3 * kOvfCap <= kRawWords, "LDS");
    const u32 slog = a.slot_log, nslot = 1u << slog;  // slots per bucket and workgroup
    // Files list entries [lo, hi) under a plan: a candidate (key >= T_guess)
    // takes the next place of its bucket; places below nslot are this
    // workgroup's slots of the bucket and are written at once, the rest wait
    // here for the overflow area.
    auto file_range = [&](u32 lo, u32 hi, u32 tg, int nb) {
      u64* const slots = a.slots;
      for (u32 i = lo + tid; i < hi; i += NT) {
        const Pair e = s_list[i];
        const u32 key = key_of_bits(e.bits);
        if (key < tg) continue;
        const int j = bucket_of(key, s_lo, nb);
        const u32 pos = atomicAdd(&s_bcnt[j], 1u);
        if (pos < nslot) {
          st_agent64(slots + (((int64_t)j * G + b) << slog) + pos, pack_pair(e));
        } else {
          const u32 q = atomicAdd(&s_novf, 1u);
          if (q < (u32)kOvfCap) {
            s_ovl[q] = e;
            s_ovt[q] = ((u32)j << 16) | (pos - nslot);
          }
        }
      }
    };
    auto keep_scalar = [&](int64_t i) {
      const float acc = r[i] + g[i];
      st_agent_f32(r + i, acc);
      const u32 bits = __float_as_uint(acc);
      if (key_of_bits(bits) >= tloc) list_keep(s_list, &s_nlist, &s_ovf, i, bits);
    };
    // One row: acc goes to residual as a float4 (whole lines, never partial);
    // entries with key >= T_loc are appended to the list at offsets from one
    // wave-wide prefix sum and one LDS atomic per wave.
    auto vec_row = [&](int64_t t, const v4f gg, const v4f rr) {
      const int64_t row0 = (int64_t)__builtin_amdgcn_readfirstlane((int)t) * NT;  // t is the same in every lane
      const int64_t i = row0 + tid;
      const bool in = i < a.nv;
      const v4f acc = rr + gg;
      if (in) st_agent_v4_nt(rv + row0, (u32)std::min<int64_t>(NT, a.nv - row0) * 16u, (u32)tid * 16u, acc);
      const u32 b0 = __float_as_uint(acc.x), b1 = __float_as_uint(acc.y);
      const u32 b2 = __float_as_uint(acc.z), b3 = __float_as_uint(acc.w);
      const u32 mk = in ? ((u32)(key_of_bits(b0) >= tloc) | ((u32)(key_of_bits(b1) >= tloc) << 1) |
                           ((u32)(key_of_bits(b2) >= tloc) << 2) | ((u32)(key_of_bits(b3) >= tloc) << 3))
                        : 0u;
      if (ballot(mk != 0) == 0) return;  // wave-uniform
      const u32 cnt = (u32)__popc(mk);
      const u32 incl = wave_inclusive_sum(cnt);
      const u32 total = __builtin_amdgcn_readlane(incl, kWave - 1);
      u32 base = 0;
      if (lane == 0) base = atomicAdd(&s_nlist, total);
      base = __builtin_amdgcn_readfirstlane(base);
      if (mk != 0) {
        u32 pos = base + incl - cnt;
        const int64_t e = a.head + 4 * i;
        const u32 bb[4] = {b0, b1, b2, b3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (mk & (1u << j)) {
            if (pos < (u32)kListCap) s_list[pos] = Pair{(int32_t)(e + j), bb[j]};
            else s_ovf = 1u;  // the list is incomplete
            ++pos;
          }
        }
      }
    };
    if (a.vec) {
      // The plan is usually published while the rows stream: lane 0 of
      // wave 0 polls its flag once per row (the answer is looked at a row
      // later), and once it is seen, wave 0's lanes load the plan (state 1)
      // and write it to LDS a row later (state 2), when the loads are back.
      u32 st0 = 0;  // wave 0: 0 plan not seen, 1 loading, 2 in LDS
      u64 pf = 0;   // lane 0 of wave 0: the flag poll in flight
      u32 pw = 0, ph = 0;
      auto poll_plan = [&]() {  // wave 0, every lane
        if (st0 == 0) {
          u32 seen = 0;
          if (lane == 0) {
            if (pf != 0) seen = 1;
            else pf = ld_agent64(&cs->plan_flag[blockIdx.x & 7].v);
          }
          if (__builtin_amdgcn_readfirstlane(seen)) {
            st0 = 1;
            pw = ld_agent(&ctl->plan.lo[lane]);
            if (lane < 3) ph = ld_agent(lane == 0 ? &ctl->plan.t_guess : lane == 1 ? &ctl->plan.nbuckets : &ctl->plan.valid);
          }
        } else if (st0 == 1) {
          st0 = 2;
          s_lo[lane] = pw;
          if (lane < 3) s_hdr[lane] = ph;
        }
      };
      // rows m, m + M, ...: buffer A holds one, B the next, and the load of
      // the row after goes out before a buffer is processed (two rows of a
      // workgroup in flight: more would cost the memory system)
      if ((int64_t)m < nrows) vec_row(m, ag, ar);
      sample_publish();
      bool arrived = false;
      for (int64_t t = (int64_t)m + M; t < nrows; t += 2 * (int64_t)M) {
        if (t + M < nrows) load_row(t + M, ag, ar);
        vec_row(t, bg, br);
        if (!arrived) {
          sample_arrive();
          arrived = true;
        }
        if (w == 0) poll_plan();
        if (t + M >= nrows) break;
        if (t + 2 * (int64_t)M < nrows) load_row(t + 2 * (int64_t)M, bg, br);
        vec_row(t + M, ag, ar);
        if (w == 0) poll_plan();
      }
      if (!arrived) sample_arrive();
      if (w == 0) {
        if (st0 == 1) {  // loaded during the last row: to LDS
          s_lo[lane] = pw;
          if (lane < 3) s_hdr[lane] = ph;
        }
        if (lane == 0) s_plan_in_lds = st0 >= 1;
      }
      if (m == 0 && tid < a.head) keep_scalar(tid);
      if (m == M - 1)
        for (int64_t i = a.head + 4 * a.nv + tid; i < a.n; i += NT) keep_scalar(i);
    } else {
      sample_publish();
      sample_arrive();
      constexpr int kU = 8;
      for (int64_t t = m; t < nrows; t += M) {
        float gg[kU], rr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t i = t * TE + u * NT + tid;
          if (i < a.n) {
            gg[u] = g[i];
            rr[u] = r[i];
          }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t i = t * TE + u * NT + tid;
          if (i < a.n) {
            const float acc = rr[u] + gg[u];
            st_agent_f32(r + i, acc);
            const u32 bits = __float_as_uint(acc);
            if (key_of_bits(bits) >= tloc) list_keep(s_list, &s_nlist, &s_ovf, i, bits);
          }
        }
      }
    }
    __syncthreads();

    // ---------------- publish ----------------
    if (!s_plan_in_lds) {
      if (tid == 0) s_flag = flag_wait(&cs->plan_flag[blockIdx.x & 7], &ctl->err);
      __syncthreads();
      if (tid < kMaxBuckets) s_lo[tid] = ld_agent(&ctl->plan.lo[tid]);
      if (tid == kMaxBuckets) s_hdr[0] = ld_agent(&ctl->plan.t_guess);
      if (tid == kMaxBuckets + 1) s_hdr[1] = ld_agent(&ctl->plan.nbuckets);
      if (tid == kMaxBuckets + 2) s_hdr[2] = ld_agent(&ctl->plan.valid);
    } else if (tid == 0) {
      s_flag = 1;
    }
    __syncthreads();
    const bool plan_ok = s_flag != 0 && s_hdr[2] == 1u && s_hdr[1] >= 1 && s_hdr[1] <= (u32)kMaxBuckets;
    const u32 tg = plan_ok ? s_hdr[0] : 0xFFFFFFFFu;
    const int nb = plan_ok ? (int)s_hdr[1] : 1;
    u32 fail = s_flag != 0 ? 0u : kWhyWait;
    if ((s_ovf || tloc > tg) && plan_ok) {
      // The list may miss keys >= T_guess (it overflowed, or T_loc lies
      // above T_guess).  This workgroup's rows of residual hold acc; after a
      // fence (so no stale cached line is read) they are re-read for the keys
      // >= T_guess.
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        s_nlist = 0;
        s_ovf = 0;
        s_novf = 0;
        atomicAdd(&ctl->rescans, 1u);
      }
      if (tid < kMaxBuckets) s_bcnt[tid] = 0;
      __syncthreads();
      auto rescan = [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo + tid; i < hi; i += NT) {
          const u32 bits = __float_as_uint(r[i]);
          if (key_of_bits(bits) >= tg) list_keep(s_list, &s_nlist, &s_ovf, i, bits);
        }
      };
      if (a.vec) {
        auto rescan_rows = [&](int64_t t, int64_t nr) {
          rescan(a.head + 4 * t * NT, a.head + 4 * std::min<int64_t>(a.nv, (t + nr) * NT));
        };
        for (int64_t t = m; t < nrows; t += M) rescan_rows(t, 1);
      } else {
        for (int64_t t = m; t < nrows; t += M) rescan(t * TE, std::min<int64_t>(a.n, (t + 1) * TE));
      }
      if (a.vec && m == 0) rescan(0, a.head);
      if (a.vec && m == M - 1) rescan(a.head + 4 * a.nv, a.n);
      __syncthreads();
      if (s_ovf) fail |= kWhyList;  // more keys >= T_guess than the list holds
    }
    const u32 nl = std::min(s_nlist, (u32)kListCap);
    if (!(fail & kWhyList)) file_range(0, nl, tg, nb);
    __syncthreads();
    if (w == 0) {  // candidates, and where each bucket's overflow starts
      const u32 c = s_bcnt[lane];
      const u32 over = c > nslot ? c - nslot : 0u;
      const u32 xo = wave_inclusive_sum(over);
      s_boff[lane] = xo - over;
      const u32 xc = wave_inclusive_sum(c);
      if (lane == kWave - 1) s_npub = xc;
    }
    __syncthreads();
    const u32 C = s_npub, novf = s_novf;
    if (C > a.region_cap || novf > (u32)kOvfCap) fail |= kWhyRegion;
    if (!fail) {
      u64* const dst = a.ovf + (int64_t)b * kOvfCap;
      for (u32 q = tid; q < novf; q += NT) {
        const u32 t = s_ovt[q];
        st_agent64(dst + s_boff[t >> 16] + (t & 0xFFFFu), pack_pair(s_ovl[q]));
      }
      if (tid < kMaxBuckets) {  // this workgroup's count of bucket tid, and the bucket's total
        const u32 c = s_bcnt[tid];
        st_agent_u16(&a.cnt_t[tid * kMaxStepBlocks + b], (u16)c);
        if (c) (void)add_agent_relaxed(&cs->tot[tid], c);
      }
    } else {
      // cannot publish: the plan fails
      if (tid < kMaxBuckets) st_agent_u16(&a.cnt_t[tid * kMaxStepBlocks + b], 0);
      if (tid == 0) or_agent((u32*)&cs->bad.v, fail);
    }
    // Every store of this workgroup -- acc included -- has completed at
    // device scope before it arrives: the finishers read the slots and counts
    // after the last arrival, and after the verdict they zero the selected
    // entries of residual, stores that must land after the acc stores.
    wait_all_memory();
    __syncthreads();
    if (tid == 0) phase_arrive(cs->main_grp, &cs->main_all, G);
  }

  // ---------------- finish ----------------
  u32 verdict;
  if (b < kMaxBuckets) {
    verdict = step_finish(a, par, s_raw, s_scan) ? 1u : 2u;
  } else {
    if (tid == 0) s_flag = flag_wait(&cs->verdict_flag[blockIdx.x & 7], &ctl->err);
    __syncthreads();
    verdict = s_flag;
  }
  if (verdict != 1u) {
    // The plan did not hold: residual holds acc everywhere (every store of
    // it was made at device scope), and the whole grid runs the exact path,
    // which reads it at device scope.
    // rarely taken: one row per tile keeps this copy of the general path small
    // (a larger one costs the fast path registers and time even unused)
    if (grid_sync(a.gen.bar)) general_path<NT, 1, false, 8, false>(a.gen);
  }
}

}  // namespace tgs

// ==================================================================== host ==
using namespace tgs;

namespace {

// Workgroups of `kernel` (NT threads) that fit on the current device at once,
// at most `cap`: resident workgroups per compute unit times the compute units.
// Cached per device (and kernel, through the caller's cache); 0 if unknown.
template <class K>
int resident_capacity(std::atomic<int>* cache, K kernel, int NT, int cap) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load();
  if (v == 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, NT, 0) != hipSuccess) occ = 0;
    v = std::max(0, std::min(cap, occ * device_cu_count()));
    if (v == 0) v = -1;
    cache[dev].store(v);
  }
  return v > 0 ? v : 0;
}

// Workgroups k_step may use: one per compute unit (its LDS allows no more),
// never above kMaxStepBlocks.
int step_capacity() {
  static std::atomic<int> cache[64];
  return resident_capacity(cache, k_step, kStepThreads, kMaxStepBlocks);
}

// Workgroups of k_general, every one resident (grid barriers).
int general_capacity() {
  static std::atomic<int> cache[64];
  return resident_capacity(cache, k_general, kGenThreads, kGenBlocks);
}

// Sampling and sizing of the fast path for (n, k) on G workgroups; false when
// the fast path does not apply.
bool step_params(int64_t n, int64_t k, int G, StepArgs& a) {
  if (k < 1 || n < kFastMinN || G < kMaxBuckets + 1 || G > kMaxStepBlocks) return false;
  const int M = G - 1;
  const double kd = (double)k, nd = (double)n;
  const double tau = std::max(1.4 * kd, kd + 8192.0);  // candidates aimed for
  const double eps = 1.0 - kd / tau;                   // relative slack below tau
  const double need_stat = 25.0 / (eps * eps);         // ~5 sigma of Poisson noise
  const double bucket_elems = std::max(512.0, 1.2 * kd / 56.0);
  if (bucket_elems > kFinishCap / 4) return false;
  const double nb_needed = std::ceil(1.1 * kd / bucket_elems);
  const double c = std::max({need_stat, 8.0 * nb_needed, 64.0});
  const double m = c * nd / tau;  // sample elements
  int64_t chunks = (int64_t)std::ceil(m / kSampleChunk);
  chunks = std::max<int64_t>(chunks, 4 * (int64_t)G);  // every workgroup samples at least 4 chunks
  chunks = std::min<int64_t>(chunks, (int64_t)G * kStepWaves * kSampleRounds);
  chunks = std::min<int64_t>(chunks, n / kSampleChunk);
  if (chunks < 4 * (int64_t)G) return false;
  a.chunks = chunks;
  a.stride = n / chunks;  // >= 64: chunks never overlap
  const double m_real = (double)chunks * kSampleChunk;
  a.c_target = (u32)std::max(1.0, std::ceil(tau * m_real / nd));
  a.bucket_samples = (u32)std::max(1.0, std::ceil(bucket_elems * m_real / nd));
  a.pub_want = 8u * ((a.c_target + G - 1) / G) + 8u;
  if (a.pub_want + 8 > (u32)kPubCap) return false;
  // T_loc: a local-sample quantile with about 1024 (and at least 4x the
  // expected candidate count) of a share's entries above it
  const double share = nd / M;
  const double f_loc = std::min(1.0, std::max(1024.0 / share, 4.0 * tau / nd));
  if (f_loc * share > kListCap / 4 || tau / M > kOvfCap / 4) return false;
  a.loc_q16 = (u32)std::min(65535.0, std::ceil(f_loc * 65536.0));
  return true;
}

}  // namespace

extern "C" size_t tgs_topk_workspace_bytes(int64_t n, int64_t k) {
  if (n < 0 || n > INT32_MAX || k < 0 || k > n) return 0;
  return topk_layout(n, k).total;
}

namespace tgs {

tgs_status topk_check_args(const char* what, const float* grad, const float* residual, int64_t n, int64_t k,
                           const int32_t* out_idx, const float* out_val) {
  if (n < 0 || n > INT32_MAX) return fail(TGS_EINVAL, "%s: n=%lld outside [0, 2^31-1]", what, (long long)n);
  if (k < 0 || k > n) return fail(TGS_EINVAL, "%s: k=%lld outside [0, n=%lld]", what, (long long)k, (long long)n);
  if (n > 0 && (!grad || !residual)) return fail(TGS_EINVAL, "%s: null grad/residual", what);
  if (k > 0 && (!out_idx || !out_val)) return fail(TGS_EINVAL, "%s: null output pointer", what);
  for (const void* p : {(const void*)grad, (const void*)residual, (const void*)out_idx, (const void*)out_val})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "%s: pointer not 4-byte aligned", what);
  const size_t nb4 = (size_t)n * 4, kb4 = (size_t)k * 4;
  if (overlaps(grad, nb4, residual, nb4) || overlaps(grad, nb4, out_idx, kb4) ||
      overlaps(grad, nb4, out_val, kb4) || overlaps(residual, nb4, out_idx, kb4) ||
      overlaps(residual, nb4, out_val, kb4) || overlaps(out_idx, kb4, out_val, kb4))
    return fail(TGS_EINVAL, "%s: overlapping buffers", what);
  return TGS_OK;
}

}  // namespace tgs

extern "C" tgs_status tgs_topk_ef_step(const float* grad, float* residual, int64_t n, int64_t k,
                                       int32_t* out_idx, float* out_val, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  const tgs_status chk = topk_check_args("topk_ef_step", grad, residual, n, k, out_idx, out_val);
  if (chk != TGS_OK) return chk;
  if (!workspace) return fail(TGS_EINVAL, "topk_ef_step: null workspace");
  const TopkLayout L = topk_layout(n, k);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "topk_ef_step: workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (n == 0) return TGS_OK;
  char* ws = (char*)workspace;
  StepCtl* ctl = (StepCtl*)(ws + L.ctl);
  GenState* gs = (GenState*)(ws + L.gstate);

  int path = (int)get_option(TGS_OPT_TOPK_PATH);
  if (path == 14) path = 0;  // (an option of rTop-k's pick)
  const int64_t gopt = get_option(TGS_OPT_MAIN_GRID);
  const bool vec = (((uintptr_t)grad) & 15u) == (((uintptr_t)residual) & 15u);
  // vector mode: up to 63 scalar entries first, so that the float4 part of
  // residual starts on a 256-byte boundary and every wave's store of 64
  // float4 covers whole cache lines (a vector cut at any offset, such as a
  // layer of a layer-wise call, would otherwise store partial lines, which
  // device-scope stores pay for dearly)
  int64_t head = 0, nv = 0;
  if (vec) {
    head = std::min<int64_t>(n, (int64_t)(((256u - (((uintptr_t)residual) & 255u)) & 255u) / 4u));
    nv = (n - head) / 4;
  }

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
  ga.cand = (u64*)(ws + L.cand);
  ga.cand_cap = L.cand_cap;
  ga.cand_ovf = &gs->cand_ovf;
  ga.bar.cnt = &gs->bar_cnt[0][0];
  ga.bar.gen = &gs->bar_gen[0][0];
  ga.bar.abort = &gs->bar_abort;
  ga.bar.err = &ctl->err;

  if (path != 1 && path < 7 && k >= 1 && k <= kSmallMaxK && n <= kSmallMaxN) {
    SmallArgs m{};
    m.grad = grad;
    m.residual = residual;
    m.out_idx = out_idx;
    m.out_val = out_val;
    m.done = ctl->seg_done;
    m.cand = (u64*)(ws + L.small);
    m.nseg = 1;
    m.seg[0] = SmallSeg{0, (u32)n, (u32)k, 0u, 0u};
    hipEvent_t e0, e1;
    take_profile_events(&e0, &e1);
    if (e0) (void)hipEventRecord(e0, stream);
    hipLaunchKernelGGL(k_small, dim3((unsigned)((n + kSmallPer - 1) / kSmallPer)), dim3(kSmallThreads), 0, stream, m);
    if (e1) (void)hipEventRecord(e1, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step: launch failed: %s", hipGetErrorString(e));
    return TGS_OK;
  }

  StepArgs sa{};
  int G = 0;
  if (path != 1 && path < 7) {
    const int cap = step_capacity();
    G = gopt > 0 ? (int)std::min<int64_t>(gopt, cap) : cap;
    if (!step_params(n, k, G, sa)) G = 0;
  }

  hipEvent_t ev0, ev1;
  take_profile_events(&ev0, &ev1);
  if (ev0) (void)hipEventRecord(ev0, stream);
  if (G > 0) {
    sa.grad = grad;
    sa.residual = residual;
    sa.n = n;
    sa.k = k;
    sa.head = head;
    sa.nv = nv;
    sa.vec = vec ? 1 : 0;
    sa.out_idx = out_idx;
    sa.out_val = out_val;
    sa.break_plan = path == 2 ? 1u : 0u;
    sa.loc_mode = path == 3 ? 1u : path == 4 ? 2u : 0u;
    sa.region_cap = path == 5 ? 1u : 0xFFFFFFFFu;
    // S = 2^slot_log slots per (bucket, workgroup), the most that keeps a
    // bucket's G * S slots within kSlotTotal (path 6: one slot, so nearly
    // every candidate goes to the overflow area)
    sa.slot_log = 0;
    while (path != 6 && ((int64_t)G << (sa.slot_log + 1)) <= kSlotTotal) ++sa.slot_log;
    sa.ctl = ctl;
    sa.pub = (u32*)(ws + L.pub);
    sa.cnt_t = (u16*)(ws + L.rcnt);
    sa.slots = (u64*)(ws + L.slots);
    sa.ovf = (u64*)(ws + L.ovf);
    sa.gstate = (u32*)gs;
    sa.gstate_words = (int)(sizeof(GenState) / sizeof(u32));
    sa.gen = ga;
    sa.gen.bar.nwg = (u32)G;
    hipLaunchKernelGGL(k_step, dim3(G), dim3(kStepThreads), 0, stream, sa);
  } else {
    AccArgs aa{};
    aa.grad = grad;
    aa.residual = residual;
    aa.n = n;
    aa.head = head;
    aa.nv = nv;
    aa.zero_ptr = (u32*)gs;
    aa.zero_words = (int)(sizeof(GenState) / sizeof(u32));
    const int64_t units = vec ? nv : n;
    const int64_t per = (int64_t)kAccThreads * (vec ? 2 : 8);
    int G1 = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxAccBlocks, (units + per - 1) / per));
    if (gopt > 0) G1 = (int)std::min<int64_t>(gopt, kMaxAccBlocks);
    aa.hist_rows = (u32*)(ws + L.hist_rows);
    ga.acc_hist = aa.hist_rows;
    ga.acc_rows = (u32)G1;
    int G2 = 0;
    if (k > 0) {
      // every workgroup of k_general must be resident at once (grid barriers)
      G2 = general_capacity();
      if (G2 <= 0) return fail(TGS_EHIP, "topk_ef_step: cannot read the device's resident capacity");
    }
    // The guided accumulate pass copies the candidates out while it streams,
    // so k_general need not read acc again: it takes one region per
    // workgroup of k_general, in index order.
    const bool guided = vec && k > 0 && path != 1 && n >= kGuideMinN && G1 <= G2;
    // the bucketed ranking (the default from kRkMinK on; path 12: a stage of
    // one candidate, so that it overflows; path 13: never)
    const RkSizes rz = rk_sizes(n, k);
    const bool bucketed = guided && L.rk_entries > 0 && (path == 0 || path == 12) && G1 <= rz.G1;
    if (guided) {
      const int64_t want = (int64_t)std::ceil(1024.0 * (double)n / (double)k);  // ~1024 expected above the k-th key
      int64_t chunks = (want + kGuessChunk - 1) / kGuessChunk;
      chunks = std::max<int64_t>(1, std::min<int64_t>({chunks, kGuessMaxChunks, nv / kGuessChunk}));  // <= 1/4 of it
      GuessArgs q{};
      q.grad = (const v4f*)(grad + head);
      q.residual = (const v4f*)(residual + head);
      q.chunks = chunks;
      q.stride = nv / chunks;
      const double f = (double)(chunks * kGuessChunk) / (double)n;
      const double c = (double)k * f;
      q.c_req = path == 7 ? 1u : (u32)std::min(4.0e9, std::ceil(c + 6.0 * std::sqrt(c) + 8.0));
      // the candidate room of all k_general waves, split over the G1
      // accumulate workgroups
      const u32 stride = (u32)((int64_t)G2 * (kGenThreads / kWave) * L.cand_cap / G1);
      const double room = (double)G1 * stride;
      q.s_max = bucketed ? 0xFFFFFFFFu : (u32)std::min(4.0e9, std::floor(0.6 * room * f));
      q.ctl = ctl;
      q.hh = header_hist(workspace);
      if (bucketed) {
        q.rk_tab = (u32*)(ws + L.rk_tab);
        q.rk_tot = (u32*)(ws + L.rk_tot);
        q.rk_samples = (float)std::max(1e-3, f * (double)L.rk_target);
      }
      // one chunk per wave where the workgroups allow: a compute unit
      // fetches only so fast, and the sample's loads are all the work
      const int gq = (int)std::min<int64_t>(kGuessBlocks, (chunks + kGuessThreads / kWave - 1) / (kGuessThreads / kWave));
      hipLaunchKernelGGL(k_guess, dim3(gq), dim3(kGuessThreads), 0, stream, q);
      GuidedArgs g{};
      g.grad = grad;
      g.residual = residual;
      g.n = n;
      g.head = head;
      g.nv = nv;
      g.zero_ptr = aa.zero_ptr;
      g.zero_words = aa.zero_words;
      g.hist_rows = aa.hist_rows;
      g.ctl = ctl;
      g.guide_ovf = &ctl->guide_ovf;
      g.guide_cnt = (u32*)(ws + L.guide_cnt);
      g.cand = ga.cand;
      g.cap = path == 8 ? 1u : stride;
      g.ticket = &ctl->acc_ticket;
      // the ticket's hand-out pays from about 32 rows per workgroup on
      const int64_t rows = (nv + kAccThreads - 1) / kAccThreads;
      const bool dyn = rows >= 32 * (int64_t)G1;
      // A long vector takes every pair after the first from the ticket; a
      // shorter one deals all but about the last two pairs of each
      // workgroup, so the ticket's atomic is rare enough not to queue.
      const int64_t pairs = (rows + 1) / 2;
      g.nstatic = dyn ? 1 : std::max<int64_t>(1, pairs / G1 - 2);
      if (bucketed) {
        g.rk_tab = q.rk_tab;
        g.rk_count = &ctl->rk_count;
        g.rk_cnt = (u32*)(ws + L.rk_cnt);
        g.rk_tot = q.rk_tot;
        g.rk_reg = (u64*)(ws + L.rk_slots);
        g.rk_ovf = &ctl->rk_ovf;
        g.rk_cap = path == 12 ? 1u : (u32)kRkStage;
        if (dyn)
          hipLaunchKernelGGL((k_acc_guided<true, true>), dim3(G1), dim3(kAccThreads), 0, stream, g);
        else
          hipLaunchKernelGGL((k_acc_guided<false, true>), dim3(G1), dim3(kAccThreads), 0, stream, g);
        RankArgs ra{};
        ra.ctl = ctl;
        ra.tot = g.rk_tot;
        ra.cnt = g.rk_cnt;
        ra.reg = g.rk_reg;
        ra.G1 = (u32)G1;
        ra.k = k;
        ra.out_idx = out_idx;
        ra.out_val = out_val;
        ra.residual = residual;
        // one ranking workgroup per compute unit (each holds ~148 KB of LDS),
        // and no more than the general path's tables are sized for
        const int gr = std::max(1, std::min({kRkBuckets, kMaxGenWG, device_cu_count()}));
        ra.gen = ga;
        ra.gen.bar.nwg = (u32)gr;
        hipLaunchKernelGGL(k_rank, dim3(gr), dim3(kRankThreads), 0, stream, ra);
        if (ev1) (void)hipEventRecord(ev1, stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step: launch failed: %s", hipGetErrorString(e));
        return TGS_OK;
      }
      if (dyn)
        hipLaunchKernelGGL((k_acc_guided<true, false>), dim3(G1), dim3(kAccThreads), 0, stream, g);
      else
        hipLaunchKernelGGL((k_acc_guided<false, false>), dim3(G1), dim3(kAccThreads), 0, stream, g);
      ga.guided = 1;
      ga.guide_stride = stride;
      ga.guide_bin = &ctl->guide_bin;
      ga.guide_ovf = &ctl->guide_ovf;
      ga.guide_cnt = g.guide_cnt;
      ga.guide_stats = &ctl->guided_used;
      ga.bkt_cnt = (u32*)(ws + L.bkt_cnt);
      ga.bkt_cur = (u32*)(ws + L.bkt_cur);
      ga.bkt_buf = (u64*)(ws + L.bkt_buf);
    } else if (vec) {
      hipLaunchKernelGGL(k_acc_pass<true>, dim3(G1), dim3(kAccThreads), 0, stream, aa);
    } else {
      hipLaunchKernelGGL(k_acc_pass<false>, dim3(G1), dim3(kAccThreads), 0, stream, aa);
    }
    if (k > 0) {
      ga.bar.nwg = (u32)G2;
      hipLaunchKernelGGL(k_general, dim3(G2), dim3(kGenThreads), 0, stream, ga);
    }
  }
  if (ev1) (void)hipEventRecord(ev1, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

// ======================================================== segmented host ==
namespace {

bool small_segment(int64_t len, int64_t k) { return len <= kSmallMaxN && k <= kSmallMaxK; }

// Checks the segment table; false (with the reason) if it is not valid.
bool segments_valid(int32_t nseg, const int64_t* offsets, const int64_t* ks, const char** why) {
  if (nseg < 0) return *why = "nseg < 0", false;
  if (nseg > 0 && (!offsets || !ks)) return *why = "null offsets/ks", false;
  if (nseg == 0) return true;
  if (offsets[0] != 0) return *why = "offsets[0] != 0", false;
  int64_t ksum = 0;
  for (int32_t s = 0; s < nseg; ++s) {
    const int64_t len = offsets[s + 1] - offsets[s];
    if (len < 0) return *why = "offsets decrease", false;
    if (ks[s] < 0 || ks[s] > len) return *why = "ks[s] outside [0, segment length]", false;
    ksum += ks[s];
  }
  if (offsets[nseg] > INT32_MAX || ksum > INT32_MAX) return *why = "total length or total k above 2^31-1", false;
  return true;
}

// A segment for the batched layer-wise path (grad and residual equally
// aligned modulo 16 bytes, at most 2^23 entries, k <= 4096).
bool mid_segment(int64_t len, int64_t k) {
  u32 a = 0, b = 0, c = 0;
  return len > 0 && mid_plan(len, k, &a, &b, &c);
}

// Workspace: a top-k workspace for the largest segment that may take a step
// of its own (its header also serves the other launches), then the candidate
// lists of the small segments' workgroups, then the batched path's region
// (sized for every batched segment; whether it is used depends on the
// pointers' alignment, so both are provided).
struct SegLayout {
  size_t big, lists, mid, total;
};

SegLayout seg_layout(int32_t nseg, const int64_t* offsets, const int64_t* ks) {
  SegLayout L{};
  L.big = kWorkspaceHeader;
  int64_t wgs = 0, blocks = 0;
  for (int32_t s = 0; s < nseg; ++s) {
    const int64_t len = offsets[s + 1] - offsets[s];
    if (len == 0) continue;
    if (mid_segment(len, ks[s])) blocks += len / 1024 + 2;
    if (small_segment(len, ks[s])) wgs += (len + kSmallPer - 1) / kSmallPer;
    else L.big = std::max(L.big, topk_layout(len, ks[s]).total);
  }
  L.big = align256(L.big);
  L.lists = L.big;
  L.mid = align256(L.lists + sizeof(u64) * (size_t)wgs * kSmallMaxK);
  L.total = L.mid + (blocks ? mid_workspace_bytes(blocks) : 0);
  return L;
}

}  // namespace

extern "C" size_t tgs_topk_segmented_workspace_bytes(int32_t nseg, const int64_t* offsets, const int64_t* ks) {
  const char* why = nullptr;
  if (!segments_valid(nseg, offsets, ks, &why)) return 0;
  return seg_layout(nseg, offsets, ks).total;
}

extern "C" tgs_status tgs_topk_ef_step_segmented(const float* grad, float* residual, int32_t nseg,
                                                 const int64_t* offsets, const int64_t* ks, int32_t* out_idx,
                                                 float* out_val, void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream) {
  const char* why = nullptr;
  if (!segments_valid(nseg, offsets, ks, &why)) return fail(TGS_EINVAL, "topk_ef_step_segmented: %s", why);
  if (!workspace) return fail(TGS_EINVAL, "topk_ef_step_segmented: null workspace");
  if (nseg == 0) return TGS_OK;
  const int64_t n = offsets[nseg];
  int64_t ksum = 0;
  for (int32_t s = 0; s < nseg; ++s) ksum += ks[s];
  if (n > 0 && (!grad || !residual)) return fail(TGS_EINVAL, "topk_ef_step_segmented: null grad/residual");
  if (ksum > 0 && (!out_idx || !out_val)) return fail(TGS_EINVAL, "topk_ef_step_segmented: null output pointer");
  for (const void* p : {(const void*)grad, (const void*)residual, (const void*)out_idx, (const void*)out_val})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "topk_ef_step_segmented: pointer not 4-byte aligned");
  const size_t nb4 = (size_t)n * 4, kb4 = (size_t)ksum * 4;
  if (overlaps(grad, nb4, residual, nb4) || overlaps(grad, nb4, out_idx, kb4) || overlaps(grad, nb4, out_val, kb4) ||
      overlaps(residual, nb4, out_idx, kb4) || overlaps(residual, nb4, out_val, kb4) ||
      overlaps(out_idx, kb4, out_val, kb4))
    return fail(TGS_EINVAL, "topk_ef_step_segmented: overlapping buffers");
  const SegLayout L = seg_layout(nseg, offsets, ks);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "topk_ef_step_segmented: workspace %zu bytes, need %zu", workspace_bytes, L.total);
  char* ws = (char*)workspace;
  StepCtl* ctl = (StepCtl*)ws;
  // grad and residual equally aligned: the segments of at most 2^23 entries
  // with k <= 4096 take the batched path; the others (and every segment
  // otherwise) as below
  const bool vec = (((uintptr_t)grad) & 15u) == (((uintptr_t)residual) & 15u);
  auto batched = [&](int32_t s) {
    const int64_t len = offsets[s + 1] - offsets[s];
    return vec && get_option(TGS_OPT_TOPK_PATH) != 11 && mid_segment(len, ks[s]);
  };
  {
    std::vector<MidSegSpec> mids;
    int64_t ko = 0;
    for (int32_t s = 0; s < nseg; ++s) {
      if (batched(s)) mids.push_back(MidSegSpec{offsets[s], offsets[s + 1] - offsets[s], ks[s], ko});
      ko += ks[s];
    }
    if (!mids.empty()) {
      const tgs_status st =
          mid_launch(grad, residual, out_idx, out_val, (int)mids.size(), mids.data(), &ctl->mid_exact, ctl->seg_done,
                     ws + L.mid, stream);
      if (st != TGS_OK) return st;
    }
  }
  // the small segments, up to kSmallMaxSeg per launch
  SmallArgs m{};
  m.grad = grad;
  m.residual = residual;
  m.out_idx = out_idx;
  m.out_val = out_val;
  m.done = ctl->seg_done;
  u64* lists = (u64*)(ws + L.lists);
  u32 wg = 0;
  auto flush = [&]() {
    if (m.nseg == 0) return;
    m.cand = lists;
    hipLaunchKernelGGL(k_small, dim3(wg), dim3(kSmallThreads), 0, stream, m);
    lists += (size_t)wg * kSmallMaxK;
    m.nseg = 0;
    wg = 0;
  };
  int64_t koff = 0;
  for (int32_t s = 0; s < nseg; ++s) {
    const int64_t len = offsets[s + 1] - offsets[s];
    if (len > 0 && !batched(s) && small_segment(len, ks[s])) {
      m.seg[m.nseg++] = SmallSeg{offsets[s], (u32)len, (u32)ks[s], (u32)koff, wg};
      wg += (u32)((len + kSmallPer - 1) / kSmallPer);
      if (m.nseg == kSmallMaxSeg) flush();
    }
    koff += ks[s];
  }
  flush();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "topk_ef_step_segmented: launch failed: %s", hipGetErrorString(e));
  // the others, one step each on the shared top-k workspace
  koff = 0;
  for (int32_t s = 0; s < nseg; ++s) {
    const int64_t len = offsets[s + 1] - offsets[s];
    if (len > 0 && !batched(s) && !small_segment(len, ks[s])) {
      const tgs_status st = tgs_topk_ef_step(grad + offsets[s], residual + offsets[s], len, ks[s],
                                             ks[s] ? out_idx + koff : nullptr, ks[s] ? out_val + koff : nullptr,
                                             workspace, L.big, stream);
      if (st != TGS_OK) return st;
    }
    koff += ks[s];
  }
  return TGS_OK;
}

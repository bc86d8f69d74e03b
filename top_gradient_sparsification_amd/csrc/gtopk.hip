// gTop-k tournament of P workers' sparse sets on one gfx950 GPU.
//
// Method (nubint review "A Distributed Synchronous SGD Algorithm with Global
// Top-k Sparsification for Low Bandwidth Networks", ABSTRACT and Method): the
// global top-k largest |values| over P workers, found by a tournament of
// O(log P) pairwise rounds; only the indices that survive keep their index
// information, and each worker learns which of its own entries survived.
//
// Every slot is held as k (index, bits) pairs sorted by index, which turns the
// per-round union into a merge:
//   rows     each worker's row copied to its slot, sorted by index (LDS
//            bitonic runs of 2048, then merge-path passes); repeated or
//            out-of-range indices set the device error word.
//   round r  for every slot s with a partner s + 2^r:
//              k_gt_union   merge-path merge of the two slots by index; a
//                           shared index keeps the A entry with value a + b
//                           (one binary32 add) and the B entry becomes a hole;
//              k_gt_select  one workgroup per merge: radix select of the k-th
//                           key over 11/11/9-bit digits, then an ordered
//                           compaction that keeps every key above it and the
//                           lowest-index ties, written back to slot s (for
//                           2k <= 65,536 the merge's keys stay in registers:
//                           k_gt_select_reg).
//   final    slot 0 sorted by (key desc, index asc) with the same run sort and
//            merge passes; the mask binary-searches every input index in the
//            index-sorted slot 0.
#include <algorithm>
#include <climits>
#include <vector>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

constexpr int kRun = 2048;          // LDS-sorted run length
constexpr int kRunThreads = 1024;
constexpr int kMergeThreads = 256;
constexpr int kMergeSpan = 16;      // outputs per thread in a merge pass
constexpr int kSelThreads = 1024;

struct ByIdx {
  __device__ static u64 key(const Pair& p) { return (u64)(u32)p.idx; }
};
struct ByRank {
  __device__ static u64 key(const Pair& p) { return pair_rank(p); }
};

template <class Cmp>
__device__ void lds_bitonic(Pair* a, int N) {
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (N >> 1); i += blockDim.x) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool up = (lo & size) == 0;
        Pair x = a[lo], y = a[hi];
        u64 kx = Cmp::key(x), ky = Cmp::key(y);
        if (up ? (kx > ky) : (kx < ky)) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Sorts every run of kRun entries of every segment in place.
template <class Cmp>
__global__ __launch_bounds__(kRunThreads) void k_run_sort(Pair* data, int64_t seg_len, int64_t runs_per_seg) {
  __shared__ Pair s[kRun];
  const int64_t seg = blockIdx.x / runs_per_seg;
  const int64_t run = blockIdx.x % runs_per_seg;
  const int64_t b0 = run * kRun;
  const int len = (int)std::min<int64_t>(kRun, seg_len - b0);
  Pair* p = data + seg * seg_len + b0;
  for (int i = threadIdx.x; i < kRun; i += kRunThreads) s[i] = i < len ? p[i] : pair_sentinel();
  __syncthreads();
  lds_bitonic<Cmp>(s, kRun);
  for (int i = threadIdx.x; i < len; i += kRunThreads) p[i] = s[i];
}

// Merge-path split of output position o between sorted A[0,la) and B[0,lb):
// the number of A entries among the first o outputs (A first on equal keys).
template <class Cmp>
__device__ __forceinline__ int64_t merge_split(const Pair* A, int64_t la, const Pair* B, int64_t lb, int64_t o) {
  int64_t lo = std::max<int64_t>(0, o - lb), hi = std::min<int64_t>(o, la);
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (Cmp::key(A[mid]) <= Cmp::key(B[o - mid - 1])) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Merges adjacent sorted runs of length L (inside segments of seg_len).
template <class Cmp>
__global__ __launch_bounds__(kMergeThreads) void k_merge_pass(const Pair* __restrict__ src, Pair* __restrict__ dst,
                                                              int64_t seg_len, int64_t nseg, int64_t L,
                                                              int64_t threads_per_seg) {
  const int64_t gt = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t seg = gt / threads_per_seg;
  if (seg >= nseg) return;
  const int64_t o0 = (gt % threads_per_seg) * kMergeSpan;  // output position in the segment
  if (o0 >= seg_len) return;
  const int64_t pair0 = (o0 / (2 * L)) * (2 * L);
  const int64_t la = std::max<int64_t>(0, std::min<int64_t>(L, seg_len - pair0));
  const int64_t lb = std::max<int64_t>(0, std::min<int64_t>(L, seg_len - pair0 - L));
  const Pair* A = src + seg * seg_len + pair0;
  const Pair* B = A + la;
  Pair* out = dst + seg * seg_len + pair0;
  const int64_t o = o0 - pair0;
  const int64_t oend = std::min<int64_t>(o + kMergeSpan, la + lb);
  int64_t i = merge_split<Cmp>(A, la, B, lb, o);
  int64_t j = o - i;
  for (int64_t q = o; q < oend; ++q) {
    bool takeA = j >= lb || (i < la && Cmp::key(A[i]) <= Cmp::key(B[j]));
    out[q] = takeA ? A[i++] : B[j++];
  }
}

// Host: sorts nseg segments of seg_len entries (in `a`, using `b` as scratch);
// returns the buffer that holds the result.
template <class Cmp>
static Pair* sort_segments(Pair* a, Pair* b, int64_t seg_len, int64_t nseg, hipStream_t st) {
  if (seg_len <= 1 || nseg == 0) return a;
  const int64_t runs = (seg_len + kRun - 1) / kRun;
  hipLaunchKernelGGL(k_run_sort<Cmp>, dim3((unsigned)(runs * nseg)), dim3(kRunThreads), 0, st, a, seg_len, runs);
  const int64_t tps = (seg_len + kMergeSpan - 1) / kMergeSpan;
  const int64_t blocks = (tps * nseg + kMergeThreads - 1) / kMergeThreads;
  for (int64_t L = kRun; L < seg_len; L *= 2) {
    hipLaunchKernelGGL(k_merge_pass<Cmp>, dim3((unsigned)blocks), dim3(kMergeThreads), 0, st, a, b, seg_len, nseg, L, tps);
    std::swap(a, b);
  }
  return a;
}

__global__ void k_gt_load_rows(const int32_t* __restrict__ idx, const float* __restrict__ val, Pair* __restrict__ out,
                               int64_t total) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) out[i] = Pair{idx[i], __float_as_uint(val[i])};
}

// Rows sorted by index: flags a repeated index or one outside [0, n).
__global__ void k_gt_validate(const Pair* __restrict__ rows, int64_t k, int64_t total, int64_t n, u32* err) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  int32_t x = rows[i].idx;
  bool bad = x < 0 || (int64_t)x >= n;
  if (i % k != 0) bad = bad || rows[i - 1].idx == x;
  if (bad) atomicOr(err, kErrBadInput);
}

// Union of slot pairs.  Merge m combines A = slots[sa[m]] and B = slots[sa[m] + half]
// (k entries each, sorted by index) into M[m] (2k entries): entries in merge
// order, a B entry whose index A also holds becomes a hole (idx -1) and that A
// entry carries a + b.
struct UnionArgs {
  Pair* slots;
  Pair* M;
  int64_t k;
  int64_t half;         // 2^r
  int64_t stride;       // 2^(r+1)
  int64_t threads_per_merge;
  int64_t nm;           // merges in this round
};

__global__ __launch_bounds__(kMergeThreads) void k_gt_union(UnionArgs a) {
  const int64_t gt = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t m = gt / a.threads_per_merge;
  const int64_t o = (gt % a.threads_per_merge) * kMergeSpan;
  const int64_t two_k = 2 * a.k;
  if (m >= a.nm || o >= two_k) return;
  const Pair* A = a.slots + (m * a.stride) * a.k;
  const Pair* B = a.slots + (m * a.stride + a.half) * a.k;
  Pair* out = a.M + m * two_k;
  const int64_t la = a.k, lb = a.k;
  const int64_t oend = std::min<int64_t>(o + kMergeSpan, two_k);
  int64_t i = merge_split<ByIdx>(A, la, B, lb, o);
  int64_t j = o - i;
  for (int64_t q = o; q < oend; ++q) {
    bool takeA = j >= lb || (i < la && (u32)A[i].idx <= (u32)B[j].idx);
    if (takeA) {
      Pair e = A[i++];
      if (j < lb && B[j].idx == e.idx) e.bits = __float_as_uint(__uint_as_float(e.bits) + __uint_as_float(B[j].bits));
      out[q] = e;
    } else {
      Pair e = B[j++];
      if (i > 0 && A[i - 1].idx == e.idx) e = pair_sentinel();
      out[q] = e;
    }
  }
}

// One workgroup per merge: keeps the k best of M[m] (holes excluded) in index
// order, written to slots[m * stride].
struct SelectArgs {
  Pair* slots;
  const Pair* M;
  int64_t k;
  int64_t stride;
};

__global__ __launch_bounds__(kSelThreads) void k_gt_select(SelectArgs a) {
  constexpr int NT = kSelThreads;
  __shared__ u32 s_hist[2048];
  __shared__ u32 s_scan[NT / kWave + 1];
  __shared__ u32 s_found[3];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const int64_t len = 2 * a.k;
  const Pair* M = a.M + m * len;
  Pair* out = a.slots + (m * a.stride) * a.k;
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  u32 prefix = 0;
  int64_t need = a.k;
  int64_t t_strict = -1;
  u32 t_eq = 0;
  int64_t r = 0;
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L], wd = widths[L];
    const u32 nbins = 1u << wd;
    for (int i = tid; i < 2048; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < len; i += NT) {
      Pair e = M[i];
      u32 key = key_of_bits(e.bits);
      if (e.idx >= 0 && (key >> (sh + wd)) == prefix) atomicAdd(&s_hist[(key >> sh) & (nbins - 1)], 1u);
    }
    __syncthreads();
    const int cpt = std::max(1, (int)nbins / NT);
    const int top = (int)nbins - cpt * tid;
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
    if (d == 0xFFFFFFFFu) return;  // fewer than k live entries: impossible for valid rows
    need -= (int64_t)s_found[1];
    const int64_t h = s_found[2];
    prefix = (prefix << wd) | d;
    if (need == h) {
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
  // ordered compaction over contiguous per-thread ranges
  const int64_t span = (len + NT - 1) / NT;
  const int64_t lo = std::min<int64_t>(len, tid * span), hi = std::min<int64_t>(len, lo + span);
  u32 gt = 0, eq = 0;
  for (int64_t i = lo; i < hi; ++i) {
    Pair e = M[i];
    u32 key = key_of_bits(e.bits);
    bool live = e.idx >= 0;
    gt += live && (int64_t)key > t_strict;
    eq += live && r > 0 && key == t_eq;
  }
  u32 gt_tot, eq_tot;
  u32 gt_ex = block_exclusive_sum<NT>(gt, s_scan, gt_tot);
  u32 eq_ex = block_exclusive_sum<NT>(eq, s_scan, eq_tot);
  int64_t pos = (int64_t)gt_ex + std::min<int64_t>((int64_t)eq_ex, r);
  int64_t eq_seen = eq_ex;
  for (int64_t i = lo; i < hi; ++i) {
    Pair e = M[i];
    u32 key = key_of_bits(e.bits);
    bool live = e.idx >= 0;
    bool g = live && (int64_t)key > t_strict;
    bool q = live && r > 0 && key == t_eq;
    bool sel = g || (q && eq_seen < r);
    eq_seen += q;
    if (sel && pos < a.k) out[pos++] = e;
  }
}

// The same selection with M's keys loaded once into registers: thread t
// holds entries j NT + t (j < EPT; coalesced rows, every load in flight at
// once).  The three histogram levels run on the registers, and the ordered
// compaction walks the rows in order (index order is (row, thread) order)
// with a ballot and per-wave counts per row; only the selected pairs are
// read again to be written out.  For 2k <= EPT NT.
template <int EPT>
__global__ __launch_bounds__(kSelThreads) void k_gt_select_reg(SelectArgs a) {
  constexpr int NT = kSelThreads;
  __shared__ u32 s_hist[2048];
  __shared__ u32 s_scan[NT / kWave + 1];
  __shared__ u32 s_found[3];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const u32 len = (u32)(2 * a.k);
  const Pair* __restrict__ M = a.M + m * (int64_t)len;
  Pair* __restrict__ out = a.slots + (m * a.stride) * a.k;
  // a hole or a place past the end gets key 0xFFFFFFFF, above every real
  // key: no histogram level counts it (its top bits never match the prefix)
  // and, compared as signed, it is below every threshold
  // (16 rows of loads in flight at a time: all EPT at once would need two
  // registers per row on top of the keys)
  static_assert(EPT % 16 == 0, "rows come in groups of 16");
  u32 key[EPT];
#pragma unroll
  for (int c = 0; c < EPT; c += 16) {
#pragma unroll
    for (int j = c; j < c + 16; ++j) {
      const u32 i = (u32)(j * NT + tid);
      const Pair e = M[i < len ? i : 0u];
      key[j] = i < len && e.idx >= 0 ? key_of_bits(e.bits) : 0xFFFFFFFFu;
    }
    asm volatile("" ::: "memory");
  }
  const int shifts[3] = {20, 9, 0};
  const int widths[3] = {11, 11, 9};
  u32 prefix = 0;
  u32 need = (u32)a.k;
  u32 t_lo = 0, t_eq = 0, r = 0;
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L], wd = widths[L];
    const u32 nbins = 1u << wd;
    for (int i = tid; i < 2048; i += NT) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if ((key[j] >> (sh + wd)) == prefix) atomicAdd(&s_hist[(key[j] >> sh) & (nbins - 1)], 1u);
    __syncthreads();
    const int cpt = std::max(1, (int)nbins / NT);
    const int top = (int)nbins - cpt * tid;
    u32 own = 0;
    if (top > 0)
      for (int d = top - 1; d >= std::max(0, top - cpt); --d) own += s_hist[d];
    u32 tot;
    const u32 above = block_exclusive_sum<NT>(own, s_scan, tot);
    if (tid == 0) s_found[0] = 0xFFFFFFFFu;
    __syncthreads();
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
    if (d == 0xFFFFFFFFu) return;  // fewer than k live entries: impossible for valid rows
    need -= s_found[1];
    const u32 h = s_found[2];
    prefix = (prefix << wd) | d;
    __syncthreads();  // s_found is rewritten by the next level
    if (need == h) {
      t_lo = prefix << sh;
      break;
    }
    if (L == 2) {
      t_lo = prefix + 1;
      t_eq = prefix;
      r = need;
    }
  }
  // ordered compaction: every key >= t_lo and the first r equal to t_eq,
  // row by row
  __shared__ u32 s_wc[2][NT / kWave][2];
  const int lane = lane_id(), w = tid / kWave;
  u32 gt_seen = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const bool g = (int)key[j] >= (int)t_lo;
    const bool q = r > 0 && key[j] == t_eq;
    const u64 bg = ballot(g), be = ballot(q);
    if (lane == 0) {
      s_wc[j & 1][w][0] = (u32)__popcll(bg);
      s_wc[j & 1][w][1] = (u32)__popcll(be);
    }
    __syncthreads();
    u32 og = 0, oe = 0, tg = 0, te = 0;
#pragma unroll
    for (int v = 0; v < NT / kWave; ++v) {
      const u32 cg = s_wc[j & 1][v][0], ce = s_wc[j & 1][v][1];
      og += v < w ? cg : 0u;
      oe += v < w ? ce : 0u;
      tg += cg;
      te += ce;
    }
    const u32 gb = gt_seen + og + lanes_below(bg), eb = eq_seen + oe + lanes_below(be);
    if (g || (q && eb < r)) {
      const u32 pos = gb + std::min(eb, r);
      if (pos < (u32)a.k) out[pos] = M[(u32)(j * NT + tid)];
    }
    gt_seen += tg;
    eq_seen += te;
    asm volatile("" ::: "memory");  // keep each row's reload in its row
  }
}

__global__ void k_gt_emit(const Pair* __restrict__ g, int64_t k, int32_t* out_idx, float* out_val) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < k) {
    out_idx[i] = g[i].idx;
    out_val[i] = __uint_as_float(g[i].bits);
  }
}

// mask[t] = 1 when idx[t] is among the k indices of `sorted0` (sorted by index).
__global__ void k_gt_mask(const int32_t* __restrict__ idx, int64_t total, const Pair* __restrict__ sorted0, int64_t k,
                          uint8_t* __restrict__ mask) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  int32_t x = idx[t];
  int64_t lo = 0, hi = k;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (sorted0[mid].idx < x) lo = mid + 1;
    else hi = mid;
  }
  mask[t] = (lo < k && sorted0[lo].idx == x) ? 1 : 0;
}

__global__ void k_gt_copy(const Pair* __restrict__ src, Pair* __restrict__ dst, int64_t len) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < len) dst[i] = src[i];
}

struct GtLayout {
  size_t slots, tmp, M, f0, f1, total;
};

static GtLayout gt_layout(int64_t P, int64_t k) {
  GtLayout L{};
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t pk = sizeof(Pair) * (size_t)P * (size_t)std::max<int64_t>(k, 1);
  L.slots = kWorkspaceHeader;  // after the header whose first word is the error word
  L.tmp = L.slots + al(pk);
  L.M = L.tmp + al(pk);
  L.f0 = L.M + al(pk);  // (P/2) merges x 2k entries <= P*k
  L.f1 = L.f0 + al(sizeof(Pair) * (size_t)std::max<int64_t>(k, 1));
  L.total = L.f1 + al(sizeof(Pair) * (size_t)std::max<int64_t>(k, 1));
  return L;
}

}  // namespace tgs

using namespace tgs;

extern "C" size_t tgs_gtopk_workspace_bytes(int32_t P, int64_t k, int64_t n) {
  if (P < 1 || k < 0 || n < 0 || n > INT32_MAX || k > n) return 0;
  return gt_layout(P, k).total;
}

extern "C" tgs_status tgs_gtopk_merge(const int32_t* idx, const float* val, int32_t P, int64_t k, int64_t n,
                                      int32_t* out_idx, float* out_val, uint8_t* out_mask, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (P < 1) return fail(TGS_EINVAL, "gtopk_merge: P=%d < 1", (int)P);
  if (n < 0 || n > INT32_MAX) return fail(TGS_EINVAL, "gtopk_merge: n=%lld outside [0, 2^31-1]", (long long)n);
  if (k < 0 || k > n) return fail(TGS_EINVAL, "gtopk_merge: k=%lld outside [0, n]", (long long)k);
  if ((int64_t)P * k > INT32_MAX) return fail(TGS_EINVAL, "gtopk_merge: P*k too large");
  if (!workspace) return fail(TGS_EINVAL, "gtopk_merge: null workspace");
  if (k > 0 && (!idx || !val || !out_idx || !out_val || !out_mask))
    return fail(TGS_EINVAL, "gtopk_merge: null array pointer");
  for (const void* p : {(const void*)idx, (const void*)val, (const void*)out_idx, (const void*)out_val})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "gtopk_merge: pointer not 4-byte aligned");
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
  Pair* slots = (Pair*)(ws + L.slots);
  Pair* tmp = (Pair*)(ws + L.tmp);
  Pair* M = (Pair*)(ws + L.M);
  const int64_t total = (int64_t)P * k;
  const unsigned eb = (unsigned)((total + 255) / 256);

  hipLaunchKernelGGL(k_gt_load_rows, dim3(eb), dim3(256), 0, stream, idx, val, slots, total);
  Pair* sorted = sort_segments<ByIdx>(slots, tmp, k, P, stream);
  if (sorted != slots) hipLaunchKernelGGL(k_gt_copy, dim3(eb), dim3(256), 0, stream, sorted, slots, total);
  hipLaunchKernelGGL(k_gt_validate, dim3(eb), dim3(256), 0, stream, slots, k, total, n, err);

  for (int64_t half = 1; half < P; half *= 2) {
    const int64_t stride = 2 * half;
    const int64_t nm = (P - half + stride - 1) / stride;  // slots s = m*stride with s + half < P
    UnionArgs ua{slots, M, k, half, stride, (2 * k + kMergeSpan - 1) / kMergeSpan, nm};
    const int64_t ublocks = (ua.threads_per_merge * nm + kMergeThreads - 1) / kMergeThreads;
    hipLaunchKernelGGL(k_gt_union, dim3((unsigned)ublocks), dim3(kMergeThreads), 0, stream, ua);
    SelectArgs sa{slots, M, k, stride};
    const int64_t ept = (2 * k + kSelThreads - 1) / kSelThreads;
    if (ept <= 16) hipLaunchKernelGGL(k_gt_select_reg<16>, dim3((unsigned)nm), dim3(kSelThreads), 0, stream, sa);
    else if (ept <= 32) hipLaunchKernelGGL(k_gt_select_reg<32>, dim3((unsigned)nm), dim3(kSelThreads), 0, stream, sa);
    else if (ept <= 48) hipLaunchKernelGGL(k_gt_select_reg<48>, dim3((unsigned)nm), dim3(kSelThreads), 0, stream, sa);
    else if (ept <= 64) hipLaunchKernelGGL(k_gt_select_reg<64>, dim3((unsigned)nm), dim3(kSelThreads), 0, stream, sa);
    else hipLaunchKernelGGL(k_gt_select, dim3((unsigned)nm), dim3(kSelThreads), 0, stream, sa);
  }
  Pair* f0 = (Pair*)(ws + L.f0);
  Pair* f1 = (Pair*)(ws + L.f1);
  const unsigned kb = (unsigned)((k + 255) / 256);
  hipLaunchKernelGGL(k_gt_copy, dim3(kb), dim3(256), 0, stream, slots, f0, k);
  Pair* g = sort_segments<ByRank>(f0, f1, k, 1, stream);
  hipLaunchKernelGGL(k_gt_emit, dim3(kb), dim3(256), 0, stream, g, k, out_idx, out_val);
  hipLaunchKernelGGL(k_gt_mask, dim3(eb), dim3(256), 0, stream, idx, total, slots, k, out_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "gtopk_merge: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

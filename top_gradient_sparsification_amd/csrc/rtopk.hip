// rTop-k with error feedback on gfx950.
//
// Method (arxivdaily listing for arXiv 2004.05298, entry "rTop-k: A
// Statistical Estimation Approach to Distributed SGD"): a sparsifier that
// chains random-k after top-k -- the k sent entries are a uniformly random
// subset of the r largest.  Entries not sent, the r - k passed over included,
// stay in the error-feedback residual (entry "Sparsified SGD with Memory").
//
//   1. the top-r step (tgs_topk_ef_step with k = r) into workspace buffers:
//      acc written back, the r largest in (key desc, index asc) order, their
//      residual set to +0;
//   2. k_rtopk_draw: entry j of the list draws u_j = word 0 of Philox4x32-10
//      (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11)
//      at counter (index_j, step low, step high, 0) under key (seed low,
//      seed high), and counts u_j >> 21 into a 2048-bin histogram; the last
//      workgroup to arrive finds the bin d0 that holds the k-th smallest
//      draw and how many of its entries are kept (need);
//   3. k_rtopk_cand: entries of bins below d0 are kept for certain (counted
//      per workgroup); those of bin d0 are listed as candidates, and the last
//      workgroup to arrive finds T, the need-th smallest composite
//      u << 32 | index among them (unique, so no tie rule is needed: the
//      index bits matter only when draws tie), by a radix select, and each
//      workgroup's place in the output;
//   4. k_rtopk_emit: the entries with composite <= T -- the k smallest --
//      are written in the list's order, (key desc, index asc), by an ordered
//      compaction; every entry passed over gets its acc back in the residual.
#include <algorithm>
#include <climits>

#include "tgs_host.h"
#include "tgs_internal.h"

namespace tgs {

constexpr int kPickThreads = 1024;

// Philox4x32-10: ten rounds on the 128-bit counter c under the key (k0, k1);
// a round multiplies words 0 and 2 by the two multipliers, mixes the high
// halves into words 1 and 3 and the key, and the key advances by the Weyl
// constants between rounds.  Returns output word 0.
__device__ __forceinline__ u32 philox_w0(u32 c0, u32 c1, u32 c2, u32 c3, u32 k0, u32 k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const u32 hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const u32 hi2 = __umulhi(0xCD9E8D57u, c2), lo2 = 0xCD9E8D57u * c2;
    const u32 n0 = hi2 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo2;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

constexpr u32 kRtCand = 8192;  // candidates the selecting workgroup orders in LDS

struct PickArgs {
  const int32_t* idx;  // [r] the top r, in (key desc, index asc) order
  const float* val;    // [r] their acc
  u32* draw;           // [r] u_j (written by k_rtopk_draw)
  u32 r, k;
  u32 seed_lo, seed_hi, step_lo, step_hi;
  int32_t* out_idx;    // [k]
  float* out_val;      // [k]
  float* residual;
  HeaderHist* hh;      // histogram of u >> 21 and its arrivals (zero on entry, left zero)
  u32* ctl;            // [0] d0, [1] need, [2] candidates, [3] arrivals of k_rtopk_cand, [4] [5] T (high, low word)
  u32* wcnt;           // [workgroups] entries kept for certain, then all kept, then the workgroup's first place
  u64* cand;           // [r] candidates: u << 32 | index
  u32* candj;          // [r] their places in the list
  u32 cand_cap;        // candidates ordered in LDS at most (fewer: from memory; to test)
};

// u_j for every entry of the top-r list, one per thread, and the histogram
// of u >> 21; the last workgroup finds d0 and need.
__global__ __launch_bounds__(kPickThreads) void k_rtopk_draw(PickArgs a) {
  constexpr int NT = kPickThreads, NW = NT / kWave;
  __shared__ u32 s_h[2048];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_last, s_d0, s_need;
  const int tid = threadIdx.x;
  const u32 j = blockIdx.x * (u32)NT + (u32)tid;
  for (int i = tid; i < 2048; i += NT) s_h[i] = 0u;
  __syncthreads();
  if (j < a.r) {
    const u32 u = philox_w0((u32)a.idx[j], a.step_lo, a.step_hi, 0u, a.seed_lo, a.seed_hi);
    a.draw[j] = u;
    atomicAdd(&s_h[u >> 21], 1u);
  }
  __syncthreads();
  for (int i = tid; i < 2048; i += NT)
    if (s_h[i]) add_agent_relaxed(&a.hh->hist[i], s_h[i]);
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_acqrel(&a.hh->done, 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  for (int i = tid; i < 2048; i += NT) s_h[i] = ld_agent(&a.hh->hist[i]);
  __syncthreads();
  // the smallest bin d0 whose count and those below it reach k (k = 0: no
  // entry is kept, d0 = need = 0); thread t owns bins 2t and 2t + 1
  static_assert(2 * NT == 2048, "two bins per thread");
  const u32 c0 = s_h[2 * tid], c1 = s_h[2 * tid + 1];
  if (tid == 0) {
    s_d0 = 0u;
    s_need = 0u;
  }
  u32 tot;
  const u32 below = block_exclusive_sum<NT>(c0 + c1, s_scan, tot);
  if (below < a.k && below + c0 + c1 >= a.k) {
    const bool first = below + c0 >= a.k;
    s_d0 = first ? 2u * tid : 2u * tid + 1u;
    s_need = a.k - (first ? below : below + c0);
  }
  __syncthreads();
  if (tid == 0) {
    st_agent(&a.ctl[0], s_d0);
    st_agent(&a.ctl[1], s_need);
    st_agent(&a.ctl[2], 0u);
    st_agent(&a.ctl[3], 0u);
    st_agent(&a.hh->done, 0u);
  }
  for (int i = tid; i < 2048; i += NT) st_agent(&a.hh->hist[i], 0u);
}

// The need-th smallest of the nc composites at src (1 <= need <= nc), all of
// whose top 11 bits are d0: a radix select over the other 53 bits (digits of
// 11, 11, 11, 11 and 9 bits).  src is in LDS, or (GLOBAL) in device memory
// written by other workgroups.  Every thread of the workgroup calls it.
template <bool GLOBAL>
__device__ u64 rt_select(const u64* src, u32 nc, u32 need, u32 d0, u32* s_h, u32* s_scan, u32* s_out) {
  constexpr int NT = kPickThreads;
  constexpr int kShift[5] = {42, 31, 20, 9, 0};
  constexpr int kWidth[5] = {11, 11, 11, 11, 9};
  const int tid = threadIdx.x;
  u64 prefix = (u64)d0 << 53;
  for (int L = 0; L < 5; ++L) {
    const int sh = kShift[L], top = sh + kWidth[L];
    const u32 nb = 1u << kWidth[L];
    for (int i = tid; i < 2048; i += NT) s_h[i] = 0u;
    __syncthreads();
    for (u32 i = tid; i < nc; i += NT) {
      const u64 c = GLOBAL ? ld_agent64(src + i) : src[i];
      if ((c >> top) == (prefix >> top)) atomicAdd(&s_h[(u32)(c >> sh) & (nb - 1u)], 1u);
    }
    __syncthreads();
    const u32 c0 = s_h[2 * tid], c1 = s_h[2 * tid + 1];  // (bins nb and above hold zero)
    u32 tot;
    const u32 below = block_exclusive_sum<NT>(c0 + c1, s_scan, tot);
    if (below < need && below + c0 + c1 >= need) {
      const bool first = below + c0 >= need;
      s_out[0] = first ? 2u * tid : 2u * tid + 1u;
      s_out[1] = first ? below : below + c0;
    }
    __syncthreads();
    const u32 d = s_out[0];
    need -= s_out[1];
    prefix |= (u64)d << sh;
    const u32 h = s_h[d];
    __syncthreads();  // s_h and s_out are rewritten by the next level
    if (h == need) return prefix | ((1ull << sh) - 1ull);  // every composite with this prefix is kept
  }
  return prefix;
}

// Entries of bins below d0 are kept for certain; those of bin d0 are listed.
// The last workgroup finds T and every workgroup's first output place.
__global__ __launch_bounds__(kPickThreads) void k_rtopk_cand(PickArgs a) {
  constexpr int NT = kPickThreads, NW = NT / kWave;
  __shared__ u64 s_c[kRtCand];
  __shared__ u32 s_h[2048];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_out[2];
  __shared__ u32 s_last;
  const int tid = threadIdx.x, lane = lane_id();
  const u32 d0 = a.ctl[0], need = a.ctl[1];
  const u32 j = blockIdx.x * (u32)NT + (u32)tid;
  const u32 u = j < a.r ? a.draw[j] : 0u;
  const bool sure = j < a.r && (u >> 21) < d0;
  const bool cnd = j < a.r && need > 0 && (u >> 21) == d0;
  u32 tot;
  (void)block_exclusive_sum<NT>(sure ? 1u : 0u, s_scan, tot);
  if (tid == 0) st_agent(&a.wcnt[blockIdx.x], tot);
  // candidates: one device add per wave that has any
  const u64 m = ballot(cnd);
  if (m) {
    u32 base = 0;
    if (lane == 0) base = add_agent_relaxed(&a.ctl[2], (u32)__popcll(m));
    base = __builtin_amdgcn_readfirstlane(base);
    if (cnd) {
      const u32 p = base + lanes_below(m);
      st_agent64(&a.cand[p], (u64)u << 32 | (u32)a.idx[j]);
      st_agent(&a.candj[p], j);
    }
  }
  wait_all_memory();
  __syncthreads();
  if (tid == 0) s_last = add_agent_acqrel(&a.ctl[3], 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  // last workgroup: T, the need-th smallest candidate (need = 0: none kept)
  const u32 nc = ld_agent(&a.ctl[2]);
  u64 T = 0;
  if (need > 0) {
    const bool lds = nc <= a.cand_cap;
    if (lds) {
      for (u32 i = tid; i < nc; i += NT) s_c[i] = ld_agent64(&a.cand[i]);
      __syncthreads();
      T = rt_select<false>(s_c, nc, need, d0, s_h, s_scan, s_out);
    } else {
      T = rt_select<true>(a.cand, nc, need, d0, s_h, s_scan, s_out);
    }
    // the kept candidates counted into their workgroups
    for (u32 i = tid; i < nc; i += NT)
      if ((lds ? s_c[i] : ld_agent64(&a.cand[i])) <= T) add_agent_relaxed(&a.wcnt[ld_agent(&a.candj[i]) / NT], 1u);
    wait_all_memory();
    __syncthreads();
  }
  // every workgroup's first place: an exclusive scan of the counts
  u32 carry = 0;
  for (u32 b0 = 0; b0 < gridDim.x; b0 += NT) {
    const u32 w = b0 + tid;
    const u32 c = w < gridDim.x ? ld_agent(&a.wcnt[w]) : 0u;
    u32 t;
    const u32 ex = block_exclusive_sum<NT>(c, s_scan, t);
    if (w < gridDim.x) st_agent(&a.wcnt[w], carry + ex);
    carry += t;
  }
  if (tid == 0) {
    st_agent(&a.ctl[4], (u32)(T >> 32));
    st_agent(&a.ctl[5], (u32)T);
  }
}

// The kept entries (composite <= T) in the list's order; the others get
// their acc back.
__global__ __launch_bounds__(kPickThreads) void k_rtopk_emit(PickArgs a) {
  constexpr int NT = kPickThreads, NW = NT / kWave;
  __shared__ u32 s_scan[NW + 1];
  const int tid = threadIdx.x;
  const u32 need = a.ctl[1];
  const u64 T = (u64)a.ctl[4] << 32 | a.ctl[5];
  const u32 off = a.wcnt[blockIdx.x];
  const u32 j = blockIdx.x * (u32)NT + (u32)tid;
  const bool in = j < a.r;
  const u32 u = in ? a.draw[j] : 0u;
  const int32_t id = in ? a.idx[j] : 0;
  const float v = in ? a.val[j] : 0.0f;
  const bool keep = in && need > 0 && ((u64)u << 32 | (u32)id) <= T;
  u32 tot;
  const u32 p = block_exclusive_sum<NT>(keep ? 1u : 0u, s_scan, tot);
  if (keep) {
    a.out_idx[off + p] = id;
    a.out_val[off + p] = v;
  } else if (in) {
    a.residual[id] = v;
  }
}

struct RtopkLayout {
  size_t idx, val, draw, ctl, wcnt, cand, candj, total;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static RtopkLayout rtopk_layout(int64_t n, int64_t r) {
  RtopkLayout L{};
  const size_t tb = tgs_topk_workspace_bytes(n, r);
  L.idx = al256(tb);
  L.val = L.idx + al256(sizeof(int32_t) * (size_t)std::max<int64_t>(r, 1));
  const size_t rr = (size_t)std::max<int64_t>(r, 1), nwg = (rr + kPickThreads - 1) / kPickThreads;
  L.draw = L.val + al256(sizeof(float) * rr);
  L.ctl = L.draw + al256(sizeof(u32) * rr);
  L.wcnt = L.ctl + 256;
  L.cand = L.wcnt + al256(sizeof(u32) * nwg);
  L.candj = L.cand + al256(sizeof(u64) * rr);
  L.total = L.candj + al256(sizeof(u32) * rr);
  return L;
}

}  // namespace tgs

using namespace tgs;

extern "C" size_t tgs_rtopk_workspace_bytes(int64_t n, int64_t r, int64_t k) {
  if (n < 0 || n > INT32_MAX || r < 0 || r > n || k < 0 || k > r) return 0;
  return rtopk_layout(n, r).total;
}

extern "C" tgs_status tgs_rtopk_ef_step(const float* grad, float* residual, int64_t n, int64_t r, int64_t k,
                                        uint64_t seed, uint64_t step, int32_t* out_idx, float* out_val,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n < 0 || n > INT32_MAX) return fail(TGS_EINVAL, "rtopk_ef_step: n=%lld outside [0, 2^31-1]", (long long)n);
  if (r < 0 || r > n || k < 0 || k > r)
    return fail(TGS_EINVAL, "rtopk_ef_step: need 0 <= k <= r <= n (r=%lld k=%lld n=%lld)", (long long)r, (long long)k,
                (long long)n);
  if (n > 0 && (!grad || !residual)) return fail(TGS_EINVAL, "rtopk_ef_step: null grad/residual");
  if (k > 0 && (!out_idx || !out_val)) return fail(TGS_EINVAL, "rtopk_ef_step: null output pointer");
  if (!workspace) return fail(TGS_EINVAL, "rtopk_ef_step: null workspace");
  for (const void* p : {(const void*)grad, (const void*)residual, (const void*)out_idx, (const void*)out_val})
    if (((uintptr_t)p & 3u) != 0) return fail(TGS_EINVAL, "rtopk_ef_step: pointer not 4-byte aligned");
  const size_t nb4 = (size_t)n * 4, kb4 = (size_t)k * 4;
  if (overlaps(grad, nb4, residual, nb4) || overlaps(grad, nb4, out_idx, kb4) || overlaps(grad, nb4, out_val, kb4) ||
      overlaps(residual, nb4, out_idx, kb4) || overlaps(residual, nb4, out_val, kb4) ||
      overlaps(out_idx, kb4, out_val, kb4))
    return fail(TGS_EINVAL, "rtopk_ef_step: overlapping buffers");
  const RtopkLayout L = rtopk_layout(n, r);
  if (workspace_bytes < L.total)
    return fail(TGS_EWORKSPACE, "rtopk_ef_step: workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (n == 0) return TGS_OK;
  char* ws = (char*)workspace;
  int32_t* ti = (int32_t*)(ws + L.idx);
  float* tv = (float*)(ws + L.val);
  const tgs_status st = tgs_topk_ef_step(grad, residual, n, r, r ? ti : nullptr, r ? tv : nullptr, workspace, L.idx,
                                         stream);
  if (st != TGS_OK) return st;
  if (r == 0) return TGS_OK;
  PickArgs a{};
  a.idx = ti;
  a.val = tv;
  a.draw = (u32*)(ws + L.draw);
  a.r = (u32)r;
  a.k = (u32)k;
  a.seed_lo = (u32)seed;
  a.seed_hi = (u32)(seed >> 32);
  a.step_lo = (u32)step;
  a.step_hi = (u32)(step >> 32);
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.residual = residual;
  a.hh = header_hist(workspace);
  a.ctl = (u32*)(ws + L.ctl);
  a.wcnt = (u32*)(ws + L.wcnt);
  a.cand = (u64*)(ws + L.cand);
  a.candj = (u32*)(ws + L.candj);
  // option 14: the last workgroup selects over the candidates in memory
  a.cand_cap = get_option(TGS_OPT_TOPK_PATH) == 14 ? 0u : kRtCand;
  const dim3 grid((unsigned)((r + kPickThreads - 1) / kPickThreads));
  hipLaunchKernelGGL(k_rtopk_draw, grid, dim3(kPickThreads), 0, stream, a);
  hipLaunchKernelGGL(k_rtopk_cand, grid, dim3(kPickThreads), 0, stream, a);
  hipLaunchKernelGGL(k_rtopk_emit, grid, dim3(kPickThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "rtopk_ef_step: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

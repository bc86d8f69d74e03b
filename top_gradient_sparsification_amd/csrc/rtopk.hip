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
//   2. k_rtopk_draw: entry i of the list draws u_i = word 0 of Philox4x32-10
//      (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11)
//      at counter (i, step low, step high, 0) under key (seed low, seed high);
//   3. k_rtopk_pick, one workgroup: the k entries with the smallest (u_i, i)
//      are kept, found by a radix select over the 64-bit composite
//      u_i << 32 | i (unique, so no tie rule is needed; the index bits are
//      looked at only when draws tie).  An ordered compaction over the top-r
//      list writes them in its order, (key desc, index asc); every entry
//      passed over gets its acc back in the residual.
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

struct PickArgs {
  const int32_t* idx;  // [r] the top r, in (key desc, index asc) order
  const float* val;    // [r] their acc
  u32* draw;           // [r] u_j (written by k_rtopk_draw)
  u32 r, k;
  u32 seed_lo, seed_hi, step_lo, step_hi;
  int32_t* out_idx;    // [k]
  float* out_val;      // [k]
  float* residual;
};

// u_j for every entry of the top-r list, one per thread.
__global__ __launch_bounds__(256) void k_rtopk_draw(PickArgs a) {
  const u32 j = blockIdx.x * 256u + threadIdx.x;
  if (j < a.r) a.draw[j] = philox_w0((u32)a.idx[j], a.step_lo, a.step_hi, 0u, a.seed_lo, a.seed_hi);
}

// One workgroup.  The entries are visited in batches of kPickBatch rows of
// 1024 (entry j = row * 1024 + tid), each batch's loads all in flight before
// any is used.
constexpr int kPickBatch = 16;

__global__ __launch_bounds__(kPickThreads) void k_rtopk_pick(PickArgs a) {
  constexpr int NT = kPickThreads, NW = NT / kWave, B = kPickBatch;
  __shared__ u32 s_h[2048];
  __shared__ u32 s_scan[NW + 1];
  __shared__ u32 s_out[2];
  __shared__ u32 s_wc[B][NW];
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const u32 r = a.r, k = a.k;
  const u32 rows = (r + NT - 1) / NT;
  // T = the k-th smallest composite u << 32 | index (1 <= k < r); kept:
  // composite <= T
  u64 T = 0;
  if (k > 0 && k < r) {
    constexpr int kShift[6] = {53, 42, 32, 21, 10, 0};
    constexpr int kWidth[6] = {11, 11, 10, 11, 11, 10};
    u64 prefix = 0;
    u32 need = k;
    for (int L = 0; L < 6; ++L) {
      const int sh = kShift[L], wd = kWidth[L];
      const u32 nb = 1u << wd;
      const int top = sh + wd;
      for (int i = tid; i < 2048; i += NT) s_h[i] = 0;
      __syncthreads();
      for (u32 b0 = 0; b0 < rows; b0 += B) {
        u32 dq[B];
#pragma unroll
        for (int e = 0; e < B; ++e) {
          const u32 j = (b0 + e) * NT + tid;
          dq[e] = j < r ? a.draw[j] : 0u;
        }
#pragma unroll
        for (int e = 0; e < B; ++e) {
          const u32 j = (b0 + e) * NT + tid;
          if (j >= r) continue;
          if (L < 3) {  // the draw's bits
            const u64 c = (u64)dq[e] << 32;
            if (top >= 64 || (c >> top) == prefix) atomicAdd(&s_h[(u32)(c >> sh) & (nb - 1u)], 1u);
          } else if ((u64)dq[e] == (prefix >> (32 - top))) {  // the draw ties the chosen one: index bits
            const u64 c = ((u64)dq[e] << 32) | (u64)(u32)a.idx[j];
            if ((c >> top) == prefix) atomicAdd(&s_h[(u32)(c >> sh) & (nb - 1u)], 1u);
          }
        }
      }
      __syncthreads();
      // the smallest digit d whose prefix count reaches need; thread t owns
      // bins 2t, 2t + 1
      const u32 c0 = 2u * tid < nb ? s_h[2 * tid] : 0u, c1 = 2u * tid + 1u < nb ? s_h[2 * tid + 1] : 0u;
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
      prefix = (prefix << wd) | d;
      const u32 h = s_h[d];
      __syncthreads();  // s_h and s_out are rewritten by the next level
      if (h == need || L == 5) {  // every composite with this prefix is kept
        T = sh == 0 ? prefix : (prefix << sh) | ((1ull << sh) - 1ull);
        break;
      }
    }
  }
  // ordered compaction over the list (rank order); entries passed over get
  // their acc back
  const u32 tu = (u32)(T >> 32);
  u32 seen = 0;
  for (u32 b0 = 0; b0 < rows; b0 += B) {
    u32 dq[B], iq[B], vq[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const u32 j = (b0 + e) * NT + tid;
      const bool in = j < r;
      dq[e] = in ? a.draw[j] : 0u;
      iq[e] = in ? (u32)a.idx[j] : 0u;
      vq[e] = in ? __float_as_uint(a.val[j]) : 0u;
    }
    u32 kmask = 0;
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const u32 j = (b0 + e) * NT + tid;
      const bool keep = j < r && k > 0 && (k == r || dq[e] < tu || (dq[e] == tu && iq[e] <= (u32)T));
      const u64 m = ballot(keep);
      if (lane == 0) s_wc[e][w] = (u32)__popcll(m);
      kmask |= (u32)keep << e;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const u32 j = (b0 + e) * NT + tid;
      u32 off = 0, tt = 0;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const u32 c = s_wc[e][q];
        off += q < w ? c : 0u;
        tt += c;
      }
      const bool keep = (kmask >> e) & 1u;
      const u64 m = ballot(keep);
      if (keep) {
        const u32 p = seen + off + lanes_below(m);
        a.out_idx[p] = (int32_t)iq[e];
        a.out_val[p] = __uint_as_float(vq[e]);
      } else if (j < r) {
        a.residual[iq[e]] = __uint_as_float(vq[e]);
      }
      seen += tt;
    }
    __syncthreads();  // s_wc is rewritten by the next batch
  }
}

struct RtopkLayout {
  size_t idx, val, draw, total;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static RtopkLayout rtopk_layout(int64_t n, int64_t r) {
  RtopkLayout L{};
  const size_t tb = tgs_topk_workspace_bytes(n, r);
  L.idx = al256(tb);
  L.val = L.idx + al256(sizeof(int32_t) * (size_t)std::max<int64_t>(r, 1));
  L.draw = L.val + al256(sizeof(float) * (size_t)std::max<int64_t>(r, 1));
  L.total = L.draw + al256(sizeof(u32) * (size_t)std::max<int64_t>(r, 1));
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
  hipLaunchKernelGGL(k_rtopk_draw, dim3((unsigned)((r + 255) / 256)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_rtopk_pick, dim3(1), dim3(kPickThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TGS_EHIP, "rtopk_ef_step: launch failed: %s", hipGetErrorString(e));
  return TGS_OK;
}

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

}  // namespace tgs

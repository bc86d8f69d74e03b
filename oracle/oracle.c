/*
 * CPU oracle for the error-feedback top-k gradient sparsifier — TEST
 * INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
 * may load or call this library.  The GPU library never links, includes or
 * calls anything here, and nothing here includes a GPU header.
 *
 * Each routine is the plain definition written out, sequential and slow on
 * purpose: full sorts instead of selection, one loop per step.
 *
 * Sources (web pages; cited by title and section):
 *   [EF]    arxivdaily listing for arXiv 2004.05298, entry "Sparsified SGD with
 *           Memory": compress (top-k) and keep the accumulated error in memory,
 *           added back before the next compression.
 *   [CONV]  same listing, entry "The Convergence of Sparsified Gradient
 *           Methods": each node sorts its gradient by magnitude, sends a subset
 *           and accumulates the rest locally.
 *   [HT]    same listing, entry "Rethinking gradient sparsification as total
 *           error minimization": hard-threshold sparsifier, i.e. top-k with k
 *           set by a constant threshold, run with error feedback.
 *   [GTOPK] nubint review "A Distributed Synchronous SGD Algorithm with Global
 *           Top-k Sparsification for Low Bandwidth Networks", sections ABSTRACT
 *           and Method: global top-k of the largest absolute values across P
 *           workers, found by a tournament of O(log P) pairwise rounds; only the
 *           globally selected indices keep their index information.
 *   [EST]   arxivdaily listing, entry "Near-Optimal Sparse Allreduce for
 *           Distributed Deep Learning" (Ok-Topk picks the top-k gradients
 *           through an estimated threshold rather than a sort); fugumt page
 *           for arXiv 2502.07634, related-paper entry "An Efficient
 *           Statistical-based Gradient Compression Technique for Distributed
 *           Training Systems" (SIDCo: threshold sparsification whose threshold
 *           estimate is as good as DGC's) and its Abstract (DGC scales better
 *           than top-k, whose sorting costs offset the communication saved).
 *   [RTOPK] arxivdaily listing, entry "rTop-k: A Statistical Estimation
 *           Approach to Distributed SGD": a sparsifier that chains top-k and
 *           random-k, i.e. a random subset of the largest entries.
 *   [PHILOX] Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
 *           as 1, 2, 3" (SC'11): the Philox4x32-10 counter-based generator,
 *           which supplies rTop-k's random draws.
 *
 * Readings where the pages are silent:
 *   - acc = residual + grad, one binary32 add, round-to-nearest-even, no
 *     fused multiply-add, subnormals kept (the x86 MXCSR FTZ and DAZ bits are
 *     cleared for the duration of every call).
 *   - "largest |acc|" compares key(x) = bits(x) & 0x7FFFFFFF as an unsigned
 *     integer; ties go to the lower index.
 *   - selected residual entries become +0.0f.
 *   - threshold test is key(acc) >= key(float(lambda)); output in ascending
 *     index order, truncated at `capacity` (entries beyond it keep acc in the
 *     residual).
 *   - gTop-k tournament: in round r slot s (s a multiple of 2^(r+1)) absorbs
 *     slot s + 2^r; coinciding indices have their values added in binary32;
 *     the k largest by (key desc, index asc) survive; a slot with no partner
 *     passes through.
 *   - threshold estimate: the q-th largest key(acc) over m sampled positions
 *     (given by the caller, repeats allowed); the hard threshold then keeps
 *     every entry whose key reaches it.
 *   - rTop-k: the top r by (key desc, index asc), then the k of them with the
 *     smallest (u_i, i), u_i = word 0 of Philox4x32-10 at counter
 *     (i, step low, step high, 0) under key (seed low, seed high): a uniform
 *     random k-subset.  Emitted in (key desc, index asc) order; every entry
 *     not emitted, the r - k left out included, keeps acc in the residual.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

/* ---- IEEE mode guard: round-to-nearest-even, no flush-to-zero, no DAZ ---- */
static unsigned int ieee_enter(void) {
  unsigned int old = _mm_getcsr();
  /* bit 15 FTZ, bit 6 DAZ, bits 13-14 rounding control (00 = nearest) */
  _mm_setcsr(old & ~(0x8000u | 0x0040u | 0x6000u));
  return old;
}
static void ieee_leave(unsigned int old) { _mm_setcsr(old); }

static uint32_t bits_of(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

/* magnitude key: monotone in |x| for every non-NaN x; -0 and +0 tie */
static uint32_t mag_key(float x) { return bits_of(x) & 0x7FFFFFFFu; }

/* one binary32 add; volatile keeps the compiler from fusing or reassociating */
static float add_f32(float a, float b) {
  volatile float s = a + b;
  return s;
}

/* composite sort key: ascending order == (key descending, index ascending) */
static uint64_t rank_key(uint32_t key, uint32_t index) {
  return ((uint64_t)(0x7FFFFFFFu - key) << 32) | (uint64_t)index;
}

static int cmp_u64(const void* a, const void* b) {
  uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
  return (x > y) - (x < y);
}

/*
 * Error-feedback top-k step ([EF], [CONV]).
 *   acc_i      = residual_i + grad_i
 *   S          = the k indices that come first when all n are ordered by
 *                (key(acc) desc, index asc)
 *   out        = S in that order, out_val = acc at that index (bitwise)
 *   residual_i = acc_i for i not in S, +0.0f for i in S
 * Returns 0, or -1 for invalid sizes, -2 if memory runs out.
 */
int oracle_topk_ef_step(const float* grad, float* residual, int64_t n, int64_t k,
                        int32_t* out_idx, float* out_val) {
  if (n < 0 || n > 0x7FFFFFFF || k < 0 || k > n) return -1;
  if (n == 0) return 0;
  float* acc = (float*)malloc((size_t)n * sizeof(float));
  uint64_t* order = (uint64_t*)malloc((size_t)n * sizeof(uint64_t));
  if (!acc || !order) { free(acc); free(order); return -2; }
  unsigned int mode = ieee_enter();

  for (int64_t i = 0; i < n; ++i) acc[i] = add_f32(residual[i], grad[i]);
  for (int64_t i = 0; i < n; ++i) order[i] = rank_key(mag_key(acc[i]), (uint32_t)i);
  qsort(order, (size_t)n, sizeof(uint64_t), cmp_u64);

  for (int64_t j = 0; j < k; ++j) {
    int32_t i = (int32_t)(order[j] & 0xFFFFFFFFu);
    out_idx[j] = i;
    out_val[j] = acc[i];
  }
  for (int64_t i = 0; i < n; ++i) residual[i] = acc[i];
  for (int64_t j = 0; j < k; ++j) residual[out_idx[j]] = 0.0f;

  ieee_leave(mode);
  free(acc);
  free(order);
  return 0;
}

/*
 * Hard-threshold step with error feedback ([HT]).
 * Scans i ascending; acc_i qualifies when key(acc_i) >= key(float(lambda)).
 * The first `capacity` qualifying entries are written as (i, acc_i) in
 * ascending index order and their residual becomes +0.0f; every other entry
 * (including qualifying ones past the capacity) keeps residual_i = acc_i.
 * Returns the total number of qualifying entries, or -1 for invalid input.
 */
int64_t oracle_threshold_ef_step_key(const float* grad, float* residual, int64_t n, uint32_t klam,
                                     int32_t* out_idx, float* out_val, int64_t capacity);

int64_t oracle_threshold_ef_step(const float* grad, float* residual, int64_t n, float lambda,
                                 int32_t* out_idx, float* out_val, int64_t capacity) {
  if (!(lambda >= 0.0f)) return -1;
  return oracle_threshold_ef_step_key(grad, residual, n, mag_key(lambda), out_idx, out_val, capacity);
}

/* The same step for a threshold given as its magnitude key (any value of
   bits & 0x7FFFFFFF; a key above infinity's is a NaN payload, which only NaNs
   of a larger or equal payload reach). */
int64_t oracle_threshold_ef_step_key(const float* grad, float* residual, int64_t n, uint32_t klam,
                                     int32_t* out_idx, float* out_val, int64_t capacity) {
  if (n < 0 || n > 0x7FFFFFFF || capacity < 0 || klam > 0x7FFFFFFFu) return -1;
  unsigned int mode = ieee_enter();
  int64_t count = 0;
  for (int64_t i = 0; i < n; ++i) {
    float acc = add_f32(residual[i], grad[i]);
    if (mag_key(acc) >= klam) {
      if (count < capacity) {
        out_idx[count] = (int32_t)i;
        out_val[count] = acc;
        residual[i] = 0.0f;
      } else {
        residual[i] = acc;
      }
      count += 1;
    } else {
      residual[i] = acc;
    }
  }
  ieee_leave(mode);
  return count;
}

/* ------------------------- threshold estimate ----------------------------- */

static int cmp_u32_desc(const void* a, const void* b) {
  uint32_t x = *(const uint32_t*)a, y = *(const uint32_t*)b;
  return (x < y) - (x > y);
}

/*
 * Threshold estimate ([EST]): the q-th largest magnitude key among the accs at
 * m sampled positions.
 *   key_j   = key(residual[s_j] + grad[s_j]) for j < m (s_j in [0, n); a
 *             position may repeat and then counts as often as it appears)
 *   *key_out = the q-th entry of the key_j sorted in descending order
 * Feeding *key_out to the hard threshold keeps about q/m of the entries.
 * Reads grad and residual only.  Returns 0, -1 for invalid input (n < 1,
 * m < 1, q outside [1, m], a position outside [0, n)), -2 if memory runs out.
 */
int oracle_threshold_estimate(const float* grad, const float* residual, int64_t n, const int32_t* sample_idx,
                              int64_t m, int64_t q, uint32_t* key_out) {
  if (n < 1 || n > 0x7FFFFFFF || m < 1 || q < 1 || q > m) return -1;
  for (int64_t j = 0; j < m; ++j)
    if (sample_idx[j] < 0 || (int64_t)sample_idx[j] >= n) return -1;
  uint32_t* k = (uint32_t*)malloc((size_t)m * sizeof(uint32_t));
  if (!k) return -2;
  unsigned int mode = ieee_enter();
  for (int64_t j = 0; j < m; ++j) {
    int32_t i = sample_idx[j];
    k[j] = mag_key(add_f32(residual[i], grad[i]));
  }
  qsort(k, (size_t)m, sizeof(uint32_t), cmp_u32_desc);
  *key_out = k[q - 1];
  ieee_leave(mode);
  free(k);
  return 0;
}

/* ------------------------------ Philox --------------------------------- */

/*
 * Philox4x32-10 ([PHILOX]): a 128-bit counter (c0..c3) is put through ten
 * rounds under a 64-bit key (k0, k1).  A round multiplies c0 and c2 by the
 * two round multipliers (0xD2511F53, 0xCD9E8D57) to 64-bit products; the new
 * counter is (high(c2 product) ^ c1 ^ k0, low(c2 product),
 * high(c0 product) ^ c3 ^ k1, low(c0 product)).  Between rounds the key words
 * grow by the Weyl constants 0x9E3779B9 and 0xBB67AE85.
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
    uint64_t p2 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
    uint32_t n0 = (uint32_t)(p2 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p2;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* rTop-k's draw for entry i: Philox word 0 at counter (i, step low, step
   high, 0) under key (seed low, seed high). */
static uint32_t rtopk_draw(uint64_t seed, uint64_t step, uint32_t i) {
  uint32_t ctr[4] = {i, (uint32_t)step, (uint32_t)(step >> 32), 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return out[0];
}

/* ------------------------------- rTop-k -------------------------------- */

/*
 * rTop-k step with error feedback ([RTOPK] with [EF]).
 *   acc_i  = residual_i + grad_i
 *   R      = the first r indices in (key(acc) desc, index asc) order
 *   S      = the k members i of R with the smallest (u_i, i), u_i the draw of
 *            entry i for (seed, step)
 *   out    = S in (key desc, index asc) order, out_val = acc there (bitwise)
 *   residual_i = +0.0f for i in S, acc_i otherwise
 * Returns 0, -1 for invalid sizes (0 <= k <= r <= n), -2 if memory runs out.
 */
int oracle_rtopk_ef_step(const float* grad, float* residual, int64_t n, int64_t r, int64_t k, uint64_t seed,
                         uint64_t step, int32_t* out_idx, float* out_val) {
  if (n < 0 || n > 0x7FFFFFFF || r < 0 || r > n || k < 0 || k > r) return -1;
  if (n == 0) return 0;
  float* acc = (float*)malloc((size_t)n * sizeof(float));
  uint64_t* order = (uint64_t*)malloc((size_t)n * sizeof(uint64_t));
  uint64_t* draw = (uint64_t*)malloc((size_t)(r > 0 ? r : 1) * sizeof(uint64_t));
  unsigned char* picked = (unsigned char*)calloc((size_t)n, 1);
  if (!acc || !order || !draw || !picked) { free(acc); free(order); free(draw); free(picked); return -2; }
  unsigned int mode = ieee_enter();

  for (int64_t i = 0; i < n; ++i) acc[i] = add_f32(residual[i], grad[i]);
  for (int64_t i = 0; i < n; ++i) order[i] = rank_key(mag_key(acc[i]), (uint32_t)i);
  qsort(order, (size_t)n, sizeof(uint64_t), cmp_u64);
  /* R = order[0 .. r); the k smallest (u, i) among them */
  for (int64_t j = 0; j < r; ++j) {
    uint32_t i = (uint32_t)(order[j] & 0xFFFFFFFFu);
    draw[j] = ((uint64_t)rtopk_draw(seed, step, i) << 32) | (uint64_t)i;
  }
  qsort(draw, (size_t)r, sizeof(uint64_t), cmp_u64);
  for (int64_t j = 0; j < k; ++j) picked[draw[j] & 0xFFFFFFFFu] = 1;
  /* emitted in R's order, which is (key desc, index asc) */
  int64_t e = 0;
  for (int64_t j = 0; j < r; ++j) {
    int32_t i = (int32_t)(order[j] & 0xFFFFFFFFu);
    if (picked[i]) {
      out_idx[e] = i;
      out_val[e] = acc[i];
      e += 1;
    }
  }
  for (int64_t i = 0; i < n; ++i) residual[i] = picked[i] ? 0.0f : acc[i];

  ieee_leave(mode);
  free(acc);
  free(order);
  free(draw);
  free(picked);
  return 0;
}

/* ---------------------------- gTop-k merge -------------------------------- */

typedef struct {
  int32_t idx;
  float val;
} pair_t;

static int cmp_pair_idx(const void* a, const void* b) {
  int32_t x = ((const pair_t*)a)->idx, y = ((const pair_t*)b)->idx;
  return (x > y) - (x < y);
}

static int cmp_pair_rank(const void* a, const void* b) {
  const pair_t* p = (const pair_t*)a;
  const pair_t* q = (const pair_t*)b;
  uint64_t x = rank_key(mag_key(p->val), (uint32_t)p->idx);
  uint64_t y = rank_key(mag_key(q->val), (uint32_t)q->idx);
  return (x > y) - (x < y);
}

/* MERGE then TOPK_k: union of two index-distinct sets of k pairs, values of a
   shared index added, then the k best by (key desc, index asc). `work` holds
   2k pairs. Result (k pairs, rank order) goes to `a`. */
static void merge_keep_topk(pair_t* a, const pair_t* b, int64_t k, pair_t* work) {
  memcpy(work, a, (size_t)k * sizeof(pair_t));
  memcpy(work + k, b, (size_t)k * sizeof(pair_t));
  qsort(work, (size_t)(2 * k), sizeof(pair_t), cmp_pair_idx);
  int64_t u = 0;
  for (int64_t i = 0; i < 2 * k; ++i) {
    if (u > 0 && work[u - 1].idx == work[i].idx) {
      work[u - 1].val = add_f32(work[u - 1].val, work[i].val);
    } else {
      work[u++] = work[i];
    }
  }
  qsort(work, (size_t)u, sizeof(pair_t), cmp_pair_rank);
  memcpy(a, work, (size_t)k * sizeof(pair_t)); /* u >= k: each side has k distinct */
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * gTop-k tournament on one host ([GTOPK]).
 * idx, val: P rows of k pairs (row p = worker p); indices distinct within a
 * row and inside [0, n).
 * out_idx/out_val: the surviving k pairs in (key desc, index asc) order.
 * out_mask[p*k + j] = 1 if idx[p*k + j] is one of the surviving indices.
 * *rounds_out (if non-null) receives the number of pairwise rounds played.
 * Returns 0, -1 for invalid input (bad sizes, index out of range, repeated
 * index within a row), -2 if memory runs out.
 */
int oracle_gtopk_merge(const int32_t* idx, const float* val, int32_t P, int64_t k, int64_t n,
                       int32_t* out_idx, float* out_val, uint8_t* out_mask, int32_t* rounds_out) {
  if (P < 1 || k < 0 || n < 0 || n > 0x7FFFFFFF || k > n) return -1;
  if (rounds_out) *rounds_out = 0;
  if (k == 0) return 0;
  size_t total = (size_t)P * (size_t)k;
  pair_t* slot = (pair_t*)malloc(total * sizeof(pair_t));
  pair_t* work = (pair_t*)malloc((size_t)(2 * k) * sizeof(pair_t));
  int32_t* sorted = (int32_t*)malloc((size_t)k * sizeof(int32_t));
  if (!slot || !work || !sorted) { free(slot); free(work); free(sorted); return -2; }

  /* precondition check: range and distinctness within each row */
  for (int32_t p = 0; p < P; ++p) {
    for (int64_t j = 0; j < k; ++j) {
      int32_t i = idx[(size_t)p * k + j];
      if (i < 0 || (int64_t)i >= n) { free(slot); free(work); free(sorted); return -1; }
      sorted[j] = i;
    }
    qsort(sorted, (size_t)k, sizeof(int32_t), cmp_i32);
    for (int64_t j = 1; j < k; ++j)
      if (sorted[j] == sorted[j - 1]) { free(slot); free(work); free(sorted); return -1; }
  }

  unsigned int mode = ieee_enter();
  for (size_t t = 0; t < total; ++t) { slot[t].idx = idx[t]; slot[t].val = val[t]; }

  int32_t rounds = 0;
  for (int64_t step = 1; step < P; step *= 2) {
    for (int64_t s = 0; s + step < P; s += 2 * step)
      merge_keep_topk(slot + (size_t)s * k, slot + (size_t)(s + step) * k, k, work);
    rounds += 1;
  }
  /* P == 1 plays no round; the single set is still reported in rank order */
  qsort(slot, (size_t)k, sizeof(pair_t), cmp_pair_rank);
  for (int64_t j = 0; j < k; ++j) { out_idx[j] = slot[j].idx; out_val[j] = slot[j].val; }

  for (int64_t j = 0; j < k; ++j) sorted[j] = slot[j].idx;
  qsort(sorted, (size_t)k, sizeof(int32_t), cmp_i32);
  for (size_t t = 0; t < total; ++t) {
    int32_t key = idx[t];
    out_mask[t] = bsearch(&key, sorted, (size_t)k, sizeof(int32_t), cmp_i32) != NULL;
  }
  if (rounds_out) *rounds_out = rounds;

  ieee_leave(mode);
  free(slot);
  free(work);
  free(sorted);
  return 0;
}

/* Reports the MXCSR bits the oracle relies on being clear during a call, as
   seen from inside one (FTZ | DAZ | rounding). Used by a self-test. */
unsigned int oracle_fp_mode_inside_call(void) {
  unsigned int mode = ieee_enter();
  unsigned int now = _mm_getcsr() & (0x8000u | 0x0040u | 0x6000u);
  ieee_leave(mode);
  return now;
}

/*
 * tgs.h -- C ABI of the MI355X (gfx950) error-feedback top-k gradient
 * sparsifier.
 *
 * The operations come from these web pages (cited by title and section):
 *   [EF]    arxivdaily listing for arXiv 2004.05298, entry "Sparsified SGD with
 *           Memory": top-k compression with the accumulated error kept in
 *           memory and added back before the next compression.
 *   [CONV]  same listing, entry "The Convergence of Sparsified Gradient
 *           Methods": sort by magnitude, send a subset, accumulate the rest
 *           locally.
 *   [SORT]  same listing, entry "Empirical Analysis on Top-k Gradient
 *           Sparsification for Distributed Deep Learning in a Supercomputing
 *           Environment": gradient sorting on the GPU is what makes top-k slow.
 *   [HT]    same listing, entry "Rethinking gradient sparsification as total
 *           error minimization": hard-threshold sparsifier (k set by a constant
 *           threshold) with error feedback.
 *   [LAYER] fugumt page for arXiv 2502.07634, related-paper entry "L-GreCo:
 *           Layerwise-Adaptive Gradient Compression for Efficient and
 *           Accurate Deep Learning": compression applied layer by layer, each
 *           layer with its own degree.
 *   [GTOPK] nubint review "A Distributed Synchronous SGD Algorithm with Global
 *           Top-k Sparsification for Low Bandwidth Networks", ABSTRACT and
 *           Method: global top-k of the largest |values| over P workers by an
 *           O(log P)-round tournament; only the selected indices survive.
 *   [EST]   arxivdaily listing, entry "Near-Optimal Sparse Allreduce for
 *           Distributed Deep Learning" (top-k picked through an estimated
 *           threshold rather than a sort); fugumt page for arXiv 2502.07634,
 *           related-paper entry "An Efficient Statistical-based Gradient
 *           Compression Technique for Distributed Training Systems"
 *           (threshold sparsification with an estimated threshold) and its
 *           Abstract (top-k's sorting costs offset what it saves).
 *   [RTOPK] arxivdaily listing, entry "rTop-k: A Statistical Estimation
 *           Approach to Distributed SGD": random-k chained after top-k.
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     keeps no pointer after the call returns and allocates no device memory.
 *   - Calls are asynchronous on `stream` (0 = the null stream); nothing waits
 *     for the device except tgs_check_device_error().
 *   - Only 4-byte alignment is required.  Inputs whose grad/residual
 *     pointers differ in alignment modulo 16 bytes take a slower scalar path.
 *   - n is at most 2^31 - 1, so every index fits in int32.  Indices are
 *     relative to the pointers passed.
 *   - `workspace` is caller-owned device memory of at least the size the
 *     matching *_workspace_bytes() query returns.  One workspace serves one
 *     call at a time; calls that share a workspace must be ordered (same
 *     stream).  Its first 32 KB (the header) hold the device error word and
 *     the synchronisation state of the top-k kernels; the rest is scratch.
 *     A workspace is ready after tgs_workspace_init() (a kernel, so it may
 *     sit in a captured graph) or after being zero-filled, and every call
 *     leaves it ready for the next one, on the host's order or replayed
 *     from a graph: the library keeps no state on the host.  Between calls
 *     the caller must not write to the header.  Any of the operations may
 *     use a workspace after any other.
 *   - Device error word (the header's first word): kernels only set bits in
 *     it, so it collects every problem since it was last read;
 *     tgs_check_device_error() reads and clears it.  After a report other
 *     than bad merge input, run tgs_workspace_init() before the next call.
 *   - Residency: the top-k kernels that synchronise their workgroups through
 *     memory (k_step, k_rank, k_general) size their grid to what fits on the device
 *     at once and assume every workgroup runs concurrently.  Kernels running
 *     on other streams at the same time can keep workgroups from starting;
 *     the waits are bounded, so the call then ends with wrong outputs and the
 *     wait-timeout bit (0x2) in the device error word, never a hang.  Run
 *     the top-k step while no other kernel occupies the device, or check
 *     the error word.
 *   - Magnitude order: key(x) = bits(x) & 0x7FFFFFFF as an unsigned integer.
 *     This matches |x| for every non-NaN value, ranks NaN above infinity and
 *     makes -0 and +0 equal.  Among equal keys the lower index comes first.
 *   - acc = residual + grad is one binary32 add, rounded to nearest even,
 *     never fused and never flushed to zero.
 *   - On a negative status nothing has been enqueued and the outputs are
 *     untouched; tgs_last_error() describes the reason.
 */
#ifndef TGS_H
#define TGS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tgs_status;
#define TGS_OK 0
#define TGS_EINVAL (-1)     /* bad size, null pointer, overlapping buffers, bad lambda */
#define TGS_EWORKSPACE (-2) /* workspace smaller than the query returned             */
#define TGS_EHIP (-3)       /* a HIP launch failed; see tgs_last_error()              */
#define TGS_EDEVICE (-4)    /* a kernel flagged a wait timeout or inconsistent counts */

/* Bytes of workspace tgs_topk_ef_step needs for this (n, k).  0 if the sizes
   are invalid. */
size_t tgs_topk_workspace_bytes(int64_t n, int64_t k);

/*
 * Error-feedback top-k step ([EF], [CONV]; the selection replaces the full
 * sort that [SORT] identifies as the bottleneck).  For k up to ~48k and
 * n >= 2^19 it is one kernel launch that reads grad and residual once;
 * n <= 2^18 with k <= 256 is one launch too; other sizes take an exact
 * radix-select path (three launches).  Every route gives the same result.
 *   grad      [n] float32, read only.
 *   residual  [n] float32, in/out: on entry the accumulated error, on exit
 *             acc with the selected entries set to +0.0f.
 *   k         0 <= k <= n entries are selected: the first k of all n indices
 *             ordered by (key(acc) descending, index ascending).
 *   out_idx   [k] int32, out: the selected indices in that order.
 *   out_val   [k] float32, out: acc at out_idx, bit for bit.
 * grad must not overlap residual or the outputs; the outputs must not overlap
 * each other or residual.  k == 0 only writes residual = acc.
 */
tgs_status tgs_topk_ef_step(const float* grad, float* residual, int64_t n, int64_t k,
                            int32_t* out_idx, float* out_val, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * tgs_topk_ef_step for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step, with no workspace argument.  Its workspace is a device array of
 * TGS_NOALLOC_WORKSPACE_BYTES inside the library, one per GPU, held until the
 * process ends; sizes whose tgs_topk_workspace_bytes(n, k) exceed it are
 * rejected with TGS_EINVAL.  The call allocates nothing: on a device's first
 * call it looks up that device's copy of the array and zero-fills its header
 * with a kernel on `stream`.  All calls on one GPU share the array (it keeps
 * the last call's contents), so calls that overlap in time on one GPU race:
 * order them on one stream.  Its device error word is not reachable; callers
 * that need it use tgs_topk_ef_step.
 */
#define TGS_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
tgs_status tgs_topk_ef_step_noalloc(const float* grad, float* residual, int64_t n, int64_t k, int32_t* out_idx,
                                    float* out_val, hipStream_t stream);

/* Bytes of workspace tgs_topk_ef_step_segmented needs for this segment table
   (HOST arrays, as below).  0 if the table is invalid. */
size_t tgs_topk_segmented_workspace_bytes(int32_t nseg, const int64_t* offsets, const int64_t* ks);

/*
 * Layer-wise error-feedback top-k ([LAYER] with [EF], [CONV]): the vector
 * grad/residual [offsets[nseg]] is cut into nseg segments (layers) and each
 * gets the top-k step of tgs_topk_ef_step with its own k, in one call.
 *   offsets   HOST int64 [nseg + 1]: segment s is [offsets[s], offsets[s+1]);
 *             offsets[0] == 0, nondecreasing, offsets[nseg] <= 2^31 - 1.
 *   ks        HOST int64 [nseg]: 0 <= ks[s] <= the segment's length.
 *   out_idx / out_val  [sum of ks]: segment s's pairs start at
 *             sum(ks[0..s)), in the order tgs_topk_ef_step gives them, with
 *             indices relative to the segment's start.
 * Segments of at most 2^18 entries with k <= 256 run together, up to 64 per
 * launch of one kernel; every other segment takes its own step.  The
 * results are those of one tgs_topk_ef_step call per segment.  Pointer and
 * overlap rules as tgs_topk_ef_step, over the whole vector and sum(ks).
 */
tgs_status tgs_topk_ef_step_segmented(const float* grad, float* residual, int32_t nseg,
                                      const int64_t* offsets, const int64_t* ks, int32_t* out_idx,
                                      float* out_val, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Bytes of workspace tgs_threshold_ef_step needs for this n (0 if invalid). */
size_t tgs_threshold_workspace_bytes(int64_t n);

/*
 * Hard-threshold step with error feedback ([HT]).
 *   An entry qualifies when key(acc_i) >= key((float)lambda); lambda must be a
 *   non-negative, non-NaN number.
 *   out_idx/out_val [capacity]: the first min(count, capacity) qualifying
 *             entries (i, acc_i) in ascending index order.
 *   d_count   device int64, out: the total number of qualifying entries
 *             (which may exceed capacity).
 *   residual  in/out: +0.0f at every emitted index, acc everywhere else
 *             (qualifying entries beyond the capacity keep acc).
 */
tgs_status tgs_threshold_ef_step(const float* grad, float* residual, int64_t n, float lambda,
                                 int32_t* out_idx, float* out_val, int64_t capacity,
                                 int64_t* d_count, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Bytes of workspace tgs_threshold_estimate needs for m samples (0 if m is
   outside [1, 2^24]).  A workspace of the larger of this and
   tgs_threshold_workspace_bytes(n) serves both calls of an estimated step. */
size_t tgs_threshold_estimate_workspace_bytes(int64_t m);

/*
 * Threshold estimate from a sample ([EST]), for the hard-threshold step.
 *   sample_idx [m] int32, device: positions in [0, n) (repeats allowed), for
 *             example drawn uniformly by the caller; 1 <= m <= 2^24.
 *   q         1 <= q <= m: the estimate is the q-th largest of
 *             key(residual[s_j] + grad[s_j]) over j < m (ties counted), so a
 *             target density rho takes q = ceil(rho * m).
 *   d_lambda  device float, out: the float whose bits are that key (>= 0).
 * grad and residual are only read.  A position outside [0, n) sets the
 * bad-input bit of the device error word (the estimate is then unspecified).
 * Two launches.  The workspace must be 256-byte aligned.
 */
tgs_status tgs_threshold_estimate(const float* grad, const float* residual, int64_t n, const int32_t* sample_idx,
                                  int64_t m, int64_t q, float* d_lambda, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * tgs_threshold_ef_step with the threshold read on the device ([HT] fed by
 * [EST]): an entry qualifies when key(acc_i) >= key(*d_lambda), read when the
 * kernels run (so tgs_threshold_estimate may write it earlier on the same
 * stream, with no host round trip).  Any bit pattern is accepted: the key of
 * a negative value is that of its magnitude; a NaN's key is only reached by
 * NaNs of at least its payload.  Everything else as tgs_threshold_ef_step.
 */
tgs_status tgs_threshold_ef_step_dev(const float* grad, float* residual, int64_t n, const float* d_lambda,
                                     int32_t* out_idx, float* out_val, int64_t capacity, int64_t* d_count,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace tgs_rtopk_ef_step needs (0 if the sizes are invalid). */
size_t tgs_rtopk_workspace_bytes(int64_t n, int64_t r, int64_t k);

/*
 * rTop-k step with error feedback ([RTOPK] with [EF]): k entries drawn
 * uniformly at random from the r of largest |acc|.
 *   0 <= k <= r <= n.  The top r are the first r by (key(acc) desc, index
 *   asc), as tgs_topk_ef_step finds them.  Entry i draws u_i = output word 0
 *   of Philox4x32-10 (Salmon et al., SC'11) at counter (i, step & 0xFFFFFFFF,
 *   step >> 32, 0) under key (seed & 0xFFFFFFFF, seed >> 32); the k of the top
 *   r with the smallest (u_i, i) are sent.
 *   out_idx/out_val [k]: the sent entries in (key desc, index asc) order,
 *             values bit for bit.
 *   residual  in/out: +0.0f at the k sent, acc everywhere else (the r - k
 *             passed over included).
 * r = k gives tgs_topk_ef_step's result.  Two more kernels follow the top-r
 * step's launches.  Pointer and overlap rules as tgs_topk_ef_step.
 */
tgs_status tgs_rtopk_ef_step(const float* grad, float* residual, int64_t n, int64_t r, int64_t k, uint64_t seed,
                             uint64_t step, int32_t* out_idx, float* out_val, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Bytes of workspace tgs_gtopk_merge needs (0 if the sizes are invalid). */
size_t tgs_gtopk_workspace_bytes(int32_t P, int64_t k, int64_t n);

/*
 * gTop-k tournament of P workers' sparse sets on one GPU ([GTOPK]).
 *   idx [P][k] int32, val [P][k] float32: worker p's k pairs, any order;
 *             indices must be distinct within a row and inside [0, n).
 *   Round r = 0, 1, ... while 2^r < P: slot s (s a multiple of 2^(r+1))
 *   absorbs slot s + 2^r when that slot exists: the union by index, values of
 *   a shared index added in binary32, keeps its first k entries by (key desc,
 *   index asc).  A slot without a partner passes through.
 *   out_idx/out_val [k]: slot 0 after the last round, in (key desc, index
 *             asc) order.
 *   out_mask [P][k] uint8: 1 where idx[p][j] is one of out_idx, else 0.
 * Rows that break the index precondition set a device error word; check it
 * with tgs_check_device_error (the outputs are then unspecified).
 * k is at most 2^20 and P k at most 2^31 - 1; the workspace must be 16-byte
 * aligned.  Each call starts by zero-filling the part of the workspace it
 * keeps its tables and counters in, so it assumes nothing of that part.
 */
tgs_status tgs_gtopk_merge(const int32_t* idx, const float* val, int32_t P, int64_t k, int64_t n,
                           int32_t* out_idx, float* out_val, uint8_t* out_mask, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Waits for `stream`, then reads and clears the device error word of
   `workspace`: TGS_OK if no kernel flagged a problem since it was last read,
   TGS_EINVAL for an input index outside its range (a merge row's index out
   of range or repeated, a sample position out of range), TGS_EDEVICE for a
   wait that timed out or inconsistent counts.  Works for every workspace.
   Synchronous: not for use inside graph capture. */
tgs_status tgs_check_device_error(const void* workspace, hipStream_t stream);

/* Makes `workspace` ready for any operation: zero-fills its header (the first
   min(workspace_bytes, 32 KB) bytes) with a kernel on `stream`.  Needed once
   for memory that is not zero-filled (and after a TGS_EDEVICE report); the
   calls themselves keep the workspace ready. */
tgs_status tgs_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* tgs_status_string(tgs_status s);

/* Thread-local description of the last failure on the calling thread ("" if
   none). */
const char* tgs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TGS_H */

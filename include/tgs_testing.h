/*
 * tgs_testing.h -- test and profiling controls of the MI355X error-feedback
 * top-k sparsifier library (libtgs.so).
 *
 * Not needed to use the library: the GPU parity tests force each route of the
 * top-k step through these controls, and the benchmark brackets a call with
 * events.  Every control is per calling thread, so a test that sets one on
 * its own thread never changes what calls on other threads do.
 */
#ifndef TGS_TESTING_H
#define TGS_TESTING_H

#include "tgs.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Controls, each set for the calling thread only (calls made on other
 * threads never see them).
 *   TGS_OPT_TOPK_PATH   0 = automatic, 1 = always the exact general path,
 *                       2 = fast path with a sample plan that cannot hold
 *                       (exercises the on-device fallback),
 *                       3 = fast path whose workgroups keep no local list
 *                       while streaming (every workgroup re-reads its rows),
 *                       4 = fast path whose workgroups keep every entry in
 *                       their local list (it overflows; they re-read),
 *                       5 = fast path whose workgroups may publish only one
 *                       candidate each (the plan fails; on-device fallback),
 *                       6 = fast path with one fixed slot per bucket and
 *                       workgroup (nearly every candidate goes through the
 *                       overflow area),
 *                       7 = guided general path whose guessed bin is the
 *                       highest one sampled (the guess fails; the general
 *                       path reads acc again),
 *                       8 = guided general path whose candidate regions
 *                       hold one pair (they overflow; the general path reads
 *                       acc again),
 *                       9 = guided general path (the accumulate pass copies
 *                       out the candidates of a sampled first-level bin)
 *                       where the fast path would otherwise run,
 *                       10 = layer-wise calls: every segment of the batched
 *                       path selects exactly from acc (as when its sampled
 *                       guess does not hold),
 *                       11 = layer-wise calls without the batched path (the
 *                       small-segment kernel and one step per segment),
 *                       12 = bucketed ranking (k >= 32768 beyond the
 *                       one-launch step) whose accumulate workgroups may
 *                       stage one candidate each: they overflow and the
 *                       general path selects from acc,
 *                       13 = no bucketed ranking: the guided general path
 *                       ranks the copied candidates itself,
 *                       14 = rTop-k: the pick's last workgroup selects over
 *                       the candidates in device memory instead of LDS (the
 *                       top-r step runs as with 0).
 *                       The guided path needs n >= 2^18, grad and residual
 *                       equally aligned modulo 16 bytes and k > 0; otherwise
 *                       7-9 run the plain general path.
 *   TGS_OPT_MAIN_GRID   0 = automatic, else the number of workgroups of the
 *                       streaming launch, capped at what can be resident;
 *                       below 65 the exact path runs (results must not
 *                       depend on it).
 */
#define TGS_OPT_TOPK_PATH 1
#define TGS_OPT_MAIN_GRID 2
tgs_status tgs_set_option(int32_t option, int64_t value);

/* One-shot profiling hook (calling thread only): the next tgs_topk_ef_step
   call on this thread records `start`
   right before its first launch and `stop` right after its last (the whole
   step); the next tgs_threshold_ef_step call brackets its streaming pass.
   Both on the call's stream.  Pass null events to clear. */
tgs_status tgs_profile_next_call(hipEvent_t start, hipEvent_t stop);

/* Milliseconds between two events recorded through tgs_profile_next_call
   (waits for `stop`).  TGS_EHIP if either has not completed. */
tgs_status tgs_profile_elapsed_ms(hipEvent_t start, hipEvent_t stop, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* TGS_TESTING_H */

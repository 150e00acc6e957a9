/*
 * msa_timeline.h — wall-clock marks along one decode step, exported only by
 * the timeline build of the library (libmsa_timeline.so: the same sources
 * compiled with -DMSA_TIMELINE; libmsa.so has neither these calls nor the
 * marks).
 *
 * The decode attention launch is a chain of dependent steps (selection,
 * block attention, hand-off, merge) whose cost is latency, which kernel
 * totals do not split.  In the timeline build, thread 0 of one watched
 * attention workgroup (sequence 0, group 0, slot 1) stores the chip's
 * constant 100 MHz clock (s_memrealtime) at each mark below; the merge mark
 * is stored by whichever workgroup merges group 0 of sequence 0, and the
 * index mark is the latest end of any decode index workgroup.  The marks of
 * the selection are stored on its fast path only (the path every randomly
 * drawn row takes).  A mark that was not reached reads 0.
 *
 * Every other entry point of msa.h behaves as in libmsa.so; each mark costs
 * one store by one thread.
 */
#ifndef MSA_TIMELINE_H
#define MSA_TIMELINE_H

#include <stdint.h>

#include "msa.h"

/* Mark numbers: entries of the array msa_timeline_read fills. */
#define MSA_MARK_START 0         /* attention workgroup begins */
#define MSA_MARK_SCORES_IN 1     /* selection: pooled scores loaded, thread maxima formed */
#define MSA_MARK_RANGE 2         /* selection: range of the thread maxima known (barrier) */
#define MSA_MARK_BIN 3           /* selection: histogram bin of the bound found (barriers) */
#define MSA_MARK_COUNTED 4       /* selection: candidates counted (barrier) */
#define MSA_MARK_GATHERED 5      /* selection: candidates gathered in LDS (barrier) */
#define MSA_MARK_SELECTED 6      /* selection: worst dropped or candidates sorted, written */
#define MSA_MARK_BLOCK_KNOWN 7   /* the workgroup's kept block is known */
#define MSA_MARK_KV_IN 8         /* block attention: page id read, K, Q and staged V in */
#define MSA_MARK_SCORES 9        /* block attention: scores and row maxima */
#define MSA_MARK_SOFTMAX 10      /* block attention: exponentials and row sums */
#define MSA_MARK_PV 11           /* block attention: P.V products issued */
#define MSA_MARK_WAVES_DONE 12   /* block attention: every wave done with V (barrier) */
#define MSA_MARK_COMBINED 13     /* block attention: wave outputs in LDS (barrier) */
#define MSA_MARK_STORED 14       /* partial stored, before the store wait */
#define MSA_MARK_COUNTED_IN 15   /* hand-off counter returned (barrier) */
#define MSA_MARK_MERGED 16       /* group 0 merged (by its last slot workgroup) */
#define MSA_MARK_INDEX_END 17    /* latest end of a decode index workgroup */
#define MSA_NUM_MARKS 18

#ifdef __cplusplus
extern "C" {
#endif

/* Sets every mark to 0 (on the current device; synchronises it).
 * MSA_ERR_HIP if the copy fails. */
msa_status msa_timeline_clear(void);

/* Copies the marks (MSA_NUM_MARKS values, in 10 ns ticks of the constant
 * clock) into the host array `marks` of `n` >= MSA_NUM_MARKS entries, after
 * the work that set them has finished (synchronises the current device).
 * MSA_ERR_INVALID_ARGUMENT for a NULL array or a short n; MSA_ERR_HIP if a
 * copy fails. */
msa_status msa_timeline_read(uint64_t *marks, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* MSA_TIMELINE_H */

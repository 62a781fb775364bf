/*
 * ps_sched.h -- C ABI of the multi-stream placement in libps: virtual ranks of
 * streams mapped onto a pool of GPUs (host-side; no device work).
 *
 * What it computes.  Each stream's per-stage work and state are packed into
 * virtual ranks, and virtual ranks are mapped onto physical GPUs, one memory
 * position each; on a GPU the tasks of the same block are batched across
 * chunks, steps and streams.  A new stream is placed on the remaining
 * capacity by Best-Fit and Limited Discrepancy Search, and admitted only if
 * all of its virtual ranks fit and it meets its SLO running alone; running
 * streams never move (AREX feed article on the PhysisServe report, section
 * "三层设计", layer 3; 163.com release, section "PhysisServe", bullets
 * "时分复用" and "虚拟 rank 的动态放置", Fig. 3 and Fig. 4).
 *
 * The model (readings where the pages are silent):
 *  - stages are (block b, step s) in block-major order p = b * n_steps + s, so
 *    that a rank holds whole blocks where it can and their steps batch
 *    together; a stream of R virtual ranks takes the groups of stages
 *    [floor(r N / R), floor((r + 1) N / R)), N = n_blocks * n_steps; R is the
 *    smallest count whose every group alone on a GPU meets the SLO, or a fixed
 *    count (finer ranks can fill capacity the fewest would leave);
 *  - a GPU's cycle (the chunk interval it sustains) is the sum over blocks, in
 *    block order, of f(n_b) = batch_fixed_ms + batch_task_ms * n_b for the
 *    n_b > 0 hosted tasks of block b;
 *  - a GPU may hold at most `positions` virtual ranks and its cycle must not
 *    exceed slo_ms;
 *  - Best-Fit orders the feasible GPUs for a rank by the slack slo_ms - cycle
 *    left after placing it, smallest first, ties to the lower GPU index; the
 *    ranks are placed in order 0..R-1; a discrepancy is any choice other than
 *    the first candidate; the search tries discrepancy limits 0..max_discrepancy
 *    in turn, depth first.
 *
 * Conventions as in ps.h: PS_OK or a negative ps_status, ps_last_error() for
 * the message; a handle is used from one host thread.
 */
#ifndef PS_SCHED_H_
#define PS_SCHED_H_

#include "ps.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ps_sched_desc {
  int32_t n_gpus;            /* physical GPUs, >= 1 */
  int32_t positions;         /* virtual ranks one GPU can hold, >= 1 */
  int32_t n_blocks;          /* Transformer blocks of the model, >= 1 */
  int32_t n_steps;           /* denoising steps, >= 1; n_blocks * n_steps <= 4096 */
  int32_t max_discrepancy;   /* LDS limit, >= 0 */
  int32_t ranks_per_stream;  /* 0: the fewest that meet the SLO alone; else exactly this many (<= stages) */
  double slo_ms;             /* chunk-interval target, > 0 */
  double batch_fixed_ms;     /* per-batch cost a, >= 0 */
  double batch_task_ms;      /* per-task cost b, > 0 */
} ps_sched_desc;

typedef struct ps_sched ps_sched;

/* Creates an empty placement over desc->n_gpus GPUs.  desc is read during the
 * call.  Errors: PS_ERR_INVALID_ARG for out-of-range fields. */
ps_status ps_sched_create(const ps_sched_desc* desc, ps_sched** out);
ps_status ps_sched_destroy(ps_sched* s);

/* Virtual ranks of a stream (*n_ranks = 0 if the split cannot meet the SLO
 * alone: then every stream is rejected). */
ps_status ps_sched_split(const ps_sched* s, int32_t* n_ranks);

/* Tries to admit stream `stream` (an id not currently admitted).  On
 * admission *n_ranks = R and gpu_of_rank[0..R) (host, capacity entries) holds
 * the GPU of each virtual rank; on rejection *n_ranks = 0 and nothing changes.
 * Errors: PS_ERR_INVALID_ARG for a null pointer, an id already admitted, or
 * capacity < the stream's rank count (nothing changes). */
ps_status ps_sched_admit(ps_sched* s, int64_t stream, int32_t* gpu_of_rank, int32_t capacity, int32_t* n_ranks);

/* Removes stream `stream`'s virtual ranks; *n_ranks = how many (0 if the id
 * was not admitted). */
ps_status ps_sched_release(ps_sched* s, int64_t stream, int32_t* n_ranks);

/* Occupancy of GPU `gpu`: virtual ranks held and the cycle in ms. */
ps_status ps_sched_gpu(const ps_sched* s, int32_t gpu, int32_t* n_ranks, double* cycle_ms);

#ifdef __cplusplus
}
#endif

#endif /* PS_SCHED_H_ */

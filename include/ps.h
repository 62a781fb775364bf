/*
 * ps.h -- C ABI of libps: the stage task of an autoregressive-denoising DiT
 * server, on one AMD Instinct MI355X (gfx950).
 *
 * What the calls compute.  A *stage* is one Transformer block at one denoising
 * step, and it is the unit of compute allocation (AREX feed article on the
 * PhysisServe report, section "三层设计", layer 1; 163.com release, section
 * "PhysisServe", bullet "Stage-wise 流水线").  Chunk c at step s reads the
 * still-noisy KV cache that earlier chunks left at that same step (AREX article,
 * section "难题"; 163.com release, section "新一代物理 AI 的基础设施", Fig. 1).
 * One GPU runs tasks of several stages in time slices and batches tasks of the
 * same block from different chunks and denoising steps against that block's
 * weights (AREX article, "三层设计", layer 2; 163.com release, bullet "时分复用",
 * Fig. 3; aicoder news, "Time-Shared Multi-Request Batching").
 *
 * Conventions for every call.
 *  - Return value: PS_OK (0) or a negative ps_status.  On failure nothing has
 *    been enqueued on the stream (see below) and ps_last_error() holds a
 *    message.
 *  - Arguments are validated on the host before any launch.  Calls that take a
 *    hipStream_t are asynchronous in that stream's order; a device fault shows
 *    up as PS_ERR_HIP on a later call.
 *  - Pointers named "device" must be device memory of the current HIP device;
 *    "host" pointers are read before the call returns.  The caller owns every
 *    tensor pointer it passes; the library owns handles, the KV pool, the
 *    cached timestep embeddings and the internal workspace.
 *  - Handles are not thread-safe: one handle is used from one host thread.
 *    ps_stage_batch calls on up to PS_MAX_STREAMS_PER_POOL different streams
 *    may run concurrently on the device (each stream has its own workspace in
 *    the pool), provided no batch reads or writes a KV slot that a concurrent
 *    batch writes; all other calls that share a handle are ordered on one
 *    stream.  Filling a timestep-embedding cache row (a timestep not cached)
 *    is stream-ordered: the fill waits on the device for the earlier reads of
 *    the row it replaces, and a call on another stream that reads the row
 *    waits on the device for the fill.  No call waits on the host, except
 *    the *_destroy calls, ps_kv_pool_release_stream and ps_trace_enable.
 *  - Calls that launch work may be captured into a HIP graph on a stream
 *    that an earlier, uncaptured call has set up: the timestep rows a call
 *    reads must already be cached and the stream's workspace large enough
 *    (else PS_ERR_UNSUPPORTED, nothing enqueued).  Reads of cached rows inside
 *    a graph are not tracked, so a graph must not be replayed after a row it
 *    reads has been replaced (keep the cache's capacity above the timesteps
 *    in use).  The arguments of a captured call are fixed in the graph.
 *  - A failing call enqueues nothing, with one exception: a HIP runtime
 *    failure part-way through a call's launches (PS_ERR_HIP) may leave the
 *    launches before it enqueued.
 *  - Element types: ps_dtype PS_BF16 (bfloat16) or PS_F32.  "compute dtype"
 *    means the dtype of the pool/block.  The residual stream (h) and the
 *    latents (x) are always fp32; biases, modulation tables and the timestep
 *    MLP are fp32.
 */
#ifndef PS_H_
#define PS_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ps_status;
#define PS_OK 0
#define PS_ERR_INVALID_ARG (-1)
#define PS_ERR_OUT_OF_MEMORY (-2)
#define PS_ERR_HIP (-3)
#define PS_ERR_SLOT_CONFLICT (-4)
#define PS_ERR_UNSUPPORTED (-5)

typedef int32_t ps_dtype;
#define PS_F32 0
#define PS_BF16 1

#define PS_MAX_WINDOW 8   /* most prior chunks one task may read */
#define PS_MAX_TASKS 32   /* most tasks in one ps_stage_batch call */
#define PS_MAX_STREAMS_PER_POOL 4   /* streams whose ps_stage_batch calls may overlap */
#define PS_FREQ_DIM 256   /* sinusoidal timestep features */

typedef struct ps_kv_pool ps_kv_pool;
typedef struct ps_block ps_block;
typedef struct ps_time_embed ps_time_embed;

/* ------------------------------------------------------------------ pool --
 * The noisy-KV pool: for every (stream, block, step) a ring of n_slots slots,
 * each holding one chunk's keys (after 3D RoPE) and values in the compute
 * dtype.  Chunk c at a step reads the entries of earlier chunks at that same
 * (block, step) (AREX article, "难题"; 163.com release, Fig. 1); the KV never
 * leaves the GPU that computed it (AREX article, "三层设计", layer 1).
 * Which slot a chunk uses is the caller's choice (ps_task); a ring of
 * window + k slots suffices for a schedule that admits k chunks per step per
 * tick.  The pool also holds, per (stream, block), the cross-attention keys
 * and values of that stream's conditioning tokens (ps_context_set).
 *
 * Token grid: a chunk has L = frames * rows * cols tokens, row-major
 * (token n = (f * rows + y) * cols + x); its frame coordinate for RoPE is
 * chunk * frames + f.  L must be a multiple of 8 and at least 64; n_ctx a
 * multiple of 8.
 * head_dim must be 64 or 128.  check_slots = 1 turns on the slot ledger:
 * each slot remembers which chunk wrote it, and ps_stage_batch rejects a task
 * whose read slots do not hold chunks c - n_read .. c - 1
 * (PS_ERR_SLOT_CONFLICT, nothing launched).
 */
typedef struct {
  int32_t n_streams, n_blocks, n_steps, n_slots;
  int32_t frames, rows, cols;
  int32_t n_heads, head_dim;
  int32_t max_ctx;          /* most conditioning tokens per stream */
  ps_dtype dtype;
  int32_t check_slots;
} ps_pool_desc;

/* Allocates the pool (device memory, uninitialised) and its RoPE tables.
 * Errors: PS_ERR_INVALID_ARG (bad sizes), PS_ERR_OUT_OF_MEMORY, PS_ERR_HIP. */
ps_status ps_kv_pool_create(const ps_pool_desc* desc, ps_kv_pool** out);
ps_status ps_kv_pool_destroy(ps_kv_pool* pool);
/* Waits for the work on hs and frees the workspace the pool keeps for calls
 * on hs (one of the PS_MAX_STREAMS_PER_POOL), so that another stream may take
 * its place.  A stream the pool has no workspace for is a no-op. */
ps_status ps_kv_pool_release_stream(ps_kv_pool* pool, hipStream_t hs);

/* Copies one chunk's cache entry into a slot, or out of it.
 * k, v: device, [L, n_heads, head_dim] row-major in the compute dtype (k after
 * RoPE).  chunk: the chunk id the ledger records for the slot (load only).
 * Used to pre-fill a pool and by tests; not needed on the hot path. */
ps_status ps_kv_pool_load(ps_kv_pool* pool, int32_t stream, int32_t block, int32_t step,
                          int32_t slot, int32_t chunk, const void* k, const void* v,
                          hipStream_t hs);
ps_status ps_kv_pool_fetch(const ps_kv_pool* pool, int32_t stream, int32_t block,
                           int32_t step, int32_t slot, void* k, void* v, hipStream_t hs);
/* Copies the cached cross-attention keys/values of (stream, block) out:
 * k, v device [n_ctx, n_heads, head_dim], compute dtype. */
ps_status ps_context_fetch(const ps_kv_pool* pool, int32_t stream, int32_t block,
                           void* k, void* v, hipStream_t hs);

/* ----------------------------------------------------------------- block --
 * A block's weights are shared by all its stages -- the block at every
 * denoising step -- which is what lets a GPU batch a block's tasks of
 * different chunks and steps against one copy of them (AREX article,
 * "三层设计", layer 2; aicoder news, "Time-Shared Multi-Request Batching":
 * heterogeneous denoising stages on one block).  The layout of the block is
 * that of the Wan-family backbones the pages evaluate (AREX article,
 * "实测数字"): AdaLN-modulated self-attention with a gate, cross-attention to
 * conditioning tokens, AdaLN-modulated GELU-tanh FFN with a gate.
 * One DiT block's weights, borrowed (device pointers, kept until
 * ps_block_destroy).  Linear weights are [out, in] row-major in the compute
 * dtype (y = x W^T + b).  With D = hidden, F = ffn:
 *   wqkv [3D, D] rows (q | k | v)   wo [D, D]
 *   wq2 [D, D]   wkv2 [2D, D] rows (k | v)   wo2 [D, D]
 *   w1 [F, D]    w2 [D, F]
 * Biases fp32: bqkv [3D], bo, bq2 [D], bkv2 [2D], bo2 [D], b1 [F], b2 [D].
 * tmod: fp32 [6, D], the block's additive modulation table T_b; a task at
 * timestep t uses m = e(t) + T_b with rows
 * (shift1, scale1, gate1, shift2, scale2, gate2).
 * block_index selects the block's region of the pool.
 * Requirements: hidden and ffn multiples of 64 (bf16) or 32 (fp32). */
typedef struct {
  int32_t hidden, n_heads, head_dim, ffn;
  int32_t block_index;
  ps_dtype dtype;
  const void *wqkv, *wo, *wq2, *wkv2, *wo2, *w1, *w2;
  const float *bqkv, *bo, *bq2, *bkv2, *bo2, *b1, *b2;
  const float* tmod;
} ps_block_desc;

ps_status ps_block_create(const ps_block_desc* desc, ps_block** out);
ps_status ps_block_destroy(ps_block* block);

/* ------------------------------------------------------ timestep embedding --
 * Tasks of one batch sit at different denoising steps, so each carries its
 * own timestep and modulation (AREX article, "三层设计", layer 2: tasks of
 * different chunks and denoising steps on one block).  Wan-style 6-way
 * modulation from a timestep embedding:
 * e(t) in R^{6 x D}, shared by all blocks:
 *   phi(t) = [cos(1000 t w_j) | sin(1000 t w_j)], w_j = 10000^(-j/128), j < 128
 *   u = SiLU(phi wt1^T + bt1) wt2^T + bt2;  e = SiLU(u) wp^T + bp.
 * Weights fp32, borrowed: wt1 [D, 256], bt1 [D], wt2 [D, D], bt2 [D],
 * wp [6D, D], bp [6D].  e(t) and u(t) are computed once per distinct t
 * (bitwise) and kept in a cache of `capacity` rows; the least recently used
 * row is replaced when the cache is full. */
typedef struct {
  int32_t hidden;
  int32_t capacity;
  const float *wt1, *bt1, *wt2, *bt2, *wp, *bp;
} ps_time_desc;

ps_status ps_time_embed_create(const ps_time_desc* desc, ps_time_embed** out);
ps_status ps_time_embed_destroy(ps_time_embed* te);
/* Writes e(t) (fp32 [6, D], device) -- computes it if not cached. */
ps_status ps_time_embed_get(ps_time_embed* te, float t, float* e, hipStream_t hs);

/* Timesteps of a schedule of n_steps denoising steps (the pages run four
 * steps per chunk -- AREX article, "实测数字" -- and give no values): the
 * uniform grid u = 1 - s / n_steps under the flow-matching time shift
 * t = a u / (1 + (a - 1) u), a = shift > 0 (a = 1 leaves it uniform).
 * out: host float [n_steps + 1], out[n_steps] = 0.  Host only. */
ps_status ps_timesteps(int32_t n_steps, float shift, float* out);

/* --------------------------------------------------------------- context --
 * Computes and caches the cross-attention keys/values of one stream's
 * conditioning tokens for one block: k2 = ctx wkv2[:D]^T + bkv2[:D],
 * v2 = ctx wkv2[D:]^T + bkv2[D:].  ctx: device [n_ctx, D], compute dtype.
 * n_ctx: 8 .. max_ctx, a multiple of 8.  Must precede any ps_stage_batch
 * whose tasks belong to that stream. */
ps_status ps_context_set(ps_kv_pool* pool, const ps_block* block, int32_t stream,
                         const void* ctx, int32_t n_ctx, hipStream_t hs);
/* Stores given cross-attention keys/values of (stream, block) instead:
 * k, v device [n_ctx, n_heads, head_dim], compute dtype; n_ctx as above. */
ps_status ps_context_load(ps_kv_pool* pool, int32_t stream, int32_t block, const void* k,
                          const void* v, int32_t n_ctx, hipStream_t hs);

/* ----------------------------------------------------------------- stage --
 * One stage task (host struct).  The task runs `block` at `step` for chunk
 * `chunk` of `stream`, with modulation e(timestep) + T_b.  Its keys/values go
 * to slot write_slot of (stream, block, step); its self-attention reads the
 * slots read_slots[0 .. n_read-1] (chronological, oldest first) followed by
 * its own write_slot. */
typedef struct {
  int32_t stream, chunk, step;
  float timestep;
  int32_t write_slot;
  int32_t n_read;
  int32_t read_slots[PS_MAX_WINDOW];
} ps_task;

/* Runs one block on a batch of stage tasks (tasks may mix chunks, steps and
 * streams):
 *   y  = LN(h)(1 + scale1) + shift1;  q, k, v = y Wqkv^T + bqkv;
 *   RoPE3D(q, k); (k, v) -> slot write_slot;
 *   h += gate1 * (SelfAttn(q, window keys/values) wo^T + bo)
 *   h += CrossAttn(LN(h) wq2^T + bq2, cached ctx keys/values) wo2^T + bo2
 *   h += gate2 * (GELU_tanh((LN(h)(1 + scale2) + shift2) w1^T + b1) w2^T + b2)
 * LN is per row without affine, eps 1e-6; attention scale 1/sqrt(head_dim).
 * All keys/values of the batch are written before any task reads (so a task
 * may read the slot another task of the same batch writes).
 * tasks: host [n_tasks].  h_in, h_out: device fp32 [n_tasks * L, D], task i
 * owning rows i*L .. i*L+L-1; h_in == h_out is allowed.  Two tasks may not
 * write the same slot, and a write slot may not be read by the same task.
 * Errors: PS_ERR_INVALID_ARG, PS_ERR_SLOT_CONFLICT (ledger on), PS_ERR_HIP,
 * PS_ERR_OUT_OF_MEMORY (workspace growth). */
ps_status ps_stage_batch(ps_kv_pool* pool, const ps_block* block, ps_time_embed* te,
                         const ps_task* tasks, int32_t n_tasks, const float* h_in,
                         float* h_out, hipStream_t hs);

/* ps_stage_batch for a batch whose tasks' hidden states are not one contiguous
 * slice: a GPU that hosts stage groups of several streams forms each block's
 * batch from whichever of their tasks are ready (163.com release, bullets
 * "时分复用" and "虚拟 rank 的动态放置", Fig. 3 right).  h_in[i], h_out[i]:
 * device fp32 [L, D] rows of task i (host arrays of n_tasks pointers, each
 * 16-byte aligned; h_in[i] == h_out[i] allowed, distinct tasks' rows must not
 * overlap).  The rows are gathered into the stream's workspace, run as one
 * batch and scattered back.  Errors as ps_stage_batch. */
ps_status ps_stage_batch_rows(ps_kv_pool* pool, const ps_block* block, ps_time_embed* te,
                              const ps_task* tasks, int32_t n_tasks, const float* const* h_in,
                              float* const* h_out, hipStream_t hs);

/* ps_stage_batch for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as ps_stage_batch; it neither allocates nor
 * frees device memory.  Its workspace is one fixed array of
 * PS_STATIC_SCRATCH_BYTES per device, held from the library's first use on
 * that device until the process ends: a batch whose workspace needs more
 * (about 43 MB per task at the 1.3B shape, 92 MB at the 14B shape) is
 * rejected with PS_ERR_INVALID_ARG before anything is enqueued.  Every call on
 * a device shares that device's array, so two calls that overlap on one
 * device (different streams, no ordering between them) race: order them. */
#define PS_STATIC_SCRATCH_BYTES (128u << 20)
ps_status ps_stage_batch_static(ps_kv_pool* pool, const ps_block* block, ps_time_embed* te,
                                const ps_task* tasks, int32_t n_tasks, const float* h_in,
                                float* h_out, hipStream_t hs);

/* Intermediate activations of one stage batch, for checking each kernel of
 * the path on its own.  Every member is a caller-owned device pointer or
 * NULL (not captured); row i*L + r belongs to task i, rows dense.  Members in
 * the compute dtype ("dt") are the values the next kernel consumes, as stored:
 *   y1    dt [n*L, D]  LN(h)(1 + scale1) + shift1
 *   q     dt [n*L, D]  self-attention queries after RoPE3D, multiplied by
 *                      log2(e)/sqrt(head_dim) (the softmax works in base 2)
 *   attn  dt [n*L, D]  self-attention output, before wo
 *   h1    fp32 [n*L, D] residual stream after the self-attention branch
 *   y2    dt [n*L, D]  LN(h1)
 *   q2    dt [n*L, D]  cross-attention queries, same scaling as q
 *   xattn dt [n*L, D]  cross-attention output, before wo2
 *   h2    fp32 [n*L, D] residual stream after the cross-attention branch
 *   y3    dt [n*L, D]  LN(h2)(1 + scale2) + shift2
 *   u     dt [n*L, F]  GELU_tanh(y3 w1^T + b1)
 * (AREX article on the PhysisServe report, section "三层设计": a stage is one
 * block at one step; the block's steps are those of ps_stage_batch.) */
typedef struct {
  void* y1;
  void* q;
  void* attn;
  float* h1;
  void* y2;
  void* q2;
  void* xattn;
  float* h2;
  void* y3;
  void* u;
} ps_stage_probe;

/* ps_stage_batch that also copies the intermediates `probe` asks for (device
 * to device, on hs, after the kernel that produces each).  Same arguments,
 * results and errors as ps_stage_batch, plus PS_ERR_INVALID_ARG for a NULL
 * probe.  The copies make it slower: it is for tests and debugging. */
ps_status ps_stage_batch_probe(ps_kv_pool* pool, const ps_block* block, ps_time_embed* te,
                               const ps_task* tasks, int32_t n_tasks, const float* h_in,
                               float* h_out, const ps_stage_probe* probe, hipStream_t hs);

/* One kernel of the stage on caller-given inputs, for checking each kernel
 * on identical inputs (the stage's steps are those of ps_stage_batch).  The
 * call does the batch's preamble (validation, timestep rows, modulation rows),
 * then runs kernel `kernel` with the launch configuration of ps_stage_batch:
 *   kernel               in (device, dense)        h_in          out (device, dense)
 *   PS_KERNEL_LN1        h fp32 [n*L, D]           -             y1 dt [n*L, D]
 *   PS_KERNEL_QKV        y1 dt [n*L, D]            -             q dt [n*L, D] (*)
 *   PS_KERNEL_ATTN_SELF  q dt [n*L, D] (*)         -             attn dt [n*L, D]
 *   PS_KERNEL_O_PROJ     attn dt [n*L, D]          h fp32        h1 fp32 [n*L, D]
 *   PS_KERNEL_LN2        h1 fp32                   -             y2 dt
 *   PS_KERNEL_XQ_PROJ    y2 dt                     -             q2 dt (*)
 *   PS_KERNEL_ATTN_CROSS q2 dt (*)                 -             xattn dt
 *   PS_KERNEL_XO_PROJ    xattn dt                  h1 fp32       h2 fp32
 *   PS_KERNEL_LN3        h2 fp32                   -             y3 dt
 *   PS_KERNEL_FFN1       y3 dt                     -             u dt [n*L, F]
 *   PS_KERNEL_FFN2       u dt [n*L, F]             h2 fp32       h_out fp32
 * (*) queries multiplied by log2(e)/sqrt(head_dim).  PS_KERNEL_QKV also
 * writes each task's keys/values into its write slot (and the slot ledger);
 * PS_KERNEL_ATTN_SELF reads the window's slots (ps_kv_pool_load fills them),
 * PS_KERNEL_ATTN_CROSS the (stream, block) context entry (ps_context_load).
 * h_in is required by the three residual kernels and ignored otherwise.
 * Errors as ps_stage_batch, plus PS_ERR_INVALID_ARG for an unknown kernel.
 * For tests: it copies its input and output, so it is not a fast path. */
#define PS_KERNEL_LN1 0
#define PS_KERNEL_QKV 1
#define PS_KERNEL_ATTN_SELF 2
#define PS_KERNEL_O_PROJ 3
#define PS_KERNEL_LN2 4
#define PS_KERNEL_XQ_PROJ 5
#define PS_KERNEL_ATTN_CROSS 6
#define PS_KERNEL_XO_PROJ 7
#define PS_KERNEL_LN3 8
#define PS_KERNEL_FFN1 9
#define PS_KERNEL_FFN2 10
ps_status ps_stage_kernel(ps_kv_pool* pool, const ps_block* block, ps_time_embed* te,
                          const ps_task* tasks, int32_t n_tasks, int32_t kernel, const void* in,
                          const float* h_in, void* out, hipStream_t hs);

/* ------------------------------------------------------------------ head --
 * The steps either side of the block stack (a Wan-style reading; the pages
 * evaluate Wan-family backbones -- AREX article on the PhysisServe report,
 * section "实测数字" -- whose latent frame of 60 x 104 in 2 x 2 patches is a
 * chunk's 30 x 52 token grid).  A chunk's latent is carried patchified:
 * x [tokens, P] fp32, P = latent channels x patch volume, a token's values
 * ordered (channel, frame, row, col) inside its patch.
 *   patch embedding: h0 = x w_embed^T + b_embed (a 3D convolution whose kernel
 *   and stride are the patch, written as a linear map);
 *   output head: (shift, scale) = u(t) + t_head, u(t) the timestep MLP output
 *   (see the timestep embedding); v = (LN(h)(1 + scale) + shift) w_head^T + b_head.
 * Weights borrowed until ps_head_destroy: w_embed [D, P] and w_head [P, D]
 * in the compute dtype ([out, in]); b_embed [D], b_head [P], t_head [2, D]
 * fp32.  Requirements: D and P multiples of 64 (bf16) or 32 (fp32). */
typedef struct {
  int32_t hidden;      /* D */
  int32_t latent_dim;  /* P */
  ps_dtype dtype;
  const void *w_embed, *w_head;
  const float *b_embed, *b_head, *t_head;
} ps_head_desc;

typedef struct ps_head ps_head;

ps_status ps_head_create(const ps_head_desc* desc, ps_head** out);
ps_status ps_head_destroy(ps_head* head);

/* h0 of n_rows tokens: x device fp32 [n_rows, P] -> h device fp32 [n_rows, D].
 * The library's workspace for the compute-dtype copy of x grows on demand
 * (PS_ERR_OUT_OF_MEMORY if it cannot). */
ps_status ps_patch_embed(ps_head* head, const float* x, float* h, int32_t n_rows, hipStream_t hs);

/* v of a batch of tasks: task i (rows i*tokens .. i*tokens+tokens-1 of h)
 * uses timestep t[i] (host fp32 [n_tasks]); h device fp32 [n_tasks * tokens,
 * D] -> v device fp32 [n_tasks * tokens, P].  te: the shared timestep
 * embedding, whose cache also keeps u(t).  Errors as ps_patch_embed, and
 * PS_ERR_INVALID_ARG if te's width is not D or a t[i] is not finite. */
ps_status ps_output_head(ps_head* head, ps_time_embed* te, const float* t, int32_t n_tasks,
                         int32_t tokens, const float* h, float* v, hipStream_t hs);

/* ----------------------------------------------------------------- euler --
 * Each chunk passes its denoising steps one after another, step s + 1
 * starting from the latent step s produced (AREX article, "难题"; 163.com
 * release, "新一代物理 AI 的基础设施", Fig. 1).  The update between steps is
 * the flow-matching Euler step of the Wan-family backbones the pages name.
 * Flow-matching Euler step after the last block: for task i,
 *   x[i] <- x[i] - dt[i] * v[i],  dt[i] = t_s - t_{s+1} (t_S = 0).
 * x: device fp32 [n_tasks * tokens, hidden]; v: device [n_tasks * tokens,
 * hidden] of v_dtype (PS_F32 or PS_BF16); dt: host fp32 [n_tasks]. */
ps_status ps_euler_update(float* x, const void* v, const float* dt, int32_t n_tasks,
                          int32_t tokens, int32_t hidden, ps_dtype v_dtype,
                          hipStream_t hs);
/* The same step with dt taken from the schedule: task i is at step steps[i]
 * of timesteps[0 .. n_steps - 1] (host float; t_{n_steps} = 0), so that
 * dt[i] = timesteps[steps[i]] - timesteps[steps[i] + 1] in fp32.  steps: host
 * int32 [n_tasks], each in [0, n_steps). */
ps_status ps_euler_update_steps(float* x, const void* v, const float* timesteps, int32_t n_steps,
                                const int32_t* steps, int32_t n_tasks, int32_t tokens,
                                int32_t hidden, ps_dtype v_dtype, hipStream_t hs);

/* Message of the last failure on this host thread ("" if none). */
const char* ps_last_error(void);

/* ----------------------------------------------------------------- trace --
 * Per-kernel timing of the stage path.  While tracing is on, every kernel
 * that ps_stage_batch and ps_euler_update launch is bracketed by HIP events
 * recorded on the caller's stream; ps_trace_collect() waits for the pending
 * events and adds each kernel's duration to its named entry.  Names:
 * "put_tasks", "modulation", "ln1", "qkv", "attn_self", "o_proj", "ln2",
 * "xq_proj", "attn_cross", "xo_proj", "ln3", "ffn1", "ffn2", "euler".
 * ps_trace_enable(1) clears the statistics; tracing adds an event pair per
 * kernel, so it is off by default. */
ps_status ps_trace_enable(int32_t on);
ps_status ps_trace_collect(void);
int32_t ps_trace_count(void);
/* Entry i (0 .. count-1): name (static string), launches, total milliseconds. */
ps_status ps_trace_entry(int32_t i, const char** name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* PS_H_ */

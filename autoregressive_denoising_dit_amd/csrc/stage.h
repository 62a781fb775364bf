// The steps of a stage call that every stage entry point shares (internal;
// not part of the ABI): validation, workspace layout, the batch preamble and
// the launch sequence of the stage's kernels.
#pragma once

#include "common.h"

namespace ps {

// A validated batch: the device image of its tasks and the pool slots it writes.
struct Batch {
  TaskTable tt{};
  int n = 0;
  size_t writes[PS_MAX_TASKS] = {};
  float t[PS_MAX_TASKS] = {};
};

// Workspace of one stage call, in device memory.
struct WsPtrs {
  float* mod = nullptr;      // [n][6][D] fp32
  float2* rope = nullptr;    // [n][frames][seg_f / 2]
  void* y = nullptr;         // [n L][D + 64] LN outputs
  void* q = nullptr;         // [n L][D] queries
  void* a = nullptr;         // [n L][D + 64] attention outputs
  void* u = nullptr;         // [n L][F + 64] FFN hidden
  DevTask* tasks = nullptr;  // [PS_MAX_TASKS]
};

// Bytes of the seven workspace buffers, in WsPtrs order.
struct WsSizes {
  size_t b[7];
};

// Every check of a stage call; nothing is enqueued or changed.
ps_status prepare_batch(const ps_kv_pool* p, const ps_block* b, const ps_time_embed* te, const ps_task* tasks,
                        int32_t n, const void* h_in, const void* h_out, const char* fn, Batch* out);
WsSizes ws_sizes(const ps_kv_pool* p, const ps_block* b, int n);
// Bytes of one contiguous region holding all buffers (each 256-byte aligned).
size_t ws_total(const WsSizes& z);
// The buffers laid out from base (ws_total(z) bytes, 256-byte aligned).
WsPtrs ws_carve(char* base, const WsSizes& z);
// Timestep rows, task table, modulation rows and RoPE frame table of the batch.
ps_status begin_batch(const ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const Batch& bt, const WsPtrs& w,
                      hipStream_t hs);
// All kernels of the stage: h_out = Block(h_in) (h_in == h_out allowed).
ps_status run_stage_all(ps_kv_pool* p, const ps_block* b, const WsPtrs& w, int n, const float* h_in, float* h_out,
                        hipStream_t hs);
// Records the batch's cache writes in the pool's slot ledger.
void commit_writes(ps_kv_pool* p, const Batch& bt, const ps_task* tasks);
// Sets the thread's error message and returns st.
ps_status set_error(ps_status st, const char* msg);

}  // namespace ps

// ps_stage_batch_static: the stage call for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops that must not
// call hipMalloc).  Its workspace is a fixed array in the library's device
// memory instead of the pool's per-stream buffers; the kernels and the launch
// sequence are those of ps_stage_batch.
#include <stdio.h>

#include <mutex>

#include "common.h"
#include "stage.h"

using namespace ps;

namespace {

// One copy per device, held from the library's first use on that device
// until the process ends.  Host code reaches it only through the address
// hipGetSymbolAddress returns on each device: the array's name on the host is
// a stand-in, not a device address.
__device__ __align__(256) unsigned char scratch[PS_STATIC_SCRATCH_BYTES];

ps_status err(ps_status st, const char* fmt, size_t a = 0, size_t b = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, fmt, a, b);
  return set_error(st, buf);
}

// Device address of this device's copy of `scratch`, looked up once per device
// with that device current.
ps_status scratch_ptr(char** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(PS_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return err(PS_ERR_UNSUPPORTED, "ps_stage_batch_static: device %zu beyond 64", (size_t)dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !q) {
      (void)hipGetLastError();
      return set_error(PS_ERR_HIP, "ps_stage_batch_static: hipGetSymbolAddress of the static workspace failed");
    }
    ptr[dev] = q;
  }
  *out = static_cast<char*>(ptr[dev]);
  return PS_OK;
}

}  // namespace

extern "C" ps_status ps_stage_batch_static(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks,
                                           int32_t n, const float* h_in, float* h_out, hipStream_t hs) {
  Batch bt;
  ps_status st = prepare_batch(p, b, te, tasks, n, h_in, h_out, "ps_stage_batch_static", &bt);
  if (st) return st;
  const WsSizes z = ws_sizes(p, b, n);
  const size_t need = ws_total(z);
  if (need > (size_t)PS_STATIC_SCRATCH_BYTES)
    return err(PS_ERR_INVALID_ARG,
               "ps_stage_batch_static: the batch needs %zu bytes of workspace, more than the static %zu",
               need, (size_t)PS_STATIC_SCRATCH_BYTES);
  char* base = nullptr;
  if ((st = scratch_ptr(&base))) return st;
  // every workspace byte a kernel reads is written earlier in the same call
  // (task table, modulation rows, then each activation before its consumer),
  // so nothing needs clearing between calls
  const WsPtrs w = ws_carve(base, z);
  if ((st = begin_batch(p, b, te, bt, w, hs))) return st;
  if ((st = run_stage_all(p, b, w, n, h_in, h_out, hs))) return st;
  commit_writes(p, bt, tasks);
  return PS_OK;
}

// C ABI of libps: handles, host-side validation, the slot ledger, the
// timestep-embedding cache and the launch sequence of one stage batch.
// Every check runs before the first launch, so a failing call enqueues nothing.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <cstdarg>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "stage.h"

using namespace ps;

namespace {

thread_local std::string g_err;

ps_status fail(ps_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace

// error reporting for the host-only parts of the library (placement)
namespace ps {
ps_status set_error(ps_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace ps

namespace {

#define PS_HIP(call)                                                                 \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) return fail(PS_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

size_t elt_size(ps_dtype t) { return t == PS_BF16 ? 2 : 4; }

// A device buffer that grows on demand (old contents are not kept).  Growth
// is stream-ordered: the old buffer is freed and the new one allocated on the
// stream whose calls use the buffer (hipFreeAsync / hipMallocAsync), so that
// growing never waits for the device.  Where the device has no stream-ordered
// allocator, the old buffer is freed after that stream alone has drained.
struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
  bool async = false;   // p came from hipMallocAsync
  void drop(hipStream_t s) {
    if (!p) return;
    if (async) {
      (void)hipFreeAsync(p, s);
    } else {
      (void)hipStreamSynchronize(s);
      (void)hipFree(p);
    }
    p = nullptr;
    bytes = 0;
  }
  ps_status reserve(size_t need, hipStream_t s) {
    if (need <= bytes) return PS_OK;
    drop(s);
    void* q = nullptr;
    hipError_t e = hipMallocAsync(&q, need, s);
    if (e == hipSuccess) {
      async = true;
    } else {
      (void)hipGetLastError();
      async = false;
      if (hipMalloc(&q, need) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PS_ERR_OUT_OF_MEMORY, "workspace: cannot allocate %zu bytes", need);
      }
    }
    p = q;
    bytes = need;
    return PS_OK;
  }
  // after all work that uses the buffer has completed
  void release() { drop(nullptr); }
};

// ---------------------------------------------------------------- tracing
struct TraceEntry {
  const char* name;
  int64_t launches = 0;
  double total_ms = 0.0;
};
struct Pending {
  int entry;
  hipEvent_t a, b;
};
struct Trace {
  bool on = false;
  std::vector<TraceEntry> entries;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> spare;
  int find(const char* name) {
    for (size_t i = 0; i < entries.size(); ++i)
      if (strcmp(entries[i].name, name) == 0) return (int)i;
    entries.push_back(TraceEntry{name});
    return (int)entries.size() - 1;
  }
  hipEvent_t take() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
  }
};
Trace g_trace;

// Brackets one launch with events when tracing is on.
struct TraceScope {
  hipStream_t s;
  int entry = -1;
  hipEvent_t a = nullptr;
  TraceScope(const char* name, hipStream_t st) : s(st) {
    if (!g_trace.on) return;
    entry = g_trace.find(name);
    a = g_trace.take();
    (void)hipEventRecord(a, s);
  }
  ~TraceScope() {
    if (entry < 0) return;
    hipEvent_t b = g_trace.take();
    (void)hipEventRecord(b, s);
    g_trace.pending.push_back(Pending{entry, a, b});
  }
};

}  // namespace

#define PS_TRACED(name, call)          \
  do {                                 \
    TraceScope ts_(name, hs);          \
    PS_HIP(call);                      \
  } while (0)

extern "C" ps_status ps_trace_enable(int32_t on) {
  (void)hipDeviceSynchronize();
  for (auto& p : g_trace.pending) {
    g_trace.spare.push_back(p.a);
    g_trace.spare.push_back(p.b);
  }
  g_trace.pending.clear();
  g_trace.entries.clear();
  g_trace.on = on != 0;
  return PS_OK;
}

extern "C" ps_status ps_trace_collect(void) {
  for (auto& p : g_trace.pending) {
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return fail(PS_ERR_HIP, "ps_trace_collect: %s", hipGetErrorString(e));
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, p.a, p.b);
    g_trace.entries[p.entry].launches += 1;
    g_trace.entries[p.entry].total_ms += ms;
    g_trace.spare.push_back(p.a);
    g_trace.spare.push_back(p.b);
  }
  g_trace.pending.clear();
  return PS_OK;
}

extern "C" int32_t ps_trace_count(void) { return (int32_t)g_trace.entries.size(); }

extern "C" ps_status ps_trace_entry(int32_t i, const char** name, int64_t* launches, double* total_ms) {
  if (i < 0 || i >= (int32_t)g_trace.entries.size() || !name || !launches || !total_ms)
    return fail(PS_ERR_INVALID_ARG, "ps_trace_entry: bad index or null argument");
  *name = g_trace.entries[i].name;
  *launches = g_trace.entries[i].launches;
  *total_ms = g_trace.entries[i].total_ms;
  return PS_OK;
}

struct ps_kv_pool {
  ps_pool_desc desc{};
  int device = 0;
  void* kv = nullptr;
  void* ctx = nullptr;
  float2* rope_y = nullptr;
  float2* rope_x = nullptr;
  int seg_f = 0, seg_h = 0, seg_w = 0;
  int64_t slot_elems = 0, ctx_elems = 0;
  std::vector<int> ctx_len;   // per (stream, block); 0 = context not set
  std::vector<int> ledger;    // per (region, slot): chunk id, -1 = empty
  // Workspace of the calls on one HIP stream.  Batches submitted on
  // different streams get different workspaces, so they may run
  // concurrently (the caller keeps their KV slots apart).
  struct Workspace {
    hipStream_t stream = nullptr;
    DevBuf mod, rope, y, q, a, u, tasks, h;
    void release() {
      for (DevBuf* b : {&mod, &rope, &y, &q, &a, &u, &tasks, &h}) b->release();
    }
  };
  std::vector<Workspace*> ws;
  Workspace* workspace(hipStream_t s) {
    for (Workspace* w : ws)
      if (w->stream == s) return w;
    if ((int)ws.size() >= PS_MAX_STREAMS_PER_POOL) return nullptr;
    Workspace* w = new (std::nothrow) Workspace;
    if (!w) return nullptr;
    w->stream = s;
    ws.push_back(w);
    return w;
  }
  int L() const { return desc.frames * desc.rows * desc.cols; }
  int D() const { return desc.n_heads * desc.head_dim; }
  PoolGeo geo() const {
    PoolGeo g{};
    g.kv = kv;
    g.ctx = ctx;
    g.slot_elems = slot_elems;
    g.ctx_elems = ctx_elems;
    g.n_slots = desc.n_slots;
    g.L = L();
    g.H = desc.n_heads;
    g.d = desc.head_dim;
    g.max_ctx = desc.max_ctx;
    g.frames = desc.frames;
    g.rows = desc.rows;
    g.cols = desc.cols;
    g.seg_f = seg_f;
    g.seg_h = seg_h;
    g.seg_w = seg_w;
    g.rope_y = rope_y;
    g.rope_x = rope_x;
    g.div_L = FastDiv((uint32_t)L());
    g.div_plane = FastDiv((uint32_t)(desc.rows * desc.cols));
    g.div_cols = FastDiv((uint32_t)desc.cols);
    g.div_rows = FastDiv((uint32_t)desc.rows);
    return g;
  }
};

struct ps_block {
  ps_block_desc d{};
};

// Streams whose calls read rows of a timestep cache; each has an event that
// is recorded after its latest read, so that a row is refilled only after
// every read of its old contents (stream-ordered: no host wait).
constexpr int TE_STREAMS = 16;

struct ps_time_embed {
  ps_time_desc d{};
  float* cache = nullptr;      // [capacity][6][D]: e(t)
  float* cache_u = nullptr;    // [capacity][D]: u(t), the timestep MLP output
  float* scratch = nullptr;    // 256 + 2 D floats
  std::vector<uint32_t> key;
  std::vector<uint64_t> used;
  std::vector<char> valid;
  uint64_t clock = 0;
  std::vector<hipEvent_t> fill_ev;        // per row: recorded after its fill
  std::vector<hipStream_t> fill_stream;   // per row: the stream of its fill
  std::vector<uint32_t> readers;          // per row: stream slots that read it since its fill
  hipStream_t rd_stream[TE_STREAMS] = {};
  hipEvent_t rd_ev[TE_STREAMS] = {};
  bool rd_used[TE_STREAMS] = {};
  hipEvent_t scratch_ev = nullptr;        // recorded after the latest fill (the scratch is free)
  hipStream_t scratch_stream = nullptr;
  bool scratch_rec = false;
};

extern "C" const char* ps_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------- pool
extern "C" ps_status ps_kv_pool_create(const ps_pool_desc* desc, ps_kv_pool** out) {
  if (!desc || !out) return fail(PS_ERR_INVALID_ARG, "ps_kv_pool_create: null argument");
  const ps_pool_desc& d = *desc;
  if (d.n_streams <= 0 || d.n_blocks <= 0 || d.n_steps <= 0 || d.n_slots <= 0)
    return fail(PS_ERR_INVALID_ARG, "pool: n_streams, n_blocks, n_steps, n_slots must be > 0");
  if (d.frames <= 0 || d.rows <= 0 || d.cols <= 0)
    return fail(PS_ERR_INVALID_ARG, "pool: token grid must be positive");
  const long long L = (long long)d.frames * d.rows * d.cols;
  if (L % 8 != 0 || L < 64 || L > (1 << 20))
    return fail(PS_ERR_INVALID_ARG, "pool: tokens per chunk (%lld) must be a multiple of 8, at least 64", L);
  if (d.head_dim != 64 && d.head_dim != 128) return fail(PS_ERR_INVALID_ARG, "pool: head_dim must be 64 or 128");
  if (d.n_heads <= 0 || d.n_heads * d.head_dim > 8192) return fail(PS_ERR_INVALID_ARG, "pool: bad n_heads");
  if (d.max_ctx <= 0 || d.max_ctx % 8 != 0) return fail(PS_ERR_INVALID_ARG, "pool: max_ctx must be a positive multiple of 8");
  if (d.dtype != PS_BF16 && d.dtype != PS_F32) return fail(PS_ERR_INVALID_ARG, "pool: bad dtype");
  if (d.n_slots > 64) return fail(PS_ERR_INVALID_ARG, "pool: at most 64 slots per ring");

  ps_kv_pool* p = new ps_kv_pool();
  p->desc = d;
  (void)hipGetDevice(&p->device);
  const int s = d.head_dim / 6;
  p->seg_f = d.head_dim - 4 * s;
  p->seg_h = 2 * s;
  p->seg_w = 2 * s;
  const size_t es = elt_size(d.dtype);
  p->slot_elems = 2LL * d.n_heads * L * d.head_dim;
  p->ctx_elems = 2LL * d.n_heads * d.max_ctx * d.head_dim;
  const size_t n_regions = (size_t)d.n_streams * d.n_blocks * d.n_steps;
  const size_t kv_bytes = n_regions * d.n_slots * p->slot_elems * es;
  const size_t ctx_bytes = (size_t)d.n_streams * d.n_blocks * p->ctx_elems * es;
  auto cleanup = [&]() {
    if (p->kv) (void)hipFree(p->kv);
    if (p->ctx) (void)hipFree(p->ctx);
    if (p->rope_y) (void)hipFree(p->rope_y);
    if (p->rope_x) (void)hipFree(p->rope_x);
    (void)hipGetLastError();
    delete p;
  };
  if (hipMalloc(&p->kv, kv_bytes) != hipSuccess || hipMalloc(&p->ctx, ctx_bytes) != hipSuccess ||
      hipMalloc(&p->rope_y, sizeof(float2) * d.rows * (p->seg_h / 2) + 16) != hipSuccess ||
      hipMalloc(&p->rope_x, sizeof(float2) * d.cols * (p->seg_w / 2) + 16) != hipSuccess) {
    cleanup();
    return fail(PS_ERR_OUT_OF_MEMORY, "pool: cannot allocate %zu + %zu bytes", kv_bytes, ctx_bytes);
  }
  hipError_t e = launch_rope_table(p->rope_y, d.rows, p->seg_h, 0);
  if (e == hipSuccess) e = launch_rope_table(p->rope_x, d.cols, p->seg_w, 0);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    cleanup();
    return fail(PS_ERR_HIP, "pool: RoPE tables: %s", hipGetErrorString(e));
  }
  p->ctx_len.assign((size_t)d.n_streams * d.n_blocks, 0);
  p->ledger.assign(n_regions * d.n_slots, -1);
  *out = p;
  return PS_OK;
}

extern "C" ps_status ps_kv_pool_destroy(ps_kv_pool* p) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "ps_kv_pool_destroy: null pool");
  (void)hipDeviceSynchronize();
  (void)hipFree(p->kv);
  (void)hipFree(p->ctx);
  (void)hipFree(p->rope_y);
  (void)hipFree(p->rope_x);
  for (auto* w : p->ws) {
    w->release();
    delete w;
  }
  p->ws.clear();
  delete p;
  return PS_OK;
}

extern "C" ps_status ps_kv_pool_release_stream(ps_kv_pool* p, hipStream_t hs) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "ps_kv_pool_release_stream: null pool");
  for (size_t i = 0; i < p->ws.size(); ++i) {
    if (p->ws[i]->stream != hs) continue;
    PS_HIP(hipStreamSynchronize(hs));
    p->ws[i]->release();
    delete p->ws[i];
    p->ws.erase(p->ws.begin() + i);
    return PS_OK;
  }
  return PS_OK;
}

static ps_status check_region(const ps_kv_pool* p, int stream, int block, int step, int slot) {
  const ps_pool_desc& d = p->desc;
  if (stream < 0 || stream >= d.n_streams) return fail(PS_ERR_INVALID_ARG, "stream %d out of range", stream);
  if (block < 0 || block >= d.n_blocks) return fail(PS_ERR_INVALID_ARG, "block %d out of range", block);
  if (step < 0 || step >= d.n_steps) return fail(PS_ERR_INVALID_ARG, "step %d out of range", step);
  if (slot < 0 || slot >= d.n_slots) return fail(PS_ERR_INVALID_ARG, "slot %d out of range", slot);
  return PS_OK;
}

static size_t region_of(const ps_kv_pool* p, int stream, int block, int step) {
  return ((size_t)stream * p->desc.n_blocks + block) * p->desc.n_steps + step;
}

extern "C" ps_status ps_kv_pool_load(ps_kv_pool* p, int32_t stream, int32_t block, int32_t step, int32_t slot,
                                     int32_t chunk, const void* k, const void* v, hipStream_t hs) {
  if (!p || !k || !v) return fail(PS_ERR_INVALID_ARG, "ps_kv_pool_load: null argument");
  ps_status st = check_region(p, stream, block, step, slot);
  if (st) return st;
  if (chunk < 0) return fail(PS_ERR_INVALID_ARG, "ps_kv_pool_load: chunk must be >= 0");
  const size_t r = region_of(p, stream, block, step);
  const size_t off = (r * p->desc.n_slots + slot) * p->slot_elems;
  const int L = p->L(), H = p->desc.n_heads, d = p->desc.head_dim;
  if (p->desc.dtype == PS_BF16)
    PS_HIP(launch_entry_load<bf16>(static_cast<bf16*>(p->kv) + off, static_cast<const bf16*>(k),
                                   static_cast<const bf16*>(v), L, L, H, d, hs));
  else
    PS_HIP(launch_entry_load<float>(static_cast<float*>(p->kv) + off, static_cast<const float*>(k),
                                    static_cast<const float*>(v), L, L, H, d, hs));
  p->ledger[r * p->desc.n_slots + slot] = chunk;
  return PS_OK;
}

extern "C" ps_status ps_kv_pool_fetch(const ps_kv_pool* p, int32_t stream, int32_t block, int32_t step,
                                      int32_t slot, void* k, void* v, hipStream_t hs) {
  if (!p || !k || !v) return fail(PS_ERR_INVALID_ARG, "ps_kv_pool_fetch: null argument");
  ps_status st = check_region(p, stream, block, step, slot);
  if (st) return st;
  const size_t r = region_of(p, stream, block, step);
  const size_t off = (r * p->desc.n_slots + slot) * p->slot_elems;
  const int L = p->L(), H = p->desc.n_heads, d = p->desc.head_dim;
  if (p->desc.dtype == PS_BF16)
    PS_HIP(launch_entry_fetch<bf16>(static_cast<const bf16*>(p->kv) + off, static_cast<bf16*>(k),
                                    static_cast<bf16*>(v), L, L, H, d, hs));
  else
    PS_HIP(launch_entry_fetch<float>(static_cast<const float*>(p->kv) + off, static_cast<float*>(k),
                                     static_cast<float*>(v), L, L, H, d, hs));
  return PS_OK;
}

extern "C" ps_status ps_context_fetch(const ps_kv_pool* p, int32_t stream, int32_t block, void* k, void* v,
                                      hipStream_t hs) {
  if (!p || !k || !v) return fail(PS_ERR_INVALID_ARG, "ps_context_fetch: null argument");
  ps_status st = check_region(p, stream, block, 0, 0);
  if (st) return st;
  const size_t cr = (size_t)stream * p->desc.n_blocks + block;
  const int n = p->ctx_len[cr];
  if (n == 0) return fail(PS_ERR_INVALID_ARG, "ps_context_fetch: context of stream %d block %d not set", stream, block);
  const size_t off = cr * p->ctx_elems;
  const int H = p->desc.n_heads, d = p->desc.head_dim;
  if (p->desc.dtype == PS_BF16)
    PS_HIP(launch_entry_fetch<bf16>(static_cast<const bf16*>(p->ctx) + off, static_cast<bf16*>(k),
                                    static_cast<bf16*>(v), n, p->desc.max_ctx, H, d, hs));
  else
    PS_HIP(launch_entry_fetch<float>(static_cast<const float*>(p->ctx) + off, static_cast<float*>(k),
                                     static_cast<float*>(v), n, p->desc.max_ctx, H, d, hs));
  return PS_OK;
}

// ------------------------------------------------------------------ block
extern "C" ps_status ps_block_create(const ps_block_desc* desc, ps_block** out) {
  if (!desc || !out) return fail(PS_ERR_INVALID_ARG, "ps_block_create: null argument");
  const ps_block_desc& d = *desc;
  if (d.dtype != PS_BF16 && d.dtype != PS_F32) return fail(PS_ERR_INVALID_ARG, "block: bad dtype");
  if (d.n_heads <= 0 || d.head_dim <= 0 || d.hidden != d.n_heads * d.head_dim)
    return fail(PS_ERR_INVALID_ARG, "block: hidden must equal n_heads * head_dim");
  const int ks = gemm_k_step(d.dtype);
  if (d.hidden % ks != 0 || d.ffn <= 0 || d.ffn % ks != 0)
    return fail(PS_ERR_INVALID_ARG, "block: hidden and ffn must be multiples of %d", ks);
  if (d.block_index < 0) return fail(PS_ERR_INVALID_ARG, "block: negative block_index");
  const void* ptrs[] = {d.wqkv, d.wo, d.wq2, d.wkv2, d.wo2, d.w1, d.w2, d.bqkv, d.bo,
                        d.bq2,  d.bkv2, d.bo2, d.b1, d.b2, d.tmod};
  for (const void* q : ptrs)
    if (!q) return fail(PS_ERR_INVALID_ARG, "block: null weight pointer");
  ps_block* b = new ps_block();
  b->d = d;
  *out = b;
  return PS_OK;
}

extern "C" ps_status ps_block_destroy(ps_block* b) {
  if (!b) return fail(PS_ERR_INVALID_ARG, "ps_block_destroy: null block");
  delete b;
  return PS_OK;
}

// Whether hs is capturing into a HIP graph.
static bool capturing(hipStream_t hs) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(hs, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

// ------------------------------------------------------ timestep embedding
static void te_free(ps_time_embed* te) {
  if (te->cache) (void)hipFree(te->cache);
  if (te->cache_u) (void)hipFree(te->cache_u);
  if (te->scratch) (void)hipFree(te->scratch);
  for (hipEvent_t e : te->fill_ev)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : te->rd_ev)
    if (e) (void)hipEventDestroy(e);
  if (te->scratch_ev) (void)hipEventDestroy(te->scratch_ev);
  (void)hipGetLastError();
  delete te;
}

extern "C" ps_status ps_time_embed_create(const ps_time_desc* desc, ps_time_embed** out) {
  if (!desc || !out) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_create: null argument");
  const ps_time_desc& d = *desc;
  if (d.hidden <= 0 || d.capacity <= 0 || d.capacity > 4096)
    return fail(PS_ERR_INVALID_ARG, "time embed: bad hidden or capacity");
  if (!d.wt1 || !d.bt1 || !d.wt2 || !d.bt2 || !d.wp || !d.bp)
    return fail(PS_ERR_INVALID_ARG, "time embed: null weight pointer");
  ps_time_embed* te = new ps_time_embed();
  te->d = d;
  te->fill_ev.assign(d.capacity, nullptr);
  bool ok = hipMalloc(&te->cache, sizeof(float) * (size_t)d.capacity * 6 * d.hidden) == hipSuccess &&
            hipMalloc(&te->cache_u, sizeof(float) * (size_t)d.capacity * d.hidden) == hipSuccess &&
            hipMalloc(&te->scratch, sizeof(float) * (PS_FREQ_DIM + 2 * (size_t)d.hidden)) == hipSuccess;
  for (int i = 0; ok && i < d.capacity; ++i)
    ok = hipEventCreateWithFlags(&te->fill_ev[i], hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < TE_STREAMS; ++i)
    ok = hipEventCreateWithFlags(&te->rd_ev[i], hipEventDisableTiming) == hipSuccess;
  if (ok) ok = hipEventCreateWithFlags(&te->scratch_ev, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    te_free(te);
    return fail(PS_ERR_OUT_OF_MEMORY, "time embed: cannot allocate the cache or its events");
  }
  te->key.assign(d.capacity, 0);
  te->used.assign(d.capacity, 0);
  te->valid.assign(d.capacity, 0);
  te->fill_stream.assign(d.capacity, nullptr);
  te->readers.assign(d.capacity, 0);
  *out = te;
  return PS_OK;
}

extern "C" ps_status ps_time_embed_destroy(ps_time_embed* te) {
  if (!te) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_destroy: null handle");
  (void)hipDeviceSynchronize();
  te_free(te);
  return PS_OK;
}

// Slot of stream hs among the streams that read the cache.  With all slots
// taken, a slot whose latest read has completed is reused (its stream's bits
// are cleared from every row); if none has, the host waits for the oldest
// slot's latest read first.
static ps_status te_stream_slot(ps_time_embed* te, hipStream_t hs, int* slot) {
  for (int i = 0; i < TE_STREAMS; ++i)
    if (te->rd_used[i] && te->rd_stream[i] == hs) {
      *slot = i;
      return PS_OK;
    }
  int pick = -1;
  for (int i = 0; i < TE_STREAMS && pick < 0; ++i)
    if (!te->rd_used[i]) pick = i;
  for (int i = 0; i < TE_STREAMS && pick < 0; ++i)
    if (hipEventQuery(te->rd_ev[i]) == hipSuccess) pick = i;
  if (pick < 0) {
    PS_HIP(hipEventSynchronize(te->rd_ev[0]));
    pick = 0;
  }
  (void)hipGetLastError();   // hipEventQuery's hipErrorNotReady
  for (uint32_t& r : te->readers) r &= ~(1u << pick);
  te->rd_used[pick] = true;
  te->rd_stream[pick] = hs;
  *slot = pick;
  return PS_OK;
}

// Cache rows of the timesteps t[0 .. n-1] (rows[i] for t[i]), filling the
// missing ones on hs.  The number of distinct timesteps is checked against
// the capacity before anything is enqueued.  A refilled row is first made to
// wait for every earlier read of it on other streams, and a stream that reads
// a row filled on another stream waits for that fill.  The rows of this call
// are never evicted by it.
static ps_status te_resolve(ps_time_embed* te, const float* t, int n, hipStream_t hs, int* rows, int* slot) {
  const int cap = te->d.capacity;
  std::vector<uint32_t> keys;
  for (int i = 0; i < n; ++i) {
    uint32_t k;
    memcpy(&k, &t[i], 4);
    bool seen = false;
    for (uint32_t x : keys) seen |= (x == k);
    if (!seen) keys.push_back(k);
  }
  if ((int)keys.size() > cap)
    return fail(PS_ERR_INVALID_ARG, "time embed: %d distinct timesteps in one call, capacity %d", (int)keys.size(), cap);
  // Under graph capture every row must already be cached and nothing waits
  // on or records events outside the graph.
  const bool cap_mode = capturing(hs);
  if (cap_mode)
    for (uint32_t k : keys) {
      bool hit = false;
      for (int j = 0; j < cap; ++j) hit |= te->valid[j] && te->key[j] == k;
      if (!hit) return fail(PS_ERR_UNSUPPORTED, "time embed: a timestep is not cached; fill it before graph capture");
    }
  ps_status st = te_stream_slot(te, hs, slot);
  if (st) return st;
  const int D = te->d.hidden;
  std::vector<int> pinned;
  for (int i = 0; i < n; ++i) {
    uint32_t k;
    memcpy(&k, &t[i], 4);
    int row = -1;
    for (int j = 0; j < cap && row < 0; ++j)
      if (te->valid[j] && te->key[j] == k) row = j;
    if (row >= 0) {
      if (te->fill_stream[row] != hs && !cap_mode) PS_HIP(hipStreamWaitEvent(hs, te->fill_ev[row], 0));
    } else {
      int victim = -1;
      for (int j = 0; j < cap; ++j) {
        bool pin = false;
        for (int pr : pinned) pin |= (pr == j);
        if (pin) continue;
        if (victim < 0 || !te->valid[j] || (te->valid[victim] && te->used[j] < te->used[victim])) victim = j;
        if (!te->valid[j]) break;
      }
      // victim >= 0: at most `cap` distinct timesteps are pinned
      for (int sl = 0; sl < TE_STREAMS; ++sl)
        if ((te->readers[victim] >> sl & 1u) && te->rd_stream[sl] != hs)
          PS_HIP(hipStreamWaitEvent(hs, te->rd_ev[sl], 0));
      if (te->scratch_rec && te->scratch_stream != hs) PS_HIP(hipStreamWaitEvent(hs, te->scratch_ev, 0));
      PS_HIP(launch_time_embed(t[i], te->d.wt1, te->d.bt1, te->d.wt2, te->d.bt2, te->d.wp, te->d.bp, D, te->scratch,
                               te->cache + (size_t)victim * 6 * D, te->cache_u + (size_t)victim * D, hs));
      PS_HIP(hipEventRecord(te->fill_ev[victim], hs));
      PS_HIP(hipEventRecord(te->scratch_ev, hs));
      te->scratch_rec = true;
      te->scratch_stream = hs;
      te->fill_stream[victim] = hs;
      te->readers[victim] = 0;
      te->valid[victim] = 1;
      te->key[victim] = k;
      row = victim;
    }
    te->used[row] = ++te->clock;
    rows[i] = row;
    pinned.push_back(row);
  }
  return PS_OK;
}

// After the kernels that read rows[0 .. n-1] have been enqueued on hs.
// Reads inside a captured graph are not tracked (no event outside the graph).
static ps_status te_mark_read(ps_time_embed* te, const int* rows, int n, int slot, hipStream_t hs) {
  if (capturing(hs)) return PS_OK;
  PS_HIP(hipEventRecord(te->rd_ev[slot], hs));
  for (int i = 0; i < n; ++i) te->readers[rows[i]] |= 1u << slot;
  return PS_OK;
}

extern "C" ps_status ps_time_embed_get(ps_time_embed* te, float t, float* e, hipStream_t hs) {
  if (!te || !e) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_get: null argument");
  if (!isfinite(t)) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_get: timestep not finite");
  int row = 0, slot = 0;
  ps_status st = te_resolve(te, &t, 1, hs, &row, &slot);
  if (st) return st;
  const size_t n = (size_t)6 * te->d.hidden;
  PS_HIP(hipMemcpyAsync(e, te->cache + row * n, n * sizeof(float), hipMemcpyDeviceToDevice, hs));
  return te_mark_read(te, &row, 1, slot, hs);
}

// Timesteps of an n_steps-step schedule: the uniform grid u = 1 - s / n_steps
// under the flow-matching time shift t = a u / (1 + (a - 1) u) (a = shift;
// a = 1 leaves the grid uniform), and t[n_steps] = 0.
extern "C" ps_status ps_timesteps(int32_t n_steps, float shift, float* out) {
  if (!out || n_steps < 1 || n_steps > 4096 || !(shift > 0.0f) || !isfinite(shift))
    return fail(PS_ERR_INVALID_ARG, "ps_timesteps: need 1 <= n_steps <= 4096, a finite shift > 0 and out");
  const double a = shift;
  for (int s = 0; s < n_steps; ++s) {
    const double u = 1.0 - (double)s / n_steps;
    out[s] = (float)(a * u / (1.0 + (a - 1.0) * u));
  }
  out[n_steps] = 0.0f;
  return PS_OK;
}

// ---------------------------------------------------------------- context
extern "C" ps_status ps_context_set(ps_kv_pool* p, const ps_block* b, int32_t stream, const void* ctx, int32_t n_ctx,
                                    hipStream_t hs) {
  if (!p || !b || !ctx) return fail(PS_ERR_INVALID_ARG, "ps_context_set: null argument");
  const ps_block_desc& bd = b->d;
  if (bd.dtype != p->desc.dtype || bd.n_heads != p->desc.n_heads || bd.head_dim != p->desc.head_dim)
    return fail(PS_ERR_INVALID_ARG, "ps_context_set: block and pool disagree on dtype or heads");
  ps_status st = check_region(p, stream, bd.block_index, 0, 0);
  if (st) return st;
  if (n_ctx < 8 || n_ctx > p->desc.max_ctx || n_ctx % 8 != 0)
    return fail(PS_ERR_INVALID_ARG, "ps_context_set: n_ctx %d must be a multiple of 8 in [8, %d]", n_ctx,
                p->desc.max_ctx);
  const size_t cr = (size_t)stream * p->desc.n_blocks + bd.block_index;
  EpiArgs ep;
  ep.bias = bd.bkv2;
  ep.pool = p->geo();
  const size_t es = elt_size(bd.dtype);
  ep.ctx_base = static_cast<char*>(p->ctx) + cr * p->ctx_elems * es;
  ep.d_shift = bd.head_dim == 128 ? 7 : 6;
  const int D = bd.hidden;
  if (bd.dtype == PS_BF16)
    PS_HIP(launch_gemm<bf16>(EPI_CTX_KV, static_cast<const bf16*>(ctx), D, static_cast<const bf16*>(bd.wkv2),
                             n_ctx, 2 * D, D, ep, nullptr, hs));
  else
    PS_HIP(launch_gemm<float>(EPI_CTX_KV, static_cast<const float*>(ctx), D, static_cast<const float*>(bd.wkv2),
                              n_ctx, 2 * D, D, ep, nullptr, hs));
  p->ctx_len[cr] = n_ctx;
  return PS_OK;
}

extern "C" ps_status ps_context_load(ps_kv_pool* p, int32_t stream, int32_t block, const void* k, const void* v,
                                     int32_t n_ctx, hipStream_t hs) {
  if (!p || !k || !v) return fail(PS_ERR_INVALID_ARG, "ps_context_load: null argument");
  ps_status st = check_region(p, stream, block, 0, 0);
  if (st) return st;
  if (n_ctx < 8 || n_ctx > p->desc.max_ctx || n_ctx % 8 != 0)
    return fail(PS_ERR_INVALID_ARG, "ps_context_load: n_ctx %d must be a multiple of 8 in [8, %d]", n_ctx,
                p->desc.max_ctx);
  const size_t cr = (size_t)stream * p->desc.n_blocks + block;
  const size_t off = cr * p->ctx_elems;
  const int H = p->desc.n_heads, d = p->desc.head_dim;
  if (p->desc.dtype == PS_BF16)
    PS_HIP(launch_entry_load<bf16>(static_cast<bf16*>(p->ctx) + off, static_cast<const bf16*>(k),
                                   static_cast<const bf16*>(v), n_ctx, p->desc.max_ctx, H, d, hs));
  else
    PS_HIP(launch_entry_load<float>(static_cast<float*>(p->ctx) + off, static_cast<const float*>(k),
                                    static_cast<const float*>(v), n_ctx, p->desc.max_ctx, H, d, hs));
  p->ctx_len[cr] = n_ctx;
  return PS_OK;
}

// ------------------------------------------------------------------ stage
// Row stride of the activation buffers that feed a GEMM as its A operand:
// padded by 64 elements so that the rows of a tile do not all begin on the
// same memory channel (a dense stride of 5120 or 13824 bf16 elements does).
static int act_ld(int cols) { return cols + 64; }

// Copy of a [rows, cols] activation stored with row stride ld into a dense
// caller buffer (a probe member; nothing when it is null).
static ps_status probe_copy(void* dst, const void* src, size_t es, size_t rows, int cols, int ld, hipStream_t hs) {
  if (!dst) return PS_OK;
  PS_HIP(hipMemcpy2DAsync(dst, cols * es, src, ld * es, cols * es, rows, hipMemcpyDeviceToDevice, hs));
  return PS_OK;
}

#define PS_PROBE(member, src, cols, ld)                                                            \
  do {                                                                                             \
    if (pr) {                                                                                      \
      ps_status ps_ = probe_copy(pr->member, src, sizeof(*(src)), (size_t)M, cols, ld, hs);         \
      if (ps_) return ps_;                                                                         \
    }                                                                                              \
  } while (0)

// Every check of a stage call; nothing is enqueued or changed.
ps_status ps::prepare_batch(const ps_kv_pool* p, const ps_block* b, const ps_time_embed* te, const ps_task* tasks,
                               int32_t n, const void* h_in, const void* h_out, const char* fn, Batch* out) {
  if (!p || !b || !te || !tasks || !h_in || !h_out) return fail(PS_ERR_INVALID_ARG, "%s: null argument", fn);
  if (n < 1 || n > PS_MAX_TASKS) return fail(PS_ERR_INVALID_ARG, "%s: n_tasks %d not in [1, %d]", fn, n, PS_MAX_TASKS);
  const ps_pool_desc& pd = p->desc;
  const ps_block_desc& bd = b->d;
  if (bd.dtype != pd.dtype || bd.n_heads != pd.n_heads || bd.head_dim != pd.head_dim)
    return fail(PS_ERR_INVALID_ARG, "%s: block and pool disagree on dtype or heads", fn);
  if (bd.block_index >= pd.n_blocks) return fail(PS_ERR_INVALID_ARG, "%s: block_index %d beyond pool", fn, bd.block_index);
  if (te->d.hidden != bd.hidden) return fail(PS_ERR_INVALID_ARG, "%s: time embedding width differs", fn);
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev != p->device) return fail(PS_ERR_INVALID_ARG, "%s: current device is not the pool's", fn);

  Batch& bt = *out;
  bt.n = n;
  bt.tt.n = n;
  for (int i = 0; i < n; ++i) {
    const ps_task& t = tasks[i];
    ps_status st = check_region(p, t.stream, bd.block_index, t.step, t.write_slot);
    if (st) return fail(st, "%s: task %d: %s", fn, i, g_err.c_str());
    if (t.chunk < 0) return fail(PS_ERR_INVALID_ARG, "%s: task %d: negative chunk", fn, i);
    if (!isfinite(t.timestep)) return fail(PS_ERR_INVALID_ARG, "%s: task %d: timestep not finite", fn, i);
    if (t.n_read < 0 || t.n_read > PS_MAX_WINDOW || t.n_read >= pd.n_slots)
      return fail(PS_ERR_INVALID_ARG, "%s: task %d: n_read %d out of range", fn, i, t.n_read);
    for (int j = 0; j < t.n_read; ++j) {
      if (t.read_slots[j] < 0 || t.read_slots[j] >= pd.n_slots)
        return fail(PS_ERR_INVALID_ARG, "%s: task %d: read slot %d out of range", fn, i, t.read_slots[j]);
      if (t.read_slots[j] == t.write_slot)
        return fail(PS_ERR_INVALID_ARG, "%s: task %d: reads its own write slot %d", fn, i, t.write_slot);
    }
    const size_t cr = (size_t)t.stream * pd.n_blocks + bd.block_index;
    if (p->ctx_len[cr] == 0)
      return fail(PS_ERR_INVALID_ARG, "%s: task %d: context of stream %d block %d not set", fn, i, t.stream,
                  bd.block_index);
    const size_t reg = region_of(p, t.stream, bd.block_index, t.step);
    const size_t wkey = reg * pd.n_slots + t.write_slot;
    for (int j = 0; j < i; ++j)
      if (bt.writes[j] == wkey) return fail(PS_ERR_SLOT_CONFLICT, "%s: task %d: two tasks of the batch write one slot", fn, i);
    bt.writes[i] = wkey;
    bt.t[i] = t.timestep;
    DevTask& dt = bt.tt.t[i];
    dt.region = (int32_t)reg;
    dt.ctx_region = (int32_t)cr;
    dt.chunk = t.chunk;
    dt.n_seg = t.n_read + 1;
    dt.ctx_len = p->ctx_len[cr];
    for (int j = 0; j < t.n_read; ++j) dt.slots[j] = t.read_slots[j];
    dt.slots[t.n_read] = t.write_slot;
  }
  if (pd.check_slots) {
    // the batch's writes land before any of its reads
    std::vector<int> led = p->ledger;
    for (int i = 0; i < n; ++i) led[bt.writes[i]] = tasks[i].chunk;
    for (int i = 0; i < n; ++i) {
      const ps_task& t = tasks[i];
      const size_t reg = bt.tt.t[i].region;
      for (int j = 0; j < t.n_read; ++j) {
        const int want = t.chunk - t.n_read + j;
        const int have = led[reg * pd.n_slots + t.read_slots[j]];
        if (have != want)
          return fail(PS_ERR_SLOT_CONFLICT, "%s: task %d (stream %d chunk %d step %d): slot %d holds chunk %d, expected %d",
                      fn, i, t.stream, t.chunk, t.step, t.read_slots[j], have, want);
      }
    }
  }
  return PS_OK;
}

WsSizes ps::ws_sizes(const ps_kv_pool* p, const ps_block* b, int n) {
  const ps_block_desc& bd = b->d;
  const size_t M = (size_t)n * p->L(), es = elt_size(bd.dtype);
  const size_t D = bd.hidden, F = bd.ffn;
  return WsSizes{{sizeof(float) * n * 6 * D, sizeof(float2) * n * p->desc.frames * (size_t)(p->seg_f / 2) + 16,
                  M * act_ld((int)D) * es, M * D * es, M * act_ld((int)D) * es, M * act_ld((int)F) * es,
                  sizeof(DevTask) * PS_MAX_TASKS}};
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ps::ws_total(const WsSizes& z) {
  size_t t = 0;
  for (size_t v : z.b) t += align256(v);
  return t;
}

WsPtrs ps::ws_carve(char* base, const WsSizes& z) {
  void* p[7];
  for (int i = 0; i < 7; ++i) {
    p[i] = base;
    base += align256(z.b[i]);
  }
  WsPtrs w;
  w.mod = static_cast<float*>(p[0]);
  w.rope = static_cast<float2*>(p[1]);
  w.y = p[2];
  w.q = p[3];
  w.a = p[4];
  w.u = p[5];
  w.tasks = static_cast<DevTask*>(p[6]);
  return w;
}

// The pool's per-stream workspace, grown to this batch (stream-ordered).
static ps_status ws_from_pool(ps_kv_pool* p, const WsSizes& z, hipStream_t hs, WsPtrs* out) {
  ps_kv_pool::Workspace* w = p->workspace(hs);
  if (!w)
    return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: more than %d streams use this pool", PS_MAX_STREAMS_PER_POOL);
  DevBuf* bufs[7] = {&w->mod, &w->rope, &w->y, &w->q, &w->a, &w->u, &w->tasks};
  for (int i = 0; i < 7; ++i)
    if (z.b[i] > bufs[i]->bytes && capturing(hs))
      return fail(PS_ERR_UNSUPPORTED, "ps_stage_batch: the workspace of this stream must grow; size it before graph capture");
  for (int i = 0; i < 7; ++i) {
    ps_status st = bufs[i]->reserve(z.b[i], hs);
    if (st) return st;
  }
  out->mod = static_cast<float*>(w->mod.p);
  out->rope = static_cast<float2*>(w->rope.p);
  out->y = w->y.p;
  out->q = w->q.p;
  out->a = w->a.p;
  out->u = w->u.p;
  out->tasks = static_cast<DevTask*>(w->tasks.p);
  return PS_OK;
}

// The batch's preamble: timestep rows (filled if missing), the task table in
// device memory, the per-task modulation rows and RoPE frame table.
ps_status ps::begin_batch(const ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const Batch& bt,
                             const WsPtrs& w, hipStream_t hs) {
  int rows[PS_MAX_TASKS], slot = 0;
  ps_status st = te_resolve(te, bt.t, bt.n, hs, rows, &slot);
  if (st) return st;
  PS_TRACED("put_tasks", launch_put_tasks(bt.tt, w.tasks, hs));
  PS_TRACED("modulation", launch_modulation(te->cache, rows, b->d.tmod, w.mod, w.rope, w.tasks, bt.n, b->d.hidden,
                                            p->desc.frames, p->seg_f, hs));
  return te_mark_read(te, rows, bt.n, slot, hs);
}

// The residual-stream buffers of the stage's steps: ln1 and the O projection
// read h_in; the O projection writes h_out, which ln2, the cross-O projection
// (in place), ln3 and FFN2 (in place) continue on.  A single-kernel call
// points them at the caller's buffers.
struct StageIO {
  const float* h_in;     // ln1 input, O-projection residual input
  float* h_out;          // O / cross-O / FFN2 output
  const float* h_ln2;    // ln2 input
  const float* h_xo;     // cross-O residual input
  const float* h_ln3;    // ln3 input
  const float* h_ffn2;   // FFN2 residual input
};

static StageIO stage_io(const float* h_in, float* h_out) {
  return StageIO{h_in, h_out, h_out, h_out, h_out, h_out};
}

// The stage's kernels in order (which < 0), or the one kernel `which`.
template <typename T>
static ps_status run_stage(ps_kv_pool* p, const ps_block* b, const WsPtrs& w, int n, const StageIO& io,
                           const ps_stage_probe* pr, int which, hipStream_t hs) {
  const ps_block_desc& bd = b->d;
  const int L = p->L(), D = bd.hidden, F = bd.ffn, M = n * L;
  T* y = static_cast<T*>(w.y);
  T* q = static_cast<T*>(w.q);
  T* a = static_cast<T*>(w.a);
  T* u = static_cast<T*>(w.u);
  const DevTask* tt = w.tasks;
  const PoolGeo pg = p->geo();
  const float qscale = 1.4426950408889634f / sqrtf((float)bd.head_dim);
  const int ldy = act_ld(D), ldu = act_ld(F);
  auto on = [&](int k) { return which < 0 || which == k; };

  // self-attention branch
  if (on(PS_KERNEL_LN1)) {
    PS_TRACED("ln1", (launch_layernorm<T>(io.h_in, y, ldy, M, D, w.mod, 0, 1, L, hs)));
    PS_PROBE(y1, y, D, ldy);
  }
  if (on(PS_KERNEL_QKV)) {
    EpiArgs e1;
    e1.bias = bd.bqkv;
    e1.out = q;
    e1.ldo = D;
    e1.out_scale = qscale;
    e1.rope_f = w.rope;
    e1.pool = pg;
    e1.d_shift = bd.head_dim == 128 ? 7 : 6;
    PS_TRACED("qkv", (launch_gemm<T>(EPI_QKV, y, ldy, static_cast<const T*>(bd.wqkv), M, 3 * D, D, e1, tt, hs)));
    PS_PROBE(q, q, D, D);
  }
  if (on(PS_KERNEL_ATTN_SELF)) {
    PS_TRACED("attn_self", (launch_attention<T>(false, q, a, ldy, pg, tt, n, hs)));
    PS_PROBE(attn, a, D, ldy);
  }
  if (on(PS_KERNEL_O_PROJ)) {
    EpiArgs e2;
    e2.bias = bd.bo;
    e2.h_in = io.h_in;
    e2.h_out = io.h_out;
    e2.mod = w.mod;
    e2.gate_row = 2;
    e2.L = L;
    e2.div_L = FastDiv((uint32_t)L);
    PS_TRACED("o_proj", (launch_gemm<T>(EPI_RES, a, ldy, static_cast<const T*>(bd.wo), M, D, D, e2, tt, hs)));
    PS_PROBE(h1, io.h_out, D, D);
  }

  // cross-attention branch
  if (on(PS_KERNEL_LN2)) {
    PS_TRACED("ln2", (launch_layernorm<T>(io.h_ln2, y, ldy, M, D, nullptr, -1, -1, L, hs)));
    PS_PROBE(y2, y, D, ldy);
  }
  if (on(PS_KERNEL_XQ_PROJ)) {
    EpiArgs e3;
    e3.bias = bd.bq2;
    e3.out = q;
    e3.ldo = D;
    e3.out_scale = qscale;
    PS_TRACED("xq_proj", (launch_gemm<T>(EPI_STORE, y, ldy, static_cast<const T*>(bd.wq2), M, D, D, e3, tt, hs)));
    PS_PROBE(q2, q, D, D);
  }
  if (on(PS_KERNEL_ATTN_CROSS)) {
    PS_TRACED("attn_cross", (launch_attention<T>(true, q, a, ldy, pg, tt, n, hs)));
    PS_PROBE(xattn, a, D, ldy);
  }
  if (on(PS_KERNEL_XO_PROJ)) {
    EpiArgs e4;
    e4.bias = bd.bo2;
    e4.h_in = io.h_xo;
    e4.h_out = io.h_out;
    e4.L = L;
    e4.div_L = FastDiv((uint32_t)L);
    PS_TRACED("xo_proj", (launch_gemm<T>(EPI_RES, a, ldy, static_cast<const T*>(bd.wo2), M, D, D, e4, tt, hs)));
    PS_PROBE(h2, io.h_out, D, D);
  }

  // FFN branch
  if (on(PS_KERNEL_LN3)) {
    PS_TRACED("ln3", (launch_layernorm<T>(io.h_ln3, y, ldy, M, D, w.mod, 3, 4, L, hs)));
    PS_PROBE(y3, y, D, ldy);
  }
  if (on(PS_KERNEL_FFN1)) {
    EpiArgs e5;
    e5.bias = bd.b1;
    e5.out = u;
    e5.ldo = ldu;
    PS_TRACED("ffn1", (launch_gemm<T>(EPI_GELU, y, ldy, static_cast<const T*>(bd.w1), M, F, D, e5, tt, hs)));
    PS_PROBE(u, u, F, ldu);
  }
  if (on(PS_KERNEL_FFN2)) {
    EpiArgs e6;
    e6.bias = bd.b2;
    e6.h_in = io.h_ffn2;
    e6.h_out = io.h_out;
    e6.mod = w.mod;
    e6.gate_row = 5;
    e6.L = L;
    e6.div_L = FastDiv((uint32_t)L);
    PS_TRACED("ffn2", (launch_gemm<T>(EPI_RES, u, ldu, static_cast<const T*>(bd.w2), M, D, F, e6, tt, hs)));
  }
  return PS_OK;
}

static ps_status run_stage_dt(ps_kv_pool* p, const ps_block* b, const WsPtrs& w, int n, const StageIO& io,
                              const ps_stage_probe* pr, int which, hipStream_t hs) {
  if (b->d.dtype == PS_BF16) return run_stage<bf16>(p, b, w, n, io, pr, which, hs);
  return run_stage<float>(p, b, w, n, io, pr, which, hs);
}

ps_status ps::run_stage_all(ps_kv_pool* p, const ps_block* b, const WsPtrs& w, int n, const float* h_in,
                            float* h_out, hipStream_t hs) {
  return run_stage_dt(p, b, w, n, stage_io(h_in, h_out), nullptr, -1, hs);
}

void ps::commit_writes(ps_kv_pool* p, const Batch& bt, const ps_task* tasks) {
  for (int i = 0; i < bt.n; ++i) p->ledger[bt.writes[i]] = tasks[i].chunk;
}

static ps_status stage_batch(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks, int32_t n,
                             const float* h_in, float* h_out, const ps_stage_probe* probe, hipStream_t hs) {
  Batch bt;
  ps_status st = prepare_batch(p, b, te, tasks, n, h_in, h_out, "ps_stage_batch", &bt);
  if (st) return st;
  WsPtrs w;
  if ((st = ws_from_pool(p, ws_sizes(p, b, n), hs, &w))) return st;
  if ((st = begin_batch(p, b, te, bt, w, hs))) return st;
  if ((st = run_stage_dt(p, b, w, n, stage_io(h_in, h_out), probe, -1, hs))) return st;
  commit_writes(p, bt, tasks);
  return PS_OK;
}

extern "C" ps_status ps_stage_batch(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks,
                                    int32_t n, const float* h_in, float* h_out, hipStream_t hs) {
  return stage_batch(p, b, te, tasks, n, h_in, h_out, nullptr, hs);
}

// The residual stream of a batch whose tasks' rows are not one contiguous
// slice: gathered into the stream's workspace, run in place, scattered back.
extern "C" ps_status ps_stage_batch_rows(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks,
                                         int32_t n, const float* const* h_in, float* const* h_out, hipStream_t hs) {
  const char* fn = "ps_stage_batch_rows";
  if (!h_in || !h_out) return fail(PS_ERR_INVALID_ARG, "%s: null argument", fn);
  if (n < 1 || n > PS_MAX_TASKS) return fail(PS_ERR_INVALID_ARG, "%s: n_tasks %d not in [1, %d]", fn, n, PS_MAX_TASKS);
  for (int i = 0; i < n; ++i) {
    if (!h_in[i] || !h_out[i]) return fail(PS_ERR_INVALID_ARG, "%s: null row pointer of task %d", fn, i);
    if ((reinterpret_cast<uintptr_t>(h_in[i]) | reinterpret_cast<uintptr_t>(h_out[i])) % 16 != 0)
      return fail(PS_ERR_INVALID_ARG, "%s: rows of task %d not 16-byte aligned", fn, i);
  }
  Batch bt;
  ps_status st = prepare_batch(p, b, te, tasks, n, h_in[0], h_out[0], fn, &bt);
  if (st) return st;
  const size_t per = (size_t)p->L() * b->d.hidden;
  WsPtrs w;
  if ((st = ws_from_pool(p, ws_sizes(p, b, n), hs, &w))) return st;
  ps_kv_pool::Workspace* ws = p->workspace(hs);
  if ((st = ws->h.reserve(sizeof(float) * per * n, hs))) return st;
  float* h = static_cast<float*>(ws->h.p);
  if ((st = begin_batch(p, b, te, bt, w, hs))) return st;
  for (int i = 0; i < n; ++i)
    PS_HIP(hipMemcpyAsync(h + per * i, h_in[i], sizeof(float) * per, hipMemcpyDeviceToDevice, hs));
  if ((st = run_stage_all(p, b, w, n, h, h, hs))) return st;
  for (int i = 0; i < n; ++i)
    PS_HIP(hipMemcpyAsync(h_out[i], h + per * i, sizeof(float) * per, hipMemcpyDeviceToDevice, hs));
  commit_writes(p, bt, tasks);
  return PS_OK;
}

extern "C" ps_status ps_stage_batch_probe(ps_kv_pool* p, const ps_block* b, ps_time_embed* te,
                                          const ps_task* tasks, int32_t n, const float* h_in, float* h_out,
                                          const ps_stage_probe* probe, hipStream_t hs) {
  if (!probe) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch_probe: null probe");
  return stage_batch(p, b, te, tasks, n, h_in, h_out, probe, hs);
}

// One kernel of the stage on caller-given inputs (dense rows).  The input is
// copied into the workspace buffer the kernel reads in a stage call (same
// strides), the kernel runs with the stage call's launch configuration, and
// its output is copied out.
extern "C" ps_status ps_stage_kernel(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks,
                                     int32_t n, int32_t kernel, const void* in, const float* h_in, void* out,
                                     hipStream_t hs) {
  const char* fn = "ps_stage_kernel";
  if (kernel < PS_KERNEL_LN1 || kernel > PS_KERNEL_FFN2) return fail(PS_ERR_INVALID_ARG, "%s: unknown kernel %d", fn, kernel);
  const bool residual = kernel == PS_KERNEL_O_PROJ || kernel == PS_KERNEL_XO_PROJ || kernel == PS_KERNEL_FFN2;
  if (residual && !h_in) return fail(PS_ERR_INVALID_ARG, "%s: the residual kernels need h_in", fn);
  Batch bt;
  ps_status st = prepare_batch(p, b, te, tasks, n, in, out, fn, &bt);
  if (st) return st;
  WsPtrs w;
  if ((st = ws_from_pool(p, ws_sizes(p, b, n), hs, &w))) return st;
  if ((st = begin_batch(p, b, te, bt, w, hs))) return st;
  const int L = p->L(), D = b->d.hidden, F = b->d.ffn;
  const size_t M = (size_t)n * L, es = elt_size(b->d.dtype);
  const int ldy = act_ld(D), ldu = act_ld(F);
  auto put = [&](void* dst, int cols, int ld) -> ps_status {
    PS_HIP(hipMemcpy2DAsync(dst, ld * es, in, cols * es, cols * es, M, hipMemcpyDeviceToDevice, hs));
    return PS_OK;
  };
  StageIO io = stage_io(static_cast<const float*>(in), static_cast<float*>(out));
  const void* res = nullptr;   // workspace output to copy out
  int res_cols = D, res_ld = ldy;
  switch (kernel) {
    case PS_KERNEL_LN1: res = w.y; break;
    case PS_KERNEL_QKV: st = put(w.y, D, ldy); res = w.q; res_ld = D; break;
    case PS_KERNEL_ATTN_SELF: st = put(w.q, D, D); res = w.a; break;
    case PS_KERNEL_O_PROJ: st = put(w.a, D, ldy); io.h_in = h_in; break;
    case PS_KERNEL_LN2: io.h_ln2 = static_cast<const float*>(in); res = w.y; break;
    case PS_KERNEL_XQ_PROJ: st = put(w.y, D, ldy); res = w.q; res_ld = D; break;
    case PS_KERNEL_ATTN_CROSS: st = put(w.q, D, D); res = w.a; break;
    case PS_KERNEL_XO_PROJ: st = put(w.a, D, ldy); io.h_xo = h_in; break;
    case PS_KERNEL_LN3: io.h_ln3 = static_cast<const float*>(in); res = w.y; break;
    case PS_KERNEL_FFN1: st = put(w.y, D, ldy); res = w.u; res_cols = F; res_ld = ldu; break;
    case PS_KERNEL_FFN2: st = put(w.u, F, ldu); io.h_ffn2 = h_in; break;
  }
  if (st) return st;
  if ((st = run_stage_dt(p, b, w, n, io, nullptr, kernel, hs))) return st;
  if (res) PS_HIP(hipMemcpy2DAsync(out, res_cols * es, res, res_ld * es, res_cols * es, M, hipMemcpyDeviceToDevice, hs));
  if (kernel == PS_KERNEL_QKV) commit_writes(p, bt, tasks);
  return PS_OK;
}

// ------------------------------------------------------------------- head
struct ps_head {
  ps_head_desc d{};
  int device = 0;
  DevBuf ws_x;     // compute-dtype copy of the latent patches (embedding's A operand)
  DevBuf ws_y;     // modulated LN of h (head's A operand), row stride D + 64
  DevBuf ws_mod;   // [n][6][D]: rows 0 and 1 = (shift, scale) of each task
};

extern "C" ps_status ps_head_create(const ps_head_desc* desc, ps_head** out) {
  if (!desc || !out) return fail(PS_ERR_INVALID_ARG, "ps_head_create: null argument");
  const ps_head_desc& d = *desc;
  if (d.dtype != PS_BF16 && d.dtype != PS_F32) return fail(PS_ERR_INVALID_ARG, "ps_head_create: bad dtype");
  const int step = gemm_k_step(d.dtype);
  if (d.hidden <= 0 || d.latent_dim <= 0 || d.hidden % step != 0 || d.latent_dim % step != 0)
    return fail(PS_ERR_INVALID_ARG, "ps_head_create: hidden %d and latent_dim %d must be positive multiples of %d",
                d.hidden, d.latent_dim, step);
  if (!d.w_embed || !d.w_head || !d.b_embed || !d.b_head || !d.t_head)
    return fail(PS_ERR_INVALID_ARG, "ps_head_create: null weight pointer");
  ps_head* h = new ps_head();
  h->d = d;
  (void)hipGetDevice(&h->device);
  *out = h;
  return PS_OK;
}

extern "C" ps_status ps_head_destroy(ps_head* h) {
  if (!h) return fail(PS_ERR_INVALID_ARG, "ps_head_destroy: null handle");
  (void)hipDeviceSynchronize();
  h->ws_x.release();
  h->ws_y.release();
  h->ws_mod.release();
  delete h;
  return PS_OK;
}

static ps_status head_device_check(const ps_head* h, const char* fn) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev != h->device) return fail(PS_ERR_INVALID_ARG, "%s: current device is not the head's", fn);
  return PS_OK;
}

extern "C" ps_status ps_patch_embed(ps_head* h, const float* x, float* out, int32_t n_rows, hipStream_t hs) {
  if (!h || !x || !out) return fail(PS_ERR_INVALID_ARG, "ps_patch_embed: null argument");
  if (n_rows <= 0) return fail(PS_ERR_INVALID_ARG, "ps_patch_embed: n_rows %d must be positive", n_rows);
  ps_status st = head_device_check(h, "ps_patch_embed");
  if (st) return st;
  const ps_head_desc& d = h->d;
  const size_t n = (size_t)n_rows * d.latent_dim;
  EpiArgs ep;
  ep.bias = d.b_embed;
  ep.out = out;
  ep.ldo = d.hidden;
  if (d.dtype == PS_BF16) {
    if ((st = h->ws_x.reserve(n * sizeof(bf16), hs))) return st;
    bf16* xb = static_cast<bf16*>(h->ws_x.p);
    PS_TRACED("embed_cast", launch_cast<bf16>(x, xb, n, hs));
    PS_TRACED("embed", (launch_gemm<bf16>(EPI_F32, xb, d.latent_dim, static_cast<const bf16*>(d.w_embed), n_rows,
                                          d.hidden, d.latent_dim, ep, nullptr, hs)));
  } else {
    PS_TRACED("embed", (launch_gemm<float>(EPI_F32, x, d.latent_dim, static_cast<const float*>(d.w_embed), n_rows,
                                           d.hidden, d.latent_dim, ep, nullptr, hs)));
  }
  return PS_OK;
}

template <typename T>
static ps_status run_head(ps_head* hd, const float* h, float* v, int M, int tokens, const float* mod, hipStream_t hs) {
  const ps_head_desc& d = hd->d;
  const int ldy = act_ld(d.hidden);
  T* y = static_cast<T*>(hd->ws_y.p);
  PS_TRACED("head_ln", (launch_layernorm<T>(h, y, ldy, M, d.hidden, mod, 0, 1, tokens, hs)));
  EpiArgs ep;
  ep.bias = d.b_head;
  ep.out = v;
  ep.ldo = d.latent_dim;
  PS_TRACED("head_gemm",
            (launch_gemm<T>(EPI_F32, y, ldy, static_cast<const T*>(d.w_head), M, d.latent_dim, d.hidden, ep, nullptr, hs)));
  return PS_OK;
}

extern "C" ps_status ps_output_head(ps_head* hd, ps_time_embed* te, const float* t, int32_t n, int32_t tokens,
                                    const float* h, float* v, hipStream_t hs) {
  if (!hd || !te || !t || !h || !v) return fail(PS_ERR_INVALID_ARG, "ps_output_head: null argument");
  if (n < 1 || n > PS_MAX_TASKS) return fail(PS_ERR_INVALID_ARG, "ps_output_head: n_tasks %d not in [1, %d]", n, PS_MAX_TASKS);
  if (tokens <= 0) return fail(PS_ERR_INVALID_ARG, "ps_output_head: tokens %d must be positive", tokens);
  ps_status st = head_device_check(hd, "ps_output_head");
  if (st) return st;
  const ps_head_desc& d = hd->d;
  if (te->d.hidden != d.hidden) return fail(PS_ERR_INVALID_ARG, "ps_output_head: time embedding width differs");
  for (int i = 0; i < n; ++i)
    if (!isfinite(t[i])) return fail(PS_ERR_INVALID_ARG, "ps_output_head: t[%d] not finite", i);
  const size_t M = (size_t)n * tokens;
  if (M > (size_t)INT32_MAX / 2) return fail(PS_ERR_INVALID_ARG, "ps_output_head: too many rows");
  if ((st = hd->ws_y.reserve(M * act_ld(d.hidden) * elt_size(d.dtype), hs))) return st;
  if ((st = hd->ws_mod.reserve(sizeof(float) * (size_t)n * 6 * d.hidden, hs))) return st;
  int rows[PS_MAX_TASKS], slot = 0;
  if ((st = te_resolve(te, t, n, hs, rows, &slot))) return st;
  float* mod = static_cast<float*>(hd->ws_mod.p);
  PS_TRACED("head_mod", launch_head_mod(te->cache_u, rows, d.t_head, mod, n, d.hidden, hs));
  if ((st = te_mark_read(te, rows, n, slot, hs))) return st;
  if (d.dtype == PS_BF16) return run_head<bf16>(hd, h, v, (int)M, tokens, mod, hs);
  return run_head<float>(hd, h, v, (int)M, tokens, mod, hs);
}

// ------------------------------------------------------------------ euler
extern "C" ps_status ps_euler_update(float* x, const void* v, const float* dt, int32_t n, int32_t tokens,
                                     int32_t hidden, ps_dtype v_dtype, hipStream_t hs) {
  if (!x || !v || !dt) return fail(PS_ERR_INVALID_ARG, "ps_euler_update: null argument");
  if (n < 1 || n > PS_MAX_TASKS) return fail(PS_ERR_INVALID_ARG, "ps_euler_update: n_tasks %d not in [1, %d]", n, PS_MAX_TASKS);
  if (tokens <= 0 || hidden <= 0 || ((long long)tokens * hidden) % 4 != 0)
    return fail(PS_ERR_INVALID_ARG, "ps_euler_update: tokens * hidden must be a positive multiple of 4");
  if (v_dtype != PS_F32 && v_dtype != PS_BF16) return fail(PS_ERR_INVALID_ARG, "ps_euler_update: bad v_dtype");
  for (int i = 0; i < n; ++i)
    if (!isfinite(dt[i])) return fail(PS_ERR_INVALID_ARG, "ps_euler_update: dt[%d] not finite", i);
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(v)) % 16 != 0)
    return fail(PS_ERR_INVALID_ARG, "ps_euler_update: x and v must be 16-byte aligned");
  PS_TRACED("euler", launch_euler(x, v, v_dtype, dt, n, tokens, hidden, hs));
  return PS_OK;
}

extern "C" ps_status ps_euler_update_steps(float* x, const void* v, const float* timesteps, int32_t n_steps,
                                           const int32_t* steps, int32_t n, int32_t tokens, int32_t hidden,
                                           ps_dtype v_dtype, hipStream_t hs) {
  if (!timesteps || !steps) return fail(PS_ERR_INVALID_ARG, "ps_euler_update_steps: null argument");
  if (n < 1 || n > PS_MAX_TASKS) return fail(PS_ERR_INVALID_ARG, "ps_euler_update_steps: n_tasks %d not in [1, %d]", n, PS_MAX_TASKS);
  if (n_steps < 1) return fail(PS_ERR_INVALID_ARG, "ps_euler_update_steps: n_steps %d must be positive", n_steps);
  float dt[PS_MAX_TASKS];
  for (int i = 0; i < n; ++i) {
    const int s = steps[i];
    if (s < 0 || s >= n_steps) return fail(PS_ERR_INVALID_ARG, "ps_euler_update_steps: step %d of task %d out of range", s, i);
    const float next = s + 1 < n_steps ? timesteps[s + 1] : 0.0f;
    dt[i] = timesteps[s] - next;
  }
  return ps_euler_update(x, v, dt, n, tokens, hidden, v_dtype, hs);
}

// C ABI of libps: handles, host-side validation, the slot ledger, the
// timestep-embedding cache and the launch sequence of one stage batch.
// Every check runs before the first launch, so a failing call enqueues nothing.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <cstdarg>
#include <new>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

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

// A device buffer that grows on demand (old contents are not kept).
struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
  ps_status reserve(size_t need) {
    if (need <= bytes) return PS_OK;
    if (p) {
      // earlier launches may still read the old buffer
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return fail(PS_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
      (void)hipFree(p);
      p = nullptr;
      bytes = 0;
    }
    if (hipMalloc(&p, need) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
      return fail(PS_ERR_OUT_OF_MEMORY, "workspace: cannot allocate %zu bytes", need);
    }
    bytes = need;
    return PS_OK;
  }
  void release() {
    if (p) (void)hipFree(p);
    p = nullptr;
    bytes = 0;
  }
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
    DevBuf mod, rope, y, q, a, u, tasks;
    void release() {
      mod.release();
      rope.release();
      y.release();
      q.release();
      a.release();
      u.release();
      tasks.release();
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

struct ps_time_embed {
  ps_time_desc d{};
  float* cache = nullptr;      // [capacity][6][D]: e(t)
  float* cache_u = nullptr;    // [capacity][D]: u(t), the timestep MLP output
  float* scratch = nullptr;    // 256 + 2 D floats
  std::vector<uint32_t> key;
  std::vector<uint64_t> used;
  std::vector<char> valid;
  uint64_t clock = 0;
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

// ------------------------------------------------------ timestep embedding
extern "C" ps_status ps_time_embed_create(const ps_time_desc* desc, ps_time_embed** out) {
  if (!desc || !out) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_create: null argument");
  const ps_time_desc& d = *desc;
  if (d.hidden <= 0 || d.capacity <= 0 || d.capacity > 4096)
    return fail(PS_ERR_INVALID_ARG, "time embed: bad hidden or capacity");
  if (!d.wt1 || !d.bt1 || !d.wt2 || !d.bt2 || !d.wp || !d.bp)
    return fail(PS_ERR_INVALID_ARG, "time embed: null weight pointer");
  ps_time_embed* te = new ps_time_embed();
  te->d = d;
  if (hipMalloc(&te->cache, sizeof(float) * (size_t)d.capacity * 6 * d.hidden) != hipSuccess ||
      hipMalloc(&te->cache_u, sizeof(float) * (size_t)d.capacity * d.hidden) != hipSuccess ||
      hipMalloc(&te->scratch, sizeof(float) * (PS_FREQ_DIM + 2 * (size_t)d.hidden)) != hipSuccess) {
    (void)hipGetLastError();
    if (te->cache) (void)hipFree(te->cache);
    if (te->cache_u) (void)hipFree(te->cache_u);
    delete te;
    return fail(PS_ERR_OUT_OF_MEMORY, "time embed: cannot allocate cache");
  }
  te->key.assign(d.capacity, 0);
  te->used.assign(d.capacity, 0);
  te->valid.assign(d.capacity, 0);
  *out = te;
  return PS_OK;
}

extern "C" ps_status ps_time_embed_destroy(ps_time_embed* te) {
  if (!te) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_destroy: null handle");
  (void)hipDeviceSynchronize();
  (void)hipFree(te->cache);
  (void)hipFree(te->cache_u);
  (void)hipFree(te->scratch);
  delete te;
  return PS_OK;
}

// Row of e(t) in the cache, computing it if absent.  `pinned` rows (used by
// the current batch) are never evicted.
static ps_status te_row(ps_time_embed* te, float t, const std::vector<int>& pinned, hipStream_t hs, int* row) {
  uint32_t k;
  memcpy(&k, &t, 4);
  const int cap = te->d.capacity;
  for (int i = 0; i < cap; ++i)
    if (te->valid[i] && te->key[i] == k) {
      te->used[i] = ++te->clock;
      *row = i;
      return PS_OK;
    }
  int victim = -1;
  for (int i = 0; i < cap; ++i) {
    bool pin = false;
    for (int pr : pinned) pin |= (pr == i);
    if (pin) continue;
    if (victim < 0 || !te->valid[i] || (te->valid[victim] && te->used[i] < te->used[victim])) victim = i;
    if (!te->valid[i]) break;
  }
  if (victim < 0) return fail(PS_ERR_INVALID_ARG, "time embed: more distinct timesteps in one batch than capacity");
  const int D = te->d.hidden;
  // A fill is rare (a new timestep).  It waits for all in-flight work, which
  // may still read the victim row or use the scratch from another stream, and
  // completes before the call returns, so that calls on any stream may read
  // the row afterwards.
  PS_HIP(hipDeviceSynchronize());
  PS_HIP(launch_time_embed(t, te->d.wt1, te->d.bt1, te->d.wt2, te->d.bt2, te->d.wp, te->d.bp, D, te->scratch,
                           te->cache + (size_t)victim * 6 * D, te->cache_u + (size_t)victim * D, hs));
  PS_HIP(hipStreamSynchronize(hs));
  te->valid[victim] = 1;
  te->key[victim] = k;
  te->used[victim] = ++te->clock;
  *row = victim;
  return PS_OK;
}

extern "C" ps_status ps_time_embed_get(ps_time_embed* te, float t, float* e, hipStream_t hs) {
  if (!te || !e) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_get: null argument");
  if (!isfinite(t)) return fail(PS_ERR_INVALID_ARG, "ps_time_embed_get: timestep not finite");
  int row = 0;
  ps_status st = te_row(te, t, {}, hs, &row);
  if (st) return st;
  const size_t n = (size_t)6 * te->d.hidden;
  PS_HIP(hipMemcpyAsync(e, te->cache + row * n, n * sizeof(float), hipMemcpyDeviceToDevice, hs));
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

template <typename T>
static ps_status run_stage(ps_kv_pool* p, ps_kv_pool::Workspace* w, const ps_block* b, const DevTask* tt, int n,
                           const float* mod, const float2* rope_f, const float* h_in, float* h_out,
                           const ps_stage_probe* pr, hipStream_t hs) {
  const ps_block_desc& bd = b->d;
  const int L = p->L(), D = bd.hidden, F = bd.ffn, M = n * L;
  T* y = static_cast<T*>(w->y.p);
  T* q = static_cast<T*>(w->q.p);
  T* a = static_cast<T*>(w->a.p);
  T* u = static_cast<T*>(w->u.p);
  const PoolGeo pg = p->geo();
  const float qscale = 1.4426950408889634f / sqrtf((float)bd.head_dim);
  const T* W = nullptr;

  // self-attention branch
  const int ldy = act_ld(D), ldu = act_ld(F);
  PS_TRACED("ln1", (launch_layernorm<T>(h_in, y, ldy, M, D, mod, 0, 1, L, hs)));
  PS_PROBE(y1, y, D, ldy);
  EpiArgs e1;
  e1.bias = bd.bqkv;
  e1.out = q;
  e1.ldo = D;
  e1.out_scale = qscale;
  e1.rope_f = rope_f;
  e1.pool = pg;
  e1.d_shift = bd.head_dim == 128 ? 7 : 6;
  W = static_cast<const T*>(bd.wqkv);
  PS_TRACED("qkv", (launch_gemm<T>(EPI_QKV, y, ldy, W, M, 3 * D, D, e1, tt, hs)));
  PS_PROBE(q, q, D, D);
  PS_TRACED("attn_self", (launch_attention<T>(false, q, a, ldy, pg, tt, n, hs)));
  PS_PROBE(attn, a, D, ldy);
  EpiArgs e2;
  e2.bias = bd.bo;
  e2.h_in = h_in;
  e2.h_out = h_out;
  e2.mod = mod;
  e2.gate_row = 2;
  e2.L = L;
  e2.div_L = FastDiv((uint32_t)L);
  PS_TRACED("o_proj", (launch_gemm<T>(EPI_RES, a, ldy, static_cast<const T*>(bd.wo), M, D, D, e2, tt, hs)));
  PS_PROBE(h1, h_out, D, D);

  // cross-attention branch
  PS_TRACED("ln2", (launch_layernorm<T>(h_out, y, ldy, M, D, nullptr, -1, -1, L, hs)));
  PS_PROBE(y2, y, D, ldy);
  EpiArgs e3;
  e3.bias = bd.bq2;
  e3.out = q;
  e3.ldo = D;
  e3.out_scale = qscale;
  PS_TRACED("xq_proj", (launch_gemm<T>(EPI_STORE, y, ldy, static_cast<const T*>(bd.wq2), M, D, D, e3, tt, hs)));
  PS_PROBE(q2, q, D, D);
  PS_TRACED("attn_cross", (launch_attention<T>(true, q, a, ldy, pg, tt, n, hs)));
  PS_PROBE(xattn, a, D, ldy);
  EpiArgs e4;
  e4.bias = bd.bo2;
  e4.h_in = h_out;
  e4.h_out = h_out;
  e4.L = L;
  e4.div_L = FastDiv((uint32_t)L);
  PS_TRACED("xo_proj", (launch_gemm<T>(EPI_RES, a, ldy, static_cast<const T*>(bd.wo2), M, D, D, e4, tt, hs)));
  PS_PROBE(h2, h_out, D, D);

  // FFN branch
  PS_TRACED("ln3", (launch_layernorm<T>(h_out, y, ldy, M, D, mod, 3, 4, L, hs)));
  PS_PROBE(y3, y, D, ldy);
  EpiArgs e5;
  e5.bias = bd.b1;
  e5.out = u;
  e5.ldo = ldu;
  PS_TRACED("ffn1", (launch_gemm<T>(EPI_GELU, y, ldy, static_cast<const T*>(bd.w1), M, F, D, e5, tt, hs)));
  PS_PROBE(u, u, F, ldu);
  EpiArgs e6;
  e6.bias = bd.b2;
  e6.h_in = h_out;
  e6.h_out = h_out;
  e6.mod = mod;
  e6.gate_row = 5;
  e6.L = L;
  e6.div_L = FastDiv((uint32_t)L);
  PS_TRACED("ffn2", (launch_gemm<T>(EPI_RES, u, ldu, static_cast<const T*>(bd.w2), M, D, F, e6, tt, hs)));
  return PS_OK;
}

static ps_status stage_batch(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks, int32_t n,
                             const float* h_in, float* h_out, const ps_stage_probe* probe, hipStream_t hs) {
  if (!p || !b || !te || !tasks || !h_in || !h_out) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: null argument");
  if (n < 1 || n > PS_MAX_TASKS) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: n_tasks %d not in [1, %d]", n, PS_MAX_TASKS);
  const ps_pool_desc& pd = p->desc;
  const ps_block_desc& bd = b->d;
  if (bd.dtype != pd.dtype || bd.n_heads != pd.n_heads || bd.head_dim != pd.head_dim)
    return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: block and pool disagree on dtype or heads");
  if (bd.block_index >= pd.n_blocks) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: block_index %d beyond pool", bd.block_index);
  if (te->d.hidden != bd.hidden) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: time embedding width differs");
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev != p->device) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: current device is not the pool's");

  TaskTable tt{};
  tt.n = n;
  std::vector<size_t> writes;
  for (int i = 0; i < n; ++i) {
    const ps_task& t = tasks[i];
    ps_status st = check_region(p, t.stream, bd.block_index, t.step, t.write_slot);
    if (st) return fail(st, "task %d: %s", i, g_err.c_str());
    if (t.chunk < 0) return fail(PS_ERR_INVALID_ARG, "task %d: negative chunk", i);
    if (!isfinite(t.timestep)) return fail(PS_ERR_INVALID_ARG, "task %d: timestep not finite", i);
    if (t.n_read < 0 || t.n_read > PS_MAX_WINDOW || t.n_read >= pd.n_slots)
      return fail(PS_ERR_INVALID_ARG, "task %d: n_read %d out of range", i, t.n_read);
    for (int j = 0; j < t.n_read; ++j) {
      if (t.read_slots[j] < 0 || t.read_slots[j] >= pd.n_slots)
        return fail(PS_ERR_INVALID_ARG, "task %d: read slot %d out of range", i, t.read_slots[j]);
      if (t.read_slots[j] == t.write_slot)
        return fail(PS_ERR_INVALID_ARG, "task %d: reads its own write slot %d", i, t.write_slot);
    }
    const size_t cr = (size_t)t.stream * pd.n_blocks + bd.block_index;
    if (p->ctx_len[cr] == 0)
      return fail(PS_ERR_INVALID_ARG, "task %d: context of stream %d block %d not set", i, t.stream, bd.block_index);
    const size_t reg = region_of(p, t.stream, bd.block_index, t.step);
    const size_t wkey = reg * pd.n_slots + t.write_slot;
    for (size_t w : writes)
      if (w == wkey) return fail(PS_ERR_SLOT_CONFLICT, "task %d: two tasks of the batch write one slot", i);
    writes.push_back(wkey);
    DevTask& dt = tt.t[i];
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
    for (int i = 0; i < n; ++i) led[writes[i]] = tasks[i].chunk;
    for (int i = 0; i < n; ++i) {
      const ps_task& t = tasks[i];
      const size_t reg = tt.t[i].region;
      for (int j = 0; j < t.n_read; ++j) {
        const int want = t.chunk - t.n_read + j;
        const int have = led[reg * pd.n_slots + t.read_slots[j]];
        if (have != want)
          return fail(PS_ERR_SLOT_CONFLICT, "task %d (stream %d chunk %d step %d): slot %d holds chunk %d, expected %d", i,
                      t.stream, t.chunk, t.step, t.read_slots[j], have, want);
      }
    }
  }

  // workspace
  const int L = p->L(), D = bd.hidden, F = bd.ffn;
  const size_t M = (size_t)n * L, es = elt_size(bd.dtype);
  ps_status st;
  ps_kv_pool::Workspace* w = p->workspace(hs);
  if (!w)
    return fail(PS_ERR_INVALID_ARG, "ps_stage_batch: more than %d streams use this pool", PS_MAX_STREAMS_PER_POOL);
  if ((st = w->mod.reserve(sizeof(float) * n * 6 * (size_t)D))) return st;
  if ((st = w->rope.reserve(sizeof(float2) * n * pd.frames * (size_t)(p->seg_f / 2) + 16))) return st;
  if ((st = w->y.reserve(M * act_ld(D) * es))) return st;
  if ((st = w->q.reserve(M * D * es))) return st;
  if ((st = w->a.reserve(M * act_ld(D) * es))) return st;
  if ((st = w->u.reserve(M * act_ld(F) * es))) return st;
  if ((st = w->tasks.reserve(sizeof(DevTask) * PS_MAX_TASKS))) return st;

  // timestep embeddings (cached per distinct t)
  std::vector<int> rows(n), pinned;
  for (int i = 0; i < n; ++i) {
    if ((st = te_row(te, tasks[i].timestep, pinned, hs, &rows[i]))) return st;
    pinned.push_back(rows[i]);
  }
  float* mod = static_cast<float*>(w->mod.p);
  float2* rope_f = static_cast<float2*>(w->rope.p);
  DevTask* dtasks = static_cast<DevTask*>(w->tasks.p);
  PS_TRACED("put_tasks", launch_put_tasks(tt, dtasks, hs));
  PS_TRACED("modulation", launch_modulation(te->cache, rows.data(), bd.tmod, mod, rope_f, dtasks, n, D, pd.frames, p->seg_f, hs));

  if (bd.dtype == PS_BF16)
    st = run_stage<bf16>(p, w, b, dtasks, n, mod, rope_f, h_in, h_out, probe, hs);
  else
    st = run_stage<float>(p, w, b, dtasks, n, mod, rope_f, h_in, h_out, probe, hs);
  if (st) return st;
  for (int i = 0; i < n; ++i) p->ledger[writes[i]] = tasks[i].chunk;
  return PS_OK;
}

extern "C" ps_status ps_stage_batch(ps_kv_pool* p, const ps_block* b, ps_time_embed* te, const ps_task* tasks,
                                    int32_t n, const float* h_in, float* h_out, hipStream_t hs) {
  return stage_batch(p, b, te, tasks, n, h_in, h_out, nullptr, hs);
}

extern "C" ps_status ps_stage_batch_probe(ps_kv_pool* p, const ps_block* b, ps_time_embed* te,
                                          const ps_task* tasks, int32_t n, const float* h_in, float* h_out,
                                          const ps_stage_probe* probe, hipStream_t hs) {
  if (!probe) return fail(PS_ERR_INVALID_ARG, "ps_stage_batch_probe: null probe");
  return stage_batch(p, b, te, tasks, n, h_in, h_out, probe, hs);
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
    if ((st = h->ws_x.reserve(n * sizeof(bf16)))) return st;
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
  if ((st = hd->ws_y.reserve(M * act_ld(d.hidden) * elt_size(d.dtype)))) return st;
  if ((st = hd->ws_mod.reserve(sizeof(float) * (size_t)n * 6 * d.hidden))) return st;
  std::vector<int> rows(n), pinned;
  for (int i = 0; i < n; ++i) {
    if ((st = te_row(te, t[i], pinned, hs, &rows[i]))) return st;
    pinned.push_back(rows[i]);
  }
  float* mod = static_cast<float*>(hd->ws_mod.p);
  PS_TRACED("head_mod", launch_head_mod(te->cache_u, rows.data(), d.t_head, mod, n, d.hidden, hs));
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

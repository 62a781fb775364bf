// Launchers of the gfx950 kernels behind libps (internal; not part of the ABI).
#pragma once

#include "common.h"

namespace ps {

// GEMM epilogues, fused into the tile store.
enum Epi {
  EPI_QKV = 0,     // bias, 3D RoPE on q and k; q (scaled) -> out, k / v -> pool write slot
  EPI_CTX_KV = 1,  // bias; k -> ctx K [H][Lc][d], v -> ctx V^T [H][d][Lc]
  EPI_STORE = 2,   // (acc + bias) * out_scale -> out (compute dtype)
  EPI_GELU = 3,    // GELU_tanh(acc + bias) -> out (compute dtype)
  EPI_RES = 4,     // h_out = h_in + gate * (acc + bias), gate = mod[task][gate_row] or 1
  EPI_F32 = 5,     // acc + bias -> out (fp32)
};

struct EpiArgs {
  const float* bias = nullptr;
  void* out = nullptr;
  int ldo = 0;                    // row stride of out (elements)
  float out_scale = 1.0f;
  const float* h_in = nullptr;
  float* h_out = nullptr;
  const float* mod = nullptr;     // [n_tasks][6][D]
  int gate_row = -1;
  int L = 1;
  const float2* rope_f = nullptr; // [n_tasks][frames][seg_f / 2]
  int rope_tab = 0;               // set by the launcher: RoPE tables fit the kernel's LDS
  void* ctx_base = nullptr;
  int d_shift = 0;                // log2(head_dim)
  FastDiv div_L;                  // rows per task
  PoolGeo pool{};
};

// Copies the batch's task list (a kernel argument) into device memory.
hipError_t launch_put_tasks(const TaskTable& tt, DevTask* dst, hipStream_t s);

template <typename T>
hipError_t launch_gemm(int epi, const T* A, int lda, const T* B, int M, int N, int K, const EpiArgs& ep,
                       const DevTask* tasks, hipStream_t s);
int gemm_k_step(int dtype);

// Flash attention of each task's queries over a list of key/value segments.
// self: segments = the task's read slots then its write slot (pool layout);
// cross: one segment = the (stream, block) context entry.
// q: [n_tasks * L, H * d] compute dtype, already multiplied by log2(e)/sqrt(d).
// out: [n_tasks * L, H * d] compute dtype.
template <typename T>
hipError_t launch_attention(bool cross, const T* q, T* out, int ldo, const PoolGeo& pg, const DevTask* tasks,
                            int n_tasks, hipStream_t s);

// y = LN(h) * (1 + mod[task][scale_row]) + mod[task][shift_row]  (rows >= 0),
// or plain LN(h) when shift_row < 0.  h fp32 [M][D], y compute dtype.
template <typename T>
hipError_t launch_layernorm(const float* h, T* y, int ldy, int M, int D, const float* mod, int shift_row,
                            int scale_row, int L, hipStream_t s);

// m[task] = e[e_row[task]] + tmod  ([6][D] fp32 each) and the per-task RoPE
// table of the frame axis, rope_f[task][f][i] = (cos, sin)((chunk * frames + f) theta_i).
hipError_t launch_modulation(const float* e_cache, const int* e_rows_host, const float* tmod,
                             float* mod, float2* rope_f, const DevTask* tasks, int n_tasks, int D,
                             int frames, int seg_f, hipStream_t s);

// Timestep embedding of one t into e (fp32 [6][D]) and the timestep MLP
// output u (fp32 [D]) using scratch (>= D + 256 floats).
hipError_t launch_time_embed(float t, const float* wt1, const float* bt1, const float* wt2,
                             const float* bt2, const float* wp, const float* bp, int D, float* scratch,
                             float* e, float* u, hipStream_t s);

// y = x in the compute dtype (n a multiple of 4).
template <typename T>
hipError_t launch_cast(const float* x, T* y, size_t n, hipStream_t s);

// Rows 0 and 1 of each task's [6][D] block of mod: u[u_rows[task]] + t_head.
hipError_t launch_head_mod(const float* u_cache, const int* u_rows_host, const float* t_head, float* mod,
                           int n_tasks, int D, hipStream_t s);

// RoPE tables of one axis: tab[p][i] = (cos, sin)(p * 10000^(-2 i / seg)), p < n_pos.
hipError_t launch_rope_table(float2* tab, int n_pos, int seg, hipStream_t s);

// x[i] -= dt[task(i)] * v[i]
hipError_t launch_euler(float* x, const void* v, int v_dtype, const float* dt_host, int n_tasks,
                        int tokens, int hidden, hipStream_t s);

// Cache entry <-> [n, H, d] layout moves.  An entry holds K [H][stride][d]
// followed by V^T [H][d][stride]; n <= stride tokens are valid.
template <typename T>
hipError_t launch_entry_load(T* entry, const T* k, const T* v, int n, int stride, int H, int d,
                             hipStream_t s);
template <typename T>
hipError_t launch_entry_fetch(const T* entry, T* k, T* v, int n, int stride, int H, int d,
                              hipStream_t s);

}  // namespace ps

// Memory-bound kernels of the stage task (gfx950): AdaLN / LayerNorm, the
// per-task modulation rows, the timestep embedding, RoPE tables, the Euler
// update and cache-entry layout moves.
//
// LayerNorm: one wave per row; the row stays in registers between the mean,
// the variance and the normalisation, so h is read from HBM once and y
// written once (16-byte loads where D % 256 == 0).  Statistics in fp32.
// For the common hidden sizes the row length is a template constant, so that
// all of a row's loads -- and the task's modulation rows, which are L2
// resident -- are in flight together before the first use.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ps {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int VW>
struct VecF;
template <>
struct VecF<4> { typedef f32x4 type; };
template <>
struct VecF<2> { typedef float __attribute__((ext_vector_type(2))) type; };

template <typename T, int VW, int MAXI>
__global__ void __launch_bounds__(256) k_layernorm(const float* __restrict__ h, T* __restrict__ y, int ldy,
                                                   int M, int D, const float* __restrict__ mod, int shift_row,
                                                   int scale_row, int L) {
  typedef typename VecF<VW>::type vf;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int ni = D / (64 * VW);
  const float* hr = h + (size_t)row * D;
  vf v[MAXI];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    if (i < ni) {
      v[i] = *reinterpret_cast<const vf*>(hr + (i * 64 + lane) * VW);
#pragma unroll
      for (int k = 0; k < VW; ++k) sum += v[i][k];
    }
  }
  const float mean = wave_sum(sum) / (float)D;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    if (i < ni) {
#pragma unroll
      for (int k = 0; k < VW; ++k) {
        const float dlt = v[i][k] - mean;
        sq += dlt * dlt;
      }
    }
  }
  const float var = wave_sum(sq) / (float)D;
  const float rstd = 1.0f / sqrtf(var + 1e-6f);
  const float* shift = nullptr;
  const float* scale = nullptr;
  if (shift_row >= 0) {
    const int ti = row / L;
    shift = mod + ((size_t)ti * 6 + shift_row) * D;
    scale = mod + ((size_t)ti * 6 + scale_row) * D;
  }
  T* yr = y + (size_t)row * ldy;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    if (i < ni) {
      const int c0 = (i * 64 + lane) * VW;
      float o[VW];
#pragma unroll
      for (int k = 0; k < VW; ++k) o[k] = (v[i][k] - mean) * rstd;
      if (shift) {
        const vf sh = *reinterpret_cast<const vf*>(shift + c0);
        const vf sc = *reinterpret_cast<const vf*>(scale + c0);
#pragma unroll
        for (int k = 0; k < VW; ++k) o[k] = o[k] * (1.0f + sc[k]) + sh[k];
      }
      if constexpr (sizeof(T) == 2) {
        bf16 w[VW];
#pragma unroll
        for (int k = 0; k < VW; ++k) w[k] = (bf16)o[k];
        if constexpr (VW == 4) {
          *reinterpret_cast<bf16x4*>(yr + c0) = bf16x4{w[0], w[1], w[2], w[3]};
        } else {
          typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<bf16x2*>(yr + c0) = bf16x2{w[0], w[1]};
        }
      } else {
        vf w;
#pragma unroll
        for (int k = 0; k < VW; ++k) w[k] = o[k];
        *reinterpret_cast<vf*>(yr + c0) = w;
      }
    }
  }
}

// Fixed-width variant: NI float4 per lane (D = 256 NI); MOD = modulated.
template <typename T, int NI, bool MOD>
__global__ void __launch_bounds__(256) k_layernorm_n(const float* __restrict__ h, T* __restrict__ y, int ldy,
                                                     int M, const float* __restrict__ mod, int shift_row,
                                                     int scale_row, FastDiv div_L) {
  constexpr int D = 256 * NI;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* hr = h + (size_t)row * D;
  f32x4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) v[i] = *reinterpret_cast<const f32x4*>(hr + (i * 64 + lane) * 4);
  f32x4 sh[MOD ? NI : 1], sc[MOD ? NI : 1];
  if constexpr (MOD) {
    const int ti = (int)div_L.div(row);
    const float* shift = mod + ((size_t)ti * 6 + shift_row) * D;
    const float* scale = mod + ((size_t)ti * 6 + scale_row) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      sh[i] = *reinterpret_cast<const f32x4*>(shift + (i * 64 + lane) * 4);
      sc[i] = *reinterpret_cast<const f32x4*>(scale + (i * 64 + lane) * 4);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  const float mean = wave_sum(sum) * (1.0f / D);
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float dlt = v[i][k] - mean;
      sq += dlt * dlt;
    }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) * (1.0f / D) + 1e-6f);
  T* yr = y + (size_t)row * ldy;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    f32x4 o = (v[i] - mean) * rstd;
    if constexpr (MOD) o = o * (1.0f + sc[i]) + sh[i];
    const int c0 = (i * 64 + lane) * 4;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x4*>(yr + c0) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
    } else {
      *reinterpret_cast<f32x4*>(yr + c0) = o;
    }
  }
}

struct Rows {
  int r[PS_MAX_TASKS];
};

__global__ void k_modulation(const float* __restrict__ e_cache, Rows rows, const float* __restrict__ tmod,
                             float* __restrict__ mod, float2* __restrict__ rope_f,
                             const DevTask* __restrict__ tasks, int n_tasks, int D, int frames, int seg_f) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int per = 6 * D;
  if (idx < n_tasks * per) {
    const int ti = idx / per, j = idx - ti * per;
    mod[idx] = e_cache[(size_t)rows.r[ti] * per + j] + tmod[j];
  }
  const int half = seg_f / 2;
  const int nr = n_tasks * frames * half;
  if (idx < nr) {
    const int ti = idx / (frames * half);
    const int rem = idx - ti * frames * half;
    const int f = rem / half, i = rem - f * half;
    const double p = (double)tasks[ti].chunk * frames + f;
    const double theta = pow(10000.0, -2.0 * i / seg_f);
    double sn, cs;
    sincos(p * theta, &sn, &cs);
    rope_f[idx] = make_float2((float)cs, (float)sn);
  }
}

__global__ void k_rope_table(float2* tab, int n_pos, int seg) {
  const int half = seg / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_pos * half) return;
  const int p = idx / half, i = idx - p * half;
  const double theta = pow(10000.0, -2.0 * i / seg);
  double sn, cs;
  sincos((double)p * theta, &sn, &cs);
  tab[idx] = make_float2((float)cs, (float)sn);
}

// phi(t): 128 cosines then 128 sines of 1000 t 10000^(-j/128)
__global__ void k_sinusoid(float t, float* phi) {
  const int j = threadIdx.x;
  if (j >= 128) return;
  const double w = pow(10000.0, -(double)j / 128.0);
  const double a = 1000.0 * (double)t * w;
  phi[j] = (float)cos(a);
  phi[128 + j] = (float)sin(a);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// y[n] = sum_k act(x[k]) W[n][k] + b[n]; act = SiLU or identity.  One wave per row.
__global__ void __launch_bounds__(256) k_gemv(const float* __restrict__ x, int K, const float* __restrict__ W,
                                              const float* __restrict__ b, float* __restrict__ y, int N,
                                              int silu_in) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* wr = W + (size_t)n * K;
  float acc = 0.0f;
  for (int k = lane; k < K; k += 64) {
    const float xv = silu_in ? silu(x[k]) : x[k];
    acc += xv * wr[k];
  }
  acc = wave_sum(acc);
  if (lane == 0) y[n] = acc + b[n];
}

// One wave copies the table: lane l takes words l, l + 64, ..., read straight
// from the kernel-argument segment (vector loads at the argument's address),
// all loads issued before the first store, so that the copy costs about one
// round trip to the argument memory instead of one per cache line.
__global__ void k_put_tasks(TaskTable tt, DevTask* dst) {
  constexpr int W = PS_MAX_TASKS * (int)(sizeof(DevTask) / 4);   // words of the whole array
  constexpr int PER = (W + 63) / 64;
  const int32_t* src = reinterpret_cast<const int32_t*>(&tt.t[0]);
  int32_t* out = reinterpret_cast<int32_t*>(dst);
  int32_t v[PER];
  // the loads do not wait for the task count: every word of the array is read
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = k * 64 + (int)threadIdx.x;
    v[k] = (k * 64 + 64 <= W || i < W) ? src[i] : 0;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) asm volatile("" : "+v"(v[k]));   // all loaded here, none sunk below
  const int words = tt.n * (int)(sizeof(DevTask) / 4);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = k * 64 + (int)threadIdx.x;
    if (i < words) out[i] = v[k];
  }
}

struct Dts {
  float dt[PS_MAX_TASKS];
};

template <typename V>
__global__ void k_euler(float* __restrict__ x, const V* __restrict__ v, Dts dts, size_t per_task4,
                        size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float dt = dts.dt[i / per_task4];
  f32x4 xv = reinterpret_cast<f32x4*>(x)[i];
  f32x4 vv;
  if constexpr (sizeof(V) == 4) {
    vv = reinterpret_cast<const f32x4*>(v)[i];
  } else {
    const bf16x4 b = reinterpret_cast<const bf16x4*>(v)[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) vv[k] = (float)b[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) xv[k] = xv[k] - dt * vv[k];
  reinterpret_cast<f32x4*>(x)[i] = xv;
}

template <typename T>
__global__ void k_entry_load(T* entry, const T* k, const T* v, int n, int stride, int H, int d) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t tot = (size_t)n * H * d;
  if (idx >= tot) return;
  const int dd = idx % d;
  const int hh = (idx / d) % H;
  const int tok = idx / ((size_t)H * d);
  entry[((size_t)hh * stride + tok) * d + dd] = k[idx];
  entry[(size_t)H * stride * d + ((size_t)hh * d + dd) * stride + tok] = v[idx];
}

template <typename T>
__global__ void k_entry_fetch(const T* entry, T* k, T* v, int n, int stride, int H, int d) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t tot = (size_t)n * H * d;
  if (idx >= tot) return;
  const int dd = idx % d;
  const int hh = (idx / d) % H;
  const int tok = idx / ((size_t)H * d);
  k[idx] = entry[((size_t)hh * stride + tok) * d + dd];
  v[idx] = entry[(size_t)H * stride * d + ((size_t)hh * d + dd) * stride + tok];
}

}  // namespace

template <typename T>
hipError_t launch_layernorm(const float* h, T* y, int ldy, int M, int D, const float* mod, int shift_row,
                            int scale_row, int L, hipStream_t s) {
  dim3 grid((M + 3) / 4), block(256);
  const bool m = shift_row >= 0;
  const FastDiv dl((uint32_t)L);
#define PS_LN_CASE(NI)                                                                                  \
  case NI:                                                                                              \
    if (m)                                                                                              \
      hipLaunchKernelGGL((k_layernorm_n<T, NI, true>), grid, block, 0, s, h, y, ldy, M, mod, shift_row,   \
                         scale_row, dl);                                                                \
    else                                                                                                \
      hipLaunchKernelGGL((k_layernorm_n<T, NI, false>), grid, block, 0, s, h, y, ldy, M, mod, shift_row,  \
                         scale_row, dl);                                                                \
    return hipGetLastError();
  if (D % 256 == 0) {
    switch (D / 256) {
      PS_LN_CASE(6)
      PS_LN_CASE(8)
      PS_LN_CASE(12)
      PS_LN_CASE(16)
      PS_LN_CASE(20)
      PS_LN_CASE(24)
      default: break;
    }
  }
#undef PS_LN_CASE
  if (D % 256 == 0 && D <= 8192) {
    hipLaunchKernelGGL((k_layernorm<T, 4, 32>), grid, block, 0, s, h, y, ldy, M, D, mod, shift_row, scale_row, L);
  } else if (D % 128 == 0 && D <= 8192) {
    hipLaunchKernelGGL((k_layernorm<T, 2, 64>), grid, block, 0, s, h, y, ldy, M, D, mod, shift_row, scale_row, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template hipError_t launch_layernorm<bf16>(const float*, bf16*, int, int, int, const float*, int, int, int,
                                           hipStream_t);
template hipError_t launch_layernorm<float>(const float*, float*, int, int, int, const float*, int, int, int,
                                            hipStream_t);

hipError_t launch_modulation(const float* e_cache, const int* e_rows_host, const float* tmod, float* mod,
                             float2* rope_f, const DevTask* tasks, int n_tasks, int D, int frames, int seg_f,
                             hipStream_t s) {
  Rows rows{};
  for (int i = 0; i < n_tasks; ++i) rows.r[i] = e_rows_host[i];
  const int n = max(n_tasks * 6 * D, n_tasks * frames * (seg_f / 2));
  hipLaunchKernelGGL(k_modulation, dim3((n + 255) / 256), dim3(256), 0, s, e_cache, rows, tmod, mod, rope_f, tasks,
                     n_tasks, D, frames, seg_f);
  return hipGetLastError();
}

hipError_t launch_put_tasks(const TaskTable& tt, DevTask* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_put_tasks, dim3(1), dim3(64), 0, s, tt, dst);
  return hipGetLastError();
}

hipError_t launch_time_embed(float t, const float* wt1, const float* bt1, const float* wt2, const float* bt2,
                             const float* wp, const float* bp, int D, float* scratch, float* e, float* u,
                             hipStream_t s) {
  float* phi = scratch;
  float* u1 = scratch + PS_FREQ_DIM;
  float* u2 = u;
  hipLaunchKernelGGL(k_sinusoid, dim3(1), dim3(128), 0, s, t, phi);
  hipLaunchKernelGGL(k_gemv, dim3((D + 3) / 4), dim3(256), 0, s, phi, PS_FREQ_DIM, wt1, bt1, u1, D, 0);
  hipLaunchKernelGGL(k_gemv, dim3((D + 3) / 4), dim3(256), 0, s, u1, D, wt2, bt2, u2, D, 1);
  hipLaunchKernelGGL(k_gemv, dim3((6 * D + 3) / 4), dim3(256), 0, s, u2, D, wp, bp, e, 6 * D, 1);
  return hipGetLastError();
}

// y[i] = x[i] in the compute dtype (round to nearest even)
template <typename T>
__global__ void k_cast(const float* __restrict__ x, T* __restrict__ y, size_t n) {
  const size_t i = (blockIdx.x * (size_t)blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4 v = *reinterpret_cast<const f32x4*>(x + i);
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(y + i) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  } else {
    *reinterpret_cast<f32x4*>(y + i) = v;
  }
}

template <typename T>
hipError_t launch_cast(const float* x, T* y, size_t n, hipStream_t s) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const size_t n4 = n / 4;
  hipLaunchKernelGGL((k_cast<T>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}
template hipError_t launch_cast<bf16>(const float*, bf16*, size_t, hipStream_t);
template hipError_t launch_cast<float>(const float*, float*, size_t, hipStream_t);

// Output-head modulation: rows 0 (shift) and 1 (scale) of task i's [6][D]
// block of mod = u(t_i) + t_head; the other four rows are not touched.
__global__ void k_head_mod(const float* __restrict__ u_cache, Rows rows, const float* __restrict__ t_head,
                           float* __restrict__ mod, int n_tasks, int D) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_tasks * 2 * D) return;
  const int ti = idx / (2 * D), j = idx - ti * 2 * D;
  mod[(size_t)ti * 6 * D + j] = u_cache[(size_t)rows.r[ti] * D + (j % D)] + t_head[j];
}

hipError_t launch_head_mod(const float* u_cache, const int* u_rows_host, const float* t_head, float* mod,
                           int n_tasks, int D, hipStream_t s) {
  if (n_tasks < 1 || n_tasks > PS_MAX_TASKS) return hipErrorInvalidValue;
  Rows rows{};
  for (int i = 0; i < n_tasks; ++i) rows.r[i] = u_rows_host[i];
  const int n = n_tasks * 2 * D;
  hipLaunchKernelGGL(k_head_mod, dim3((n + 255) / 256), dim3(256), 0, s, u_cache, rows, t_head, mod, n_tasks, D);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int n_pos, int seg, hipStream_t s) {
  const int n = n_pos * (seg / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, s, tab, n_pos, seg);
  return hipGetLastError();
}

hipError_t launch_euler(float* x, const void* v, int v_dtype, const float* dt_host, int n_tasks, int tokens,
                        int hidden, hipStream_t s) {
  Dts dts{};
  for (int i = 0; i < n_tasks; ++i) dts.dt[i] = dt_host[i];
  const size_t per4 = (size_t)tokens * hidden / 4;
  const size_t n4 = per4 * n_tasks;
  const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
  if (v_dtype == PS_F32) {
    hipLaunchKernelGGL((k_euler<float>), grid, block, 0, s, x, static_cast<const float*>(v), dts, per4, n4);
  } else {
    hipLaunchKernelGGL((k_euler<bf16>), grid, block, 0, s, x, static_cast<const bf16*>(v), dts, per4, n4);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_entry_load(T* entry, const T* k, const T* v, int n, int stride, int H, int d, hipStream_t s) {
  const size_t tot = (size_t)n * H * d;
  hipLaunchKernelGGL((k_entry_load<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, entry, k, v, n,
                     stride, H, d);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_entry_fetch(const T* entry, T* k, T* v, int n, int stride, int H, int d, hipStream_t s) {
  const size_t tot = (size_t)n * H * d;
  hipLaunchKernelGGL((k_entry_fetch<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, entry, k, v, n,
                     stride, H, d);
  return hipGetLastError();
}
template hipError_t launch_entry_load<bf16>(bf16*, const bf16*, const bf16*, int, int, int, int, hipStream_t);
template hipError_t launch_entry_load<float>(float*, const float*, const float*, int, int, int, int, hipStream_t);
template hipError_t launch_entry_fetch<bf16>(const bf16*, bf16*, bf16*, int, int, int, int, hipStream_t);
template hipError_t launch_entry_fetch<float>(const float*, float*, float*, int, int, int, int, hipStream_t);

}  // namespace ps

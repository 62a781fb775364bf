// Dense contractions of the stage task on gfx950 MFMA, with fused epilogues.
//
// C[M, N] = A[M, K] * B[N, K]^T, A = activations (row-major, K contiguous),
// B = weights in [out, in] layout (K contiguous).  M = n_tasks * L rows: the
// whole batch of stage tasks is one GEMM against the block's weights, which is
// what time-sharing buys (tasks of one block from different chunks and steps
// share one weight pass: AREX article on the PhysisServe report, section
// "三层设计", layer 2).
//
// Tiling: 256 x 256 macro tile, 128 bytes of K per stage (64 bf16 / 32 fp32),
// 4 waves in a 2 x 2 grid, each owning a 128 x 128 sub-tile = 4 x 4 MFMA
// 32x32 accumulators.  Operand tiles are double-buffered in LDS (2 x 64 KB)
// with a 16-byte-chunk XOR swizzle (chunk ^ (row & 7)) so that the MFMA
// fragment reads of 32 consecutive rows hit distinct banks.  The next K stage
// is fetched into registers while the current one is multiplied.
//
// Tile order: the linear workgroup id is first remapped so that consecutive
// ids land on the same XCD (the dispatcher deals workgroups to the 8 XCDs
// round-robin, each XCD has its own L2), then walked in groups of 8 tile rows
// so that the tiles an XCD runs together share operand panels in its L2.
#include "common.h"
#include "kernels.h"

namespace ps {

namespace {

constexpr int BM = 256, BN = 256, ROWB = 128, NT = 256;
constexpr int CPR = ROWB / 16;  // 16-byte chunks per LDS row (8)
constexpr int EPITCH = 65;      // fp32 row pitch of the epilogue staging (64 columns + 1)
constexpr int OPER_BYTES = 2 * (BM + BN) * ROWB;        // double-buffered operand tiles
constexpr int STAGE_BYTES = 4 * 128 * EPITCH * 4;      // 4 waves x 128 rows x pitch
constexpr int SMEM_BYTES = OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES;

__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int full = (total / 8) * 8;
  if (id >= full) return id;
  return (id % 8) * (total / 8) + id / 8;
}

__device__ __forceinline__ float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * z * (1.0f + tanhf(k0 * (z + 0.044715f * z * z * z)));
}

// Epilogue of one wave's 128 x 64 staged block (rows rbase.., columns cbase..).
template <typename T, int EPI>
__device__ __forceinline__ void epilogue_half(const float* stg, int rbase, int cbase, int lane, int M, int N,
                                              const EpiArgs& ep, const DevTask* __restrict__ tasks) {
  const int col = cbase + lane;
  const bool col_ok = col < N;
  if (cbase >= N) return;
  const int nrows = min(128, M - rbase);
  const PoolGeo& pg = ep.pool;
  if constexpr (EPI == EPI_QKV || EPI == EPI_CTX_KV) {
    const int D = pg.H * pg.d;
    const int part = cbase / D;  // a 64-column block lies inside one of q / k / v
    const bool transposed = (EPI == EPI_QKV) ? part == 2 : part == 1;
    if (transposed) {
      // values -> V^T [H][d][tokens]: one lane per row (token), columns in turn
      const int stride = (EPI == EPI_QKV) ? pg.L : pg.max_ctx;
      for (int half = 0; half < 2; ++half) {
        const int rr = half * 64 + lane;
        if (half * 64 >= nrows) break;
        const bool row_ok = rr < nrows;
        const int row = rbase + rr;
        T* vt;
        int tok;
        if constexpr (EPI == EPI_QKV) {
          const int ti = row_ok ? (int)pg.div_L.div(row) : 0;
          tok = row - ti * pg.L;
          const DevTask& tk = tasks[ti];
          vt = static_cast<T*>(pg.kv) +
               ((size_t)tk.region * pg.n_slots + tk.slots[tk.n_seg - 1]) * pg.slot_elems +
               (size_t)pg.H * pg.L * pg.d;
        } else {
          tok = row;
          vt = static_cast<T*>(ep.ctx_base) + (size_t)pg.H * pg.max_ctx * pg.d;
        }
        for (int c2 = 0; c2 < 64; ++c2) {
          const int cg = cbase + c2;
          if (cg >= N) break;
          const float val = stg[rr * EPITCH + c2] + ep.bias[cg];
          const int cc = cg - part * D;
          const int hh = cc >> ep.d_shift, dd = cc & (pg.d - 1);
          if (row_ok) vt[((size_t)hh * pg.d + dd) * stride + tok] = from_f32<T>(val);
        }
      }
      return;
    }
    // q or k (QKV) / k (context): one lane per column, rows in turn
    const float bias = col_ok ? ep.bias[col] : 0.0f;
    const int cc = col - part * D;
    const int hh = cc >> ep.d_shift, dd = cc & (pg.d - 1);
    if constexpr (EPI == EPI_CTX_KV) {
      T* kb = static_cast<T*>(ep.ctx_base);
      for (int rr = 0; rr < nrows; ++rr) {
        const float val = stg[rr * EPITCH + lane] + bias;
        if (col_ok) kb[((size_t)hh * pg.max_ctx + rbase + rr) * pg.d + dd] = from_f32<T>(val);
      }
      return;
    } else {
      const float bias_p = (col ^ 1) < N ? ep.bias[col ^ 1] : 0.0f;
      const float sgn = (dd & 1) ? 1.0f : -1.0f;
      int seg, pi;
      if (dd < pg.seg_f) {
        seg = 0; pi = dd >> 1;
      } else if (dd < pg.seg_f + pg.seg_h) {
        seg = 1; pi = (dd - pg.seg_f) >> 1;
      } else {
        seg = 2; pi = (dd - pg.seg_f - pg.seg_h) >> 1;
      }
      for (int rr = 0; rr < nrows; ++rr) {
        const int row = rbase + rr;
        const int ti = (int)pg.div_L.div(row);
        const int tok = row - ti * pg.L;
        const int yx = (int)pg.div_cols.div(tok);
        float2 cs;
        if (seg == 0) {
          const int fl = (int)pg.div_plane.div(tok);
          cs = ep.rope_f[(ti * pg.frames + fl) * (pg.seg_f / 2) + pi];
        } else if (seg == 1) {
          const int yy = yx - (int)pg.div_rows.div(yx) * pg.rows;
          cs = pg.rope_y[yy * (pg.seg_h / 2) + pi];
        } else {
          const int xx = tok - yx * pg.cols;
          cs = pg.rope_x[xx * (pg.seg_w / 2) + pi];
        }
        const float val = stg[rr * EPITCH + lane] + bias;
        const float partner = stg[rr * EPITCH + (lane ^ 1)] + bias_p;
        const float out = val * cs.x + sgn * partner * cs.y;
        if (!col_ok) continue;
        if (part == 0) {
          static_cast<T*>(ep.out)[(size_t)row * D + cc] = from_f32<T>(out * ep.out_scale);
        } else {
          const DevTask& tk = tasks[ti];
          T* kb = static_cast<T*>(pg.kv) +
                  ((size_t)tk.region * pg.n_slots + tk.slots[tk.n_seg - 1]) * pg.slot_elems;
          kb[((size_t)hh * pg.L + tok) * pg.d + dd] = from_f32<T>(out);
        }
      }
      return;
    }
  } else {
    const float bias = col_ok ? ep.bias[col] : 0.0f;
    for (int rr = 0; rr < nrows; ++rr) {
      const int row = rbase + rr;
      const float val = stg[rr * EPITCH + lane] + bias;
      if (!col_ok) continue;
      const size_t o = (size_t)row * N + col;
      if constexpr (EPI == EPI_STORE) {
        static_cast<T*>(ep.out)[o] = from_f32<T>(val * ep.out_scale);
      } else if constexpr (EPI == EPI_GELU) {
        static_cast<T*>(ep.out)[o] = from_f32<T>(gelu_tanh(val));
      } else {  // EPI_RES: h_out = h_in + gate * val
        float gate = 1.0f;
        if (ep.gate_row >= 0) {
          const int ti = (int)ep.div_L.div(row);
          gate = ep.mod[((size_t)ti * 6 + ep.gate_row) * N + col];
        }
        ep.h_out[o] = ep.h_in[o] + gate * val;
      }
    }
  }
}

template <typename T, int EPI>
__global__ void __launch_bounds__(NT) k_gemm(const T* __restrict__ A, const T* __restrict__ B,
                                             int M, int N, int K, EpiArgs ep,
                                             const DevTask* __restrict__ tasks) {
  constexpr int BK = ROWB / sizeof(T);
  __shared__ u32x4 smem[SMEM_BYTES / 16];
  u32x4(*lds)[(BM + BN) * CPR] = reinterpret_cast<u32x4(*)[(BM + BN) * CPR]>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int pid = xcd_remap(blockIdx.x, total);
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int first_m = (pid / per_group) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // Operand fetch through buffer resources: rows past M (or N) lie past the
  // resource's end and read as zero, so ragged tiles need no clamping.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(A), 0, (int)((size_t)M * K * sizeof(T)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(B), 0, (int)((size_t)N * K * sizeof(T)), 0x00020000);
  // this thread moves 16-byte chunk c of rows r0 + 32 i of each operand tile
  const int c = tid & 7, r0 = tid >> 3;
  const int pc = c ^ (r0 & 7);
  const uint32_t row_bytes = (uint32_t)K * sizeof(T);
  const uint32_t a_off = (uint32_t)(m0 + r0) * row_bytes + c * 16;
  const uint32_t b_off = (uint32_t)(n0 + r0) * row_bytes + c * 16;
  const uint32_t step32 = 32u * row_bytes;
  u32x4 ra_[8], rb_[8];
  auto fetch = [&](int kt) {
    const int koff = kt * ROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra_[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(a_off + i * step32), koff, 0);
      rb_[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(b_off + i * step32), koff, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds[buf][(r0 + 32 * i) * CPR + pc] = ra_[i];
      lds[buf][(BM + r0 + 32 * i) * CPR + pc] = rb_[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave >> 1, wn = wave & 1;
  const int nk = K / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch(kt + 1);
#pragma unroll
    for (int u = 0; u < CPR / 2; ++u) {
      const int ch = (2 * u + g) ^ (l32 & 7);
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds[buf][(wm * 128 + i * 32 + l32) * CPR + ch];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = lds[buf][(BM + wn * 128 + j * 32 + l32) * CPR + ch];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mfma<T>::unit(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // The accumulators go through LDS, 64 columns at a time (row pitch 65
  // floats), so that the epilogue walks rows (or columns) with one lane per
  // element and every global store is a contiguous run.
  float* stg = reinterpret_cast<float*>(smem) + wave * (128 * EPITCH);
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          stg[row * EPITCH + jj * 32 + l32] = acc[i][2 * hlf + jj][r];
        }
    __syncthreads();
    epilogue_half<T, EPI>(stg, m0 + wm * 128, n0 + wn * 128 + hlf * 64, lane, M, N, ep, tasks);
    __syncthreads();
  }
}

}  // namespace

template <typename T>
hipError_t launch_gemm(int epi, const T* A, const T* B, int M, int N, int K, const EpiArgs& ep,
                       const DevTask* tt, hipStream_t s) {
  // 32-bit buffer offsets: every operand byte (plus one tile of overrun) must be addressable
  const uint64_t lim = 1ull << 32;
  if ((uint64_t)(M + BM) * K * sizeof(T) >= lim || (uint64_t)(N + BN) * K * sizeof(T) >= lim ||
      K % (ROWB / (int)sizeof(T)) != 0 || M <= 0 || N <= 0)
    return hipErrorInvalidValue;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid(tiles), block(NT);
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((k_gemm<T, EPI_QKV>), grid, block, 0, s, A, B, M, N, K, ep, tt); break;
    case EPI_CTX_KV: hipLaunchKernelGGL((k_gemm<T, EPI_CTX_KV>), grid, block, 0, s, A, B, M, N, K, ep, tt); break;
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<T, EPI_STORE>), grid, block, 0, s, A, B, M, N, K, ep, tt); break;
    case EPI_GELU: hipLaunchKernelGGL((k_gemm<T, EPI_GELU>), grid, block, 0, s, A, B, M, N, K, ep, tt); break;
    case EPI_RES: hipLaunchKernelGGL((k_gemm<T, EPI_RES>), grid, block, 0, s, A, B, M, N, K, ep, tt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_gemm<bf16>(int, const bf16*, const bf16*, int, int, int, const EpiArgs&,
                                      const DevTask*, hipStream_t);
template hipError_t launch_gemm<float>(int, const float*, const float*, int, int, int, const EpiArgs&,
                                       const DevTask*, hipStream_t);

int gemm_k_step(int dtype) { return dtype == PS_BF16 ? ROWB / 2 : ROWB / 4; }

}  // namespace ps

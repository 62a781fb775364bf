// Dense contractions of the stage task on gfx950 MFMA, with fused epilogues.
//
// C[M, N] = A[M, K] * B[N, K]^T, A = activations (row-major, K contiguous),
// B = weights in [out, in] layout (K contiguous).  M = n_tasks * L rows: the
// whole batch of stage tasks is one GEMM against the block's weights, which is
// what time-sharing buys (tasks of one block from different chunks and steps
// share one weight pass: AREX article on the PhysisServe report, section
// "三层设计", layer 2).
//
// Tiling: 256 x 256 macro tile, 4 waves in a 2 x 2 grid, each owning a
// 128 x 128 sub-tile = 4 x 4 MFMA 32x32 accumulators (in AGPRs).  K advances
// in stages of 64 bytes per row (32 bf16 / 16 fp32) through a ring of 4 LDS
// stages; operand chunks are XOR-swizzled so that fragment reads of
// consecutive rows hit distinct banks.  Stage kt is multiplied while the
// first fragments of stage kt + 1 are read, stage kt + 2 is written to LDS
// and stage kt + 4 is fetched into registers.
//
// Tile order: the linear workgroup id is first remapped so that consecutive
// ids land on the same XCD (the dispatcher deals workgroups to the 8 XCDs
// round-robin, each XCD has its own L2), then walked in groups of 8 tile rows
// so that the tiles an XCD runs together share operand panels in its L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ps {

namespace {

constexpr int BM = 256, BN = 256, ROWB = 128, NT = 256;
constexpr int CPR = ROWB / 16;  // 16-byte chunks per LDS row (8)
constexpr int NSTAGE = 2;       // LDS stages of operands
constexpr int EPITCH = 65;      // fp32 row pitch of the epilogue staging (64 columns + 1)
constexpr int STAGE_CH = (BM + BN) * CPR;               // 16-byte chunks per stage
constexpr int OPER_BYTES = NSTAGE * STAGE_CH * 16;      // 2 x 64 KB
constexpr int STAGE_BYTES = 4 * 128 * EPITCH * 4;      // 4 waves x 128 rows x pitch
constexpr int SMEM_BYTES = OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a raw buffer straight into LDS at lds_addr + 16 * lane.
// Written as inline assembly so that the compiler does not treat every later
// LDS read as dependent on it (it would wait for all copies in flight); the
// kernel orders these copies itself with vm_wait + barriers.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// s_waitcnt vmcnt(n) for n in {0, 8, 16} (memory operations still in flight).
__device__ __forceinline__ void vm_wait(int n) {
  if (n >= 16) {
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  } else if (n >= 8) {
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

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
// Rows (or columns) are processed EB at a time so that EB independent global
// loads and stores are in flight per lane instead of one.
constexpr int EB = 8;

template <typename T, int EPI>
__device__ __forceinline__ void epilogue_half(const float* stg, int rbase, int cbase, int lane, int M, int N,
                                              const EpiArgs& ep, const DevTask* __restrict__ tasks) {
  const int col = cbase + lane;
  const bool col_ok = col < N;
  if (cbase >= N) return;
  const int nrows = min(128, M - rbase);
  if (nrows <= 0) return;
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
        const int ncol = min(64, N - cbase);
        for (int c0 = 0; c0 < ncol; c0 += EB) {
          float val[EB];
#pragma unroll
          for (int k = 0; k < EB; ++k) val[k] = stg[rr * EPITCH + c0 + k] + ep.bias[min(cbase + c0 + k, N - 1)];
#pragma unroll
          for (int k = 0; k < EB; ++k) {
            const int cc = cbase + c0 + k - part * D;
            const int hh = cc >> ep.d_shift, dd = cc & (pg.d - 1);
            if (row_ok && c0 + k < ncol) vt[((size_t)hh * pg.d + dd) * stride + tok] = from_f32<T>(val[k]);
          }
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
      for (int r0 = 0; r0 < nrows; r0 += EB) {
        float2 cs[EB];
        int tis[EB], toks[EB];
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          const int row = rbase + min(r0 + k, nrows - 1);
          const int ti = (int)pg.div_L.div(row);
          const int tok = row - ti * pg.L;
          const int yx = (int)pg.div_cols.div(tok);
          tis[k] = ti;
          toks[k] = tok;
          if (seg == 0) {
            const int fl = (int)pg.div_plane.div(tok);
            cs[k] = ep.rope_f[(ti * pg.frames + fl) * (pg.seg_f / 2) + pi];
          } else if (seg == 1) {
            const int yy = yx - (int)pg.div_rows.div(yx) * pg.rows;
            cs[k] = pg.rope_y[yy * (pg.seg_h / 2) + pi];
          } else {
            const int xx = tok - yx * pg.cols;
            cs[k] = pg.rope_x[xx * (pg.seg_w / 2) + pi];
          }
        }
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          const int rr = r0 + k;
          if (rr >= nrows || !col_ok) continue;
          const int row = rbase + rr;
          const float val = stg[rr * EPITCH + lane] + bias;
          const float partner = stg[rr * EPITCH + (lane ^ 1)] + bias_p;
          const float o = val * cs[k].x + sgn * partner * cs[k].y;
          if (part == 0) {
            static_cast<T*>(ep.out)[(size_t)row * D + cc] = from_f32<T>(o * ep.out_scale);
          } else {
            const DevTask& tk = tasks[tis[k]];
            T* kb = static_cast<T*>(pg.kv) +
                    ((size_t)tk.region * pg.n_slots + tk.slots[tk.n_seg - 1]) * pg.slot_elems;
            kb[((size_t)hh * pg.L + toks[k]) * pg.d + dd] = from_f32<T>(o);
          }
        }
      }
      return;
    }
  } else {
    const float bias = col_ok ? ep.bias[col] : 0.0f;
    for (int r0 = 0; r0 < nrows; r0 += EB) {
      float val[EB];
#pragma unroll
      for (int k = 0; k < EB; ++k) val[k] = stg[min(r0 + k, 127) * EPITCH + lane] + bias;
      if constexpr (EPI == EPI_RES) {
        float hv[EB], gv[EB];
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          const int row = rbase + min(r0 + k, nrows - 1);
          const size_t o = (size_t)row * N + (col_ok ? col : 0);
          hv[k] = ep.h_in[o];
          gv[k] = 1.0f;
          if (ep.gate_row >= 0) {
            const int ti = (int)ep.div_L.div(row);
            gv[k] = ep.mod[((size_t)ti * 6 + ep.gate_row) * N + (col_ok ? col : 0)];
          }
        }
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          if (r0 + k >= nrows || !col_ok) continue;
          const size_t o = (size_t)(rbase + r0 + k) * N + col;
          ep.h_out[o] = hv[k] + gv[k] * val[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          if (r0 + k >= nrows || !col_ok) continue;
          const size_t o = (size_t)(rbase + r0 + k) * ep.ldo + col;
          if constexpr (EPI == EPI_STORE) {
            static_cast<T*>(ep.out)[o] = from_f32<T>(val[k] * ep.out_scale);
          } else {
            static_cast<T*>(ep.out)[o] = from_f32<T>(gelu_tanh(val[k]));
          }
        }
      }
    }
  }
}

template <typename T, int EPI>
__global__ void __launch_bounds__(NT) k_gemm(const T* __restrict__ A, const T* __restrict__ B,
                                             int M, int N, int K, int lda, EpiArgs ep,
                                             const DevTask* __restrict__ tasks) {
  constexpr int BK = ROWB / sizeof(T);
  __shared__ u32x4 smem[SMEM_BYTES / 16];

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

  // Operands stream from memory straight into LDS (buffer_load ... lds): each
  // instruction moves 64 lanes x 16 bytes into one contiguous 1 KB block =
  // 8 rows of a stage (128 bytes of K each: whole cache lines).  Rows past M
  // (or N) lie past the buffer resource's end and arrive as zeros, so ragged
  // tiles need no clamping.  The chunk a lane fetches is chosen so that the
  // block lands already swizzled.  A's row stride is lda elements (the
  // activation buffers are padded so that rows do not all start on the same
  // memory channel); B is dense.
  const uint64_t a_base = (uint64_t)(uintptr_t)A, b_base = (uint64_t)(uintptr_t)B;
  const i32x4 rsa = {(int)(uint32_t)a_base, (int)(uint32_t)(a_base >> 32), (int)((size_t)M * lda * sizeof(T)),
                     0x00020000};
  const i32x4 rsb = {(int)(uint32_t)b_base, (int)(uint32_t)(b_base >> 32), (int)((size_t)N * K * sizeof(T)),
                     0x00020000};
  const uint32_t a_row = (uint32_t)lda * sizeof(T), b_row = (uint32_t)K * sizeof(T);
  uint32_t voa[8], vob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int cl = (lane & 7) ^ lds_swz<CPR>(row);
    voa[i] = (uint32_t)(m0 + row) * a_row + cl * 16;
    vob[i] = (uint32_t)(n0 + row) * b_row + cl * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t wblk = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 8 * 1024);
  auto dma_stage = [&](int kt) {
    const uint32_t dst = lds0 + (kt & (NSTAGE - 1)) * (STAGE_CH * 16) + wblk;
    const uint32_t koff = (uint32_t)kt * ROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_dma16(rsa, voa[i], koff, dst + i * 1024);
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_dma16(rsb, vob[i], koff, dst + BM * ROWB + i * 1024);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave >> 1, wn = wave & 1;
  const int fsw = lds_swz<CPR>(l32);
  u32x4 fr[2][8];   // MFMA fragments of two k-units (A 0..3, B 4..7)
  auto frags = [&](int set, int buf, int u) {
    const u32x4* st = smem + buf * STAGE_CH;
    const int ch = (2 * u + g) ^ fsw;
#pragma unroll
    for (int i = 0; i < 4; ++i) fr[set][i] = st[(wm * 128 + i * 32 + l32) * CPR + ch];
#pragma unroll
    for (int j = 0; j < 4; ++j) fr[set][4 + j] = st[(BM + wn * 128 + j * 32 + l32) * CPR + ch];
  };
  auto mma = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) Mfma<T>::unit(acc[i][j], fr[set][i], fr[set][4 + j]);
  };
  // Instruction order: LDS fragment reads and the memory-to-LDS copies spread
  // between the MFMAs so that their latencies hide behind matrix work.
  auto interleave = [&]() {
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // Pipeline over stages of 128 bytes of K (four MFMA k-units), two LDS
  // buffers.  Stage kt + 1 is copied in while stage kt is multiplied; the
  // barrier sits before the last k-unit of stage kt, so that the first
  // fragments of stage kt + 1 are read while that unit's MFMAs run, and the
  // copy of stage kt + 2 (into the buffer just finished) starts right after it.
  const int nk = K / BK;
  dma_stage(0);
  if (nk > 1) {
    dma_stage(1);
    vm_wait(16);
  } else {
    vm_wait(0);
  }
  __syncthreads();
  frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    frags(1, buf, 1);
    mma(0);
    interleave();
    frags(0, buf, 2);
    mma(1);
    interleave();
    frags(1, buf, 3);
    mma(0);
    interleave();
    if (kt + 1 < nk) {
      vm_wait(0);
      __syncthreads();
      if (kt + 2 < nk) dma_stage(kt + 2);
      frags(0, buf ^ 1, 0);
    }
    mma(1);
    interleave();
  }
  __syncthreads();

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
hipError_t launch_gemm(int epi, const T* A, int lda, const T* B, int M, int N, int K, const EpiArgs& ep,
                       const DevTask* tt, hipStream_t s) {
  // 32-bit buffer offsets: every operand byte (plus one tile of overrun) must be addressable
  const uint64_t lim = 1ull << 32;
  if ((uint64_t)(M + BM) * lda * sizeof(T) >= lim || (uint64_t)(N + BN) * K * sizeof(T) >= lim ||
      K % (ROWB / (int)sizeof(T)) != 0 || M <= 0 || N <= 0 || lda < K || (lda * sizeof(T)) % 16 != 0)
    return hipErrorInvalidValue;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid(tiles), block(NT);
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((k_gemm<T, EPI_QKV>), grid, block, 0, s, A, B, M, N, K, lda, ep, tt); break;
    case EPI_CTX_KV: hipLaunchKernelGGL((k_gemm<T, EPI_CTX_KV>), grid, block, 0, s, A, B, M, N, K, lda, ep, tt); break;
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<T, EPI_STORE>), grid, block, 0, s, A, B, M, N, K, lda, ep, tt); break;
    case EPI_GELU: hipLaunchKernelGGL((k_gemm<T, EPI_GELU>), grid, block, 0, s, A, B, M, N, K, lda, ep, tt); break;
    case EPI_RES: hipLaunchKernelGGL((k_gemm<T, EPI_RES>), grid, block, 0, s, A, B, M, N, K, lda, ep, tt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_gemm<bf16>(int, const bf16*, int, const bf16*, int, int, int, const EpiArgs&,
                                      const DevTask*, hipStream_t);
template hipError_t launch_gemm<float>(int, const float*, int, const float*, int, int, int, const EpiArgs&,
                                       const DevTask*, hipStream_t);

int gemm_k_step(int dtype) { return dtype == PS_BF16 ? ROWB / 2 : ROWB / 4; }

}  // namespace ps

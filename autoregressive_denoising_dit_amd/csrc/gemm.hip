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
// in stages of 128 bytes per row (64 bf16 / 32 fp32 = four MFMA k-units)
// through two LDS stages filled by memory-to-LDS copies.  Operand chunks are
// XOR-swizzled so that fragment reads of consecutive rows hit distinct banks.
//
// The copies of a stage are spread over the k-loop, a few between every four
// MFMAs, instead of issued in one burst per stage: a burst of copies from all
// waves stalls instruction issue while the memory pipeline drains it, and with
// one wave per SIMD nothing else keeps the matrix cores busy meanwhile.
//
// Tile order: workgroups walk the tile grid in groups of two tile rows, in
// dispatch order (the dispatcher deals consecutive workgroups to the 8 XCDs
// round-robin, so each XCD sees a spread of tiles).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ps {

namespace {

constexpr int BM = 256, BN = 256, ROWB = 128, NT = 256;
constexpr int CPR = ROWB / 16;  // 16-byte chunks per LDS row (8)
constexpr int NSTAGE = 2;       // LDS stages of operands
constexpr int U = ROWB / 32;    // MFMA k-units per stage (4)
constexpr int RPI = 64 / CPR;   // rows per copy instruction (8)
constexpr int IPW = (BM / 4) / RPI;   // copy instructions per wave per operand per stage (8)
constexpr int CPG = IPW / 4;    // copies per group of four MFMAs (2)
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
  constexpr int GROUP = 2;
  const int pid = blockIdx.x;
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
  uint32_t voa[IPW], vob[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (wave * IPW + i) * RPI + lane / CPR;
    const int cl = (lane % CPR) ^ lds_swz<CPR>(row);
    voa[i] = (uint32_t)(m0 + row) * a_row + cl * 16;
    vob[i] = (uint32_t)(n0 + row) * b_row + cl * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t wblk = (uint32_t)__builtin_amdgcn_readfirstlane(wave * IPW * 1024);
  // copy instruction c of stage kt: c < IPW are A blocks, the rest B blocks
  auto dma_one = [&](int kt, int c) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + (kt & (NSTAGE - 1)) * (STAGE_CH * 16) + wblk;
    const uint32_t koff = (uint32_t)kt * ROWB;
    if (c < IPW) lds_dma16(rsa, voa[c], koff, dst + c * 1024);
    else lds_dma16(rsb, vob[c - IPW], koff, dst + BM * ROWB + (c - IPW) * 1024);
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
  // One k-unit: 16 MFMAs on fragment set ms in four groups of four.  Each
  // group also reads two fragments of the next k-unit (set fs, LDS buffer
  // fbuf, unit fu: the four B fragments first, as every group of the next
  // unit needs them, then A in order) and issues CPG copy instructions of
  // operand half dh of stage dkt (none when dkt < 0).
  auto unit = [&](int ms, int fs, int fbuf, int fu, bool rd, int dkt, int dh) __attribute__((always_inline)) {
    const u32x4* st = smem + fbuf * STAGE_CH;
    const int ch = (2 * fu + g) ^ fsw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) Mfma<T>::unit(acc[i][j], fr[ms][i], fr[ms][4 + j]);
      if (rd) {
        if (i < 2) {
          fr[fs][4 + 2 * i] = st[(BM + wn * 128 + (2 * i) * 32 + l32) * CPR + ch];
          fr[fs][5 + 2 * i] = st[(BM + wn * 128 + (2 * i + 1) * 32 + l32) * CPR + ch];
        } else {
          fr[fs][2 * (i - 2)] = st[(wm * 128 + (2 * (i - 2)) * 32 + l32) * CPR + ch];
          fr[fs][2 * (i - 2) + 1] = st[(wm * 128 + (2 * (i - 2) + 1) * 32 + l32) * CPR + ch];
        }
      }
      if (dkt >= 0)
#pragma unroll
        for (int c = 0; c < CPG; ++c) dma_one(dkt, dh * IPW + i * CPG + c);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline over stages of 128 bytes of K, two LDS buffers.  The barrier of
  // stage kt sits before its last k-unit: by then every wave holds all of
  // stage kt's fragments in registers, so its buffer is refilled with stage
  // kt + 2 -- the A half of the copies during that last k-unit, the B half
  // during the first k-unit of stage kt + 1 -- while the first fragments of
  // stage kt + 1 are read.  Stage kt + 1 must have landed at the barrier.
  auto stage = [&](int kt, bool copy_b, bool copy_a, bool last) __attribute__((always_inline)) {
    const int buf = kt & 1;
    if (last) {
#pragma unroll
      for (int u = 0; u + 1 < U; ++u) unit(u & 1, (u + 1) & 1, buf, u + 1, true, -1, 0);
      unit((U - 1) & 1, 0, 0, 0, false, -1, 0);
      return;
    }
    unit(0, 1, buf, 1, true, copy_b ? kt + 1 : -1, 1);
#pragma unroll
    for (int u = 1; u + 1 < U; ++u) unit(u & 1, (u + 1) & 1, buf, u + 1, true, -1, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    unit((U - 1) & 1, U & 1, buf ^ 1, 0, true, copy_a ? kt + 2 : -1, 0);
  };

  const int nk = K / BK;
  for (int st = 0; st < NSTAGE && st < nk; ++st)
#pragma unroll
    for (int c = 0; c < 2 * IPW; ++c) dma_one(st, c);
  if (nk > 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // stage 0 landed, stage 1 may fly
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) fr[0][i] = smem[((i < 4 ? wm * 128 + i * 32 : BM + wn * 128 + (i - 4) * 32) + l32) * CPR + (g ^ fsw)];
  int kt = 0;
  if (nk > 1) {
    stage(0, false, nk > 2, false);
    for (kt = 1; kt + 2 < nk; ++kt) stage(kt, true, true, false);   // steady state
    for (; kt + 1 < nk; ++kt) stage(kt, true, false, false);
  }
  stage(kt, false, false, true);
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

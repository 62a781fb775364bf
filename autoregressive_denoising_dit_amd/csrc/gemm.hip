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
// 128 x 128 sub-tile = 4 x 4 MFMA 32x32 accumulators (in AGPRs); or, where it
// fills the CUs' rounds better, 192 x 256 or 128 x 256 tiles of 96 x 128 or
// 64 x 128 per wave (3 x 4 or 2 x 4 accumulators).  The 256 x 256 tile also
// runs as 8 waves in a 2 x 4 grid (128 x 64 each, 4 x 2 accumulators): two
// waves per SIMD, so that one wave's MFMAs cover the other's fragment reads
// and copies, at half the fragment reuse per wave.  Every output element sees
// the same MFMA sequence over K in every layout, so the choice never changes a
// result.  K advances
// in stages of 128 bytes per row (64 bf16 / 32 fp32 = four MFMA k-units)
// through two LDS stages filled by memory-to-LDS copies.  Operand chunks are
// XOR-swizzled so that fragment reads of consecutive rows hit distinct banks.
//
// The copies of a stage are spread over the k-loop, a few between every four
// MFMAs, instead of issued in one burst per stage: a burst of copies from all
// waves stalls instruction issue while the memory pipeline drains it, and with
// one wave per SIMD nothing else keeps the matrix cores busy meanwhile.
//
// Tile order: workgroups walk the tile grid in groups of two tile rows; for
// QKV and with 32 or more tile columns each XCD takes a contiguous range of
// that order, else the dispatch order deals the tiles round-robin over the
// 8 XCDs.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ps {

namespace {

constexpr int BMX = 256, BN = 256, ROWB = 128;   // largest row tile, column tile
constexpr int CPR = ROWB / 16;  // 16-byte chunks per LDS row (8)
constexpr int NSTAGE = 2;       // LDS stages of operands
constexpr int U = ROWB / 32;    // MFMA k-units per stage (4)
constexpr int RPI = 64 / CPR;   // rows per copy instruction (8)
constexpr int EP = 68;          // fp32 row pitch of the epilogue staging (64 columns, 16-byte rows)
constexpr int OPER_BYTES = NSTAGE * (BMX + BN) * CPR * 16;   // 2 x 64 KB

// Tile of 64 MI rows x 256 columns: NW waves, two down and NW / 2 across; a
// wave owns MI x NJ MFMA tiles of 32 x 32.
template <int MI, int NW>
struct Tile {
  static constexpr int NT = 64 * NW;                  // threads
  static constexpr int BM = 64 * MI;                  // rows per tile
  static constexpr int MR = 32 * MI;                  // rows per wave
  static constexpr int WN = NW / 2;                   // waves across
  static constexpr int WC = BN / WN;                  // columns per wave
  static constexpr int NJ = WC / 32;                  // MFMA tiles across per wave
  static constexpr int IPWA = (BM / NW) / RPI;        // A copy instructions per wave per stage
  static constexpr int IPWB = (BN / NW) / RPI;        // B copy instructions per wave per stage
  static constexpr int STAGE_CH = (BM + BN) * CPR;    // 16-byte chunks per stage
  static_assert(IPWA * RPI * NW == BM && IPWB * RPI * NW == BN, "tile must split evenly over the copies");
  static_assert(NW == 4 || (NW == 8 && MI >= 3), "eight waves only with 192- and 256-row tiles");
};
constexpr int STAGE_BYTES = 4 * 128 * EP * 4;          // 4 waves x 128 rows (or 8 x 64) x pitch
constexpr int SMEM_BYTES = OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES;
constexpr int TAB_BYTES = 160 * 1024 - SMEM_BYTES;     // LDS side tables of the epilogues
constexpr int TAB_BIAS = 512, TAB_DATA = TAB_BIAS + BN * 4;   // table offsets (bytes)



// GELU, tanh form: z/2 (1 + tanh(u)) with u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated as z / (1 + e^(-2u)) (the same function: 1 + tanh(u) = 2 / (1 + e^(-2u)))
// with the hardware base-2 exponential and reciprocal; saturates to z or 0
// through inf instead of overflowing.
__device__ __forceinline__ float gelu_tanh(float z) {
  constexpr float c = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float t = __builtin_amdgcn_exp2f(c * z * (1.0f + 0.044715f * z * z));
  return z * __builtin_amdgcn_rcpf(1.0f + t);
}

// ------------------------------------------------------------ epilogues
// After the k-loop each wave stages its 128 x 128 accumulator block in LDS,
// 64 columns at a time (row pitch EP floats), and stores it with lanes that
// own 4 consecutive columns (16 lanes per row, 4 rows per instruction), so
// that every global access is a 16-byte (fp32) or 8-byte (bf16) vector and
// rows are contiguous runs.  Side data that would otherwise be fetched from
// memory during the epilogue -- the tile's bias columns, the pool offset of
// each task's write slot, the RoPE cos/sin tables, the gate rows of the
// modulation -- is copied into LDS before the k-loop.  A global load issued
// after the epilogue's first stores would wait for those stores as well (one
// in-order counter covers both), so the epilogue reads side data from LDS
// only, and the residual epilogue issues each batch of residual loads before
// the previous batch's stores.

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 w = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4*>(p) = w;
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// LDS side tables: bytes [0, 256) the pool offset (elements) of each task's
// write slot, [256, 512) a TabGeo, [512, 1536) the bias of the tile's 256
// columns (zeros past N), [1536, TAB_BYTES) the data -- RoPE tables (float2)
// for the QKV epilogue, gate rows (float) for the residual one.
struct TabGeo {
  int t0;                      // first task (row block) the tile touches
  int off_f, off_y, off_x;     // RoPE tables in float2 units from byte 512
};

// RoPE (cos, sin) of pair dd / 2 of the head dim at token tok of task ti:
// the frame axis first (seg_f dims), then rows (seg_h), then columns (seg_w).
template <typename P>
__device__ __forceinline__ float2 rope_cs(const P& tb, const PoolGeo& pg, int ti, int fl, int yy, int xx,
                                          int dd) {
  if (dd < pg.seg_f) return tb.f[(ti * pg.frames + fl) * (pg.seg_f / 2) + (dd >> 1)];
  if (dd < pg.seg_f + pg.seg_h) return tb.y[yy * (pg.seg_h / 2) + ((dd - pg.seg_f) >> 1)];
  return tb.x[xx * (pg.seg_w / 2) + ((dd - pg.seg_f - pg.seg_h) >> 1)];
}
struct RopePtrs {
  const float2* f;   // indexed from the first task of the tile
  const float2* y;
  const float2* x;
};

// One wave's staged MR x 64 block: rows rbase.., columns cbase.. of C.
template <typename T, int EPI, int MR>
__device__ __forceinline__ void epilogue_block(const float* stg, int rbase, int cbase, int lane, int M, int N,
                                               const EpiArgs& ep, const char* tab, int n0) {
  if (cbase >= N) return;
  const int nrows = min(MR, M - rbase);
  if (nrows <= 0) return;
  const PoolGeo& pg = ep.pool;
  const int rq = lane >> 4, cq = lane & 15;   // row within a step of 4, column quad
  const int col = cbase + 4 * cq;
  const bool col_ok = col < N;                // N is a multiple of 4
  const float* btab = reinterpret_cast<const float*>(tab + TAB_BIAS) - n0;   // indexed by column
  const f32x4 bias = ld4(btab + col);

  if constexpr (EPI == EPI_QKV || EPI == EPI_CTX_KV) {
    const int D = pg.H * pg.d;
    const int part = cbase / D;   // a 64-column block lies inside one of q / k / v
    const bool transposed = (EPI == EPI_QKV) ? part == 2 : part == 1;
    const int64_t* soff = reinterpret_cast<const int64_t*>(tab);
    if (transposed) {
      // values -> V^T [H][d][tokens]: one lane per row (token), 4 columns at a time
      const int stride = (EPI == EPI_QKV) ? pg.L : pg.max_ctx;
      const int ncol = min(64, N - cbase);
      for (int half = 0; half < 2 && half * 64 < nrows; ++half) {
        const int rr = half * 64 + lane;
        const bool row_ok = rr < nrows;
        const int row = rbase + rr;
        T* vt;
        int tok;
        if constexpr (EPI == EPI_QKV) {
          const int ti = row_ok ? (int)pg.div_L.div(row) : 0;
          tok = row - ti * pg.L;
          vt = static_cast<T*>(pg.kv) + soff[ti] + (size_t)pg.H * pg.L * pg.d;
        } else {
          tok = row;
          vt = static_cast<T*>(ep.ctx_base) + (size_t)pg.H * pg.max_ctx * pg.d;
        }
        for (int c0 = 0; c0 < ncol; c0 += 4) {
          const f32x4 v = ld4(stg + min(rr, MR - 1) * EP + c0) + ld4(btab + cbase + c0);
          const int cc = cbase + c0 - part * D;
          const int hh = cc >> ep.d_shift, dd = cc & (pg.d - 1);
          if (row_ok) {
            T* dst = vt + ((size_t)hh * pg.d + dd) * stride + tok;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(size_t)j * stride] = from_f32<T>(v[j]);
          }
        }
      }
      return;
    }
    // q or k (QKV) / k (context): lanes own column quads, rows in steps of 4
    const int cc = col - part * D;
    const int hh = cc >> ep.d_shift, dd = cc & (pg.d - 1);
    if constexpr (EPI == EPI_CTX_KV) {
      T* kb = static_cast<T*>(ep.ctx_base);
      for (int r = rq; r < nrows; r += 4) {
        const f32x4 v = ld4(stg + r * EP + 4 * cq) + bias;
        if (col_ok) store4(kb + ((size_t)hh * pg.max_ctx + rbase + r) * pg.d + dd, v);
      }
      return;
    } else {
      const TabGeo& tg = *reinterpret_cast<const TabGeo*>(tab + 256);
      RopePtrs lt;
      const float2* tb2 = reinterpret_cast<const float2*>(tab + TAB_DATA);
      lt.f = tb2 + tg.off_f;
      lt.y = tb2 + tg.off_y;
      lt.x = tb2 + tg.off_x;
      RopePtrs gt{ep.rope_f + (size_t)tg.t0 * pg.frames * (pg.seg_f / 2), pg.rope_y, pg.rope_x};
      // One loop per table location, so that the tables' pointers keep their
      // address space: a pointer that may be either LDS or global memory is
      // read with a flat load, and the wait for a flat load also waits for
      // every store issued before it -- each row would wait for the previous
      // rows' stores to complete.
      auto rows = [&](const RopePtrs& tb) __attribute__((always_inline)) {
        for (int r = rq; r < nrows; r += 4) {
          const int row = rbase + r;
          const int ti = (int)pg.div_L.div(row);
          const int tok = row - ti * pg.L;
          const int yx = (int)pg.div_cols.div(tok);
          const int fl = (int)pg.div_plane.div(tok);
          const int yy = yx - (int)pg.div_rows.div(yx) * pg.rows;
          const int xx = tok - yx * pg.cols;
          const float2 c0 = rope_cs(tb, pg, ti - tg.t0, fl, yy, xx, dd);
          const float2 c1 = rope_cs(tb, pg, ti - tg.t0, fl, yy, xx, dd + 2);
          const f32x4 v = ld4(stg + r * EP + 4 * cq) + bias;
          // rotate the pairs (dd, dd + 1) and (dd + 2, dd + 3)
          f32x4 o;
          o[0] = v[0] * c0.x - v[1] * c0.y;
          o[1] = v[1] * c0.x + v[0] * c0.y;
          o[2] = v[2] * c1.x - v[3] * c1.y;
          o[3] = v[3] * c1.x + v[2] * c1.y;
          if (!col_ok) continue;
          if (part == 0) {
            store4(static_cast<T*>(ep.out) + (size_t)row * ep.ldo + cc, o * ep.out_scale);
          } else {
            T* kb = static_cast<T*>(pg.kv) + soff[ti];
            store4(kb + ((size_t)hh * pg.L + tok) * pg.d + dd, o);
          }
        }
      };
      if (ep.rope_tab != 0) rows(lt);
      else rows(gt);
      return;
    }
  } else {
    for (int r = rq; r < nrows; r += 4) {
      const f32x4 v = ld4(stg + r * EP + 4 * cq) + bias;
      if (!col_ok) continue;
      if constexpr (EPI == EPI_F32) {
        store4(static_cast<float*>(ep.out) + (size_t)(rbase + r) * ep.ldo + col, v);
        continue;
      }
      f32x4 o;
      if constexpr (EPI == EPI_STORE) {
        o = v * ep.out_scale;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = gelu_tanh(v[j]);
      }
      store4(static_cast<T*>(ep.out) + (size_t)(rbase + r) * ep.ldo + col, o);
    }
  }
}

// Gated residual epilogue of one wave over its whole MR x 128 block:
// h_out = h_in + gate * (acc + bias).  The block goes through the staging
// area in two halves of 64 columns; the residual rows are read in batches of
// 4 * EB rows, each batch loaded before the previous batch is stored, so that
// a load never waits for earlier stores.
template <int EB>
__device__ __forceinline__ void load_res(f32x4 (&h)[EB], const float* h_in, int rbase, int nrows, int r0, int rq,
                                         int col, int N) {
  // lanes past the last column load a valid one (and store nothing): the
  // loads stay unconditional, so the compiler counts them in order instead
  // of waiting for each one where branches join
  const int cc = min(col, N - 4);
#pragma unroll
  for (int k = 0; k < EB; ++k) {
    const int r = min(r0 + 4 * k + rq, nrows - 1);
    h[k] = ld4(h_in + (size_t)(rbase + r) * N + cc);
  }
}

template <int MR, typename StageFn>
__device__ __forceinline__ void epilogue_res(float* stg, StageFn stage_half, int rbase, int cbase, int lane, int M,
                                             int N, const EpiArgs& ep, const char* tab, int n0) {
  constexpr int EB = 8, RB = 4 * EB, NB = MR / RB;   // rows per batch, batches per half
  const int nrows = min(MR, M - rbase);
  if (nrows <= 0 || cbase >= N) return;
  const int rq = lane >> 4, cq = lane & 15;
  const float* btab = reinterpret_cast<const float*>(tab + TAB_BIAS) - n0;
  const float* gtab = reinterpret_cast<const float*>(tab + TAB_DATA);
  const int t0 = reinterpret_cast<const TabGeo*>(tab + 256)->t0;
  // every batch runs (rows past nrows are clamped loads and skipped
  // stores), so that batch n always lives in register set n % 2
  f32x4 hv[2][EB];
  stage_half(0);
  load_res<EB>(hv[0], ep.h_in, rbase, nrows, 0, rq, cbase + 4 * cq, N);
#pragma unroll
  for (int n = 0; n < 2 * NB; ++n) {
    const int hlf = n / NB, b = n % NB;
    if (n == NB) stage_half(1);   // the wave's reads of half 0 are done (LDS accesses complete in order)
    if (n + 1 < 2 * NB) {
      const int nn = n + 1;
      load_res<EB>(hv[nn & 1], ep.h_in, rbase, nrows, (nn % NB) * RB, rq, cbase + (nn / NB) * 64 + 4 * cq, N);
    }
    const int col = cbase + hlf * 64 + 4 * cq;
    if (col >= N) continue;
    const f32x4 bias = ld4(btab + col);
#pragma unroll
    for (int k = 0; k < EB; ++k) {
      const int r = b * RB + 4 * k + rq;
      if (r >= nrows) continue;
      const int row = rbase + r;
      f32x4 gv = {1.0f, 1.0f, 1.0f, 1.0f};
      if (ep.gate_row >= 0) {
        const int tl = (int)ep.div_L.div(row) - t0;
        gv = ld4(gtab + tl * BN + (col - n0));
      }
      const f32x4 v = ld4(stg + r * EP + 4 * cq) + bias;
      *reinterpret_cast<f32x4*>(ep.h_out + (size_t)row * N + col) = hv[n & 1][k] + gv * v;
    }
  }
}

// The same over a wave's MR x 64 block (eight-wave tiles, MR = 96 or 128),
// staged in two halves of 64 rows (the second one partly filled when MR = 96).
template <int MR, typename StageFn>
__device__ __forceinline__ void epilogue_res_rows(float* stg, StageFn stage_half, int rbase, int cbase, int lane,
                                                  int M, int N, const EpiArgs& ep, const char* tab, int n0) {
  constexpr int EB = 8, RB = 4 * EB, NB = 64 / RB;   // rows per batch, batches per half
  const int nrows = min(MR, M - rbase);
  if (nrows <= 0 || cbase >= N) return;
  const int rq = lane >> 4, cq = lane & 15;
  const int col = cbase + 4 * cq;
  const float* btab = reinterpret_cast<const float*>(tab + TAB_BIAS) - n0;
  const float* gtab = reinterpret_cast<const float*>(tab + TAB_DATA);
  const int t0 = reinterpret_cast<const TabGeo*>(tab + 256)->t0;
  f32x4 hv[2][EB];
  stage_half(0);
  load_res<EB>(hv[0], ep.h_in, rbase, nrows, 0, rq, col, N);
  const f32x4 bias = ld4(btab + col);
#pragma unroll
  for (int n = 0; n < 2 * NB; ++n) {
    const int hlf = n / NB;
    if (n == NB) stage_half(1);   // the wave's reads of half 0 are done (LDS accesses complete in order)
    if (n + 1 < 2 * NB) load_res<EB>(hv[(n + 1) & 1], ep.h_in, rbase, nrows, (n + 1) * RB, rq, col, N);
    if (col >= N) continue;
#pragma unroll
    for (int k = 0; k < EB; ++k) {
      const int r = n * RB + 4 * k + rq;
      if (r >= nrows) continue;
      const int row = rbase + r;
      f32x4 gv = {1.0f, 1.0f, 1.0f, 1.0f};
      if (ep.gate_row >= 0) {
        const int tl = (int)ep.div_L.div(row) - t0;
        gv = ld4(gtab + tl * BN + (col - n0));
      }
      const f32x4 v = ld4(stg + (r - hlf * 64) * EP + 4 * cq) + bias;
      *reinterpret_cast<f32x4*>(ep.h_out + (size_t)row * N + col) = hv[n & 1][k] + gv * v;
    }
  }
}

template <typename T, int EPI, int MI, int NW>
__global__ void __launch_bounds__(64 * NW) k_gemm(const T* __restrict__ A, const T* __restrict__ B,
                                                           int M, int N, int K, int lda, EpiArgs ep,
                                                           const DevTask* __restrict__ tasks) {
  using TL = Tile<MI, NW>;
  constexpr int BK = ROWB / sizeof(T);
  constexpr int NT = TL::NT, BM = TL::BM, MR = TL::MR, WN = TL::WN, WC = TL::WC, NJ = TL::NJ;
  constexpr int IPWA = TL::IPWA, IPWB = TL::IPWB, STAGE_CH = TL::STAGE_CH;
  __shared__ u32x4 smem[(SMEM_BYTES + TAB_BYTES) / 16];
  char* tab = reinterpret_cast<char*>(smem) + SMEM_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  constexpr int GROUP = 2;
  // Consecutive workgroups go to the 8 XCDs in turn.  With many tile columns,
  // and always for QKV, each XCD takes a contiguous range of the grouped order
  // instead, so that the tiles its CUs run at one time share few A and B
  // panels in its L2 and the QKV epilogue writes a task's keys and values
  // from the XCD whose L2 the task's attention reads them from; with few tile
  // columns the dispatch order measured faster for the other GEMMs.
  const int total = tiles_m * tiles_n;
  const int full = (total / 8) * 8;
  const int bid = blockIdx.x;
  const int pid = ((tiles_n < 32 && EPI != EPI_QKV) || bid >= full) ? bid : (bid % 8) * (total / 8) + bid / 8;
  const int per_group = GROUP * tiles_n;
  const int first_m = (pid / per_group) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // epilogue side tables (read only after the k-loop's barriers)
  if (tid < BN / 4) {
    const int c = n0 + 4 * tid;
    reinterpret_cast<f32x4*>(tab + TAB_BIAS)[tid] =
        c < N && ep.bias ? ld4(ep.bias + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if constexpr (EPI == EPI_QKV) {
    const PoolGeo& pg = ep.pool;
    const int n_tasks = (int)pg.div_L.div(M - 1) + 1;
    if (tid < n_tasks) {
      const DevTask& tk = tasks[tid];
      reinterpret_cast<int64_t*>(tab)[tid] =
          ((int64_t)tk.region * pg.n_slots + tk.slots[tk.n_seg - 1]) * pg.slot_elems;
    }
    const int t0 = (int)pg.div_L.div(m0);
    const int t1 = (int)pg.div_L.div(min(M, m0 + BM) - 1);
    const int nf = (t1 - t0 + 1) * pg.frames * (pg.seg_f / 2);
    const int ny = pg.rows * (pg.seg_h / 2), nx = pg.cols * (pg.seg_w / 2);
    if (tid == 0) {
      TabGeo* tg = reinterpret_cast<TabGeo*>(tab + 256);
      tg->t0 = t0;
      tg->off_f = 0;
      tg->off_y = nf;
      tg->off_x = nf + ny;
    }
    if (ep.rope_tab) {
      float2* d2 = reinterpret_cast<float2*>(tab + TAB_DATA);
      const float2* f0 = ep.rope_f + (size_t)t0 * pg.frames * (pg.seg_f / 2);
      for (int i = tid; i < nf + ny + nx; i += NT)
        d2[i] = i < nf ? f0[i] : i < nf + ny ? pg.rope_y[i - nf] : pg.rope_x[i - nf - ny];
    }
  } else if constexpr (EPI == EPI_RES) {
    if (ep.gate_row >= 0) {
      const int t0 = (int)ep.div_L.div(m0);
      const int t1 = (int)ep.div_L.div(min(M, m0 + BM) - 1);
      if (tid == 0) reinterpret_cast<TabGeo*>(tab + 256)->t0 = t0;
      float* gt = reinterpret_cast<float*>(tab + TAB_DATA);
      for (int i = tid; i < (t1 - t0 + 1) * (BN / 4); i += NT) {
        const int t = t0 + i / (BN / 4), c4 = (i % (BN / 4)) * 4;
        const f32x4 v = n0 + c4 < N ? ld4(ep.mod + ((size_t)t * 6 + ep.gate_row) * N + n0 + c4)
                                    : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        *reinterpret_cast<f32x4*>(gt + (t - t0) * BN + c4) = v;
      }
    }
  }

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
  uint32_t voa[IPWA], vob[IPWB];
#pragma unroll
  for (int i = 0; i < IPWA; ++i) {
    const int row = (wave * IPWA + i) * RPI + lane / CPR;
    const int cl = (lane % CPR) ^ lds_swz<CPR>(row);
    voa[i] = (uint32_t)(m0 + row) * a_row + cl * 16;
  }
#pragma unroll
  for (int i = 0; i < IPWB; ++i) {
    const int row = (wave * IPWB + i) * RPI + lane / CPR;
    const int cl = (lane % CPR) ^ lds_swz<CPR>(row);
    vob[i] = (uint32_t)(n0 + row) * b_row + cl * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t wblk_a = (uint32_t)__builtin_amdgcn_readfirstlane(wave * IPWA * 1024);
  const uint32_t wblk_b = (uint32_t)__builtin_amdgcn_readfirstlane(BM * ROWB + wave * IPWB * 1024);
  // copy instruction c of stage kt: c < IPWA are A blocks, the rest B blocks
  auto dma_one = [&](int kt, int c) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + (kt & (NSTAGE - 1)) * (STAGE_CH * 16);
    const uint32_t koff = (uint32_t)kt * ROWB;
    if (c < IPWA) lds_dma16_buf(rsa, voa[c], koff, dst + wblk_a + c * 1024);
    else lds_dma16_buf(rsb, vob[c - IPWA], koff, dst + wblk_b + (c - IPWA) * 1024);
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave / WN, wn = wave % WN;
  const int fsw = lds_swz<CPR>(l32);
  u32x4 fr[2][8];   // MFMA fragments of two k-units (A 0..MI-1, B 4..4+NJ-1)
  // One k-unit: MI NJ MFMAs on fragment set ms in MI groups of NJ.  The
  // groups also read the fragments of the next k-unit (set fs, LDS buffer
  // fbuf, unit fu: the B fragments first, as every group of the next unit
  // needs them, then A in order) and issue the copy instructions of operand
  // dh (0 = A, 1 = B) of stage dkt, spread evenly (none when dkt < 0).
  auto unit = [&](int ms, int fs, int fbuf, int fu, bool rd, int dkt, int dh) __attribute__((always_inline)) {
    const u32x4* st = smem + fbuf * STAGE_CH;
    const int ch = (2 * fu + g) ^ fsw;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) Mfma<T>::unit(acc[i][j], fr[ms][i], fr[ms][4 + j]);
      if (rd) {
        if constexpr (NJ == 2) {
          // eight waves: B in group 0, A 0 and 1 in group 1, then one A per group
          if (i == 0) {
            fr[fs][4] = st[(BM + wn * WC + l32) * CPR + ch];
            fr[fs][5] = st[(BM + wn * WC + 32 + l32) * CPR + ch];
          } else if (i == 1) {
            fr[fs][0] = st[(wm * MR + l32) * CPR + ch];
            fr[fs][1] = st[(wm * MR + 32 + l32) * CPR + ch];
          } else {
            fr[fs][i] = st[(wm * MR + i * 32 + l32) * CPR + ch];
          }
        } else if (i < 2) {
          fr[fs][4 + 2 * i] = st[(BM + wn * WC + (2 * i) * 32 + l32) * CPR + ch];
          fr[fs][5 + 2 * i] = st[(BM + wn * WC + (2 * i + 1) * 32 + l32) * CPR + ch];
          // two groups only (128-row tiles): each also reads its A fragment
          if constexpr (MI == 2) fr[fs][i] = st[(wm * MR + i * 32 + l32) * CPR + ch];
        } else if constexpr (MI > 2) {
          // A fragments [a0, a1) of the next unit in group i
          const int a0 = (i - 2) * MI / (MI - 2), a1 = (i - 1) * MI / (MI - 2);
#pragma unroll
          for (int a = a0; a < a1; ++a) fr[fs][a] = st[(wm * MR + a * 32 + l32) * CPR + ch];
        }
      }
      if (dkt >= 0) {
        const int n = dh ? IPWB : IPWA;
        const int c0 = i * n / MI, c1 = (i + 1) * n / MI;
#pragma unroll
        for (int c = c0; c < c1; ++c) dma_one(dkt, dh * IPWA + c);
      }
      if constexpr (NJ == 2) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
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
    for (int c = 0; c < IPWA + IPWB; ++c) dma_one(st, c);
  static_assert(IPWA + IPWB == 7 || IPWA + IPWB == 8 || IPWA + IPWB == 12 || IPWA + IPWB == 14 ||
                    IPWA + IPWB == 16,
                "prologue waits for 7, 8, 12, 14 or 16");
  if (nk > 1) {   // stage 0 landed, stage 1 may fly
    if constexpr (IPWA + IPWB == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (IPWA + IPWB == 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    else if constexpr (IPWA + IPWB == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (IPWA + IPWB == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  }
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < MI || (i >= 4 && i < 4 + NJ))
      fr[0][i] = smem[((i < 4 ? wm * MR + i * 32 : BM + wn * WC + (i - 4) * 32) + l32) * CPR + (g ^ fsw)];
  int kt = 0;
  if (nk > 1) {
    stage(0, false, nk > 2, false);
    for (kt = 1; kt + 2 < nk; ++kt) stage(kt, true, true, false);   // steady state
    for (; kt + 1 < nk; ++kt) stage(kt, true, false, false);
  }
  stage(kt, false, false, true);
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  // each wave stages into and reads back its own region only; LDS accesses
  // of one wave complete in order, so no barrier is needed between halves
  if constexpr (NW == 4) {
    // half h: columns 64 h .. 64 h + 63 of the wave's MR x 128 block
    float* stg = reinterpret_cast<float*>(smem) + wave * (128 * EP);
    auto stage_half = [&](int hlf) __attribute__((always_inline)) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            stg[row * EP + jj * 32 + l32] = acc[i][2 * hlf + jj][r];
          }
    };
    if constexpr (EPI == EPI_RES) {
      epilogue_res<MR>(stg, stage_half, m0 + wm * MR, n0 + wn * WC, lane, M, N, ep, tab, n0);
    } else {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        stage_half(hlf);
        epilogue_block<T, EPI, MR>(stg, m0 + wm * MR, n0 + wn * WC + hlf * 64, lane, M, N, ep, tab, n0);
      }
    }
  } else {
    // half h: rows 64 h .. 64 h + 63 of the wave's MR x 64 block (the second
    // half holds 32 rows when MR = 96)
    float* stg = reinterpret_cast<float*>(smem) + wave * (64 * EP);
    auto stage_half = [&](int hlf) __attribute__((always_inline)) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          if (2 * hlf + ii >= MI) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = ii * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            stg[row * EP + jj * 32 + l32] = acc[2 * hlf + ii][jj][r];
          }
        }
    };
    if constexpr (EPI == EPI_RES) {
      epilogue_res_rows<MR>(stg, stage_half, m0 + wm * MR, n0 + wn * WC, lane, M, N, ep, tab, n0);
    } else {
      stage_half(0);
      epilogue_block<T, EPI, 64>(stg, m0 + wm * MR, n0 + wn * WC, lane, M, N, ep, tab, n0);
      stage_half(1);
      epilogue_block<T, EPI, MR - 64>(stg, m0 + wm * MR + 64, n0 + wn * WC, lane, M, N, ep, tab, n0);
    }
  }
}

}  // namespace

// Compute units of the current device, read once per device.
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] <= 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

template <typename T, int MI, int NW>
static hipError_t launch_gemm_mi(int epi, const T* A, int lda, const T* B, int M, int N, int K, const EpiArgs& ep,
                                 const DevTask* tt, hipStream_t s) {
  constexpr int BM = Tile<MI, NW>::BM;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid(tiles), block(Tile<MI, NW>::NT);
  // LDS side tables of the epilogue: a tile's rows span at most BM / L + 2 tasks
  EpiArgs e = ep;
  if (epi == EPI_QKV || epi == EPI_RES) {
    const int L = epi == EPI_QKV ? ep.pool.L : ep.L;
    if (L < 64) return hipErrorInvalidValue;
    const int span = BM / L + 2;
    if (epi == EPI_RES && span * BN * 4 > TAB_BYTES - TAB_DATA) return hipErrorInvalidValue;
    if (epi == EPI_QKV) {
      const PoolGeo& pg = ep.pool;
      const int64_t pairs = (int64_t)span * pg.frames * (pg.seg_f / 2) + (int64_t)pg.rows * (pg.seg_h / 2) +
                            (int64_t)pg.cols * (pg.seg_w / 2);
      e.rope_tab = pairs * 8 <= TAB_BYTES - TAB_DATA ? 1 : 0;
      if (M / L > 32) return hipErrorInvalidValue;   // one write-slot offset per task
    }
  }
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((k_gemm<T, EPI_QKV, MI, NW>), grid, block, 0, s, A, B, M, N, K, lda, e, tt); break;
    case EPI_CTX_KV: hipLaunchKernelGGL((k_gemm<T, EPI_CTX_KV, MI, NW>), grid, block, 0, s, A, B, M, N, K, lda, e, tt); break;
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<T, EPI_STORE, MI, NW>), grid, block, 0, s, A, B, M, N, K, lda, e, tt); break;
    case EPI_GELU: hipLaunchKernelGGL((k_gemm<T, EPI_GELU, MI, NW>), grid, block, 0, s, A, B, M, N, K, lda, e, tt); break;
    case EPI_RES: hipLaunchKernelGGL((k_gemm<T, EPI_RES, MI, NW>), grid, block, 0, s, A, B, M, N, K, lda, e, tt); break;
    case EPI_F32: hipLaunchKernelGGL((k_gemm<T, EPI_F32, MI, NW>), grid, block, 0, s, A, B, M, N, K, lda, e, tt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm(int epi, const T* A, int lda, const T* B, int M, int N, int K, const EpiArgs& ep,
                       const DevTask* tt, hipStream_t s) {
  // 32-bit buffer offsets: every operand byte (plus one tile of overrun) must be addressable
  const uint64_t lim = 1ull << 32;
  if ((uint64_t)(M + BMX) * lda * sizeof(T) >= lim || (uint64_t)(N + BN) * K * sizeof(T) >= lim ||
      K % (ROWB / (int)sizeof(T)) != 0 || M <= 0 || N <= 0 || N % 4 != 0 || lda < K ||
      (lda * sizeof(T)) % 16 != 0)
    return hipErrorInvalidValue;
  // Row tile: the one with the shorter estimated run, in rounds of tiles
  // over all CUs.  A round of 192-row tiles measured 0.82-0.91 of a round of
  // 256-row ones (fewer rows per copied byte) and is counted as 0.85 (17/20);
  // a round of 128-row tiles measured 0.69 and is counted as 0.7 (14/20).
  // The 128-row tile only wins when few tiles leave CUs idle (small batches).
  // Ties keep the larger tile.
  const int cu = cu_count(), tn = (N + BN - 1) / BN;
  auto rounds = [&](int bm) { return (int64_t)((((M + bm - 1) / bm) * tn + cu - 1) / cu); };
  const int64_t c4 = rounds(Tile<4, 4>::BM) * 20, c3 = rounds(Tile<3, 4>::BM) * 17, c2 = rounds(Tile<2, 4>::BM) * 14;
  if (c2 < c3 && c2 < c4) return launch_gemm_mi<T, 2, 4>(epi, A, lda, B, M, N, K, ep, tt, s);
  // 192- and 256-row tiles in bf16: eight waves up to K = 8192 (measured 2-13%
  // faster on the 1.3B, 5B and 14B shapes there), four beyond (the long-K
  // FFN2 shapes ran 1-2% slower with eight)
  const bool eight = std::is_same<T, bf16>::value && K <= 8192;
  if (c3 < c4) {
    if constexpr (std::is_same<T, bf16>::value)
      if (eight) return launch_gemm_mi<T, 3, 8>(epi, A, lda, B, M, N, K, ep, tt, s);
    return launch_gemm_mi<T, 3, 4>(epi, A, lda, B, M, N, K, ep, tt, s);
  }
  if constexpr (std::is_same<T, bf16>::value)
    if (eight) return launch_gemm_mi<T, 4, 8>(epi, A, lda, B, M, N, K, ep, tt, s);
  return launch_gemm_mi<T, 4, 4>(epi, A, lda, B, M, N, K, ep, tt, s);
}

template hipError_t launch_gemm<bf16>(int, const bf16*, int, const bf16*, int, int, int, const EpiArgs&,
                                      const DevTask*, hipStream_t);
template hipError_t launch_gemm<float>(int, const float*, int, const float*, int, int, int, const EpiArgs&,
                                       const DevTask*, hipStream_t);

int gemm_k_step(int dtype) { return dtype == PS_BF16 ? ROWB / 2 : ROWB / 4; }

}  // namespace ps

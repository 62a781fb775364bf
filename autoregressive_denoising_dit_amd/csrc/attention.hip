// Flash-style attention of a stage task over its noisy-KV window (gfx950).
//
// Self-attention: chunk c at step s attends to the keys/values that chunks
// c - n_read .. c - 1 left at the same (block, step) -- still noisy -- and to
// its own (AREX article on the PhysisServe report, section "难题"; 163.com
// release, section "新一代物理 AI 的基础设施", Fig. 1).  Those entries sit in
// ring slots of the pool, so the key sequence is a list of segments (read
// slots oldest first, then the write slot).  Cross-attention uses the same
// kernel with one segment, the stream's cached conditioning keys/values.
//
// Formulation: the kernel computes S^T = K Q^T and O^T = V^T P^T with MFMA
// 32x32 tiles.  In the accumulator layout a lane then holds one query (its
// column) and several keys, so (i) the softmax row statistics are lane-local
// plus one exchange between the two half-waves, (ii) rescaling O^T by the
// running max touches only the lane's own registers, and (iii) the
// probabilities P^T are already in the B-operand layout of the next MFMA --
// no LDS round trip for P.  V is stored transposed in the pool (V^T [d][L])
// so that P V contracts along contiguous memory.
//
// Work split: one workgroup = (query tile, head, task), one wave per 32
// queries: in bf16 4 waves (128 queries) with a ring of two 64-key tiles, two
// workgroups per CU; in fp32 8 waves (256 queries) with a deeper ring.  Key /
// value tiles are copied from the pool straight into LDS (no register
// staging).  Softmax runs in fp32 with exp2 on logits pre-scaled
// by log2(e)/sqrt(d) (the scale is folded into q by the producing GEMM).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ps {

namespace {

constexpr int KT = 64;
// Lazy rescaling: the running max m used in exp2(s - m) is raised only when a
// tile's logits exceed it by more than this (log2 units), so probabilities stay
// <= 2^8 and the O / l rescale is skipped on most tiles.  O / l is unchanged.
constexpr float kLazy = 8.0f;

__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int full = (total / 8) * 8;
  if (id >= full) return id;
  return (id % 8) * (total / 8) + id / 8;
}

// bf16: LDS row r of a key tile holds key perm16(r): within each group of 16
// rows the middle two quads are swapped, so that the S^T accumulator rows a
// half-wave holds ({4g..4g+3, 8+4g..8+4g+3}) are keys 8g..8g+7 -- exactly the
// 8 contiguous keys of its V^T operand chunk in the P V product.
__device__ __forceinline__ int perm16(int r) {
  const int q = (r >> 2) & 3;
  const int qs = (q == 1) ? 2 : (q == 2) ? 1 : q;
  return (r & ~15) | (qs << 2) | (r & 3);
}

// NT threads (NT / 64 waves of 32 queries each) per workgroup, a ring of RING
// key/value tiles (0: the deepest that fits 128 KB of LDS).
template <typename T, int HD, int NT, int RING>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
k_attn(const T* __restrict__ q, T* __restrict__ out, int ldo, PoolGeo pg, const DevTask* __restrict__ tasks,
       int cross, int n_qt, int n_tasks) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KCH = HD / VEC;     // 16-byte chunks per K row
  constexpr int VCH = KT / VEC;     // 16-byte chunks per V^T row
  constexpr int NU_QK = KCH / 2;    // k-units of the QK contraction
  constexpr int NU_PV = VCH / 2;    // k-units of the PV contraction
  constexpr bool kBf16 = sizeof(T) == 2;
  // LDS ring of NSTG key/value tiles; each tile = K [KT][KCH] then V^T [HD][VCH]
  constexpr int TILE_CH = KT * KCH + HD * VCH;
  constexpr int KB = KT * KCH / 64, VB = HD * VCH / 64;   // 1 KB copy blocks per tile
  constexpr int DPW = (KB + VB) / (NT / 64);              // copies per wave per tile
  constexpr int QT = NT / 2;   // queries per workgroup
  constexpr int NSTG = RING ? RING : TILE_CH * 16 * 4 <= 128 * 1024 ? 4 : 2;
  static_assert((KB + VB) % (NT / 64) == 0, "copy blocks must split evenly over waves");
  __shared__ u32x4 smem[NSTG * TILE_CH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int total = n_qt * pg.H * n_tasks;
  const int pid = xcd_remap(blockIdx.x, total);   // a (task, head)'s query tiles share an XCD
  const int qt = pid % n_qt;
  const int h = (pid / n_qt) % pg.H;
  const int task = pid / (n_qt * pg.H);
  const DevTask& tk = tasks[task];
  const int L = pg.L, D = pg.H * HD;

  // Key segments: self = read slots (oldest first) then the write slot, each
  // L tokens (L >= the 64-key tile, so a tile spans at most two segments);
  // cross = the stream's context entry.  The fetch position (segment, offset)
  // advances tile by tile in scalar registers.
  const int n_seg = cross ? 1 : __builtin_amdgcn_readfirstlane(tk.n_seg);
  const int seg_len = cross ? (1 << 30) : L;
  const int seg_stride = cross ? pg.max_ctx : L;
  const int n_keys = cross ? __builtin_amdgcn_readfirstlane(tk.ctx_len) : n_seg * L;
  // task fields are read once into registers (the copy instructions clobber
  // memory as far as the compiler knows, which would force reloads)
  const T* const region_base = cross ? static_cast<const T*>(pg.ctx) + (size_t)tk.ctx_region * pg.ctx_elems
                                     : static_cast<const T*>(pg.kv) + (size_t)tk.region * pg.n_slots * pg.slot_elems;
  auto seg_base = [&](int i) -> const T* {
    if (cross) return region_base;
    return region_base + (size_t)tk.slots[i] * pg.slot_elems;
  };
  const size_t k_off = (size_t)h * seg_stride * HD;
  const size_t v_off = (size_t)pg.H * seg_stride * HD + (size_t)h * HD * seg_stride;

  // this lane's query and its Q fragments (B operand of S^T = K Q^T); a wave
  // whose 32 queries all lie past the chunk only helps load key tiles
  const bool wave_active = qt * QT + wave * 32 < L;
  const int qi = qt * QT + wave * 32 + l32;
  const int qc = min(qi, L - 1);
  const T* qrow = q + ((size_t)task * L + qc) * D + (size_t)h * HD;

  // Key/value tiles are copied from the pool straight into LDS: each copy
  // instruction moves one 1 KB block (64 lanes x 16 bytes); a lane fetches the
  // chunk that lands swizzled at its position.  Wave w issues blocks
  // w * DPW .. w * DPW + DPW - 1 of the tile's [K blocks | V blocks].
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  int f_seg = 0, f_off = 0;   // segment and offset of the next tile to copy
  // Per-lane byte offsets of this wave's copy blocks inside a tile that lies
  // in one segment (all but the tiles that straddle a segment boundary and
  // the ragged last one): the source of such a tile is a scalar base plus
  // these constants, so a copy costs one 64-bit add instead of the full
  // per-lane index arithmetic.
  uint32_t lane_off[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int bi = wave * DPW + i;
    if (bi < KB) {
      const int row = bi * (64 / KCH) + lane / KCH;
      const int c = (lane % KCH) ^ lds_swz<KCH>(row);
      lane_off[i] = (uint32_t)(((kBf16 ? perm16(row) : row) * HD + c * VEC) * sizeof(T));
    } else {
      const int vb = bi - KB;
      const int f = vb * (64 / VCH) + lane / VCH;
      const int c = (lane % VCH) ^ lds_swz<VCH>(f);
      lane_off[i] = (uint32_t)(((size_t)f * seg_stride + c * VEC) * sizeof(T));
    }
  }
  // this wave's copy blocks: all K or all V^T (KB is a multiple of DPW)
  static_assert(KB % DPW == 0, "a wave's copy blocks must not straddle K and V^T");
  const bool k_wave = wave * DPW < KB;
  const size_t my_off = k_wave ? k_off : v_off;
  const uint32_t my_step = k_wave ? HD * sizeof(T) : sizeof(T);   // bytes per key
  const uint32_t my_dst = (uint32_t)__builtin_amdgcn_readfirstlane(
      k_wave ? wave * DPW * 1024 : KT * KCH * 16 + (wave * DPW - KB) * 1024);
  const T* cur_base = seg_base(0);   // base of segment f_seg
  auto copy_tile = [&](int tile, int stg) {
    const int t0 = tile * KT;
    const T* b0 = cur_base;
    const int split = seg_len - f_off;   // tile-relative key where the next segment starts
    const uint32_t stage = lds0 + (uint32_t)(stg * TILE_CH * 16);
    if (split >= KT && t0 + KT <= n_keys) {
      // a buffer resource over this head's K (or V^T) of the segment; the tile
      // offset goes in the scalar offset, the lane's in the 32-bit vector one.
      // A wave copies K blocks only or V^T blocks only, so the copies of a
      // tile are straight-line code.
      const i32x4 rs = make_rsrc(b0 + my_off, 0xffffffffu);
      const uint32_t so = (uint32_t)f_off * my_step;
      const uint32_t d0 = stage + my_dst;
#pragma unroll
      for (int i = 0; i < DPW; ++i) lds_dma16_buf(rs, lane_off[i], so, d0 + i * 1024);
    } else {
      const T* b1 = seg_base(min(f_seg + 1, n_seg - 1));
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int bi = wave * DPW + i;   // wave-uniform
        const T* src;
        uint32_t dst;
        if (bi < KB) {
          const int row = bi * (64 / KCH) + lane / KCH;
          const int c = (lane % KCH) ^ lds_swz<KCH>(row);
          const int rel = min(kBf16 ? perm16(row) : row, n_keys - 1 - t0);
          const bool nx = rel >= split;
          const int tok = f_off + rel - (nx ? seg_len : 0);
          src = (nx ? b1 : b0) + k_off + (size_t)tok * HD + c * VEC;
          dst = stage + bi * 1024;
        } else {
          const int vb = bi - KB;
          const int f = vb * (64 / VCH) + lane / VCH;
          const int c = (lane % VCH) ^ lds_swz<VCH>(f);
          const int rel = min(c * VEC, n_keys - VEC - t0);
          const bool nx = rel >= split;
          const int tok = f_off + rel - (nx ? seg_len : 0);
          src = (nx ? b1 : b0) + v_off + (size_t)f * seg_stride + tok;
          dst = stage + KT * KCH * 16 + vb * 1024;
        }
        lds_dma16_global(src, (uint32_t)__builtin_amdgcn_readfirstlane(dst));
      }
    }
    f_off += KT;
    if (f_off >= seg_len) {
      f_off -= seg_len;
      ++f_seg;
      cur_base = seg_base(min(f_seg, n_seg - 1));
    }
  };

  f32x16 o[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m_run = 0.0f, l_run = 0.0f;
  f32x16 negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.0f;

  const int n_tiles = (n_keys + KT - 1) / KT;
  for (int t = 0; t < NSTG - 1 && t < n_tiles; ++t) copy_tile(t, t);
  // The Q fragments load while the first tiles' copies are in flight; their
  // wait is taken here together with the first tile's (a wait first inside
  // the tile loop would also wait for the next tile's copies).
  u32x4 qf[NU_QK];
#pragma unroll
  for (int u = 0; u < NU_QK; ++u) qf[u] = *reinterpret_cast<const u32x4*>(qrow + (2 * u + g) * VEC);
  vm_wait_n((min(NSTG - 2, n_tiles - 1)) * DPW);
#pragma unroll
  for (int u = 0; u < NU_QK; ++u) asm volatile("" : "+v"(qf[u]));
  // In bf16 the loop runs NSTG tiles per iteration, one per LDS stage, so
  // that each stage's LDS offset is a constant folded into the fragment
  // reads' offset field instead of an address add per read.
  constexpr int UNR = kBf16 ? NSTG : 1;
  for (int tile0 = 0; tile0 < n_tiles; tile0 += UNR) {
#pragma unroll
  for (int su = 0; su < UNR; ++su) {
    const int tile = tile0 + su;
    if (tile >= n_tiles) break;
    const int st = kBf16 ? su : tile % NSTG;   // LDS stage of this tile
    // tile lands (copies of later tiles may stay in flight); the barrier also
    // tells every wave that all reads of the stage about to be refilled are done
    vm_wait_n((min(tile + NSTG - 2, n_tiles - 1) - tile) * DPW);
    __syncthreads();
    if (tile + NSTG - 1 < n_tiles) copy_tile(tile + NSTG - 1, (st + NSTG - 1) % NSTG);
    const u32x4* ks = smem + st * TILE_CH;
    const u32x4* vs = ks + KT * KCH;

    if (wave_active) {
    // S^T - m for the 64 keys of this tile (the accumulators start at -m)
    f32x16 s[2];
    s[0] = negm;
    s[1] = negm;
#pragma unroll
    for (int u = 0; u < NU_QK; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 kf = ks[(t * 32 + l32) * KCH + ((2 * u + g) ^ lds_swz<KCH>(l32))];
        Mfma<T>::unit(s[t], kf, qf[u]);
      }
    if constexpr (kBf16) {
      // keep KLA key-fragment reads in flight ahead of the MFMAs: the reads
      // first, then one MFMA per read, then the last KLA MFMAs (left to
      // itself the scheduler issues each read right before its MFMA, which
      // then waits the full LDS latency; two ahead measured about 1% faster
      // than four, with fewer registers)
      constexpr int NM = 2 * NU_QK, KLA = 2;
      __builtin_amdgcn_sched_group_barrier(0x100, KLA, 0);
#pragma unroll
      for (int i = 0; i < NM - KLA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KLA, 0);
    }
    if ((tile + 1) * KT > n_keys) {   // ragged last tile
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = t * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          const int key = tile * KT + (kBf16 ? perm16(row) : row);
          if (key >= n_keys) s[t][r] = -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = __builtin_elementwise_maximum(mt, s[t][r]);
    {
      // the other half-wave's keys of the same query: swap the lane halves in
      // registers (v_permlane32_swap) instead of a round trip through LDS,
      // which would also wait for the fragment reads in flight
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mt), __float_as_int(mt), false, false);
      mt = __builtin_elementwise_maximum(__int_as_float(sw[0]), __int_as_float(sw[1]));
    }
    const bool need = (tile == 0) || (mt > kLazy);
    if (__any(need)) {
      const float shift = need ? mt : 0.0f;
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      m_run += shift;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m_run;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] -= shift;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = __builtin_amdgcn_exp2f(s[t][r]);

    // O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < NU_PV; ++u) {
      u32x4 pf;
      if constexpr (kBf16) {
        const int t = u >> 1, r0 = (u & 1) * 8;
        bf16x8 pb;
#pragma unroll
        for (int r = 0; r < 8; ++r) pb[r] = (bf16)s[t][r0 + r];
        pf = __builtin_bit_cast(u32x4, pb);
        // row sum of the probabilities as the MFMA sees them (bf16)
        typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bf16x2 pr = {pb[2 * r], pb[2 * r + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l_run, false);
        }
      } else {
        const int t = u >> 2, r0 = (u & 3) * 4;
        const f32x4 p4 = {s[t][r0], s[t][r0 + 1], s[t][r0 + 2], s[t][r0 + 3]};
        l_run += (p4[0] + p4[1]) + (p4[2] + p4[3]);
        pf = __builtin_bit_cast(u32x4, p4);
      }
#pragma unroll
      for (int i = 0; i < HD / 32; ++i) {
        const int f = i * 32 + l32;
        const u32x4 vf = vs[f * VCH + ((2 * u + g) ^ lds_swz<VCH>(f))];
        Mfma<T>::unit(o[i], vf, pf);
      }
    }
    if constexpr (kBf16) {
      // the same for the value fragments of O^T += V^T P^T
      constexpr int NM = NU_PV * HD / 32, VLA = 2;
      __builtin_amdgcn_sched_group_barrier(0x100, VLA, 0);
#pragma unroll
      for (int i = 0; i < NM - VLA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, VLA, 0);
    }

    }
  }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qi < L) {
    T* orow = out + ((size_t)task * L + qi) * ldo + (size_t)h * HD;
#pragma unroll
    for (int i = 0; i < HD / 32; ++i)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int f = i * 32 + rg * 8 + g * 4;
        if constexpr (kBf16) {
          bf16x4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (bf16)(o[i][rg * 4 + r] * inv);
          *reinterpret_cast<bf16x4*>(orow + f) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = o[i][rg * 4 + r] * inv;
          *reinterpret_cast<f32x4*>(orow + f) = w;
        }
      }
  }
}

}  // namespace

template <typename T, int HD>
hipError_t launch_attention_hd(bool cross, const T* q, T* out, int ldo, const PoolGeo& pg, const DevTask* tt,
                               int n_tasks, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // 4-wave workgroups with a two-tile ring: two of them share a CU, and as
    // they run unsynchronised, one's softmax and start-up (query loads, first
    // tiles) overlap the other's matrix work.  (Measured a little faster than
    // 8-wave workgroups with a four-tile ring, which load each key/value tile
    // once per 256 queries instead of 128.)
    const int n_qt = (pg.L + 127) / 128;
    hipLaunchKernelGGL((k_attn<T, HD, 256, 2>), dim3(n_qt * pg.H * n_tasks), dim3(256), 0, s, q, out, ldo, pg, tt,
                       cross ? 1 : 0, n_qt, n_tasks);
  } else {
    const int n_qt = (pg.L + 255) / 256;
    hipLaunchKernelGGL((k_attn<T, HD, 512, 0>), dim3(n_qt * pg.H * n_tasks), dim3(512), 0, s, q, out, ldo, pg, tt,
                       cross ? 1 : 0, n_qt, n_tasks);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attention(bool cross, const T* q, T* out, int ldo, const PoolGeo& pg, const DevTask* tt,
                            int n_tasks, hipStream_t s) {
  if (pg.d == 128) return launch_attention_hd<T, 128>(cross, q, out, ldo, pg, tt, n_tasks, s);
  if (pg.d == 64) return launch_attention_hd<T, 64>(cross, q, out, ldo, pg, tt, n_tasks, s);
  return hipErrorInvalidValue;
}

template hipError_t launch_attention<bf16>(bool, const bf16*, bf16*, int, const PoolGeo&, const DevTask*,
                                           int, hipStream_t);
template hipError_t launch_attention<float>(bool, const float*, float*, int, const PoolGeo&,
                                            const DevTask*, int, hipStream_t);

}  // namespace ps

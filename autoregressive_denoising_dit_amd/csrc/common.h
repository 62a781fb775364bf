// Internal types shared by the gfx950 kernels and the C-ABI layer of libps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ps.h"

namespace ps {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------------------
// MFMA building block.  A "k-unit" is one 16-byte chunk per lane from each
// operand (lanes 0-31 and 32-63 supply different chunks).  For bf16 that is
// one v_mfma_f32_32x32x16_bf16 (16 k values); for fp32 four
// v_mfma_f32_32x32x2_f32 (8 k values).  A and B use the same k order, so any
// permutation of k inside the unit gives the same product.
//
// Output layout of a 32x32 accumulator (f32x16 per lane): lane l holds column
// l % 32 and rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int kPerUnit = 16;
  __device__ __forceinline__ static void unit(f32x16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int kPerUnit = 8;
  __device__ __forceinline__ static void unit(f32x16& acc, u32x4 a, u32x4 b) {
    // bit-cast whole vectors: a bit-cast of a single vector element would read
    // the vector's first element
    const f32x4 fa = __builtin_bit_cast(f32x4, a);
    const f32x4 fb = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
  }
};

// XOR swizzle of 16-byte chunks in an LDS row holding CH chunks, chosen so
// that MFMA fragment reads -- consecutive rows at one logical chunk -- hit
// distinct banks both when 8 lanes share a 128-byte bank cycle and when 16
// lanes share a 256-byte one.
template <int CH>
__device__ __forceinline__ int lds_swz(int row) {
  if constexpr (CH >= 16) {
    return row & 15;
  } else if constexpr (CH == 8) {
    return (row & 7) ^ ((row >> 3) & 1);
  } else {
    static_assert(CH == 4, "unsupported LDS row width");
    return ((row >> 1) ^ (row >> 3)) & 3;
  }
}

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16 *
// lane (global_load_lds_dwordx4).  Inline assembly so that the compiler does
// not make every later LDS read wait for all copies in flight; callers order
// the copies with vm_wait_n and barriers.
__device__ __forceinline__ void lds_dma16_global(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr), "v"(src) : "memory");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes) with raw (unstrided) addressing;
// reads past the end return zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)bytes, 0x00020000};
}

// 16 bytes per lane from rsrc + voff + soff straight into LDS at lds_addr +
// 16 * lane (buffer_load_dwordx4 ... lds): no per-lane address arithmetic
// beyond the 32-bit lane offset.
__device__ __forceinline__ void lds_dma16_buf(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// s_waitcnt vmcnt(n): at most n memory operations of this wave still in flight.
__device__ __forceinline__ void vm_wait_n(int n) {
  if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

// --------------------------------------------------------------------------
// Stage tasks as the kernels see them (passed by value as a kernel argument).
struct DevTask {
  int32_t region;       // ((stream * n_blocks) + block) * n_steps + step
  int32_t ctx_region;   // stream * n_blocks + block
  int32_t chunk;
  int32_t n_seg;        // n_read + 1 chunks of keys
  int32_t ctx_len;      // conditioning tokens of the stream
  int32_t slots[PS_MAX_WINDOW + 1];  // read slots (oldest first), then the write slot
};

// Host-side image of the batch's task list; it travels to device memory as
// the argument of a one-wave copy kernel (stream-ordered, no host staging).
struct TaskTable {
  DevTask t[PS_MAX_TASKS];
  int32_t n;
};

// Division by a runtime-constant divisor d (n < 2^31):
// q = (umulhi(n, mul) + n) >> shift with shift = ceil(log2 d) and
// mul = floor(2^32 (2^shift - d) / d) + 1.
struct FastDiv {
  uint32_t d = 1, mul = 1, shift = 0;
  FastDiv() = default;
  explicit FastDiv(uint32_t div) : d(div) {
    shift = 0;
    while ((1ull << shift) < div) ++shift;
    mul = (uint32_t)(((1ull << 32) * ((1ull << shift) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const { return (__umulhi(n, mul) + n) >> shift; }
};

// Pool geometry.  Slot layout: K [H][L][d] then V^T [H][d][L].  Context
// layout per (stream, block): K [H][Lc][d] then V^T [H][d][Lc], Lc = max_ctx.
struct PoolGeo {
  void* kv;
  void* ctx;
  int64_t slot_elems;
  int64_t ctx_elems;
  int32_t n_slots, L, H, d, max_ctx;
  int32_t frames, rows, cols;
  int32_t seg_f, seg_h, seg_w;     // RoPE segments of the head dim
  const float2* rope_y;            // [rows][seg_h / 2] (cos, sin)
  const float2* rope_x;            // [cols][seg_w / 2]
  FastDiv div_L, div_plane, div_cols, div_rows;  // L, rows * cols, cols, rows
};

}  // namespace ps

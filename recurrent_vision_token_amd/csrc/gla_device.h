// Device-side building blocks shared by the HIP kernels of the library
// (gfx950): vector types, buffer resources, MFMA wrappers, explicit waits,
// LDS-writing loads and transposed LDS reads of swizzled tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {
namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes from `base`: loads at offsets at or past
// the end return zeros and stores there are dropped.
constexpr int kRawBufferWord3 = 0x00020000;  // untyped buffer, 32-bit elements (gfx9 family)

__device__ __forceinline__ rsrc_t seq_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferWord3);
}

__device__ __forceinline__ f32x4 mma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Row-major chunk tiles in LDS, filled straight from memory by buffer loads
// that write LDS: one wave instruction moves 1 KB, lane l's 16 bytes landing at
// byte 16 l of the block, and a lane whose offset is out of range writes zeros.
// A tile row holds one token's d values (RB = 2d bytes); its 16-byte piece p is
// stored at piece p ^ (row & 7), which spreads row reads and the transposed
// reads below evenly over the LDS banks.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __fp16 lds_h4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): at most n vector-memory operations outstanding, or no LDS
// operation outstanding.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}
constexpr int kLgkmZero = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Waits and barriers are explicit around the LDS-writing loads: the fence in
// __syncthreads would wait for every such load in flight, including the ones
// filling the other buffer.  The empty asm statements keep the compiler from
// moving memory accesses across the wait and the barrier.
template <int WAITCNT>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(WAITCNT);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate: at most n vector-memory operations and no LDS
// operation outstanding.
__host__ __device__ constexpr int vmcnt_lgkm0_imm(int n) {
  return (n & 15) | (7 << 4) | ((n >> 4) << 14);
}

// Wave priority that falls as the workgroup gets through its work (`done`
// of `total` units, both uniform): 3 in the first quarter, then 2, 1, 0.
// The issue arbiter of a SIMD picks the oldest ready wave among those of the
// highest priority, so workgroups of equal work sharing a CU would otherwise
// finish in dispatch order, the last one running alone at the end; falling
// priorities let the ones behind catch up.
__device__ __forceinline__ void prio_by_progress(int done, int total) {
  const int level = (4 * done) / total;
  if (level <= 0)
    __builtin_amdgcn_s_setprio(3);
  else if (level == 1)
    __builtin_amdgcn_s_setprio(2);
  else if (level == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// LDS-writing load of 16 bytes per lane into a 1 KB block of a tile.
__device__ __forceinline__ void dma16(rsrc_t src, f16* block, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)block, 16, off, 0, 0, 0);
}
// The same written as assembly, so that the compiler adds no waits of its
// own for it (it cannot tell the LDS this load fills from the LDS that later
// reads touch, and would wait for the load before them): every wait on these
// loads must be explicit (s_waitcnt vmcnt), and the LDS they fill read only
// after such a wait and a barrier.  The block address goes to m0, which the
// calling kernel must use for nothing else; one wait state separates the m0
// write from the load that reads it.  NT marks the data non-temporal.
template <bool NT>
__device__ __forceinline__ void dma16_asm(rsrc_t src, const f16* block, uint32_t off) {
  const uint32_t lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)const_cast<f16*>(block));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(lds), "v"(off), "s"(src)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(off), "s"(src)
                 : "memory", "m0");
}

// The same with a cache policy: AUX bit 1 marks the data non-temporal (read
// for the last time; the caches need not keep it).
constexpr int kAuxNT = 2;
template <int AUX>
__device__ __forceinline__ void dma16p(rsrc_t src, f16* block, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)block, 16, off, 0, 0, AUX);
}

// Transposed read of the 16 x 16 block at (row0, col0) of a swizzled tile
// (ds_read_b64_tr_b16): lane (i, g) = (lane % 16, lane / 16) receives rows
// row0 + 4g .. row0 + 4g + 3 of column col0 + i, i.e. the MFMA operand that
// reduces over rows.  Lane j of each 16-lane group addresses row 4g + j / 4,
// columns 4 (j % 4) .. + 3 of the block.
template <int RB>
__device__ __forceinline__ f16x4 tr_read(const f16* tile, int row0, int col0) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int row = row0 + 4 * g + (j >> 2);
  const int col = col0 + 4 * (j & 3);
  const f16* a = tile + row * (RB / 2) + (((col >> 3) ^ (row & 7)) << 3) + (col & 4);
  const lds_h4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) lds_h4_t*)(lds_void_t*)a);
  return __builtin_bit_cast(f16x4, x);
}

__device__ __forceinline__ f16x8 cat8(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// element offset of (row, col) in a swizzled tile with RB-byte rows (col % 4 == 0)
template <int RB>
__device__ __forceinline__ int swz(int row, int col) {
  return row * (RB / 2) + (((col >> 3) ^ (row & 7)) << 3) + (col & 7);
}

__device__ __forceinline__ f16x4 ld64(const f16* a) { return *reinterpret_cast<const f16x4*>(a); }
__device__ __forceinline__ f16x8 ld128(const f16* a) { return *reinterpret_cast<const f16x8*>(a); }
__device__ __forceinline__ void st64(f16* a, f16x4 x) { *reinterpret_cast<f16x4*>(a) = x; }
__device__ __forceinline__ f16x4 to_f16(f32x4 x) { return __builtin_convertvector(x, f16x4); }

}  // namespace
}  // namespace gla

// Device helpers shared by the IKBO kernels (gfx950): vector types, bf16
// packing, the HBM -> LDS copy, explicit vmcnt waits, the LDS chunk swizzle and
// XCD-aware workgroup ids.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ikbo {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Per-row XOR applied to the 16-byte chunk index.  Over 16 consecutive rows it
// takes 16 distinct values, and over 4 consecutive rows (aligned) its bits 2-3
// differ, which keeps both the K-operand reads and the transposed V reads
// free of bank conflicts.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

__device__ __forceinline__ u32x2_t pack4_bf16(float a, float b, float c, float d) {
  u32x2_t r;
  r.x = bf16_bits(a) | (bf16_bits(b) << 16);
  r.y = bf16_bits(c) | (bf16_bits(d) << 16);
  return r;
}

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane l's 16
// bytes land at LDS byte address lds_byte + 16*l.  Written as inline assembly so
// that the compiler's wait insertion, which cannot tell ring stages apart and
// would wait for every copy in flight before any LDS read, leaves the ring
// alone; completion is awaited explicitly with wait_vmcnt before a barrier.
// M0 holds the LDS base; nothing else in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_byte) : "memory", "m0");
}
// The same copy from a wave-uniform base held in SGPRs plus a per-lane byte
// offset (the saddr form): the per-tile address then costs no vector
// arithmetic, only the scalar base moves.
__device__ __forceinline__ void copy16_to_lds_s(const void* sbase, uint32_t voff_bytes, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff_bytes), "s"(sbase), "s"(lds_byte)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Logical workgroup id: ids w and w+1 share an XCD when the grid is a multiple of 8.
__device__ __forceinline__ int logical_wg() {
  const int G = gridDim.x, b = blockIdx.x;
  return (G & 7) ? b : (b & 7) * (G >> 3) + (b >> 3);
}

}  // namespace dev
}  // namespace ikbo

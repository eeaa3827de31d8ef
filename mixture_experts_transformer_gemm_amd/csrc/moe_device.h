// Device-side helpers shared by the GEMM translation units (internal).
#pragma once

#include "moe_internal.h"

namespace gmoe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 2 signed bytes (bits sh.. of w) -> 2 bf16 (exact: |q| <= 128 needs at
// most 8 significant bits): each byte converts to fp32, and one byte permute
// takes the upper halves of both (v_perm_b32 selectors 0-3 pick bytes of its
// second operand, 4-7 of its first)
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int sh) {
  const float a = (float)(int)(int8_t)(w >> sh);
  const float b = (float)(int)(int8_t)(w >> (sh + 8));
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// 16 int8 (one 16-byte load) -> two fragments of 8 bf16
__device__ __forceinline__ void i8x16_to_frags(u32x4 q, u32x4& lo, u32x4& hi) {
  lo.x = i8x2_to_bf16x2(q.x, 0);
  lo.y = i8x2_to_bf16x2(q.x, 16);
  lo.z = i8x2_to_bf16x2(q.y, 0);
  lo.w = i8x2_to_bf16x2(q.y, 16);
  hi.x = i8x2_to_bf16x2(q.z, 0);
  hi.y = i8x2_to_bf16x2(q.z, 16);
  hi.z = i8x2_to_bf16x2(q.w, 0);
  hi.w = i8x2_to_bf16x2(q.w, 16);
}

// Reduction offset (within a 64-wide block) of the 8 values lane group g
// supplies to MFMA step s. bf16 weights: step s covers [32s, 32s+32), so one
// load instruction reads 64 contiguous bytes of each of 16 weight rows.
// 8-bit weights: group g owns [16g, 16g+16), one 16-byte load, split in two.
template <bool W8>
__device__ __forceinline__ int koff(int s, int g) {
  return W8 ? 16 * g + 8 * s : 32 * s + 8 * g;
}

// Loads the two weight fragments (steps 0 and 1) of one 64-wide block.
template <bool W8>
__device__ __forceinline__ void load_wfrags(const void* wrow, int kb, int g, u32x4& f0, u32x4& f1) {
  if (W8) {
    const u32x4 q = ld16((const int8_t*)wrow + kb + 16 * g);
    i8x16_to_frags(q, f0, f1);
  } else {
    const bf16_bits* p = (const bf16_bits*)wrow + kb;
    f0 = ld16(p + koff<false>(0, g));
    f1 = ld16(p + koff<false>(1, g));
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Workgroup barrier without the vmcnt(0) a __syncthreads() fence implies (the
// caller waits for exactly the loads it needs). The empty asm statements with
// a memory clobber stop the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds):
// lane i of the wavefront writes lds_base + 16 i (lds_base must be
// wavefront-uniform). POLICY is the instruction's cache-policy field (0
// default, 2 nontemporal). The builtin only exists in the device pass.
template <int POLICY>
__device__ __forceinline__ void dma16_policy(const void* src, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, POLICY);
#endif
}

// slot of 16-byte chunk c of LDS row r for 128-byte rows (conflict-free for
// fragment reads of 16 consecutive rows at one chunk, and of 32 rows at two
// chunks, measured on gfx950)
__device__ __forceinline__ int rslot(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt vmcnt(n), other counters left alone
#define GMOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// s_waitcnt with vmcnt(n) and lgkmcnt(0) (expcnt left at its maximum)
#define GMOE_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14))

}  // namespace gmoe

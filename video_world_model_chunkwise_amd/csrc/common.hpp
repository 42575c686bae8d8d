// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// packing, and the matrix-core (MFMA) instructions with their operand layouts.
//
// Wave64 MFMA layouts used throughout (lane = threadIdx.x % 64):
//   16x16x32 bf16   A: lane holds row (lane % 16), k-slots 8*(lane/16) + 0..7
//                   B: lane holds col (lane % 16), k-slots 8*(lane/16) + 0..7
//                   C: lane holds rows 4*(lane/16) + 0..3 of col (lane % 16)
//   32x32x16 bf16   A: row (lane % 32), k-slots 8*(lane/32) + 0..7
//                   B: col (lane % 32), k-slots 8*(lane/32) + 0..7
//                   C: reg r -> row 8*(r/4) + 4*(lane/32) + r%4, col (lane % 32)
//   32x32x64 fp8    A/B: row/col (lane % 32), 32 bytes = k-slots 32*(lane/32) + 0..31
//                   C: as 32x32x16
// A k-slot is a position in the reduction; any bijection between slots and
// the true reduction index works as long as A and B use the same one.  The
// kernels exploit that: the C registers of two vertically adjacent 16x16
// tiles (rows 4g+r and 16+4g+r) are exactly the operand registers of a
// 16x16x32 product reducing over those 32 rows under the slot map
//   slot 8g + r     <-> k = 4g + r          (r = 0..3)
//   slot 8g + 4 + r <-> k = 16 + 4g + r     (r = 0..3),
// so chained products pass results through registers instead of LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kairos {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Two fp32 -> packed bf16x2 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = bf16x2{(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint2 lo, uint2 hi) {
  uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// 8 fp32 -> bf16x8 operand
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  uint4 u = make_uint4(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5),
                       pack_bf16x2(a6, a7));
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 (OCP E4M3) x fp8 -> fp32, 32x32x64; scale operands 0 select the unscaled form.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// fp4 (OCP E2M1) x fp4 -> fp32, 32x32x64: format 4 for both operands; each
// lane's 32 codes occupy the low four registers of the operand.
__device__ __forceinline__ f32x16 mfma32x32x64_fp4(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would drain the next
// block's prefetch at each barrier; here only LDS operations are completed
// before the barrier and global loads stay in flight (their own uses are
// guarded by the compiler's waits).  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Linear block id -> (xcd-major) id so that consecutive logical ids of one
// group land on one XCD (blocks are dispatched round-robin over 8 XCDs).
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  const int nx = 8;
  if (nblocks % nx != 0) return bid;
  return (bid % nx) * (nblocks / nx) + bid / nx;
}

}  // namespace kairos

// Shared device helpers for the gfx950 kernels (bf16 fragments, wave reductions, timing).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte global load of 8 bf16 values (one dwordx4).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streaming 16-byte load: non-temporal hint for data read exactly once (the KV stream).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] * B[32x16].  Lane l supplies row (l % 16) of A
// and column (l % 16) of B, eight consecutive k values each, k group l / 16; it receives C rows
// 4 (l / 16) .. +3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// v_mfma_f32_16x16x32_f16: the same operand layout as the bf16 form, fp16 elements.
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// Pack two floats into bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane exchange through ds_bpermute (lane ^ mask).
__device__ __forceinline__ float xor_lane(float v, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Workgroup timing record: start/end device realtime clock, HW_ID and XCC_ID registers.
__device__ __forceinline__ uint64_t realtime() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t hw_id() {
  // s_getreg_b32 HW_REG_HW_ID (id 4), offset 0, 32 bits
  return __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
}
__device__ __forceinline__ uint32_t xcc_id() {
  // s_getreg_b32 HW_REG_XCC_ID (id 20), offset 0, 4 bits
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);
}

}  // namespace lbsa

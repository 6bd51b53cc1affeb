// Shared device helpers for the gfx950 MoE kernels (HIP, CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

namespace moe {

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dispatched round-robin

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16 bit pattern, round to nearest even (hardware v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float sigmoidf_acc(float z) { return 1.0f / (1.0f + expf(-z)); }

// Maps a linear workgroup id so that each XCD receives a contiguous range of
// logical tiles (the hardware hands consecutive ids to different XCDs).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  int q = nblocks / kNumXcd, rem = nblocks % kNumXcd;
  int xcd = bid % kNumXcd, slot = bid / kNumXcd;
  return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace moe

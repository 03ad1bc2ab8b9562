// device_common.h -- small gfx950 device helpers shared by the kernels of
// libpagedkv.so (bf16 packing, DPP lane exchange, bf16 dot products).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// v_dot2_f32_bf16: c + a.lo*b.lo + a.hi*b.hi, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 -> packed bf16 pair (lo, hi), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP controls (GFX9 encoding).
enum : int {
  kQuadXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kQuadXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kQuadXor3 = 0x1B,        // quad_perm [3,2,1,0]
  kRowHalfMirror = 0x141,  // lane i <-> 7-i inside each group of 8
  kRowMirror = 0x140,      // lane i <-> 15-i inside each row of 16
  kRowRor8 = 0x128,        // lane i <- lane (i+8) mod 16 inside each row of 16
  kRowRor4 = 0x124,        // rotations of a row of 16 by 4, 2, 1 lanes
  kRowRor2 = 0x122,
  kRowRor1 = 0x121,
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true));
}
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kCtrl, 0xf, 0xf, true);
}

// Wave-uniform read of an int32 array that no kernel of this launch writes
// (block tables, lengths): through the constant address space, so the
// compiler issues a scalar load even where the kernel also stores to global
// memory.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int64_t idx) {
  return ((const_i32_ptr)p)[idx];
}

// Value of x held by lane (lane ^ mask) for any mask < 64 (ds_bpermute).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float shfl(float x, int src_lane) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, x)));
}

}  // namespace pkv

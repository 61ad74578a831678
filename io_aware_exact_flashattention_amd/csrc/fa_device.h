// fa_device.h - device-side helpers shared by the gfx950 attention kernels:
// vector types, MFMA wrappers, 16-bit <-> float conversion and LDS swizzles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type tags. Storage on the device is 16-bit raw bits for both
// half types; the tag selects the MFMA and the conversions.
struct Bf16 {};
struct F16 {};

template <typename T> struct Elem;

template <> struct Elem<Bf16> {
  // D(32x32, f32) += A(32x16) * B(16x32); 8 bf16 per lane per operand.
  __device__ static __forceinline__ f32x16 mma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two floats -> two bf16 (round to nearest even), low half = lo.
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
};

template <> struct Elem<F16> {
  __device__ static __forceinline__ f32x16 mma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Lane value exchange within a wavefront (64 lanes).
__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// The values of lanes i and i^32, both in every lane: v_permlane32_swap
// exchanges the two 32-lane halves inside the vector ALU, with no LDS round
// trip (a ds_bpermute would queue behind the LDS reads of other waves).
// After the swap, lanes below 32 hold (x[i], x[i+32]) and lanes from 32 on
// hold (x[i-32], x[i]).
__device__ __forceinline__ void half_pair(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];  // copy out before the bit cast
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// The values of lanes i and i^16, both in every lane: v_permlane16_swap
// exchanges the odd 16-lane rows of one copy of x with the even rows of the
// other, so every lane ends with its own value and its partner's (in either
// order).
__device__ __forceinline__ void row_pair(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// max / sum of lanes i and i^32 (the same value in both lanes of a pair)
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  half_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  half_pair(x, a, b);
  return a + b;
}

// Byte-select of two 32-bit words (v_perm_b32): result byte i is byte
// sel[i] of the 8-byte value (hi:lo).
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Byte address of a __shared__ object in the LDS aperture.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global -> LDS 16-byte load (global_load_lds_dwordx4): lane i of
// the wave writes LDS bytes [lds_wave_base + 16 i, +16); lds_wave_base is a
// wave-uniform LDS byte address (goes to M0). Written as inline assembly so
// that the compiler's wait-count pass does not treat every later LDS read as
// possibly aliasing it; completion is awaited explicitly with s_waitcnt
// vmcnt by the caller before the LDS bytes are read.
__device__ __forceinline__ void load_to_lds(const void* gsrc, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds_wave_base)
               : "memory", "m0");
}

// The same copy from a wave-uniform base (an SGPR pair) plus a 32-bit
// per-lane byte offset: no 64-bit address arithmetic per lane.
__device__ __forceinline__ void load_to_lds_sv(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_wave_base)
               : "memory", "m0");
}

// The same copy with the non-temporal hint, for bytes that are read once
// (streamed K/V pages): they do not displace cache lines that are reused.
__device__ __forceinline__ void stream_to_lds(const void* gsrc, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gsrc), "s"(lds_wave_base)
               : "memory", "m0");
}

}  // namespace fa

// Device-side helpers for the gfx950 paged-attention kernels: storage-type
// traits (fp16 / bf16 as raw 16-bit words), packed dot products on the
// v_dot2 instructions, DPP reductions inside 8-lane token rows, and fp32 ->
// storage rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Fp16 {};
struct Bf16 {};

template <class DT> struct Storage;

template <> struct Storage<Fp16> {
  // acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2c_f32_f16).
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                  __builtin_bit_cast(f16x2_t, b), acc, false);
  }
  static __device__ __forceinline__ float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
  // Round to nearest even (v_cvt_f16_f32 under the default round mode).
  static __device__ __forceinline__ uint16_t from_float(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
};

template <> struct Storage<Bf16> {
  // acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2c_f32_bf16).
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
  // bf16 is the upper half of a binary32: widening is a shift.
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
  // Round to nearest even on the dropped 16 bits; NaN stays a quiet NaN.
  static __device__ __forceinline__ uint16_t from_float(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  }
};

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // row_mirror: lane i <-> 15-i within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over LANES (8 or 16) consecutive lanes -- one token row -- holding
// slices of one dot product. Butterfly: xor 1 and xor 2 inside quads, the
// half-row mirror pairs quad 0 with quad 1, the row mirror pairs the two
// halves of a 16-lane row. Every lane of the row ends with the full sum.
// All 64 lanes must be active.
template <int LANES>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "row width");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if (LANES == 16) x += dpp<kDppMirror>(x);
  return x;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: K/V rows are streamed once per step, so
// they should not displace anything else from the caches.
__device__ __forceinline__ u32x4_t load_stream16(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa

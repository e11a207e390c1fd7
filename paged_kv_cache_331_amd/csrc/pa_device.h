// Device-side helpers for the gfx950 paged-attention kernels: storage-type
// traits (fp16 / bf16 as raw 16-bit words), cache-element traits (the
// query's 2-byte type, or FP8 E4M3 codes), packed dot products on the v_dot2
// instructions, DPP reductions inside token rows, and fp32 -> storage
// rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Fp16 {};
struct Bf16 {};
struct Fp8 {};   // OCP E4M3 codes (cache element type only)

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
  // Two finite values rounded to nearest even and packed (lo, hi): one
  // v_cvt_pk_f16_f32.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static constexpr uint32_t kOnes = 0x3c003c00u;   // (1, 1)
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
  // Two finite values rounded to nearest even and packed (lo, hi): one
  // v_cvt_pk_bf16_f32.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static constexpr uint32_t kOnes = 0x3f803f80u;   // (1, 1)
};

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // row_mirror: lane i <-> 15-i within 16 lanes
constexpr int kDppRowRor8 = 0x128;    // row_ror:8: lane i <-> i ^ 8 within 16 lanes

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

// gfx950 lane swaps on a pair (a, b) holding one value per lane each:
// lane_swap32 trades lanes 32-63 of a with lanes 0-31 of b, lane_swap16 the
// odd 16-lane rows of a with the even rows of b. Afterwards a lane whose bit
// 5 (resp. 4) is clear holds (its own a, its partner's a) and a lane whose
// bit is set holds (its partner's b, its own b), the partner being lane ^ 32
// (resp. ^ 16). With a == b both lanes see both values.
__device__ __forceinline__ void lane_swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void lane_swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Loads marked non-temporal: K/V rows are streamed once per step, so they
// should not displace anything else from the caches.
__device__ __forceinline__ u32x4_t load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
// 16 bytes through a global-address-space pointer: a load whose address is
// chosen between a buffer and a constant (the zero chunk) stays a global
// load instead of a flat one.
__device__ __forceinline__ u32x4_t load_global16(const void* p) {
  return *(const __attribute__((address_space(1))) u32x4_t*)p;
}
__device__ __forceinline__ u32x2_t load_stream8(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

// Eight 2-byte source values -> eight E4M3 codes (two words, lowest
// dimension in the lowest byte): y = fp32(x) / scale (IEEE division),
// clamped to +-448, rounded to nearest even by v_cvt_pk_fp8_f32; NaN -> 0x7F.
template <class ST>
__device__ __forceinline__ u32x2_t encode_fp8x8(uint4 x, float scale) {
  const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
  u32x2_t out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      y[2 * j] = Storage<ST>::lo(xw[2 * w + j]) / scale;
      y[2 * j + 1] = Storage<ST>::hi(xw[2 * w + j]) / scale;
    }
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = fminf(fmaxf(y[j], -448.f), 448.f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], packed, true);
    uint32_t p = (uint32_t)packed;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (y[j] != y[j]) p = (p & ~(0xffu << (8 * j))) | (0x7fu << (8 * j));
    out[w] = p;
  }
  return out;
}

// The slice of one cached K or V row a lane holds: DL consecutive dimensions.
// QT is the query's type (fp16 / bf16), KT the cache element type.
template <class QT, class KT, int DL> struct Kv;

// Dimensions per lane: 16-byte loads throughout, so 8 dimensions of a 2-byte
// cache and 16 of an FP8 one (8 at head size 64, where 16 would leave a token
// row of 4 lanes and an odd number of rows per tile).
template <class KT, int D> struct LaneDims { static constexpr int value = 8; };
template <> struct LaneDims<Fp8, 128> { static constexpr int value = 16; };

// Cache in the query's 2-byte type: 16 bytes per lane.
template <class QT> struct Kv<QT, QT, 8> {
  typedef uint16_t elem;
  typedef u32x4_t row;
  static __device__ __forceinline__ row load(const elem* p) { return load_stream16(p); }
  // acc + q . k over the 8 dimensions (q as 4 packed pairs of QT).
  static __device__ __forceinline__ float dot(const uint32_t (&q)[4], row k, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = Storage<QT>::dot2(q[e], k[e], acc);
    return acc;
  }
  // The dimensions as packed QT pairs (dimensions 2e, 2e+1 in word e).
  static __device__ __forceinline__ void pairs(row v, uint32_t (&w)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = v[e];
  }
  static __device__ __forceinline__ row zero() { return row{0u, 0u, 0u, 0u}; }
  // The lane's slice of a new token's row in the query's type (src points at
  // its first dimension), as the cache stores it: a copy (scale unused).
  static __device__ __forceinline__ row from_src(const uint16_t* src, float) {
    return *reinterpret_cast<const u32x4_t*>(src);
  }
  static __device__ __forceinline__ void store(elem* dst, row r) {
    *reinterpret_cast<u32x4_t*>(dst) = r;
  }
};

// Two E4M3 codes (the low or high 16 bits of w, lower address first) as a
// pair of QT. Every E4M3 value is exact in fp16 and in bf16, so the unit
// scale leaves the conversion exact.
template <class QT> struct Fp8Pair;
template <> struct Fp8Pair<Fp16> {
  template <bool HIGH> static __device__ __forceinline__ uint32_t get(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
  }
};
template <> struct Fp8Pair<Bf16> {
  template <bool HIGH> static __device__ __forceinline__ uint32_t get(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
  }
};

// FP8 E4M3 cache: DL codes (DL bytes) per lane, W = DL / 4 words. The
// tensor's scale is applied outside (folded into the logit scale for K, into
// the output for V).
template <class QT, int DL> struct Kv<QT, Fp8, DL> {
  static_assert(DL == 8 || DL == 16, "lane width");
  static constexpr int W = DL / 4;
  typedef uint8_t elem;
  typedef uint32_t row __attribute__((ext_vector_type(W)));
  static __device__ __forceinline__ row load(const elem* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const row*>(p));
  }
  static __device__ __forceinline__ float dot(const uint32_t (&q)[DL / 2], row k, float acc) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      acc = Storage<QT>::dot2(q[2 * w], Fp8Pair<QT>::template get<false>(k[w]), acc);
      acc = Storage<QT>::dot2(q[2 * w + 1], Fp8Pair<QT>::template get<true>(k[w]), acc);
    }
    return acc;
  }
  static __device__ __forceinline__ void pairs(row v, uint32_t (&w)[DL / 2]) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      w[2 * i] = Fp8Pair<QT>::template get<false>(v[i]);
      w[2 * i + 1] = Fp8Pair<QT>::template get<true>(v[i]);
    }
  }
  static __device__ __forceinline__ row zero() { return row{}; }
  // The lane's DL dimensions of a new token's row quantized as the FP8 cache
  // write does: e4m3(fp32(x) / scale).
  static __device__ __forceinline__ row from_src(const uint16_t* src, float scale) {
    row r;
#pragma unroll
    for (int c = 0; c < DL / 8; ++c) {
      const u32x2_t w = encode_fp8x8<QT>(*reinterpret_cast<const uint4*>(src + 8 * c), scale);
      r[2 * c] = w[0];
      r[2 * c + 1] = w[1];
    }
    return r;
  }
  static __device__ __forceinline__ void store(elem* dst, row r) {
    *reinterpret_cast<row*>(dst) = r;
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa

// codec.hpp -- register-level decoding of prepacked 2-/4-bit fields on gfx950.
//
// A 16-bit float whose exponent makes its mantissa bit p weigh exactly 1 turns
// a field u written into mantissa bits [p, p+bits) into the exact value
// base + u ("magic number" conversion): one AND-OR per two weights, because
// the prepack puts weight 2j of a dword in the low half-word and weight 2j+1
// at the same offset of the high half-word.  The resulting pair feeds
// v_dot2_f32_{bf16,f16} against an activation pair, so a dot product over a
// block yields sum_k (base_k + u_k) x_k; the block epilogue subtracts
// sum_k (base_k + zero_point) x_k, which depends on the activations only and
// is computed once per row and block (see gemv.hip).
//
// Field positions and bases (bits of each half-word; p = mantissa bit offset):
//   4-bit, bf16 pairs: pair j from (w >> 4j), field at bits 0..3, base 128
//   4-bit, f16 pairs : pair j from (w << 6 >> 4j), field at bits 6..9, base 16
//   2-bit, bf16 pairs: pairs 0-2 from w, 3-5 from w>>6, 6-7 from w>>12, fields
//                      at bits 0-1 / 2-3 / 4-5 -> bases 128 / 32 / 8
//   2-bit, f16 pairs : pairs 0-3 from w<<2, 4-7 from w>>6, fields at bits
//                      2-3 / 4-5 / 6-7 / 8-9 -> bases 256 / 64 / 16 / 4
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qmoe {

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1, so that
// register arrays indexed by i never fall back to scratch memory.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int BITS, bool F16>
struct Codec;

template <>
struct Codec<4, false> {
  static constexpr int kPairs = 4;  // pairs per dword
  static constexpr int kPeriod = 8; // weights per dword
  __host__ __device__ static constexpr float base(int) { return 128.f; }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    constexpr uint32_t M = 0x000F000Fu, C = 0x43004300u;
    p[0] = (w & M) | C;
    p[1] = ((w >> 4) & M) | C;
    p[2] = ((w >> 8) & M) | C;
    p[3] = ((w >> 12) & M) | C;
  }
};

template <>
struct Codec<4, true> {
  static constexpr int kPairs = 4;
  static constexpr int kPeriod = 8;
  __host__ __device__ static constexpr float base(int) { return 16.f; }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    constexpr uint32_t M = 0x03C003C0u, C = 0x4C004C00u;
    p[0] = ((w << 6) & M) | C;
    p[1] = ((w << 2) & M) | C;
    p[2] = ((w >> 2) & M) | C;
    p[3] = ((w >> 6) & M) | C;
  }
};

template <>
struct Codec<2, false> {
  static constexpr int kPairs = 8;
  static constexpr int kPeriod = 16;
  __host__ __device__ static constexpr float base(int j) {
    return (j % 3 == 0) ? 128.f : (j % 3 == 1) ? 32.f : 8.f;
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    constexpr uint32_t M0 = 0x00030003u, C0 = 0x43004300u;  // bits 0-1 -> 128 + u
    constexpr uint32_t M1 = 0x000C000Cu, C1 = 0x42004200u;  // bits 2-3 ->  32 + u
    constexpr uint32_t M2 = 0x00300030u, C2 = 0x41004100u;  // bits 4-5 ->   8 + u
    const uint32_t w6 = w >> 6, w12 = w >> 12;
    p[0] = (w & M0) | C0;
    p[1] = (w & M1) | C1;
    p[2] = (w & M2) | C2;
    p[3] = (w6 & M0) | C0;
    p[4] = (w6 & M1) | C1;
    p[5] = (w6 & M2) | C2;
    p[6] = (w12 & M0) | C0;
    p[7] = (w12 & M1) | C1;
  }
};

template <>
struct Codec<2, true> {
  static constexpr int kPairs = 8;
  static constexpr int kPeriod = 16;
  __host__ __device__ static constexpr float base(int j) {
    return (j % 4 == 0) ? 256.f : (j % 4 == 1) ? 64.f : (j % 4 == 2) ? 16.f : 4.f;
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    constexpr uint32_t M0 = 0x000C000Cu, C0 = 0x5C005C00u;  // bits 2-3 -> 256 + u
    constexpr uint32_t M1 = 0x00300030u, C1 = 0x54005400u;  // bits 4-5 ->  64 + u
    constexpr uint32_t M2 = 0x00C000C0u, C2 = 0x4C004C00u;  // bits 6-7 ->  16 + u
    constexpr uint32_t M3 = 0x03000300u, C3 = 0x44004400u;  // bits 8-9 ->   4 + u
    const uint32_t a = w << 2, b = w >> 6;
    p[0] = (a & M0) | C0;
    p[1] = (a & M1) | C1;
    p[2] = (a & M2) | C2;
    p[3] = (a & M3) | C3;
    p[4] = (b & M0) | C0;
    p[5] = (b & M1) | C1;
    p[6] = (b & M2) | C2;
    p[7] = (b & M3) | C3;
  }
};

// v_dot2_f32_{bf16,f16}: acc + lo(a)*lo(b) + hi(a)*hi(b).
template <bool F16>
__device__ inline float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), acc,
                                  false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
}

__device__ inline float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ inline float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
template <bool F16>
__device__ inline float half_to_f32(uint32_t h) {
  if constexpr (F16) return f16_to_f32(h);
  else return bf16_to_f32(h);
}
__device__ inline float half_to_f32_rt(uint32_t h, int is_f16) {
  return is_f16 ? f16_to_f32(h) : bf16_to_f32(h);
}

// Round to nearest even.  bf16: integer rounding of the float32 pattern.
__device__ inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline uint16_t f32_to_f16_rne(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);  // v_cvt_f16_f32, round-to-nearest-even mode
}
__device__ inline uint16_t f32_to_act(float v, int is_f16) {
  return is_f16 ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
}

}  // namespace qmoe

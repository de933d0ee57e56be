// codec.hpp -- register-level decoding of prepacked 2-/4-bit fields on gfx950.
//
// A 16-bit float whose exponent makes its mantissa bit p weigh exactly 1 turns
// a field u written into mantissa bits [p, p+bits) into the exact value
// base + u ("magic number" conversion): one AND-OR per two weights, because
// the prepack puts weight 2j of a dword in the low half-word and weight 2j+1
// at the same offset of the high half-word.  The resulting pairs are exact
// 16-bit float operands of the matrix cores, so a dot product over a block
// yields sum_k (base_k + u_k) x_k; the block epilogue subtracts
// sum_k (base_k + zero_point) x_k, which depends on the activations only
// (gemv_impl.hpp).
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

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Masks and float constants of a decoder held in registers.  CDNA VOP3
// encodings take no 32-bit literal, so with literal masks the compiler splits
// (x & m) | c into v_and_b32 + v_or_b32; once the constants are opaque
// register values (an empty asm statement that touches only the constant
// itself) it selects one v_and_or_b32 per weight pair, and its own wait
// counting stays in charge of every loaded register.
template <int N>
struct RegConsts {
  uint32_t m[N], c[N];
};
__device__ inline uint32_t opaque_s(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ inline uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int BITS, bool F16>
struct Codec;

// Every decoder: kNC (mask, constant) pairs; extract(w, p, k) decodes one
// dword into kPairs 16-bit float pairs with (x & m) | c per pair, from the
// constants k (literal by default, or opaque registers for the GEMV).
template <typename CD>
struct CodecOps {
  __device__ static inline RegConsts<CD::kNC> literal() {
    RegConsts<CD::kNC> k;
#pragma unroll
    for (int i = 0; i < CD::kNC; ++i) {
      k.m[i] = CD::kM[i];
      k.c[i] = CD::kC[i];
    }
    return k;
  }
  __device__ static inline RegConsts<CD::kNC> in_registers() {
    RegConsts<CD::kNC> k;
#pragma unroll
    for (int i = 0; i < CD::kNC; ++i) {
      k.m[i] = opaque_s(CD::kM[i]);
      k.c[i] = opaque_v(CD::kC[i]);
    }
    return k;
  }
};

template <>
struct Codec<4, false> {
  static constexpr int kPairs = 4;  // pairs per dword
  static constexpr int kPeriod = 8; // weights per dword
  static constexpr int kNC = 1;
  static constexpr uint32_t kM[kNC] = {0x000F000Fu}, kC[kNC] = {0x43004300u};  // bits 0-3 -> 128 + u
  __host__ __device__ static constexpr float base(int) { return 128.f; }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs], const RegConsts<kNC> &k) {
    p[0] = (w & k.m[0]) | k.c[0];
    p[1] = ((w >> 4) & k.m[0]) | k.c[0];
    p[2] = ((w >> 8) & k.m[0]) | k.c[0];
    p[3] = ((w >> 12) & k.m[0]) | k.c[0];
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    extract(w, p, CodecOps<Codec>::literal());
  }
};

template <>
struct Codec<4, true> {
  static constexpr int kPairs = 4;
  static constexpr int kPeriod = 8;
  static constexpr int kNC = 1;
  static constexpr uint32_t kM[kNC] = {0x03C003C0u}, kC[kNC] = {0x4C004C00u};  // bits 6-9 -> 16 + u
  __host__ __device__ static constexpr float base(int) { return 16.f; }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs], const RegConsts<kNC> &k) {
    p[0] = ((w << 6) & k.m[0]) | k.c[0];
    p[1] = ((w << 2) & k.m[0]) | k.c[0];
    p[2] = ((w >> 2) & k.m[0]) | k.c[0];
    p[3] = ((w >> 6) & k.m[0]) | k.c[0];
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    extract(w, p, CodecOps<Codec>::literal());
  }
};

template <>
struct Codec<2, false> {
  static constexpr int kPairs = 8;
  static constexpr int kPeriod = 16;
  static constexpr int kNC = 3;
  // bits 0-1 -> 128 + u, bits 2-3 -> 32 + u, bits 4-5 -> 8 + u
  static constexpr uint32_t kM[kNC] = {0x00030003u, 0x000C000Cu, 0x00300030u};
  static constexpr uint32_t kC[kNC] = {0x43004300u, 0x42004200u, 0x41004100u};
  __host__ __device__ static constexpr float base(int j) {
    return (j % 3 == 0) ? 128.f : (j % 3 == 1) ? 32.f : 8.f;
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs], const RegConsts<kNC> &k) {
    const uint32_t w6 = w >> 6, w12 = w >> 12;
    p[0] = (w & k.m[0]) | k.c[0];
    p[1] = (w & k.m[1]) | k.c[1];
    p[2] = (w & k.m[2]) | k.c[2];
    p[3] = (w6 & k.m[0]) | k.c[0];
    p[4] = (w6 & k.m[1]) | k.c[1];
    p[5] = (w6 & k.m[2]) | k.c[2];
    p[6] = (w12 & k.m[0]) | k.c[0];
    p[7] = (w12 & k.m[1]) | k.c[1];
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    extract(w, p, CodecOps<Codec>::literal());
  }
};

template <>
struct Codec<2, true> {
  static constexpr int kPairs = 8;
  static constexpr int kPeriod = 16;
  static constexpr int kNC = 4;
  // bits 2-3 -> 256 + u, 4-5 -> 64 + u, 6-7 -> 16 + u, 8-9 -> 4 + u
  static constexpr uint32_t kM[kNC] = {0x000C000Cu, 0x00300030u, 0x00C000C0u, 0x03000300u};
  static constexpr uint32_t kC[kNC] = {0x5C005C00u, 0x54005400u, 0x4C004C00u, 0x44004400u};
  __host__ __device__ static constexpr float base(int j) {
    return (j % 4 == 0) ? 256.f : (j % 4 == 1) ? 64.f : (j % 4 == 2) ? 16.f : 4.f;
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs], const RegConsts<kNC> &k) {
    const uint32_t a = w << 2, b = w >> 6;
    p[0] = (a & k.m[0]) | k.c[0];
    p[1] = (a & k.m[1]) | k.c[1];
    p[2] = (a & k.m[2]) | k.c[2];
    p[3] = (a & k.m[3]) | k.c[3];
    p[4] = (b & k.m[0]) | k.c[0];
    p[5] = (b & k.m[1]) | k.c[1];
    p[6] = (b & k.m[2]) | k.c[2];
    p[7] = (b & k.m[3]) | k.c[3];
  }
  __device__ static inline void extract(uint32_t w, uint32_t (&p)[kPairs]) {
    extract(w, p, CodecOps<Codec>::literal());
  }
};

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
// Branch-free variant for loops that must not split on the (wave-uniform)
// scale type: `f16_mask` is all ones for f16, zero for bf16, and should come
// from opaque_v so the compiler cannot turn the bit select back into a branch.
__device__ inline float half_to_f32_sel(uint32_t h, uint32_t f16_mask) {
  const uint32_t f = __float_as_uint(f16_to_f32(h & 0xFFFFu));
  const uint32_t b = h << 16;
  return __uint_as_float((f & f16_mask) | (b & ~f16_mask));
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

// Configurable SwiGLU: with limit > 0 the gate is clipped from above and the
// up value to [-limit, limit]; then g * sigmoid(alpha g) * (u + beta).
__device__ inline float swiglu_cfg(float g, float u, float alpha, float beta, float limit) {
  if (limit > 0.f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  return g / (1.f + expf(-alpha * g)) * (u + beta);
}

}  // namespace qmoe

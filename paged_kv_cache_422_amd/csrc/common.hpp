// Device-side helpers shared by the gfx950 kernels: 16-bit storage types,
// conversions with round-to-nearest-even, and thin wrappers over the CDNA4
// matrix-core (MFMA) instructions the kernels use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage tags.  Both formats are moved as raw uint16_t.
struct F16 {};
struct BF16 {};

template <class T> __device__ __forceinline__ float to_f32(uint16_t x);
template <> __device__ __forceinline__ float to_f32<F16>(uint16_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, x));
}
template <> __device__ __forceinline__ float to_f32<BF16>(uint16_t x) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
}

// fp32 -> 16-bit, round to nearest even (the language's conversion, which
// gfx950 performs with its hardware convert instructions).
template <class T> __device__ __forceinline__ uint16_t from_f32(float x);
template <> __device__ __forceinline__ uint16_t from_f32<F16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <> __device__ __forceinline__ uint16_t from_f32<BF16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// D(16x16, f32) += A(16x32) * B(32x16); each lane supplies 8 values of A
// (row lane%16, k = 8*(lane/16) .. +7) and 8 of B (column lane%16, same k).
// The accumulator holds rows 4*(lane/16) .. +3 of column lane%16.
template <class T> __device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma16x16x32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16x16x32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16, f32) += A(16x16) * B(16x16); each lane supplies 4 values of A
// (row lane%16, k = 4*(lane/16) .. +3) and 4 of B (column lane%16, same k).
template <class T> __device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma16x16x16<F16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16x16x16<BF16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// D(32x32, f32) += A(32x16) * B(16x32); each lane supplies 8 values of A
// (row lane%32, k = 8*(lane/32) .. +7) and 8 of B (column lane%32, same k).
// Accumulator element i of lane l holds row 8*(i/4) + 4*(l/32) + i%4,
// column l%32.
template <class T> __device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma32x32x16<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma32x32x16<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Probabilities go into the matrix cores as 16-bit values.  fp16 keeps 11
// significant bits, enough on its own.  bf16 keeps 8 (relative error up to
// 2^-9 per weight), which is too coarse when only a few keys carry the
// softmax, so a bf16 weight is sent as hi + lo with lo = bf16(p - hi): two
// products, about 16 significant bits.
template <class T> struct SplitP { static constexpr bool kSplit = false; };
template <> struct SplitP<BF16> { static constexpr bool kSplit = true; };

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one 32 lanes away (lane l with l ^ 32) in VALU.
// v_permlane32_swap moves lanes 32..63 of its first operand into lanes
// 0..31 of its second and back, so given the same value twice its two
// results are (low half, low half) and (high half, high half): every lane
// sees both halves, with no LDS round trip (unlike a bpermute).  Both halves
// get the same result (max and + are commutative, bit for bit).
__device__ __forceinline__ void halves32(float x, float& lo, float& hi) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // Elements into scalars first: bit-casting a vector element in place reads
  // element 0 for both.
  const uint32_t r0 = r[0], r1 = r[1];
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_xor32(float x) {
  float lo, hi;
  halves32(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float add_xor32(float x) {
  float lo, hi;
  halves32(x, lo, hi);
  return lo + hi;
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa

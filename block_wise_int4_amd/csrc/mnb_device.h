// Device helpers shared by every kernel of the library: nibble extraction,
// exact (q - zp) pairs, dequantization with one rounding, and conversions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb_layout.h"

namespace mnb {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Nibble position of input t (0..7) inside a device word (k0 k2 k4 k6 k1 k3 k5 k7).
__host__ __device__ __forceinline__ int nibble_pos(int t) { return (t >> 1) + 4 * (t & 1); }

// 4-bit code of input t (0..7) of a device word.
__device__ __forceinline__ uint32_t code_at(uint32_t w, int t) { return (w >> (4 * nibble_pos(t))) & 15u; }

// Canonical word (nibble p = input p) -> device word (nibble order above).
__host__ __device__ __forceinline__ uint32_t to_device_word(uint32_t c) {
    uint32_t d = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) d |= ((c >> (4 * t)) & 15u) << (4 * nibble_pos(t));
    return d;
}

// Device word -> canonical word.
__host__ __device__ __forceinline__ uint32_t to_canonical_word(uint32_t d) {
    uint32_t c = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) c |= ((d >> (4 * nibble_pos(t))) & 15u) << (4 * t);
    return c;
}

// Float16 pair (1024 + q_2h, 1024 + q_2h+1) from device word w, pair h (0..3):
// 0x6400 is 1024.0 in float16, whose unit in the last place is 1, so OR-ing
// a 4-bit integer into the low mantissa bits adds it exactly.
__device__ __forceinline__ uint32_t magic_pair(uint32_t w, int h) {
    return ((w >> (4 * h)) & 0x000F000Fu) | 0x64006400u;
}

// The same offset form of a zero point, in both halves.
__device__ __forceinline__ h2 zp_magic(uint32_t zp) { return as_h2(0x64006400u | zp | (zp << 16)); }

// Exact float16 pair (q - zp) for inputs (2h, 2h+1): both operands lie in
// [1024, 1039], so their difference is an exactly representable integer.
__device__ __forceinline__ h2 centered_pair(uint32_t w, int h, h2 zm) { return as_h2(magic_pair(w, h)) - zm; }

// Dequantized float16 pair: the exact (q - zp) times the scale, one rounding
// (round half to even) in the float16 multiply.
__device__ __forceinline__ h2 dequant_pair_f16(uint32_t w, int h, h2 zm, h2 s2) {
    return centered_pair(w, h, zm) * s2;
}

// Dequantized float32 value: exact integer difference, one float32 multiply.
__device__ __forceinline__ float dequant_f32(uint32_t code, uint32_t zp, float s) {
    return (float)((int)code - (int)zp) * s;
}

// Zero point of entry e of a tile's packed zero-point bytes.
__device__ __forceinline__ uint32_t zp_nibble(const uint8_t *tile_zp, int e) {
    return (tile_zp[e >> 1] >> (4 * (e & 1))) & 15u;
}

// float64 -> float16 bits, round half to even, with subnormals, overflow to
// infinity and NaN kept NaN. Written out on integers so that the result is a
// single rounding of the float64 value.
__host__ __device__ __forceinline__ uint16_t f64_to_f16_bits(double d) {
    const uint64_t b = __builtin_bit_cast(uint64_t, d);
    const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    const int e = (int)((b >> 52) & 0x7FF);
    const uint64_t m = b & ((1ull << 52) - 1);
    if (e == 0x7FF) return sign | (m ? 0x7E00u : 0x7C00u);
    if (e == 0) return sign;                     // float64 subnormal: far below 2^-25
    const int E = e - 1023;                      // value = 1.m * 2^E
    if (E > 15) return sign | 0x7C00u;
    const uint64_t full = m | (1ull << 52);      // 53-bit significand
    const int shift = (E >= -14) ? 42 : 42 + (-14 - E);
    if (shift > 54) return sign;                 // below half the smallest subnormal
    uint64_t q = full >> shift;
    const uint64_t rem = full & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    uint32_t bits;
    if (E >= -14) bits = (uint32_t)((E + 15) << 10) + (uint32_t)q - 1024u;  // carry bumps the exponent
    else bits = (uint32_t)q;                                                 // subnormal (1024 = min normal)
    if (bits >= 0x7C00u) return sign | 0x7C00u;
    return sign | (uint16_t)bits;
}

template <typename T> struct Io;
template <> struct Io<float> {
    static constexpr int kScaleBytes = 4;
    __device__ static float load(const float *p) { return *p; }
    __device__ static float to_f32(float v) { return v; }
    __device__ static float from_f32(float v) { return v; }
    __device__ static float round_f64(double v) { return (float)v; }
};
template <> struct Io<_Float16> {
    static constexpr int kScaleBytes = 2;
    __device__ static float to_f32(_Float16 v) { return (float)v; }
    __device__ static _Float16 from_f32(float v) { return (_Float16)v; }
    __device__ static _Float16 round_f64(double v) { return __builtin_bit_cast(_Float16, f64_to_f16_bits(v)); }
};

}  // namespace mnb

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

// ---------------------------------------------------------------------------
// Pair forms. Inputs 2h and 2h+1 (h = 0..3) of a device word sit at bits 4h
// and 4h + 16, so pairs h = 0 and 2 land in the low nibble of each 16-bit
// half (after a shift by 8 for h = 2) and pairs h = 1 and 3 one nibble
// higher. Each form below takes a pair out with one mask and no per-pair
// shift; the kernels run these helpers and nothing else, and the read-back
// exports (mnb_unpack, mnb_dequant) run them too, so their bit-exact tests
// check the code the products execute.
// ---------------------------------------------------------------------------

// Masks and float16 offsets of the dequant pair form. The MFMA kernel pins
// them in registers (three-operand v_and_or_b32 takes no literal), other
// callers use the literals.
struct PairForm {
    uint32_t mask_lo, mask_hi;    // 0x000F000F, 0x00F000F0
    uint32_t magic_lo, magic_hi;  // 0x6400 = 1024.0 (ulp 1), 0x5400 = 64.0 (ulp 1/16), in both halves
};
__device__ __forceinline__ PairForm pair_form_literal() {
    return PairForm{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
}

// Dequantized float16 pair h of device word w. Pairs h = 0, 2 become
// 1024 + q under the 0x6400 exponent (whose ulp is 1); pairs h = 1, 3,
// masked in place, become 64 + q under 0x5400 (ulp 1/16). Subtracting the
// zero point in the same offset form (1024 + zp or 64 + zp) leaves the
// exact integer q - zp, and the one multiply by the scale rounds once (to
// nearest even): the value (q - zp) * s rounded to float16.
__device__ __forceinline__ h2 dequant_pair_f16(uint32_t w, int h, uint32_t zp, h2 s2, const PairForm &f) {
    const uint32_t word = h >= 2 ? w >> 8 : w;
    h2 x, zm;
    if (h & 1) {
        x = as_h2((word & f.mask_hi) | f.magic_hi);
        zm = as_h2(0x54005400u | (zp << 4) | (zp << 20));
    } else {
        x = as_h2((word & f.mask_lo) | f.magic_lo);
        zm = as_h2(0x64006400u | zp | (zp << 16));
    }
    return (x - zm) * s2;
}

// Decode form of pair h: the two codes left in place under a zero exponent,
// i.e. the exact float16 subnormals q * 2^-24 (h = 0, 2) or q * 2^-20
// (h = 1, 3, one nibble higher). w8 = w >> 8. A dot product of these with
// activations is exact up to its float32 accumulation; multiplying the
// h = 1, 3 sum by 1/16 and then everything by 2^24 restores the codes.
__device__ __forceinline__ uint32_t subnormal_pair(uint32_t w, uint32_t w8, int h) {
    const uint32_t v = h >= 2 ? w8 : w;
    return (h & 1) ? (v & 0x00F000F0u) : (v & 0x000F000Fu);
}
constexpr float kSubnormalUnscale = 16777216.0f;  // 2^24
constexpr float kHighPairScale = 0.0625f;         // 2^-20 -> 2^-24

// Dequantized float32 value: exact integer difference, one float32 multiply.
__device__ __forceinline__ float dequant_f32(uint32_t code, uint32_t zp, float s) {
    return (float)((int)code - (int)zp) * s;
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

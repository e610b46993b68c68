// Embedding-row gather with int8 dequantization: out[t][h] = table[id][h] *
// scale[id] for id = ids[t], rounded once to the output dtype.
//
// One wave per output row; each lane moves 16 table bytes per step, so a
// step is one fully coalesced kilobyte of the row. The product of an int8
// and a float32 needs at most 31 significant bits:
//  - float32 output: the float32 multiply is that single rounding;
//  - float16 output: the float32 product is first rounded to odd (the exact
//    error from an FMA says on which side the exact value lies), and the
//    float16 conversion then rounds to nearest even. With 13 spare bits
//    between the two formats, rounding to odd first gives the correctly
//    rounded float16 (Boldo and Melquiond, "Emulation of FMA and correctly
//    rounded sums: proved algorithms using rounding to odd", 2008).
// Ids outside [0, V) produce rows of zeros.
//
// After the fused LM-head argmax, the gather can take the argmax's
// per-workgroup partial results instead of an id: one workgroup reduces
// them to the index (the finishing launch of the argmax, moved into the
// consumer) and gathers that row.
#include "mnb_decode.h"

namespace mnb {

constexpr int kEmbedWaves = 4;

// float32 product q * s rounded to odd.
__device__ __forceinline__ float mul_round_odd(float q, float s) {
    const float p = q * s;
    if (p == 0.0f || __builtin_isinf(p)) return p;  // (a float16 zero or infinity either way)
    const float e = __builtin_fmaf(q, s, -p);  // q * s - p, exact
    uint32_t u = __builtin_bit_cast(uint32_t, p);
    if (e != 0.0f && (u & 1u) == 0u) u += ((e > 0.0f) == (p > 0.0f)) ? 1u : 0xFFFFFFFFu;
    return __builtin_bit_cast(float, u);
}

// 16 consecutive entries of one row: table bytes raw (zeros for an invalid
// id) times the row's scale s, written to dst[0, 16).
template <typename T>
__device__ __forceinline__ void gather16(u32x4 raw, float s, T *dst) {
    T v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float q = (float)(int8_t)((raw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        if constexpr (sizeof(T) == 4) v[i] = q * s;
        else v[i] = (T)mul_round_odd(q, s);
    }
#pragma unroll
    for (int i = 0; i < (int)(16 * sizeof(T) / 16); ++i)
        reinterpret_cast<u32x4 *>(dst)[i] = reinterpret_cast<const u32x4 *>(v)[i];
}

template <typename T>
__global__ __launch_bounds__(64 * kEmbedWaves) void embed_gather_kernel(const int8_t *__restrict__ table,
                                                                        const float *__restrict__ scales,
                                                                        const int64_t *__restrict__ ids, int64_t rows,
                                                                        int64_t vocab, int64_t h, T *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kEmbedWaves + (threadIdx.x >> 6);
    if (t >= rows) return;
    const int64_t id = ids[t];
    const bool valid = id >= 0 && id < vocab;
    const float s = valid ? scales[id] : 0.0f;
    const int8_t *src = table + (valid ? id : 0) * h;
    T *dst = out + t * h;
    for (int64_t c = (int64_t)lane * 16; c < h; c += 64 * 16) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (valid) raw = *reinterpret_cast<const u32x4 *>(src + c);
        gather16<T>(raw, s, dst + c);
    }
}

// One workgroup: the argmax index from the product's slots, then its row.
static_assert(kGemvThreads == 64 * kEmbedWaves, "the slot reduction runs on the gather's workgroup");
template <typename T>
__global__ __launch_bounds__(kGemvThreads) void embed_gather_argmax_kernel(
    const int8_t *__restrict__ table, const float *__restrict__ scales, const unsigned long long *__restrict__ slots,
    int count, int64_t *__restrict__ index, int64_t vocab, int64_t h, T *__restrict__ out) {
    const int64_t id = argmax_key_index(argmax_reduce_slots(slots, count));
    if (index && threadIdx.x == 0) *index = id;
    const bool valid = id >= 0 && id < vocab;
    const float s = valid ? scales[id] : 0.0f;
    const int8_t *src = table + (valid ? id : 0) * h;
    for (int64_t c = (int64_t)threadIdx.x * 16; c < h; c += kGemvThreads * 16) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (valid) raw = *reinterpret_cast<const u32x4 *>(src + c);
        gather16<T>(raw, s, out + c);
    }
}

hipError_t launch_embed_gather_argmax(const int8_t *table, const float *scales, const void *slots, int64_t count,
                                      int64_t *index, int64_t vocab, int64_t h, int dtype, void *out,
                                      hipStream_t st) {
    const auto *sl = static_cast<const unsigned long long *>(slots);
    if (dtype == kF16)
        embed_gather_argmax_kernel<_Float16><<<1, kGemvThreads, 0, st>>>(table, scales, sl, (int)count, index, vocab,
                                                                          h, static_cast<_Float16 *>(out));
    else
        embed_gather_argmax_kernel<float><<<1, kGemvThreads, 0, st>>>(table, scales, sl, (int)count, index, vocab, h,
                                                                       static_cast<float *>(out));
    return hipGetLastError();
}

hipError_t launch_embed_gather(const int8_t *table, const float *scales, const int64_t *ids, int64_t rows,
                               int64_t vocab, int64_t h, int dtype, void *out, hipStream_t st) {
    const unsigned grid = (unsigned)((rows + kEmbedWaves - 1) / kEmbedWaves);
    if (dtype == kF16)
        embed_gather_kernel<_Float16><<<grid, 64 * kEmbedWaves, 0, st>>>(table, scales, ids, rows, vocab, h,
                                                                         static_cast<_Float16 *>(out));
    else
        embed_gather_kernel<float><<<grid, 64 * kEmbedWaves, 0, st>>>(table, scales, ids, rows, vocab, h,
                                                                      static_cast<float *>(out));
    return hipGetLastError();
}

}  // namespace mnb

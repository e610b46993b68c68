// Pieces shared by the decode-shaped kernels (the float decode kernel and
// the int8-activation decode kernel): the workgroup shape, wave-uniform
// helpers, the weight stream of one row group in load groups of 8 tiles,
// and the host-side LDS opt-in.
#pragma once
#include <atomic>

#include "mnb_internal.h"

namespace mnb {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kTG = 8;  // tiles per load group: one metadata group
static_assert(kMetaGroup == kTG, "a load group is one metadata group");
constexpr int kDecodeOcc = 3;  // decode workgroups per CU (12 waves)

// Buffer resource over [base, base + bytes): loads at or past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;  // buffer-load cache policy: streamed once, not kept

// A value made wave-uniform (kept in a scalar register).
__device__ __forceinline__ int uniform_int(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_readfirstlane(v);
#else
    return v;
#endif
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
#else
    return v;
#endif
}

// Scales of TG consecutive tiles, read with one (float16) or two (float32)
// 16-byte vector loads.
template <typename T, int TG>
struct ScaleVec {
    static constexpr int kWords = TG * (int)sizeof(T) / 4;
    static_assert(kWords % 4 == 0, "whole 16-byte loads");
    uint32_t w[kWords];
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
#pragma unroll
        for (int i = 0; i < kWords / 4; ++i) {
            const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * i, soff, 0));
            w[4 * i + 0] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    }
    __device__ float get(int u) const {
        if constexpr (sizeof(T) == 2) {
            const uint32_t x = w[u >> 1];
            return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> (16 * (u & 1))));
        } else {
            return __builtin_bit_cast(float, w[u]);
        }
    }
};

template <typename T>
struct Group {
    u32x4 codes[kTG];
    ScaleVec<T, kTG> s;
    uint32_t z;
};

// Loads tiles [c0, c0 + kTG) of row group g: its scales and zero points
// first (tile 0 needs them), then the codes in tile order, all
// unconditionally, so that the compiler waits for exactly the loads a tile
// uses. Codes of tiles past kg read zero (they lie past the row group's
// buffer range), and their metadata is the layout's zero padding.
// With valid false every load has an empty range: nothing is read and the
// group holds zeros (so that the loads need no branch around them).
template <typename T>
__device__ __forceinline__ void load_group(const Problem &p, int64_t g_, int64_t c0_, bool valid, uint32_t lane_code_off,
                                           uint32_t e, Group<T> &G) {
    // (every value below is the same in all lanes; read from the problem
    // descriptor they may sit in vector registers, and a buffer resource must
    // be scalar, so they are made wave-uniform explicitly)
    const int64_t g = uniform_i64(g_), c0 = uniform_i64(c0_), kg = uniform_i64(p.kg);
    const uint8_t *packed = reinterpret_cast<const uint8_t *>(uniform_i64(reinterpret_cast<int64_t>(p.packed)));
    // the metadata block of (row group g, tile group c0 / 8): entry e's scales
    // of the 8 tiles at e * 8 elements, its zero points at e * 4 bytes
    const int64_t entries = uniform_i64(p.nbt) * kTileRows;
    const int64_t blk = (g * (uniform_i64(p.kgp) / kMetaGroup) + c0 / kMetaGroup) * entries;
    const __amdgpu_buffer_rsrc_t ms =
        buffer_over(packed + uniform_i64(p.scales_off) + blk * kMetaGroup * (int64_t)sizeof(T),
                    valid ? (uint32_t)(entries * kMetaGroup * (int64_t)sizeof(T)) : 0u);
    const __amdgpu_buffer_rsrc_t mz = buffer_over(packed + uniform_i64(p.zp_off) + blk * (kMetaGroup / 2),
                                                  valid ? (uint32_t)(entries * (kMetaGroup / 2)) : 0u);
    G.s.load(ms, e * kMetaGroup * (uint32_t)sizeof(T), 0);
    G.z = __builtin_amdgcn_raw_buffer_load_b32(mz, e * (kMetaGroup / 2), 0, 0);
    const __amdgpu_buffer_rsrc_t codes =
        buffer_over(packed + g * kg * kTileCodeBytes, valid ? (uint32_t)(kg * kTileCodeBytes) : 0u);
#pragma unroll
    for (int u = 0; u < kTG; ++u)
        G.codes[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   codes, lane_code_off, (uint32_t)((c0 + u) * kTileCodeBytes),
                                                   kNonTemporal));
}

// Inputs the decode kernel stages: K padded to whole load groups.
__host__ __device__ __forceinline__ int64_t decode_staged_k(int64_t kg) { return (kg + kTG - 1) / kTG * kTG * kTileK; }

constexpr int kGemvMaxLds = 160 * 1024;     // LDS of one CU
constexpr int kDefaultLds = 64 * 1024;      // above this a launch must opt in

// Relative streaming rates of the persistent decode workgroups, and the
// split of a launch's work by them. Workgroups are dispatched one per CU in
// block order (workgroup w is in slot w / 256 of its CU) and round-robin over
// the XCDs (w % 8). Timestamps of every workgroup of the decode steps gave
// the same rates on the 0.6B and the 1.7B step: a CU's first workgroup
// streams fastest, its second at about 0.9 and its third at 0.75 of that
// rate (the CU issues older waves first), and workgroups on the odd XCDs at
// 0.935 of the even ones' (measured with equal work per workgroup, then
// corrected once from the end times the weighted split gave).
// decode_rate_prefix(v, wgs): the summed rates of workgroups [0, v).
__host__ __device__ inline double decode_rate_prefix(int64_t v, int64_t wgs) {
    const double kSlot[3] = {1.0, 0.895, 0.75};
    const double kOdd = 0.935;
    const double per8 = 4.0 + 4.0 * kOdd;  // eight consecutive workgroups
    const bool slots = wgs > 256;          // more than one workgroup per CU
    const int64_t s = v / 256, j = v % 256, r = j % 8;
    double sum = 0.0;
    for (int64_t k = 0; k < s; ++k) sum += (slots ? kSlot[k < 2 ? k : 2] : 1.0) * 32.0 * per8;
    const double rs = slots ? kSlot[s < 2 ? s : 2] : 1.0;
    return sum + rs * ((double)(j / 8) * per8 + (double)((r + 1) / 2) + (double)(r / 2) * kOdd);
}

// First batch of workgroup w when `nbat` batches of one product are split
// over `wgs` workgroups: by rate when there are at least four batches per
// workgroup, evenly otherwise (where rounding to whole batches would cost
// more than the rates gain).
__host__ __device__ inline int64_t decode_split(int64_t nbat, int64_t w, int64_t wgs) {
    if (nbat < 4 * wgs) return nbat * w / wgs;
    if (w >= wgs) return nbat;
    return (int64_t)((double)nbat * decode_rate_prefix(w, wgs) / decode_rate_prefix(wgs, wgs));
}

// The fused LM-head argmax leaves one 64-bit key per workgroup of its
// launch (the best of the outputs that workgroup produced; larger key =
// larger value, equal values = lower index). argmax_reduce_slots: the
// largest of slots[0, count), computed by all kGemvThreads threads of a
// workgroup together and returned to every thread. The slot array holds
// kGemvMaxWgs slots, so all of them are loaded at once and those past
// `count` (left from earlier calls) are dropped afterwards.
__device__ __forceinline__ unsigned long long argmax_reduce_slots(const unsigned long long *slots, int count) {
    __shared__ unsigned long long wave_best[kGemvWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int kPer = (kGemvMaxWgs + kGemvThreads - 1) / kGemvThreads;
    static_assert(kPer * kGemvThreads == kGemvMaxWgs, "whole passes over the slots");
    unsigned long long v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = slots[threadIdx.x + i * kGemvThreads];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if ((int)threadIdx.x + i * kGemvThreads >= count) v[i] = 0ull;
    unsigned long long b = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) b = v[i] > b ? v[i] : b;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(b, off);
        b = o > b ? o : b;
    }
    if (lane == 0) wave_best[wave] = b;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) b = wave_best[w] > b ? wave_best[w] : b;
    return b;
}

// The output index a key names (-1 for the empty key).
__device__ __forceinline__ int64_t argmax_key_index(unsigned long long key) {
    return key == 0 ? -1 : (int64_t)(0xFFFFFFFFu - (uint32_t)key);
}

// Kernels whose dynamic LDS may exceed the default must opt in. Each kernel's
// limit is raised once per device, to the largest size any call can ask
// for, and never lowered, so concurrent callers cannot undo each other's
// setting and later calls skip the runtime call.
template <auto Kernel>
static hipError_t allow_lds(size_t lds) {
    if (lds <= (size_t)kDefaultLds) return hipSuccess;
    static std::atomic<uint64_t> raised{0};  // bit d: raised on device d (devices 0..63)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
    if (bit && (raised.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kGemvMaxLds);
    if (e == hipSuccess && bit) raised.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace mnb

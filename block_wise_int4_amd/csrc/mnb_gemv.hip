// Decode-step kernel (M = 1) and the float32 vector kernel (M >= 2).
//
// One wave owns one 16-row group of the weight and walks its 128-input
// tiles: per tile each lane issues one fully coalesced 128-bit load (its row
// r = lane & 15, chunk j = lane >> 4), one scale load and one zero-point
// byte, turns the 32 codes into exact float16 (q - zp) pairs with the
// 1024-offset trick, and folds them into a float32 dot product with the
// activation slice it reads from LDS. The block scale multiplies the chunk's
// partial sum once. After the last tile the four chunk lanes of each row are
// summed with two cross-lane exchanges and lanes 0..15 store the 16 outputs.
//
// The activation vector is staged in LDS once per workgroup (zero-filled past
// K), so every wave of the workgroup reads it from there.
#include "mnb_internal.h"

namespace mnb {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGemvUnroll = 4;  // tiles whose loads are issued together

struct GemvTileData {
    u32x4 codes;
    uint32_t zb;   // zero-point byte
    float s;
};

template <typename T>
__device__ __forceinline__ void gemv_load_tile(const Problem &p, int64_t g, int64_t c, int lane, int e,
                                               GemvTileData &d) {
    const int64_t tile = g * p.kg + c;
    d.codes = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4 *>(p.packed + tile * kTileCodeBytes) + lane);
    const T *sc = reinterpret_cast<const T *>(p.packed + p.scales_off) + tile * p.nbt * kTileRows + e;
    d.s = (float)*sc;
    d.zb = p.packed[p.zp_off + tile * (p.nbt * kTileRows / 2) + (e >> 1)];
}

template <typename T, int MR>
__device__ __forceinline__ void gemv_tile_math(const GemvTileData &d, int e, const T *xs, int64_t kp, int64_t c,
                                               int j, float (&acc)[MR]) {
    const uint32_t z = (d.zb >> (4 * (e & 1))) & 15u;
    const uint32_t w[4] = {d.codes.x, d.codes.y, d.codes.z, d.codes.w};
    if constexpr (sizeof(T) == 2) {
        const h2 zm = zp_magic(z);
        h2 cp[16];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int h = 0; h < 4; ++h) cp[4 * t + h] = centered_pair(w[t], h, zm);
#pragma unroll
        for (int row = 0; row < MR; ++row) {
            const uint4 *xv = reinterpret_cast<const uint4 *>(xs + row * kp + c * kTileK + j * kChunk);
            float part = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 xx = xv[t];
                const uint32_t xw[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) part = __builtin_amdgcn_fdot2(cp[4 * t + h], as_h2(xw[h]), part, false);
            }
            acc[row] = __builtin_fmaf(d.s, part, acc[row]);
        }
    } else {
        float dv[32];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 8; ++u) dv[8 * t + u] = (float)((int)code_at(w[t], u) - (int)z);
#pragma unroll
        for (int row = 0; row < MR; ++row) {
            const float4 *xv = reinterpret_cast<const float4 *>(xs + row * kp + c * kTileK + j * kChunk);
            float part = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 xx = xv[q];
                part = __builtin_fmaf(dv[4 * q + 0], xx.x, part);
                part = __builtin_fmaf(dv[4 * q + 1], xx.y, part);
                part = __builtin_fmaf(dv[4 * q + 2], xx.z, part);
                part = __builtin_fmaf(dv[4 * q + 3], xx.w, part);
            }
            acc[row] = __builtin_fmaf(d.s, part, acc[row]);
        }
    }
}

// One workgroup: row groups [4 * wq, 4 * wq + 4) of the weight, activation
// rows [m0, m0 + MR).
template <typename T, int MR>
__device__ __forceinline__ void gemv_workgroup(const Problem &p, int64_t wg, T *xs) {
    const int64_t mchunks = (p.m + MR - 1) / MR;
    const int64_t wq = wg / mchunks;
    const int64_t m0 = (wg % mchunks) * MR;
    const int64_t kp = p.kg * kTileK;
    const T *x = static_cast<const T *>(p.x);

    // Stage X[m0 .. m0 + MR) into LDS in 16-byte pieces, zero past K and M.
    constexpr int kPer = 16 / sizeof(T);
    const int64_t pieces = MR * kp / kPer;
    for (int64_t i = threadIdx.x; i < pieces; i += kGemvThreads) {
        const int64_t row = i / (kp / kPer);
        const int64_t k = (i % (kp / kPer)) * kPer;
        uint4 v = {0u, 0u, 0u, 0u};
        if (m0 + row < p.m && k < p.k) v = *reinterpret_cast<const uint4 *>(x + (m0 + row) * p.k + k);
        *reinterpret_cast<uint4 *>(xs + row * kp + k) = v;
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, j = lane >> 4;
    const int64_t g = wq * kGemvWaves + wave;
    if (g >= p.rg) return;
    const int e = (j / (p.bs / kChunk)) * kTileRows + r;

    float acc[MR];
#pragma unroll
    for (int row = 0; row < MR; ++row) acc[row] = 0.0f;

    int64_t c = 0;
    for (; c + kGemvUnroll <= p.kg; c += kGemvUnroll) {
        GemvTileData d[kGemvUnroll];
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u) gemv_load_tile<T>(p, g, c + u, lane, e, d[u]);
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u) gemv_tile_math<T, MR>(d[u], e, xs, kp, c + u, j, acc);
    }
    for (; c < p.kg; ++c) {
        GemvTileData d;
        gemv_load_tile<T>(p, g, c, lane, e, d);
        gemv_tile_math<T, MR>(d, e, xs, kp, c, j, acc);
    }

#pragma unroll
    for (int row = 0; row < MR; ++row) {
        float v = acc[row];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[row] = v;
    }
    const int64_t n = g * kTileRows + r;
    if (j == 0 && n < p.n) {
        T *y = static_cast<T *>(p.y);
#pragma unroll
        for (int row = 0; row < MR; ++row)
            if (m0 + row < p.m) y[(m0 + row) * p.n + n] = (T)acc[row];
    }
}

template <typename T, int MR>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(Problem p) {
    extern __shared__ __align__(16) uint8_t smem[];
    gemv_workgroup<T, MR>(p, blockIdx.x, reinterpret_cast<T *>(smem));
}

// Index of the problem owning workgroup `wg`: the last entry whose wg_begin
// is <= wg (entries are sorted by wg_begin).
__device__ __forceinline__ int find_problem(const Problem *entries, int count, int64_t wg) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (entries[mid].wg_begin <= wg) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <typename T, int MR>
__global__ __launch_bounds__(kGemvThreads) void gemv_grouped_kernel(const Problem *entries, int count) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int i = find_problem(entries, count, blockIdx.x);
    const Problem p = entries[i];
    gemv_workgroup<T, MR>(p, (int64_t)blockIdx.x - p.wg_begin, reinterpret_cast<T *>(smem));
}

// Variants: 0 = fp16 x1, 1 = fp32 x1, 2 = fp32 x4 activation rows per pass.
constexpr int kGemvMaxLds = 65536;

int gemv_variant(int dtype, int64_t m) {
    if (dtype == kF16) return 0;
    return m >= 2 ? 2 : 1;
}

static int gemv_rows(int variant) { return variant == 2 ? 4 : 1; }
static int gemv_elem(int variant) { return variant == 0 ? 2 : 4; }

static size_t gemv_lds(const Problem &p, int variant) {
    return (size_t)gemv_rows(variant) * (size_t)(p.kg * kTileK) * gemv_elem(variant);
}

int64_t gemv_workgroups(const Problem &p, int variant) {
    const int mr = gemv_rows(variant);
    return ((p.rg + kGemvWaves - 1) / kGemvWaves) * ((p.m + mr - 1) / mr);
}

// Largest K (padded) the LDS staging allows for a variant.
int64_t gemv_max_kpad(int variant) { return kGemvMaxLds / (gemv_rows(variant) * gemv_elem(variant)); }

hipError_t launch_gemv(const Problem &p, int dtype, int variant, hipStream_t st) {
    (void)dtype;
    const unsigned grid = (unsigned)gemv_workgroups(p, variant);
    const size_t lds = gemv_lds(p, variant);
    switch (variant) {
    case 0: gemv_kernel<_Float16, 1><<<grid, kGemvThreads, lds, st>>>(p); break;
    case 1: gemv_kernel<float, 1><<<grid, kGemvThreads, lds, st>>>(p); break;
    default: gemv_kernel<float, 4><<<grid, kGemvThreads, lds, st>>>(p); break;
    }
    return hipGetLastError();
}

size_t gemv_lds_bytes(const Problem &p, int variant) { return gemv_lds(p, variant); }

hipError_t launch_gemv_grouped(const Problem *dev_entries, int count, int64_t wgs, int variant, size_t lds,
                               hipStream_t st) {
    switch (variant) {
    case 0: gemv_grouped_kernel<_Float16, 1><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, count); break;
    case 1: gemv_grouped_kernel<float, 1><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, count); break;
    default: gemv_grouped_kernel<float, 4><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, count); break;
    }
    return hipGetLastError();
}

}  // namespace mnb

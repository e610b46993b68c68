// Int8 compute mode (the exports' accuracy level 4): activations are
// quantized per (row, block of block_size inputs) to symmetric int8, and the
// products run as integer dot products of the 4-bit codes with those int8
// values, each block's integer sum scaled by the weight scale times the
// activation scale.
//
// Two kernels per product:
//  1. quantize_act_kernel: a_s = amax / 127 and qa = clamp(rint(x / a_s),
//     -127, 127) per block, both in float32 (IEEE division, round to nearest
//     even), written to the caller's workspace together with the integer sum
//     of every 32-input chunk of qa (the zero-point term). In the workspace
//     the 8 codes of each 8 inputs x0..x7 are stored as x0 x4 x1 x5 x2 x6 x3
//     x7, the byte order in which one mask of a device code word yields the
//     matching weight codes (below).
//  2. i8_rows_kernel: one wave per 16-row group of the weight and MR
//     activation rows per pass; per 128-input tile a lane (row r, chunk j)
//     expands its 32 codes to bytes with two masks per word, w & 0x0F0F0F0F
//     -> codes k0 k4 k1 k5 and (w >> 4) & 0x0F0F0F0F -> k2 k6 k3 k7 (the
//     device word holds k0 k2 k4 k6 k1 k3 k5 k7), and runs 8 v_dot4_i32_i8
//     per activation row. The zero point enters once per chunk as
//     zp * sum(qa); the chunk's integer sum, times s * a_s, is accumulated in
//     float32. The four chunk lanes of a row are summed with two cross-lane
//     exchanges.
#include "mnb_internal.h"

namespace mnb {

constexpr int kA8Max = 127;

// Byte position, inside the stored 8 codes of inputs 8t..8t+7, of input u.
__host__ __device__ __forceinline__ int a8_slot(int u) { return ((u & 3) << 1) | (u >> 2); }

template <typename T, bool kDeviceOrder>
__global__ __launch_bounds__(256) void quantize_act_kernel(const T *__restrict__ x, int64_t m_rows, int64_t k, int bs,
                                                           int8_t *__restrict__ qa, float *__restrict__ scales,
                                                           int32_t *__restrict__ chunk_sums) {
    // thread = 8 consecutive inputs; the bs / 8 threads of a block are
    // consecutive lanes of one wave (bs divides 256, 8 divides bs)
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = k / 8;
    const bool live = t < m_rows * per_row;
    const int64_t tt = live ? t : 0;
    const int64_t m = tt / per_row, k0 = (tt % per_row) * 8;
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = live ? (float)x[m * k + k0 + u] : 0.0f;
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) amax = fmaxf(amax, fabsf(v[u]));
    const int group = bs / 8;  // lanes per block: 4, 8, 16 or 32
    for (int off = 1; off < group; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float a_s = amax / (float)kA8Max;
    int code[8];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        float q = a_s > 0.0f ? __builtin_rintf(v[u] / a_s) : 0.0f;
        q = fminf(fmaxf(q, -(float)kA8Max), (float)kA8Max);
        code[u] = (int)q;
        sum += code[u];
    }
    // chunk sums: 4 lanes per 32 inputs
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    if (!live) return;
    uint32_t word[2] = {0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int pos = kDeviceOrder ? a8_slot(u) : u;
        word[pos >> 2] |= ((uint32_t)code[u] & 0xFFu) << (8 * (pos & 3));
    }
    *reinterpret_cast<uint2 *>(qa + m * k + k0) = uint2{word[0], word[1]};
    if (k0 % bs == 0) scales[m * (k / bs) + k0 / bs] = a_s;
    if (chunk_sums && k0 % kChunk == 0) chunk_sums[m * (k / kChunk) + k0 / kChunk] = sum;
}

// Workspace regions for M rows of K inputs at block size bs.
struct A8Workspace {
    int64_t qa_bytes, scales_off, sums_off, total;
};
inline A8Workspace a8_workspace(int64_t m, int64_t k, int bs) {
    A8Workspace w;
    w.qa_bytes = m * k;
    w.scales_off = align_up(w.qa_bytes, kAlign);
    w.sums_off = align_up(w.scales_off + m * (k / bs) * 4, kAlign);
    w.total = align_up(w.sums_off + m * (k / kChunk) * 4, kAlign);
    return w;
}

constexpr int kA8Waves = 4;

template <typename T, int MR>
__global__ __launch_bounds__(64 * kA8Waves) void i8_rows_kernel(Problem p, const int8_t *__restrict__ qa,
                                                                 const float *__restrict__ a_scales,
                                                                 const int32_t *__restrict__ chunk_sums) {
    const int64_t mchunks = (p.m + MR - 1) / MR;
    const int64_t wq = blockIdx.x / mchunks;
    const int64_t m0 = (blockIdx.x % mchunks) * MR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, j = lane >> 4;
    const int64_t g = wq * kA8Waves + wave;
    if (g >= p.rg) return;
    const int e = (j / (p.bs / kChunk)) * kTileRows + r;
    const int64_t nb = p.k / p.bs;
    float acc[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) acc[i] = 0.0f;
    for (int64_t c = 0; c < p.kg; ++c) {
        const int64_t kc = c * kTileK + j * kChunk;  // the lane's first input
        if (kc >= p.k) break;                        // the K tail lies on whole chunks
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p.packed + (g * p.kg + c) * kTileCodeBytes + lane * 16);
        const int64_t mi = meta_index(g, p.nbt, p.kgp, e, c);
        const float s = Io<T>::to_f32(reinterpret_cast<const T *>(p.packed + p.scales_off)[mi]);
        const int zp = (int)((p.packed[p.zp_off + (mi >> 1)] >> (4 * (mi & 1))) & 15u);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            lo[t] = w[t] & 0x0F0F0F0Fu;
            hi[t] = (w[t] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int i = 0; i < MR; ++i) {
            const int64_t m = m0 + i;
            if (m >= p.m) break;
            const u32x4 *a = reinterpret_cast<const u32x4 *>(qa + m * p.k + kc);
            const u32x4 a0 = a[0], a1 = a[1];  // inputs kc .. kc + 15, kc + 16 .. kc + 31
            const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            int isum = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                isum = __builtin_amdgcn_sdot4((int)lo[t], (int)aw[2 * t], isum, false);
                isum = __builtin_amdgcn_sdot4((int)hi[t], (int)aw[2 * t + 1], isum, false);
            }
            isum -= zp * chunk_sums[m * (p.k / kChunk) + kc / kChunk];
            const float f = s * a_scales[m * nb + kc / p.bs];
            acc[i] = __builtin_fmaf(f, (float)isum, acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < MR; ++i) {
        float v = acc[i];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[i] = v;
    }
    const int64_t n = g * kTileRows + r;
    if (j == 0 && n < p.n) {
        T *y = static_cast<T *>(p.y);
#pragma unroll
        for (int i = 0; i < MR; ++i)
            if (m0 + i < p.m) y[(m0 + i) * p.n + n] = Io<T>::from_f32(acc[i]);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
int64_t a8_workspace_bytes(int64_t m, int64_t k, int bs) { return a8_workspace(m, k, bs).total; }

static unsigned grid_256(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_quantize_act(const void *x, int64_t m, int64_t k, int bs, int dtype, int8_t *qa, float *scales,
                               hipStream_t st) {
    const unsigned grid = grid_256(m * (k / 8));
    if (dtype == kF16)
        quantize_act_kernel<_Float16, false><<<grid, 256, 0, st>>>(static_cast<const _Float16 *>(x), m, k, bs, qa,
                                                                   scales, nullptr);
    else
        quantize_act_kernel<float, false><<<grid, 256, 0, st>>>(static_cast<const float *>(x), m, k, bs, qa, scales,
                                                                nullptr);
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const Problem &p, int dtype, void *workspace, hipStream_t st) {
    const A8Workspace ws = a8_workspace(p.m, p.k, p.bs);
    uint8_t *base = static_cast<uint8_t *>(workspace);
    int8_t *qa = reinterpret_cast<int8_t *>(base);
    float *a_s = reinterpret_cast<float *>(base + ws.scales_off);
    int32_t *sums = reinterpret_cast<int32_t *>(base + ws.sums_off);
    const unsigned qgrid = grid_256(p.m * (p.k / 8));
    if (dtype == kF16)
        quantize_act_kernel<_Float16, true><<<qgrid, 256, 0, st>>>(static_cast<const _Float16 *>(p.x), p.m, p.k,
                                                                   p.bs, qa, a_s, sums);
    else
        quantize_act_kernel<float, true><<<qgrid, 256, 0, st>>>(static_cast<const float *>(p.x), p.m, p.k, p.bs, qa,
                                                                a_s, sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t groups = (p.rg + kA8Waves - 1) / kA8Waves;
    if (p.m >= 4) {
        const unsigned grid = (unsigned)(groups * ((p.m + 3) / 4));
        if (dtype == kF16) i8_rows_kernel<_Float16, 4><<<grid, 64 * kA8Waves, 0, st>>>(p, qa, a_s, sums);
        else i8_rows_kernel<float, 4><<<grid, 64 * kA8Waves, 0, st>>>(p, qa, a_s, sums);
    } else {
        const unsigned grid = (unsigned)(groups * p.m);
        if (dtype == kF16) i8_rows_kernel<_Float16, 1><<<grid, 64 * kA8Waves, 0, st>>>(p, qa, a_s, sums);
        else i8_rows_kernel<float, 1><<<grid, 64 * kA8Waves, 0, st>>>(p, qa, a_s, sums);
    }
    return hipGetLastError();
}

int64_t gemm_i8_workgroups(const Problem &p) {
    const int64_t groups = (p.rg + kA8Waves - 1) / kA8Waves;
    return p.m >= 4 ? groups * ((p.m + 3) / 4) : groups * p.m;
}

}  // namespace mnb

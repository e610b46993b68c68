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
//
// M = 1 (decode): one launch. The decode kernel's workgroups (4 waves,
// persistent, host-balanced batches of 4 row groups, single products or a
// grouped plan) quantize the activation vector themselves into LDS with the
// same arithmetic as quantize_act_kernel (so the same codes, scales and
// chunk sums, bit for bit), then stream the weights in load groups of 8
// tiles and run the same per-tile integer dot products as i8_rows_kernel,
// accumulated in the same order, so a decode call gives the bits the
// two-launch form would.
#include "mnb_decode.h"

namespace mnb {

constexpr int kA8Max = 127;

// Byte position, inside the stored 8 codes of inputs 8t..8t+7, of input u.
__host__ __device__ __forceinline__ int a8_slot(int u) { return ((u & 3) << 1) | (u >> 2); }

// Quantizes 8 consecutive inputs of one block. The block's bs / 8 threads
// are consecutive lanes of one wave (bs divides 256 and 8 divides bs), and
// every lane of the wave calls this together (lanes past the data pass
// zeros). Returns the 8 codes packed in the order given by kDeviceOrder,
// the block's scale, and the sum of the lane's 32-input chunk of codes.
template <bool kDeviceOrder>
__device__ __forceinline__ uint2 quantize8(const float (&v)[8], int bs, float *a_s_out, int *chunk_sum) {
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) amax = fmaxf(amax, fabsf(v[u]));
    const int group = bs / 8;  // lanes per block: 4, 8, 16 or 32
    for (int off = 1; off < group; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float a_s = amax / (float)kA8Max;
    uint32_t word[2] = {0u, 0u};
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        float q = a_s > 0.0f ? __builtin_rintf(v[u] / a_s) : 0.0f;
        q = fminf(fmaxf(q, -(float)kA8Max), (float)kA8Max);
        const int code = (int)q;
        sum += code;
        const int pos = kDeviceOrder ? a8_slot(u) : u;
        word[pos >> 2] |= ((uint32_t)code & 0xFFu) << (8 * (pos & 3));
    }
    // chunk sums: 4 lanes per 32 inputs
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    *a_s_out = a_s;
    *chunk_sum = sum;
    return uint2{word[0], word[1]};
}

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
    float a_s;
    int sum;
    const uint2 word = quantize8<kDeviceOrder>(v, bs, &a_s, &sum);
    if (!live) return;
    *reinterpret_cast<uint2 *>(qa + m * k + k0) = word;
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
// M = 1: the decode-shaped int8 kernel.
// ---------------------------------------------------------------------------
// LDS: the quantized vector (staged K bytes, device order), then the block
// scales (float), then the chunk sums (int), all zero past K.
struct A8Lds {
    int64_t kp, scales_off, sums_off, total;
};
__host__ __device__ __forceinline__ A8Lds a8_lds(int64_t kg, int bs) {
    A8Lds l;
    l.kp = decode_staged_k(kg);
    l.scales_off = l.kp;
    l.sums_off = l.scales_off + l.kp / bs * 4;
    l.total = l.sums_off + l.kp / kChunk * 4;
    return l;
}

// log2 of the block size (32, 64, 128 or 256)
__device__ __forceinline__ int bs_shift(int bs) { return __builtin_ctz((unsigned)bs); }

template <typename T>
__device__ __forceinline__ void stage_x_i8(const Problem &p, uint8_t *smem) {
    __syncthreads();  // every wave is done with the previous vector
    const A8Lds l = a8_lds(p.kg, p.bs);
    const T *x = static_cast<const T *>(p.x);
    float *scales = reinterpret_cast<float *>(smem + l.scales_off);
    int32_t *sums = reinterpret_cast<int32_t *>(smem + l.sums_off);
    const int sh = bs_shift(p.bs);
    const int kx = (int)p.k, kp8 = (int)(l.kp / 8);
    // 8 inputs per thread per pass (the staged length is a multiple of 1024
    // inputs, so waves are either wholly inside it or wholly past it)
    for (int base = 0; base < kp8; base += kGemvThreads) {
        const int t = base + (int)threadIdx.x;
        const int k0 = t * 8;
        const bool live = k0 < kx;
        float v[8];
        u32x4 raw[sizeof(T) / 2];
        if (live) {
#pragma unroll
            for (int i = 0; i < (int)(sizeof(T) / 2); ++i) raw[i] = reinterpret_cast<const u32x4 *>(x + k0)[i];
        } else {
#pragma unroll
            for (int i = 0; i < (int)(sizeof(T) / 2); ++i) raw[i] = u32x4{0u, 0u, 0u, 0u};
        }
        const T *xv = reinterpret_cast<const T *>(raw);
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (float)xv[u];
        float a_s;
        int sum;
        const uint2 word = quantize8<true>(v, p.bs, &a_s, &sum);
        if (t < kp8) {
            *reinterpret_cast<uint2 *>(smem + k0) = word;
            if ((k0 & (p.bs - 1)) == 0) scales[k0 >> sh] = a_s;
            if ((k0 & (kChunk - 1)) == 0) sums[k0 / kChunk] = sum;
        }
    }
    __syncthreads();
}

// Tiles [c0, c0 + kTG) of the lane's row and chunk, accumulated into acc
// tile by tile (the order i8_rows_kernel uses). Tiles and chunks past K
// add exactly nothing: zero codes, scales and zero points against zero
// activation codes and scales.
template <typename T>
__device__ __forceinline__ void group_math_i8(const Group<T> &G, const uint8_t *smem, const A8Lds &l, int sh,
                                              int64_t c0, int j, float &acc) {
    const float *scales = reinterpret_cast<const float *>(smem + l.scales_off);
    const int32_t *sums = reinterpret_cast<const int32_t *>(smem + l.sums_off);
    const int kc0 = (int)c0 * kTileK + j * kChunk;  // the lane's first input in the group
#pragma unroll
    for (int u = 0; u < kTG; ++u) {
        const int kc = kc0 + u * kTileK;
        const u32x4 w = G.codes[u];
        const u32x4 *a = reinterpret_cast<const u32x4 *>(smem + kc);
        const u32x4 a0 = a[0], a1 = a[1];
        const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        int isum = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            isum = __builtin_amdgcn_sdot4((int)(w[t] & 0x0F0F0F0Fu), (int)aw[2 * t], isum, false);
            isum = __builtin_amdgcn_sdot4((int)((w[t] >> 4) & 0x0F0F0F0Fu), (int)aw[2 * t + 1], isum, false);
        }
        const int zp = (int)((G.z >> (4 * u)) & 15u);
        isum -= zp * sums[kc / kChunk];
        const float f = G.s.get(u) * scales[kc >> sh];
        acc = __builtin_fmaf(f, (float)isum, acc);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <typename T, bool kGrouped>
__device__ __forceinline__ void decode_i8_range(const Problem *entries, Problem p, int pi, int64_t b0, int64_t b1,
                                                uint8_t *smem) {
    const int wave = uniform_int((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const int r = lane & 15, j = lane >> 4;
    const uint32_t lane_code_off = (uint32_t)lane * 16u;
    int64_t b = b0;
    while (b < b1) {
        if constexpr (kGrouped) {
            while (b >= p.batch_end) p = entries[++pi];
        }
        const int64_t bend = b1 < p.batch_end ? b1 : p.batch_end;
        const A8Lds l = a8_lds(p.kg, p.bs);
        const uint32_t e = (uint32_t)((j / (p.bs / kChunk)) * kTileRows + r);
        const int64_t ngroups = (p.kg + kTG - 1) / kTG;

        int64_t sb = b, g = (b - p.batch_begin) * kGemvWaves + wave;
        int64_t c0 = 0;
        const bool have = g < p.rg;
        Group<T> cur;
        // the first weight group is in flight while x is quantized
        load_group<T>(p, g, 0, have, lane_code_off, e, cur);
        stage_x_i8<T>(p, smem);

        float acc = 0.0f;
        while (have) {
            group_math_i8<T>(cur, smem, l, bs_shift(p.bs), c0, j, acc);
            int64_t nb = sb, nc0 = c0 + kTG;
            if (nc0 >= ngroups * kTG) {
                nc0 = 0;
                nb = sb + 1;
            }
            const int64_t ng = (nb - p.batch_begin) * kGemvWaves + wave;
            const bool nvalid = nb < bend && ng < p.rg;
            load_group<T>(p, ng, nc0, nvalid, lane_code_off, e, cur);
            if (nc0 == 0) {  // row group finished
                float v = acc;
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                const int64_t n = g * kTileRows + r;
                if (j == 0 && n < p.n) static_cast<T *>(p.y)[n] = Io<T>::from_f32(v);
                acc = 0.0f;
            }
            if (!nvalid) break;
            sb = nb;
            c0 = nc0;
            g = ng;
        }
        b = bend;
    }
}

template <typename T>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(kDecodeOcc)))
void decode_i8_kernel(Problem p, int64_t wgs) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int64_t nbat = p.batch_end;
    const int64_t b0 = nbat * blockIdx.x / wgs, b1 = nbat * (blockIdx.x + 1) / wgs;
    decode_i8_range<T, false>(nullptr, p, 0, b0, b1, smem);
}

template <typename T>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(kDecodeOcc)))
void decode_i8_grouped_kernel(const Problem *entries, const GemvWg *table) {
    extern __shared__ __align__(16) uint8_t smem[];
    const GemvWg w = table[blockIdx.x];
    if (w.b0 >= w.b1) return;
    decode_i8_range<T, true>(entries, entries[w.p], w.p, w.b0, w.b1, smem);
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
size_t gemv_i8_lds_bytes(const Problem &p) { return (size_t)a8_lds(p.kg, p.bs).total; }

hipError_t launch_gemv_i8(const Problem &p0, int dtype, hipStream_t st) {
    Problem p = p0;
    p.batch_begin = 0;
    p.batch_end = (p.rg + kGemvWaves - 1) / kGemvWaves;
    const int64_t wgs = p.batch_end < kGemvMaxWgs ? p.batch_end : kGemvMaxWgs;
    const size_t lds = gemv_i8_lds_bytes(p);
    hipError_t e = hipSuccess;
    if (dtype == kF16) {
        if ((e = allow_lds<decode_i8_kernel<_Float16>>(lds)) != hipSuccess) return e;
        decode_i8_kernel<_Float16><<<(unsigned)wgs, kGemvThreads, lds, st>>>(p, wgs);
    } else {
        if ((e = allow_lds<decode_i8_kernel<float>>(lds)) != hipSuccess) return e;
        decode_i8_kernel<float><<<(unsigned)wgs, kGemvThreads, lds, st>>>(p, wgs);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_i8_grouped(const Problem *dev_entries, const GemvWg *dev_table, int64_t wgs, int dtype,
                                  size_t lds, hipStream_t st) {
    hipError_t e = hipSuccess;
    if (dtype == kF16) {
        if ((e = allow_lds<decode_i8_grouped_kernel<_Float16>>(lds)) != hipSuccess) return e;
        decode_i8_grouped_kernel<_Float16><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, dev_table);
    } else {
        if ((e = allow_lds<decode_i8_grouped_kernel<float>>(lds)) != hipSuccess) return e;
        decode_i8_grouped_kernel<float><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, dev_table);
    }
    return hipGetLastError();
}

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

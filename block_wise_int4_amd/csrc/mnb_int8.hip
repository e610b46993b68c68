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

// scales: [m][K / bs], or with m_pad > 0 transposed, [K / bs][m_pad].
// With m_pad > 0 the codes also take the matrix-core kernel's order: rows
// of qa_stride bytes (K rounded up to whole tiles), and inside each
// 128-input tile the 8-byte pieces of chunk k32, lane group g at position
// g * 4 + k32 (a lane's four pieces of a tile are contiguous).
template <typename T, bool kDeviceOrder>
__global__ __launch_bounds__(256) void quantize_act_kernel(const T *__restrict__ x, int64_t m_rows, int64_t k, int bs,
                                                           int8_t *__restrict__ qa, float *__restrict__ scales,
                                                           int32_t *__restrict__ chunk_sums, int64_t m_pad,
                                                           int64_t qa_stride) {
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
    if (m_pad > 0) {
        const int64_t t8 = (k0 % kTileK) / 8;  // = k32 * 4 + g
        const int64_t pos = (k0 / kTileK) * kTileK + ((t8 % 4) * 4 + t8 / 4) * 8;
        *reinterpret_cast<uint2 *>(qa + m * qa_stride + pos) = word;
    } else {
        *reinterpret_cast<uint2 *>(qa + m * k + k0) = word;
    }
    if (k0 % bs == 0) {
        if (m_pad > 0) scales[(k0 / bs) * m_pad + m] = a_s;
        else scales[m * (k / bs) + k0 / bs] = a_s;
    }
    if (chunk_sums && k0 % kChunk == 0) chunk_sums[m * (k / kChunk) + k0 / kChunk] = sum;
}

// Workspace regions for M rows of K inputs at block size bs.
struct A8Workspace {
    int64_t qa_bytes, scales_off, sums_off, total;
};
// The matrix-core path (M >= kA8MfmaMinRows) reads the activation scales
// transposed, [K / bs][m_pad], m_pad = M rounded up to whole row tiles.
constexpr int kA8MfmaMinRows = 16;
constexpr int kA8MPad = 128;
inline int64_t a8_m_pad(int64_t m) { return align_up(m, kA8MPad); }
inline A8Workspace a8_workspace(int64_t m, int64_t k, int bs) {
    A8Workspace w;
    w.qa_bytes = m * align_up(k, kTileK);  // rows padded to whole tiles for the matrix-core kernel
    w.scales_off = align_up(w.qa_bytes, kAlign);
    w.sums_off = align_up(w.scales_off + a8_m_pad(m) * (k / bs) * 4, kAlign);
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
// M >= 16: the int8 matrix-core kernel.
//
// v_mfma_i32_16x16x32_i8 takes, per lane, 8 bytes of A (activation row
// lane & 15) and 8 bytes of B (weight row lane & 15) for the same 8 of its
// 32 K positions (lane group lane >> 4). A lane loads word g = lane >> 4 of
// its weight row's 32-input chunk (8 codes, k0 k2 k4 k6 k1 k3 k5 k7) and
// expands it to bytes with two masks (k0 k4 k1 k5 | k2 k6 k3 k7); the
// quantizer stores the activations in that same byte order, so one MFMA is
// exactly one 32-input chunk of both operands, and chunks of one block never
// mix with another block's. The zero point is folded into the bytes:
// (nibble + 0x80 - zp) ^ 0x80 is nibble - zp as a signed byte, four at a
// time with no carries. A block's chunks chain into one integer accumulator
// (exact: |sum| <= 256 * 15 * 127); at the block's end each of the lane's 4
// outputs takes s[n] * a_s[m] * sum in float32.
// Workgroup: 2 x 2 waves, a wave computes (MF * 16) x (NF * 16) outputs.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int64_t a8_xcd_logical_wg(int64_t b, int64_t n) {
    // block b runs on XCD b % 8; give each XCD a contiguous range of tiles
    const int64_t q = n / 8, rem = n % 8;
    const int64_t x = b % 8, i = b / 8;
    return x * q + (x < rem ? x : rem) + i;
}

// Inputs of one 128-input tile for a wave: per weight row group its 4 code
// words (one per 32-input chunk), per activation fragment its 32 bytes (the
// quantizer groups a lane's four 8-byte pieces of a tile together), and the
// scales and zero points of the tile's blocks.
template <int BS, int MF, int NF>
struct A8Tile {
    static constexpr int kBlocks = BS >= kTileK ? 1 : kTileK / BS;  // blocks (or parts of one) per tile
    uint32_t w[NF][4];
    u32x4 a[MF][2];
    f4 as[MF][kBlocks];
    float s[NF][kBlocks];
    uint32_t zb[NF][kBlocks];  // (0x80 - zp) in every byte
};

template <typename T, int BS, int MF, int NF>
__global__ __launch_bounds__(256) void i8_mfma_kernel(Problem p, const int8_t *__restrict__ qa, int64_t qa_stride,
                                                      const float *__restrict__ a_scales_t, int64_t m_pad) {
    constexpr int WM = 2, WN = 2;
    using Tile = A8Tile<BS, MF, NF>;
    constexpr int kBlocks = Tile::kBlocks;
    constexpr int kChunksPerBlock = BS / kChunk;
    const int64_t tiles_n = (p.rg + WN * NF - 1) / (WN * NF);
    const int64_t wg = a8_xcd_logical_wg(blockIdx.x, gridDim.x);
    const int64_t tn = wg % tiles_n, tm = wg / tiles_n;
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m_base = (tm * WM + wm) * MF * 16;   // the wave's first activation row
    const int64_t g_base = (tn * WN + wn) * NF;        // the wave's first weight row group
    const int64_t nb = p.k / BS;
    // rows past M read zero (buffer range); row groups past N have an empty range
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(qa), 0, (int)(p.m * qa_stride), 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a_scales_t), 0, (int)(nb * m_pad * 4), 0x00020000);
    __amdgpu_buffer_rsrc_t cr[NF];
#pragma unroll
    for (int b = 0; b < NF; ++b) {
        const int64_t g = g_base + b;
        const bool in = g < p.rg;
        cr[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.packed + (in ? g : 0) * p.kg * kTileCodeBytes),
                                                  0, in ? (int)(p.kg * kTileCodeBytes) : 0, 0x00020000);
    }
    // each row group's scales and zero points: one contiguous metadata span
    // (empty for row groups past N, whose loads then read zero)
    const int64_t meta_span = (p.kgp / kMetaGroup) * (int64_t)p.nbt * kTileRows * kMetaGroup;  // entries
    __amdgpu_buffer_rsrc_t msr[NF], mzr[NF];
#pragma unroll
    for (int b = 0; b < NF; ++b) {
        const int64_t g = g_base + b;
        const bool in = g < p.rg;
        const int64_t first = (in ? g : 0) * meta_span;
        msr[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.packed + p.scales_off + first * sizeof(T)), 0,
                                                   in ? (int)(meta_span * sizeof(T)) : 0, 0x00020000);
        mzr[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.packed + p.zp_off + first / 2), 0,
                                                   in ? (int)(meta_span / 2) : 0, 0x00020000);
    }

    // every load is issued for every tile (a tile past K reads zeros or
    // unused bytes inside the buffers), so the compiler counts them exactly
    auto load_tile = [&](int64_t c, Tile &t) {
        const int64_t cm = c < p.kg ? c : p.kg - 1;  // metadata index kept inside the layout
#pragma unroll
        for (int b = 0; b < NF; ++b)
#pragma unroll
            for (int k32 = 0; k32 < 4; ++k32)
                t.w[b][k32] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr[b], (int)(c * kTileCodeBytes) + (k32 * kTileRows + r) * 16 + grp * 4, 0, 0);
#pragma unroll
        for (int a = 0; a < MF; ++a) {
            const uint32_t off = (uint32_t)((m_base + a * 16 + r) * qa_stride + c * kTileK + grp * 32);
            t.a[a][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, (int)off, 0, 0));
            t.a[a][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, (int)off + 16, 0, 0));
        }
#pragma unroll
        for (int jb = 0; jb < kBlocks; ++jb) {
            const int64_t blk = BS >= kTileK ? c * kTileK / BS : c * kBlocks + jb;
#pragma unroll
            for (int a = 0; a < MF; ++a) {
                const uint32_t soff = (uint32_t)((blk * m_pad + m_base + a * 16 + grp * 4) * 4);
                t.as[a][jb] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(sr, (int)soff, 0, 0));
            }
            // entry of (this lane's row, block jb) of tile cm inside a row group's span
            const int64_t li = ((cm / kMetaGroup) * p.nbt * kTileRows + jb * kTileRows + r) * kMetaGroup +
                               cm % kMetaGroup;
#pragma unroll
            for (int b = 0; b < NF; ++b) {
                float sv;
                if constexpr (sizeof(T) == 2)
                    sv = (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                                                                 msr[b], (int)(li * 2), 0, 0));
                else
                    sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(msr[b], (int)(li * 4), 0, 0));
                const uint32_t zbyte = __builtin_amdgcn_raw_buffer_load_b8(mzr[b], (int)(li >> 1), 0, 0);
                const uint32_t zp = (zbyte >> (4 * (uint32_t)(li & 1))) & 15u;
                t.s[b][jb] = sv;
                t.zb[b][jb] = 0x80808080u - zp * 0x01010101u;
            }
        }
    };

    float acc[MF][NF][4];
    i32x4 ci[MF][NF];
#pragma unroll
    for (int a = 0; a < MF; ++a)
#pragma unroll
        for (int b = 0; b < NF; ++b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;
            ci[a][b] = i32x4{0, 0, 0, 0};
        }
    auto compute_tile = [&](int64_t c, const Tile &t) {
#pragma unroll
        for (int k32 = 0; k32 < 4; ++k32) {
            const int64_t kk = c * kTileK + k32 * kChunk;  // the chunk's first input (uniform)
            if (kk >= p.k) break;                          // the K tail lies on whole chunks
            const int jb = BS >= kTileK ? 0 : k32 / kChunksPerBlock;
            long bop[NF];
#pragma unroll
            for (int b = 0; b < NF; ++b) {
                const uint32_t w = t.w[b][k32];
                const uint32_t lo = ((w & 0x0F0F0F0Fu) + t.zb[b][jb]) ^ 0x80808080u;
                const uint32_t hi = (((w >> 4) & 0x0F0F0F0Fu) + t.zb[b][jb]) ^ 0x80808080u;
                bop[b] = (long)(((uint64_t)hi << 32) | lo);
            }
#pragma unroll
            for (int a = 0; a < MF; ++a) {
                const u32x4 v = t.a[a][k32 >> 1];
                const uint32_t x0 = (k32 & 1) ? v.z : v.x, x1 = (k32 & 1) ? v.w : v.y;
                const long aop = (long)(((uint64_t)x1 << 32) | x0);
#pragma unroll
                for (int b = 0; b < NF; ++b)
                    ci[a][b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop[b], ci[a][b], 0, 0, 0);
            }
            if (((kk + kChunk) % BS) == 0) {  // the block ends: scale its integer sums
#pragma unroll
                for (int a = 0; a < MF; ++a) {
                    const f4 as4 = t.as[a][jb];
                    const float asv[4] = {as4.x, as4.y, as4.z, as4.w};
#pragma unroll
                    for (int b = 0; b < NF; ++b) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[a][b][i] = __builtin_fmaf(t.s[b][jb] * asv[i], (float)ci[a][b][i], acc[a][b][i]);
                        ci[a][b] = i32x4{0, 0, 0, 0};
                    }
                }
            }
        }
    };

    Tile t0, t1;
    load_tile(0, t0);
    for (int64_t c = 0; c < p.kg; c += 2) {
        load_tile(c + 1, t1);
        compute_tile(c, t0);
        load_tile(c + 2, t0);
        if (c + 1 < p.kg) compute_tile(c + 1, t1);
    }

    T *y = static_cast<T *>(p.y);
#pragma unroll
    for (int b = 0; b < NF; ++b) {
        const int64_t n = (g_base + b) * kTileRows + r;
        if (n >= p.n) continue;
#pragma unroll
        for (int a = 0; a < MF; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = m_base + a * 16 + grp * 4 + i;
                if (m < p.m) y[m * p.n + n] = Io<T>::from_f32(acc[a][b][i]);
            }
    }
}

constexpr int kA8MF = 2, kA8NF = 2;  // wave tile 32 x 32, workgroup tile 64 x 64

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
    const int64_t b0 = decode_split(nbat, blockIdx.x, wgs), b1 = decode_split(nbat, blockIdx.x + 1, wgs);
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
                                                                   scales, nullptr, 0, k);
    else
        quantize_act_kernel<float, false><<<grid, 256, 0, st>>>(static_cast<const float *>(x), m, k, bs, qa, scales,
                                                                nullptr, 0, k);
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const Problem &p, int dtype, void *workspace, hipStream_t st) {
    const A8Workspace ws = a8_workspace(p.m, p.k, p.bs);
    uint8_t *base = static_cast<uint8_t *>(workspace);
    int8_t *qa = reinterpret_cast<int8_t *>(base);
    float *a_s = reinterpret_cast<float *>(base + ws.scales_off);
    int32_t *sums = reinterpret_cast<int32_t *>(base + ws.sums_off);
    const unsigned qgrid = grid_256(p.m * (p.k / 8));
    const bool mfma = p.m >= kA8MfmaMinRows;
    const int64_t m_pad = mfma ? a8_m_pad(p.m) : 0;  // the matrix-core kernel reads the scales transposed
    const int64_t qa_stride = mfma ? p.kg * kTileK : p.k;
    if (dtype == kF16)
        quantize_act_kernel<_Float16, true><<<qgrid, 256, 0, st>>>(static_cast<const _Float16 *>(p.x), p.m, p.k,
                                                                   p.bs, qa, a_s, sums, m_pad, qa_stride);
    else
        quantize_act_kernel<float, true><<<qgrid, 256, 0, st>>>(static_cast<const float *>(p.x), p.m, p.k, p.bs, qa,
                                                                a_s, sums, m_pad, qa_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mfma) {
        const unsigned grid = (unsigned)gemm_i8_workgroups(p);
#define MNB_I8_MFMA(BS)                                                                                       \
    case BS:                                                                                                  \
        if (dtype == kF16)                                                                                    \
            i8_mfma_kernel<_Float16, BS, kA8MF, kA8NF><<<grid, 256, 0, st>>>(p, qa, qa_stride, a_s, m_pad);   \
        else                                                                                                  \
            i8_mfma_kernel<float, BS, kA8MF, kA8NF><<<grid, 256, 0, st>>>(p, qa, qa_stride, a_s, m_pad);      \
        break;
        switch (p.bs) {
            MNB_I8_MFMA(32)
            MNB_I8_MFMA(64)
            MNB_I8_MFMA(128)
            MNB_I8_MFMA(256)
        default: return hipErrorInvalidValue;
        }
#undef MNB_I8_MFMA
        return hipGetLastError();
    }
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

// The matrix-core path addresses the activations and their scales with
// 32-bit buffer offsets.
bool gemm_i8_fits(const Problem &p) {
    if (p.m < kA8MfmaMinRows) return true;
    return p.m * p.kg * kTileK < 0x7FFFFFFFLL && (p.k / p.bs) * a8_m_pad(p.m) * 4 < 0x7FFFFFFFLL;
}

int64_t gemm_i8_workgroups(const Problem &p) {
    if (p.m >= kA8MfmaMinRows) {
        const int64_t tiles_n = (p.rg + 2 * kA8NF - 1) / (2 * kA8NF);
        const int64_t tiles_m = (p.m + 2 * kA8MF * 16 - 1) / (2 * kA8MF * 16);
        return tiles_m * tiles_n;
    }
    const int64_t groups = (p.rg + kA8Waves - 1) / kA8Waves;
    return p.m >= 4 ? groups * ((p.m + 3) / 4) : groups * p.m;
}

}  // namespace mnb

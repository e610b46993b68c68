// Weight-side kernels that run once per weight or only in tests: RTN
// quantization into the canonical format, canonical -> device layout
// (pack), and the bit-exact read-back exports (unpack, dequant).
#include "mnb_internal.h"

namespace mnb {

// ---------------------------------------------------------------------------
// RTN quantization, one thread per (row, pair of blocks) so that each thread
// owns whole zero-point bytes. Decisions are taken in float64:
//  - asymmetric: the block extent including zero, the scale (hi - lo) / 15
//    rounded once to the scale dtype, zp = clamp(rint(-lo / s), 0, 15);
//  - symmetric (no zero points written): the scale max|w| / 7 rounded once
//    to the scale dtype and the fixed zero point 8;
// then q = clamp(rint(w / s) + zp, 0, 15); a block whose stored scale is 0
// gets q = zp.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quantize_rtn_kernel(const float *__restrict__ w, int64_t n_rows,
                                                           int64_t k, int bs, uint8_t *__restrict__ qweight,
                                                           T *__restrict__ scales, uint8_t *__restrict__ zps) {
    const int64_t nb = k / bs;
    const int64_t npairs = (nb + 1) / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_rows * npairs) return;
    const int64_t n = idx / npairs;
    const int64_t p = idx % npairs;
    uint32_t zbyte = 0;
    for (int e = 0; e < 2; ++e) {
        const int64_t b = 2 * p + e;
        if (b >= nb) break;
        const float *src = w + n * k + b * bs;
        double lo = 0.0, hi = 0.0;
        for (int i = 0; i < bs; ++i) {
            const double v = (double)src[i];
            lo = v < lo ? v : lo;
            hi = v > hi ? v : hi;
        }
        const bool sym = zps == nullptr;
        const double amax = -lo > hi ? -lo : hi;
        const T stored = Io<T>::round_f64(sym ? amax / 7.0 : (hi - lo) / 15.0);
        const double s = (double)stored;
        uint32_t zp = sym ? 8u : 0u;
        if (s != 0.0 && !sym) {
            const double z = __builtin_rint(-lo / s);
            zp = (uint32_t)(z < 0.0 ? 0.0 : (z > 15.0 ? 15.0 : z));
        }
        uint8_t *dst = qweight + n * (k / 2) + b * bs / 2;
        for (int i = 0; i < bs; i += 2) {
            uint32_t c[2] = {zp, zp};
            if (s != 0.0) {
                for (int t = 0; t < 2; ++t) {
                    const double q = __builtin_rint((double)src[i + t] / s) + (double)zp;
                    c[t] = (uint32_t)(q < 0.0 ? 0.0 : (q > 15.0 ? 15.0 : q));
                }
            }
            dst[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
        }
        scales[n * nb + b] = stored;
        zbyte |= zp << (4 * e);
    }
    if (zps) zps[n * ((nb + 1) / 2) + p] = (uint8_t)zbyte;
}

// ---------------------------------------------------------------------------
// Pack: one thread per 16-byte code slot of a tile (row r, chunk j).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t *__restrict__ qweight, Layout L,
                                                         uint8_t *__restrict__ packed) {
    const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tiles = L.rg * L.kg;
    if (slot >= tiles * 64) return;
    const int64_t tile = slot >> 6;
    const int l = (int)(slot & 63);
    const int r = l & 15, j = l >> 4;
    const int64_t g = tile / L.kg, c = tile % L.kg;
    const int64_t n = g * kTileRows + r;
    const int64_t k0 = c * kTileK + j * kChunk;
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    if (n < L.n && k0 < L.k) {
        // k0 is a multiple of 32 and K a multiple of 32: the chunk is whole.
        const uint32_t *src = reinterpret_cast<const uint32_t *>(qweight + n * (L.k / 2) + k0 / 2);
        for (int t = 0; t < 4; ++t) {
            uint32_t cw;
            __builtin_memcpy(&cw, reinterpret_cast<const uint8_t *>(src) + 4 * t, 4);
            out[t] = to_device_word(cw);
        }
    }
    uint32_t *dst = reinterpret_cast<uint32_t *>(packed + tile * kTileCodeBytes + l * 16);
    for (int t = 0; t < 4; ++t) dst[t] = out[t];
}

// Scales and zero points: one thread per zero-point byte, i.e. per (row
// group g, entry e, pair of tiles): entry e = jb * 16 + r is block jb of row
// r inside each tile; tiles past kg (up to kgp) get zeros.
template <typename T>
__global__ __launch_bounds__(256) void pack_meta_kernel(const T *__restrict__ scales,
                                                        const uint8_t *__restrict__ zero_points, Layout L,
                                                        uint8_t *__restrict__ packed) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int E = L.nbt * kTileRows;
    const int64_t pairs = L.kgp / 2;
    if (idx >= L.rg * E * pairs) return;
    const int64_t g = idx / (E * pairs);
    const int e = (int)((idx / pairs) % E);
    const int64_t cp = idx % pairs;
    const int jb = e / kTileRows, r = e % kTileRows;
    const int64_t n = g * kTileRows + r;
    const int64_t nb = L.k / L.bs;
    const int64_t zpb = (nb + 1) / 2;
    T *sdst = reinterpret_cast<T *>(packed + L.scales_off);
    uint32_t zbyte = 0;
    for (int h = 0; h < 2; ++h) {
        const int64_t c = 2 * cp + h;
        const int64_t b = c * kTileK / L.bs + jb;  // the block of entry jb of tile c
        T s = (T)0.0f;
        uint32_t z = 0;
        if (n < L.n && c < L.kg && b < nb) {
            s = scales[n * nb + b];
            // no zero points: the symmetric format's fixed 8
            z = zero_points ? (zero_points[n * zpb + b / 2] >> (4 * (b & 1))) & 15u : 8u;
        }
        sdst[meta_index(g, L.nbt, L.kgp, e, c)] = s;
        zbyte |= z << (4 * h);
    }
    packed[L.zp_off + meta_index(g, L.nbt, L.kgp, e, 2 * cp) / 2] = (uint8_t)zbyte;
}

// ---------------------------------------------------------------------------
// Read-back exports, one thread per code slot. They run the helpers the
// compute kernels run: unpack reads each code through the decode kernel's
// subnormal pair form (and the float32 paths' code_at must agree with it),
// dequant forms float16 weights with the MFMA kernel's dequant pair form
// and float32 weights with dequant_f32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed, Layout L,
                                                     uint8_t *__restrict__ q, uint8_t *__restrict__ zp) {
    const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tiles = L.rg * L.kg;
    if (slot >= tiles * 64) return;
    const int64_t tile = slot >> 6;
    const int l = (int)(slot & 63);
    const int r = l & 15, j = l >> 4;
    const int64_t g = tile / L.kg, c = tile % L.kg;
    const int64_t n = g * kTileRows + r;
    const int64_t k0 = c * kTileK + j * kChunk;
    if (n >= L.n || k0 >= L.k) return;
    const uint4 v = *reinterpret_cast<const uint4 *>(packed + tile * kTileCodeBytes + l * 16);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    for (int t = 0; t < 4; ++t) {
        for (int h = 0; h < 4; ++h) {
            // the pair as the decode kernel's dot products see it, scaled back
            const h2 sub = as_h2(subnormal_pair(wv[t], wv[t] >> 8, h));
            const float unscale = (h & 1) ? kSubnormalUnscale * kHighPairScale : kSubnormalUnscale;
            const uint32_t c0 = (uint32_t)((float)sub.x * unscale), c1 = (uint32_t)((float)sub.y * unscale);
            // code_at (the float32 kernels' reader) names the same codes, or the
            // slot reads 0xFF, which no valid code equals
            const bool agree = c0 == code_at(wv[t], 2 * h) && c1 == code_at(wv[t], 2 * h + 1);
            q[n * L.k + k0 + 8 * t + 2 * h] = agree ? (uint8_t)c0 : 0xFFu;
            q[n * L.k + k0 + 8 * t + 2 * h + 1] = agree ? (uint8_t)c1 : 0xFFu;
        }
    }
    const int chunks_per_block = L.bs / kChunk;
    if (j % chunks_per_block == 0) {
        const int e = (j / chunks_per_block) * kTileRows + r;
        const int64_t mi = meta_index(g, L.nbt, L.kgp, e, c);
        zp[n * (L.k / L.bs) + k0 / L.bs] = (uint8_t)((packed[L.zp_off + (mi >> 1)] >> (4 * (mi & 1))) & 15u);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ packed, Layout L,
                                                      T *__restrict__ w) {
    const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tiles = L.rg * L.kg;
    if (slot >= tiles * 64) return;
    const int64_t tile = slot >> 6;
    const int l = (int)(slot & 63);
    const int r = l & 15, j = l >> 4;
    const int64_t g = tile / L.kg, c = tile % L.kg;
    const int64_t n = g * kTileRows + r;
    const int64_t k0 = c * kTileK + j * kChunk;
    if (n >= L.n || k0 >= L.k) return;
    const uint4 v = *reinterpret_cast<const uint4 *>(packed + tile * kTileCodeBytes + l * 16);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    const int e = (j / (L.bs / kChunk)) * kTileRows + r;
    const int64_t mi = meta_index(g, L.nbt, L.kgp, e, c);
    const T s = reinterpret_cast<const T *>(packed + L.scales_off)[mi];
    const uint32_t z = (packed[L.zp_off + (mi >> 1)] >> (4 * (mi & 1))) & 15u;
    T *dst = w + n * L.k + k0;
    if constexpr (sizeof(T) == 2) {
        const h2 s2 = {s, s};
        const PairForm pf = pair_form_literal();
        for (int t = 0; t < 4; ++t)
            for (int h = 0; h < 4; ++h) {
                const h2 d = dequant_pair_f16(wv[t], h, z, s2, pf);
                dst[8 * t + 2 * h] = d.x;
                dst[8 * t + 2 * h + 1] = d.y;
            }
    } else {
        for (int t = 0; t < 4; ++t)
            for (int u = 0; u < 8; ++u) dst[8 * t + u] = dequant_f32(code_at(wv[t], u), z, s);
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_quantize_rtn(const float *w, int64_t n, int64_t k, int bs, int dtype, uint8_t *qweight,
                               void *scales, uint8_t *zps, hipStream_t st) {
    const int64_t threads = n * ((k / bs + 1) / 2);
    if (dtype == kF16)
        quantize_rtn_kernel<_Float16><<<grid_for(threads), 256, 0, st>>>(w, n, k, bs, qweight,
                                                                         (_Float16 *)scales, zps);
    else
        quantize_rtn_kernel<float><<<grid_for(threads), 256, 0, st>>>(w, n, k, bs, qweight, (float *)scales,
                                                                      zps);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *qweight, const void *scales, const uint8_t *zps, const Layout &L,
                       int dtype, uint8_t *packed, hipStream_t st) {
    const int64_t tiles = L.rg * L.kg;
    pack_codes_kernel<<<grid_for(tiles * 64), 256, 0, st>>>(qweight, L, packed);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t meta = L.rg * (L.nbt * kTileRows) * (L.kgp / 2);
    if (dtype == kF16)
        pack_meta_kernel<_Float16><<<grid_for(meta), 256, 0, st>>>((const _Float16 *)scales, zps, L, packed);
    else
        pack_meta_kernel<float><<<grid_for(meta), 256, 0, st>>>((const float *)scales, zps, L, packed);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, const Layout &L, uint8_t *q, uint8_t *zp, hipStream_t st) {
    unpack_kernel<<<grid_for(L.rg * L.kg * 64), 256, 0, st>>>(packed, L, q, zp);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *packed, const Layout &L, int dtype, void *w, hipStream_t st) {
    if (dtype == kF16)
        dequant_kernel<_Float16><<<grid_for(L.rg * L.kg * 64), 256, 0, st>>>(packed, L, (_Float16 *)w);
    else
        dequant_kernel<float><<<grid_for(L.rg * L.kg * 64), 256, 0, st>>>(packed, L, (float *)w);
    return hipGetLastError();
}

}  // namespace mnb

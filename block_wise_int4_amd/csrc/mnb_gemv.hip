// Decode kernel (M = 1) and the float32 multi-row vector kernel (M >= 2).
//
// Decode kernel. A workgroup of 4 waves walks a contiguous range of
// "batches"; a batch is 4 consecutive 16-row groups of one weight, one per
// wave, so the 4 waves always work on the same weight and share its
// activation vector, staged once in LDS together with the sum of every
// 32-input chunk. The ranges are balanced by bytes on the host, so a few
// workgroups per CU stay busy until the end of the launch and every
// workgroup pays the staging cost only when its range crosses into another
// weight.
//
// A wave streams its row group 8 tiles at a time: per tile one fully
// coalesced, non-temporal 128-bit load per lane (row r = lane & 15, chunk
// j = lane >> 4), and per 8 tiles one 16-byte scale load and one 4-byte
// zero-point load; it then computes those tiles. The CU's other waves keep
// the memory busy meanwhile: with 12 waves per CU, also keeping the next 8
// tiles in flight during the arithmetic measured slower (more bytes in
// flight than HBM serves best).
//
// Arithmetic per 32-input chunk: (w >> 4h) & 0x000F000F places two 4-bit
// codes in the low bits of two float16 halves with a zero exponent, i.e. the
// exact subnormals q * 2^-24; v_dot2_f32_f16 multiplies them by the
// activation pair exactly and accumulates in float32. The zero point never
// touches the codes: sum_k (q_k - zp) x_k = 2^24 * sum_k (q_k 2^-24) x_k
// - zp * sum_k x_k, with the chunk sum of x read from LDS, and the block
// scale multiplies the chunk result once. The four chunk lanes of each row
// are summed with two cross-lane exchanges at the end of the row group.
#include <mutex>

#include "../../include/mnb.h"
#include "mnb_decode.h"

namespace mnb {

// Contribution of tiles [c0, c0 + kTG) to the lane's partial dot product.
// Tiles past kg contribute exactly zero: zero codes, scales and zero points
// against activations staged as zeros.
template <typename T>
__device__ __forceinline__ float group_math(const Group<T> &G, const T *xs, const float *xsum, int64_t c0, int j) {
    float acc = 0.0f;
    // the group's first tile in LDS; tile u sits at a constant offset from it
    const T *xg = xs + c0 * kTileK + j * kChunk;
    const float *sg = xsum + c0 * 4 + j;
#pragma unroll
    for (int u = 0; u < kTG; ++u) {
        const float s = G.s.get(u);
        const float zs = (float)((G.z >> (4 * u)) & 15u) * sg[u * 4];
        const u32x4 w = G.codes[u];
        float part = 0.0f;
        if constexpr (sizeof(T) == 2) {
            const u32x4 *xv = reinterpret_cast<const u32x4 *>(xg + u * kTileK);
            // pairs 0 and 2 in place (q * 2^-24), pairs 1 and 3 one nibble
            // higher (q * 2^-20) into a second sum scaled back at the end: one
            // shift per word instead of three
            float part_hi = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 xx = xv[t];
                const uint32_t w0 = w[t], w8 = w[t] >> 8;
                part = __builtin_amdgcn_fdot2(as_h2(subnormal_pair(w0, w8, 0)), as_h2(xx[0]), part, false);
                part_hi = __builtin_amdgcn_fdot2(as_h2(subnormal_pair(w0, w8, 1)), as_h2(xx[1]), part_hi, false);
                part = __builtin_amdgcn_fdot2(as_h2(subnormal_pair(w0, w8, 2)), as_h2(xx[2]), part, false);
                part_hi = __builtin_amdgcn_fdot2(as_h2(subnormal_pair(w0, w8, 3)), as_h2(xx[3]), part_hi, false);
            }
            part = __builtin_fmaf(part_hi, kHighPairScale, part);
            part = __builtin_fmaf(part, kSubnormalUnscale, -zs);  // 2^24 undoes the subnormal scaling exactly
        } else {
            const float4 *xv = reinterpret_cast<const float4 *>(xg + u * kTileK);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float4 xa = xv[2 * t], xb = xv[2 * t + 1];
                const float xf[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                for (int u2 = 0; u2 < 8; ++u2) part = __builtin_fmaf((float)code_at(w[t], u2), xf[u2], part);
            }
            part -= zs;
        }
        acc = __builtin_fmaf(s, part, acc);
        // each tile's activation reads stay with its arithmetic: hoisted
        // ahead of the code loads they would hold 128 more registers
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

// Stage x[0 .. K) (zero-filled to whole load groups) and its 32-input chunk
// sums in LDS.
template <typename T>
__device__ __forceinline__ void stage_x(const Problem &p, T *xs, float *xsum) {
    __syncthreads();  // every wave is done with the previous vector
    const int64_t kp = decode_staged_k(p.kg);
    const T *x = static_cast<const T *>(p.x);
    constexpr int kPer = 16 / sizeof(T);
    for (int64_t i = threadIdx.x; i < kp / kPer; i += kGemvThreads) {
        const int64_t k = i * kPer;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k < p.k) v = *reinterpret_cast<const u32x4 *>(x + k);
        *reinterpret_cast<u32x4 *>(xs + k) = v;
    }
    __syncthreads();
    for (int64_t ch = threadIdx.x; ch < kp / kChunk; ch += kGemvThreads) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) sum += (float)xs[ch * kChunk + i];
        xsum[ch] = sum;
    }
    __syncthreads();
}

// Greedy-argmax key of output n with value v (already rounded to the
// output dtype): larger key = larger value, equal values = lower index.
// -0 counts as +0; the values are taken to be finite.
template <typename T>
__device__ __forceinline__ uint64_t argmax_key(T v, int64_t n) {
    uint32_t ord;
    if constexpr (sizeof(T) == 2) {
        uint32_t h = __builtin_bit_cast(uint16_t, v);
        if (h == 0x8000u) h = 0u;
        ord = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
    } else {
        uint32_t u = __builtin_bit_cast(uint32_t, v);
        if (u == 0x80000000u) u = 0u;
        ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
}

// Runs batches [b0, b1) starting in problem `pi`. With kArgmax, y is
// written only when the problem has one, and the result is the largest
// argmax key among the outputs this lane finished (0 if none).
template <typename T, bool kGrouped, bool kArgmax = false>
__device__ __forceinline__ uint64_t decode_range(const Problem *entries, Problem p, int pi, int64_t b0, int64_t b1,
                                                 uint8_t *smem) {
    uint64_t best = 0;
    const int wave = uniform_int((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const int r = lane & 15, j = lane >> 4;
    const uint32_t lane_code_off = (uint32_t)lane * 16u;
    int64_t b = b0;
    while (b < b1) {
        if constexpr (kGrouped) {
            while (b >= p.batch_end) p = entries[++pi];
        }
        const int64_t bend = b1 < p.batch_end ? b1 : p.batch_end;
        const int64_t kp = decode_staged_k(p.kg);
        T *xs = reinterpret_cast<T *>(smem);
        float *xsum = reinterpret_cast<float *>(smem + kp * sizeof(T));
        const uint32_t e = (uint32_t)((j / (p.bs / kChunk)) * kTileRows + r);
        const int64_t ngroups = (p.kg + kTG - 1) / kTG;

        int64_t sb = b, g = (b - p.batch_begin) * kGemvWaves + wave;
        int64_t c0 = 0;
        const bool have = g < p.rg;
        Group<T> cur;
        // the first weight group is in flight while x is staged
        load_group<T>(p, g, 0, have, lane_code_off, e, cur);
        stage_x<T>(p, xs, xsum);

        float acc = 0.0f;
        while (have) {
            acc += group_math<T>(cur, xs, xsum, c0, j);
            // the step after this one: next 8 tiles, or the next batch's row group
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
                if constexpr (kArgmax) {
                    if (j == 0 && n < p.n) {
                        const T yv = (T)v;
                        if (p.y) static_cast<T *>(p.y)[n] = yv;
                        const uint64_t key = argmax_key<T>(yv, n);
                        best = key > best ? key : best;
                    }
                } else {
                    if (j == 0 && n < p.n) static_cast<T *>(p.y)[n] = (T)v;
                }
                acc = 0.0f;
            }
            if (!nvalid) break;
            sb = nb;
            c0 = nc0;
            g = ng;
        }
        b = bend;
    }
    return best;
}

template <typename T>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(kDecodeOcc)))
void decode_kernel(Problem p, int64_t wgs) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int64_t nbat = p.batch_end;  // batch_begin = 0 for a single problem
    const int64_t b0 = decode_split(nbat, blockIdx.x, wgs), b1 = decode_split(nbat, blockIdx.x + 1, wgs);
    decode_range<T, false>(nullptr, p, 0, b0, b1, smem);
}

// Single products that fill at most one round of workgroups (every decode
// linear but the LM head) have too few waves to keep the memory and the
// ALUs busy: with one wave per row group, a row group of K inputs waits for
// K / 1024 load groups' round trips and arithmetic in sequence, about 2 us
// per 1024 inputs. Here the S waves of a workgroup (S = 1, 2 or 4) share
// one row group: the wave with sub-index s takes load groups s, s + S,
// s + 2S, ..., with two of them in flight at a time, and keeps each group's
// per-lane result. The first wave of the row group then adds the results
// of groups 0, 1, 2, ... in order, which is the exact sequence of float
// additions decode_range makes for the same row group, so the outputs equal
// the grouped kernel's bit for bit. With S = 1 each wave owns one row group
// (four per workgroup), as in decode_kernel, with the next load group in
// flight during the current one's arithmetic.
template <typename T, int S>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(kDecodeOcc)))
void decode_split_kernel(Problem p) {
    static_assert(S == 1 || S == 2 || S == 4, "waves per row group");
    constexpr int kRowGroups = kGemvWaves / S;  // row groups per workgroup
    extern __shared__ __align__(16) uint8_t smem[];
    const int wave = uniform_int((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const int r = lane & 15, j = lane >> 4;
    const int rgw = wave / S, sub = wave % S;
    const uint32_t lane_code_off = (uint32_t)lane * 16u;
    const int64_t kp = decode_staged_k(p.kg);
    T *xs = reinterpret_cast<T *>(smem);
    float *xsum = reinterpret_cast<float *>(smem + kp * sizeof(T));
    const uint32_t e = (uint32_t)((j / (p.bs / kChunk)) * kTileRows + r);
    const int64_t ngroups = (p.kg + kTG - 1) / kTG;
    const int64_t g = (int64_t)blockIdx.x * kRowGroups + rgw;
    const bool have = g < p.rg;
    // per-lane results of every load group of the workgroup's row groups
    // (S > 1): [row group of the workgroup][load group][lane]
    float *parts = xsum + kp / kChunk + (int64_t)rgw * ngroups * 64;

    // this wave's i-th load group is t = sub + i * S; ring slot i % 2
    Group<T> ring[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = sub + (int64_t)i * S;
        load_group<T>(p, g, t * kTG, have && t < ngroups, lane_code_off, e, ring[i]);
    }
    stage_x<T>(p, xs, xsum);

    float acc = 0.0f;
    for (int64_t t0 = sub; t0 < ngroups; t0 += 2 * S) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t t = t0 + (int64_t)i * S;
            if (t < ngroups) {
                const float gm = group_math<T>(ring[i], xs, xsum, t * kTG, j);
                if constexpr (S == 1) acc += gm;
                else parts[t * 64 + lane] = gm;
            }
            const int64_t tn = t + 2 * S;
            load_group<T>(p, g, tn * kTG, have && tn < ngroups, lane_code_off, e, ring[i]);
        }
    }
    if constexpr (S > 1) {
        __syncthreads();
        if (sub != 0) return;
        for (int64_t t = 0; t < ngroups; ++t) acc += parts[t * 64 + lane];
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    const int64_t n = g * kTileRows + r;
    if (j == 0 && n < p.n) static_cast<T *>(p.y)[n] = (T)acc;
}

// Waves per row group for a single decode product, 0 where the split kernel
// does not apply (more than one round of workgroups even at S = 1, or the
// per-group results do not fit next to the staged activations).
int decode_split_waves(const Problem &p, size_t base_lds, size_t *lds) {
    const int64_t ngroups = (p.kg + kTG - 1) / kTG;
    // (three load groups also take four waves: one round trip, one wave idle)
    for (int s = 4; s >= 1; s /= 2) {
        if ((s == 4 && ngroups < 3) || (s == 2 && ngroups < 2)) continue;
        const int64_t wgs = (p.rg * s + kGemvWaves - 1) / kGemvWaves;
        if (wgs > kGemvMaxWgs) continue;
        const size_t need = base_lds + (s > 1 ? (size_t)(kGemvWaves / s) * ngroups * 64 * 4 : 0);
        if (need > (size_t)kGemvMaxLds) continue;
        *lds = need;
        return s;
    }
    return 0;
}

template <typename T>
static hipError_t launch_decode_split(const Problem &p, int s, size_t lds, hipStream_t st) {
    const unsigned grid = (unsigned)((p.rg * s + kGemvWaves - 1) / kGemvWaves);
    hipError_t e = hipSuccess;
    switch (s) {
    case 4:
        if ((e = allow_lds<decode_split_kernel<T, 4>>(lds)) != hipSuccess) return e;
        decode_split_kernel<T, 4><<<grid, kGemvThreads, lds, st>>>(p);
        break;
    case 2:
        if ((e = allow_lds<decode_split_kernel<T, 2>>(lds)) != hipSuccess) return e;
        decode_split_kernel<T, 2><<<grid, kGemvThreads, lds, st>>>(p);
        break;
    default:
        if ((e = allow_lds<decode_split_kernel<T, 1>>(lds)) != hipSuccess) return e;
        decode_split_kernel<T, 1><<<grid, kGemvThreads, lds, st>>>(p);
        break;
    }
    return hipGetLastError();
}

// Argmax workspace: one 8-byte slot per workgroup of the product launch.
static_assert(kGemvMaxWgs * 8 <= MNB_ARGMAX_WORKSPACE_BYTES, "argmax workspace too small");

// Decode product fused with a greedy argmax over its outputs: each
// workgroup stores the best key of the outputs it produced in its slot.
template <typename T>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(kDecodeOcc)))
void decode_argmax_kernel(Problem p, int64_t wgs, unsigned long long *slots) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ unsigned long long wave_best[kGemvWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nbat = p.batch_end;
    const int64_t b0 = decode_split(nbat, blockIdx.x, wgs), b1 = decode_split(nbat, blockIdx.x + 1, wgs);
    uint64_t best = decode_range<T, false, true>(nullptr, p, 0, b0, b1, smem);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off);
        best = o > best ? o : best;
    }
    if (lane == 0) wave_best[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long b = wave_best[0];
#pragma unroll
        for (int w = 1; w < kGemvWaves; ++w) b = wave_best[w] > b ? wave_best[w] : b;
        slots[blockIdx.x] = b;
    }
}

// Second launch on the same stream (so every slot is visible): the largest
// key of `count` slots, turned back into its output index.
__global__ __launch_bounds__(kGemvThreads) void argmax_finish_kernel(const unsigned long long *slots, int count,
                                                                     int64_t *index) {
    const unsigned long long b = argmax_reduce_slots(slots, count);
    if (threadIdx.x == 0) *index = argmax_key_index(b);
}

template <typename T>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(kDecodeOcc)))
void decode_grouped_kernel(const Problem *entries, const GemvWg *table) {
    extern __shared__ __align__(16) uint8_t smem[];
    const GemvWg w = table[blockIdx.x];
    if (w.b0 >= w.b1) return;
    decode_range<T, true>(entries, entries[w.p], w.p, w.b0, w.b1, smem);
}

// ---------------------------------------------------------------------------
// float32 multi-row kernel (M >= 2): one wave per row group, 4 activation
// rows per pass, activations staged in LDS.
// ---------------------------------------------------------------------------
template <int MR>
__device__ __forceinline__ void rows_workgroup(const Problem &p, int64_t wg, float *xs) {
    const int64_t mchunks = (p.m + MR - 1) / MR;
    const int64_t wq = wg / mchunks;
    const int64_t m0 = (wg % mchunks) * MR;
    const int64_t kp = p.kg * kTileK;
    const float *x = static_cast<const float *>(p.x);
    for (int64_t i = threadIdx.x; i < MR * kp / 4; i += kGemvThreads) {
        const int64_t row = i / (kp / 4);
        const int64_t k = (i % (kp / 4)) * 4;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m0 + row < p.m && k < p.k) v = *reinterpret_cast<const u32x4 *>(x + (m0 + row) * p.k + k);
        *reinterpret_cast<u32x4 *>(xs + row * kp + k) = v;
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, j = lane >> 4;
    const int64_t g = wq * kGemvWaves + wave;
    if (g >= p.rg) return;
    const int e = (j / (p.bs / kChunk)) * kTileRows + r;
    float acc[MR];
#pragma unroll
    for (int row = 0; row < MR; ++row) acc[row] = 0.0f;
    for (int64_t c = 0; c < p.kg; ++c) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p.packed + (g * p.kg + c) * kTileCodeBytes + lane * 16);
        const int64_t mi = meta_index(g, p.nbt, p.kgp, e, c);
        const float s = reinterpret_cast<const float *>(p.packed + p.scales_off)[mi];
        const uint32_t z = (p.packed[p.zp_off + (mi >> 1)] >> (4 * (mi & 1))) & 15u;
        float dv[32];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 8; ++u) dv[8 * t + u] = (float)((int)code_at(w[t], u) - (int)z);
#pragma unroll
        for (int row = 0; row < MR; ++row) {
            const float *xr = xs + row * kp + c * kTileK + j * kChunk;
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) part = __builtin_fmaf(dv[i], xr[i], part);
            acc[row] = __builtin_fmaf(s, part, acc[row]);
        }
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
        float *y = static_cast<float *>(p.y);
#pragma unroll
        for (int row = 0; row < MR; ++row)
            if (m0 + row < p.m) y[(m0 + row) * p.n + n] = acc[row];
    }
}

template <int MR>
__global__ __launch_bounds__(kGemvThreads) void rows_kernel(Problem p) {
    extern __shared__ __align__(16) uint8_t smem[];
    rows_workgroup<MR>(p, blockIdx.x, reinterpret_cast<float *>(smem));
}

__device__ __forceinline__ int find_problem(const Problem *entries, int count, int64_t wg) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (entries[mid].wg_begin <= wg) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int MR>
__global__ __launch_bounds__(kGemvThreads) void rows_grouped_kernel(const Problem *entries, int count) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int i = find_problem(entries, count, blockIdx.x);
    const Problem p = entries[i];
    rows_workgroup<MR>(p, (int64_t)blockIdx.x - p.wg_begin, reinterpret_cast<float *>(smem));
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kRowsMR = 4;
// Variants: 0 = fp16 decode, 1 = fp32 decode, 2 = fp32 4 rows per pass,
// 3 = fp32 1 row per pass (K too long to stage 4 rows).
int gemv_variant(int dtype, int64_t m) {
    if (m >= 2) return 2;
    return dtype == kF16 ? 0 : 1;
}

static int elem_bytes(int variant) { return variant == 0 ? 2 : 4; }
static int rows_per_pass(int variant) { return variant == 2 ? kRowsMR : 1; }

size_t gemv_lds_bytes(const Problem &p, int variant) {
    if (variant >= 2) return (size_t)(rows_per_pass(variant) * p.kg * kTileK * 4);
    const int64_t kp = decode_staged_k(p.kg);
    return (size_t)(kp * elem_bytes(variant) + kp / kChunk * 4);
}

bool gemv_lds_fits(const Problem &p, int variant) { return gemv_lds_bytes(p, variant) <= (size_t)kGemvMaxLds; }

int64_t gemv_workgroups(const Problem &p, int variant) {
    const int mr = rows_per_pass(variant);
    return ((p.rg + kGemvWaves - 1) / kGemvWaves) * ((p.m + mr - 1) / mr);
}

int64_t gemv_schedule(Problem *entries, int count, GemvWg *table, int max_wgs) {
    // batches and their cost (tiles per row group, plus one for the row end)
    int64_t nbat = 0, cost = 0;
    for (int i = 0; i < count; ++i) {
        Problem &p = entries[i];
        p.batch_begin = nbat;
        nbat += (p.rg + kGemvWaves - 1) / kGemvWaves;
        p.batch_end = nbat;
        cost += (p.batch_end - p.batch_begin) * (p.kg + 1);
    }
    const int64_t wgs = nbat < max_wgs ? nbat : max_wgs;
    // workgroup w starts at the first batch whose cost prefix reaches its
    // share of the cost (shares proportional to the workgroups' rates)
    const double total_rate = decode_rate_prefix(wgs, wgs);
    int pi = 0;
    int64_t b = 0, prefix = 0;
    for (int64_t w = 0; w <= wgs; ++w) {
        const int64_t target = w == wgs ? cost : (int64_t)((double)cost * decode_rate_prefix(w, wgs) / total_rate);
        while (b < nbat && prefix < target) {
            while (b >= entries[pi].batch_end) ++pi;
            prefix += entries[pi].kg + 1;
            ++b;
        }
        if (w < wgs) {
            int q = pi;
            while (q < count - 1 && b >= entries[q].batch_end) ++q;
            table[w].b0 = (int32_t)b;
            table[w].p = q;
            table[w].pad_ = 0;
        }
        if (w > 0) table[w - 1].b1 = (int32_t)b;
    }
    return wgs;
}

hipError_t launch_gemv(const Problem &p0, int dtype, int variant, hipStream_t st) {
    (void)dtype;
    const size_t lds = gemv_lds_bytes(p0, variant);
    hipError_t e = hipSuccess;
    if (variant >= 2) {
        const unsigned grid = (unsigned)gemv_workgroups(p0, variant);
        if (variant == 2) {
            if ((e = allow_lds<rows_kernel<kRowsMR>>(lds)) != hipSuccess) return e;
            rows_kernel<kRowsMR><<<grid, kGemvThreads, lds, st>>>(p0);
        } else {
            if ((e = allow_lds<rows_kernel<1>>(lds)) != hipSuccess) return e;
            rows_kernel<1><<<grid, kGemvThreads, lds, st>>>(p0);
        }
        return hipGetLastError();
    }
    Problem p = p0;
    p.batch_begin = 0;
    p.batch_end = (p.rg + kGemvWaves - 1) / kGemvWaves;
    const int64_t wgs = p.batch_end < kGemvMaxWgs ? p.batch_end : kGemvMaxWgs;
    size_t split_lds = 0;
    if (const int sw = decode_split_waves(p, lds, &split_lds)) {  // a product of one round of workgroups
        return variant == 0 ? launch_decode_split<_Float16>(p, sw, split_lds, st)
                            : launch_decode_split<float>(p, sw, split_lds, st);
    }
    if (variant == 0) {
        if ((e = allow_lds<decode_kernel<_Float16>>(lds)) != hipSuccess) return e;
        decode_kernel<_Float16><<<(unsigned)wgs, kGemvThreads, lds, st>>>(p, wgs);
    } else {
        if ((e = allow_lds<decode_kernel<float>>(lds)) != hipSuccess) return e;
        decode_kernel<float><<<(unsigned)wgs, kGemvThreads, lds, st>>>(p, wgs);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_argmax(const Problem &p0, int variant, void *workspace, int64_t *index, hipStream_t st) {
    const size_t lds = gemv_lds_bytes(p0, variant);
    Problem p = p0;
    p.batch_begin = 0;
    p.batch_end = (p.rg + kGemvWaves - 1) / kGemvWaves;
    const int64_t wgs = p.batch_end < kGemvMaxWgs ? p.batch_end : kGemvMaxWgs;
    unsigned long long *slots = static_cast<unsigned long long *>(workspace);
    hipError_t e = hipSuccess;
    if (variant == 0) {
        if ((e = allow_lds<decode_argmax_kernel<_Float16>>(lds)) != hipSuccess) return e;
        decode_argmax_kernel<_Float16><<<(unsigned)wgs, kGemvThreads, lds, st>>>(p, wgs, slots);
    } else if (variant == 1) {
        if ((e = allow_lds<decode_argmax_kernel<float>>(lds)) != hipSuccess) return e;
        decode_argmax_kernel<float><<<(unsigned)wgs, kGemvThreads, lds, st>>>(p, wgs, slots);
    } else {
        return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!index) return hipSuccess;  // the slots stay for a consumer that reduces them (the embedding gather)
    argmax_finish_kernel<<<1, kGemvThreads, 0, st>>>(slots, (int)wgs, index);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Library-held argmax slots for callers that cannot allocate: one array per
// device (the runtime gives each device its own copy), holding one slot per
// workgroup of the largest argmax launch. Host code never passes the
// array's name to a kernel: in host code it is a stand-in, not a device
// address. Its address on each device comes from hipGetSymbolAddress, once
// per device, with that device current.
// ---------------------------------------------------------------------------
constexpr int kScratchSlots = kGemvMaxWgs;
static __device__ __align__(256) unsigned long long scratch[kScratchSlots];

constexpr int kMaxScratchDevices = 64;
static std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
static std::mutex g_scratch_mu;

hipError_t argmax_scratch(void **slots, int64_t *n_slots) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!ptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *slots = ptr;
    *n_slots = kScratchSlots;
    return hipSuccess;
}

int64_t gemv_argmax_slots(const Problem &p) { return argmax_slot_count(p.n); }

int64_t argmax_slot_count(int64_t n) {
    const int64_t rg = (n + kTileRows - 1) / kTileRows;
    const int64_t batches = (rg + kGemvWaves - 1) / kGemvWaves;
    return batches < kGemvMaxWgs ? batches : kGemvMaxWgs;
}

hipError_t launch_gemv_grouped(const Problem *dev_entries, int count, const GemvWg *dev_table, int64_t wgs,
                               int variant, size_t lds, hipStream_t st) {
    hipError_t e = hipSuccess;
    switch (variant) {
    case 0:
        if ((e = allow_lds<decode_grouped_kernel<_Float16>>(lds)) != hipSuccess) return e;
        decode_grouped_kernel<_Float16><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, dev_table);
        break;
    case 1:
        if ((e = allow_lds<decode_grouped_kernel<float>>(lds)) != hipSuccess) return e;
        decode_grouped_kernel<float><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, dev_table);
        break;
    case 2:
        if ((e = allow_lds<rows_grouped_kernel<kRowsMR>>(lds)) != hipSuccess) return e;
        rows_grouped_kernel<kRowsMR><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, count);
        break;
    default:
        if ((e = allow_lds<rows_grouped_kernel<1>>(lds)) != hipSuccess) return e;
        rows_grouped_kernel<1><<<(unsigned)wgs, kGemvThreads, lds, st>>>(dev_entries, count);
        break;
    }
    return hipGetLastError();
}

}  // namespace mnb

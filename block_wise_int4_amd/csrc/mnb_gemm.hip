// Prefill kernel (float16, M >= 2): int4 weight tiles dequantized in
// registers feed v_mfma_f32_16x16x32_f16, activations are staged in LDS.
//
// Workgroup = WM x WN waves; wave (wm, wn) computes an (MF * 16) x (NF * 16)
// block of Y, so the workgroup tile is (WM * MF * 16) x (WN * NF * 16).
//
// Weight side: a wave owns NF 16-row groups of W (= NF 16-column fragments
// of Y). For each 128-input tile it issues one coalesced 128-bit load per
// lane and fragment (lane l holds row l & 15, chunk l >> 4: 32 codes), forms
// exact (q - zp) float16 pairs with the 1024-offset trick and multiplies by
// the block scale with one rounding. Those 32 values are the lane's B
// operands for the four MFMAs of the tile: MFMA t uses inputs t*8 .. t*8+7
// of the lane's chunk. The sum over K does not care which inputs an MFMA
// groups together, as long as A and B agree; A is read from LDS with the
// same grouping, so no lane shuffles are needed on either side.
//
// Activation side: the 128-input tile is split in two LDS stages of 64
// inputs (stage h holds inputs j*32 + h*16 + [0, 16) of each chunk j), which
// keeps a double-buffered 416-row stage inside the 160 KB LDS. Global loads
// of the next stage are issued before the MFMAs of the current one; one
// barrier per stage.
#include "mnb_internal.h"

namespace mnb {

constexpr int kLdaHalves = 72;  // 64 inputs + 8 halves of padding per LDS row

template <int MF, int NF, int WM, int WN>
struct GemmCfg {
    static constexpr int kMT = WM * MF * 16;
    static constexpr int kNT = WN * NF * 16;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kPieces = kMT * 8;  // 16-byte pieces per A stage
    static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
    static constexpr int kStageHalves = kMT * kLdaHalves;
};

template <int MF, int NF, int WM, int WN>
__device__ __forceinline__ void gemm_workgroup(const Problem &p, int64_t wg, _Float16 *lds) {
    using C = GemmCfg<MF, NF, WM, WN>;
    const int64_t tn = wg % p.tiles_n;
    const int64_t tm = wg / p.tiles_n;
    const int64_t m0 = tm * C::kMT;
    const int64_t g0 = tn * (WN * NF);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 15, j = lane >> 4;
    const int e = (j / (p.bs / kChunk)) * kTileRows + r;
    const _Float16 *x = static_cast<const _Float16 *>(p.x);
    const int64_t n_stages = 2 * p.kg;

    // ---- activation stages -------------------------------------------------
    uint4 areg[C::kPPT];
    auto load_a = [&](int64_t stage) {
        const int64_t c = stage >> 1;
        const int h = (int)(stage & 1);
#pragma unroll
        for (int i = 0; i < C::kPPT; ++i) {
            const int pc = tid + i * C::kThreads;
            uint4 v = {0u, 0u, 0u, 0u};
            if (pc < C::kPieces) {
                const int row = pc >> 3, seg = pc & 7;
                const int64_t m = m0 + row;
                const int64_t k = c * kTileK + (seg >> 1) * kChunk + h * 16 + (seg & 1) * 8;
                if (m < p.m && k < p.k) v = *reinterpret_cast<const uint4 *>(x + m * p.k + k);
            }
            areg[i] = v;
        }
    };
    auto store_a = [&](int buf) {
        _Float16 *dst = lds + buf * C::kStageHalves;
#pragma unroll
        for (int i = 0; i < C::kPPT; ++i) {
            const int pc = tid + i * C::kThreads;
            if (pc < C::kPieces)
                *reinterpret_cast<uint4 *>(dst + (pc >> 3) * kLdaHalves + (pc & 7) * 8) = areg[i];
        }
    };

    // ---- weight tiles -------------------------------------------------------
    uint4 braw[NF];
    _Float16 sraw[NF];
    uint32_t zraw[NF];
    auto load_b = [&](int64_t c) {
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const int64_t g = g0 + wn * NF + b;
            if (g < p.rg) {
                const int64_t tile = g * p.kg + c;
                braw[b] = *(reinterpret_cast<const uint4 *>(p.packed + tile * kTileCodeBytes) + lane);
                const int64_t mi = meta_index(g, p.nbt, p.kgp, e, c);
                sraw[b] = reinterpret_cast<const _Float16 *>(p.packed + p.scales_off)[mi];
                zraw[b] = (p.packed[p.zp_off + (mi >> 1)] >> (4 * (mi & 1))) & 15u;
            } else {
                braw[b] = {0u, 0u, 0u, 0u};
                sraw[b] = (_Float16)0.0f;
                zraw[b] = 0u;
            }
        }
    };
    h8 bw[NF][4];
    auto dequant_b = [&]() {
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const h2 zm = zp_magic(zraw[b]);
            const h2 s2 = {sraw[b], sraw[b]};
            const uint32_t w[4] = {braw[b].x, braw[b].y, braw[b].z, braw[b].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                h8 v;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const h2 d = dequant_pair_f16(w[t], h, zm, s2);
                    v[2 * h] = d.x;
                    v[2 * h + 1] = d.y;
                }
                bw[b][t] = v;
            }
        }
    };

    f4 acc[MF][NF];
#pragma unroll
    for (int a = 0; a < MF; ++a)
#pragma unroll
        for (int b = 0; b < NF; ++b) acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    load_a(0);
    load_b(0);
    store_a(0);
    __syncthreads();

    for (int64_t c = 0; c < p.kg; ++c) {
        dequant_b();
        if (c + 1 < p.kg) load_b(c + 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t stage = 2 * c + h;
            const bool more = stage + 1 < n_stages;
            if (more) load_a(stage + 1);
            const _Float16 *As = lds + (int)(stage & 1) * C::kStageHalves + (wm * MF * 16 + r) * kLdaHalves + j * 16;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int a = 0; a < MF; ++a) {
                    const h8 av = *reinterpret_cast<const h8 *>(As + a * 16 * kLdaHalves + tt * 8);
#pragma unroll
                    for (int b = 0; b < NF; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bw[b][2 * h + tt], acc[a][b], 0, 0, 0);
                }
            }
            if (more) store_a((int)((stage + 1) & 1));
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds rows j*4 + i, column r of each fragment ------
    _Float16 *y = static_cast<_Float16 *>(p.y);
#pragma unroll
    for (int b = 0; b < NF; ++b) {
        const int64_t n = (g0 + wn * NF + b) * kTileRows + r;
        if (n >= p.n) continue;
#pragma unroll
        for (int a = 0; a < MF; ++a) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = m0 + wm * MF * 16 + a * 16 + j * 4 + i;
                if (m < p.m) y[m * p.n + n] = (_Float16)acc[a][b][i];
            }
        }
    }
}

template <int MF, int NF, int WM, int WN>
__global__ __launch_bounds__(64 * WM *WN) void gemm_kernel(Problem p) {
    __shared__ __align__(16) _Float16 lds[2 * GemmCfg<MF, NF, WM, WN>::kStageHalves];
    gemm_workgroup<MF, NF, WM, WN>(p, blockIdx.x, lds);
}

__device__ __forceinline__ int find_gemm_problem(const Problem *entries, int count, int64_t wg) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (entries[mid].wg_begin <= wg) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int MF, int NF, int WM, int WN>
__global__ __launch_bounds__(64 * WM *WN) void gemm_grouped_kernel(const Problem *entries, int count) {
    __shared__ __align__(16) _Float16 lds[2 * GemmCfg<MF, NF, WM, WN>::kStageHalves];
    const int i = find_gemm_problem(entries, count, blockIdx.x);
    const Problem p = entries[i];
    gemm_workgroup<MF, NF, WM, WN>(p, (int64_t)blockIdx.x - p.wg_begin, lds);
}

// ---------------------------------------------------------------------------
// Variants and their selection.
// ---------------------------------------------------------------------------
struct VariantInfo {
    int mt, nt;
};
static const VariantInfo kVariants[] = {
    {16, 64},    // 0: MF 1,  NF 1, 1x4 waves
    {32, 64},    // 1: MF 2,  NF 1, 1x4 waves
    {64, 128},   // 2: MF 4,  NF 2, 1x4 waves
    {128, 128},  // 3: MF 4,  NF 4, 2x2 waves
    {256, 128},  // 4: MF 8,  NF 4, 2x2 waves
    {384, 128},  // 5: MF 12, NF 4, 2x2 waves
    {416, 128},  // 6: MF 13, NF 4, 2x2 waves
};
constexpr int kNumVariants = 7;

int gemm_variant(int64_t m) {
    if (m <= 16) return 0;
    if (m <= 32) return 1;
    if (m <= 64) return 2;
    // fewest padded rows; on a tie the taller tile (less weight dequant work)
    int best = 3;
    int64_t best_rows = -1;
    for (int v = 3; v < kNumVariants; ++v) {
        const int64_t mt = kVariants[v].mt;
        const int64_t rows = (m + mt - 1) / mt * mt;
        if (best_rows < 0 || rows <= best_rows) {
            best = v;
            best_rows = rows;
        }
    }
    return best;
}

void gemm_tiles(const Problem &p, int variant, int32_t *tiles_m, int32_t *tiles_n) {
    const int64_t mt = kVariants[variant].mt;
    const int64_t rg_per_tile = kVariants[variant].nt / kTileRows;
    *tiles_m = (int32_t)((p.m + mt - 1) / mt);
    *tiles_n = (int32_t)((p.rg + rg_per_tile - 1) / rg_per_tile);
}

#define MNB_GEMM_VARIANTS(X) \
    X(0, 1, 1, 1, 4)         \
    X(1, 2, 1, 1, 4)         \
    X(2, 4, 2, 1, 4)         \
    X(3, 4, 4, 2, 2)         \
    X(4, 8, 4, 2, 2)         \
    X(5, 12, 4, 2, 2)        \
    X(6, 13, 4, 2, 2)

hipError_t launch_gemm(const Problem &p, int variant, hipStream_t st) {
    const unsigned grid = (unsigned)((int64_t)p.tiles_m * p.tiles_n);
    switch (variant) {
#define X(V, MF, NF, WM, WN) \
    case V: gemm_kernel<MF, NF, WM, WN><<<grid, 64 * WM * WN, 0, st>>>(p); break;
        MNB_GEMM_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_grouped(const Problem *dev_entries, int count, int64_t wgs, int variant, hipStream_t st) {
    switch (variant) {
#define X(V, MF, NF, WM, WN) \
    case V: gemm_grouped_kernel<MF, NF, WM, WN><<<(unsigned)wgs, 64 * WM * WN, 0, st>>>(dev_entries, count); break;
        MNB_GEMM_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mnb

// Prefill kernel (float16, M >= 2): int4 weight tiles dequantized in
// registers feed v_mfma_f32_16x16x32_f16; activations reach LDS by direct
// buffer-to-LDS loads.
//
// Workgroup = WM x WN waves; wave (wm, wn) computes an (MF * 16) x (NF * 16)
// block of Y, so the workgroup tile is (WM * MF * 16) x (WN * NF * 16).
//
// Weight side: a wave owns NF 16-row groups of W (= NF 16-column fragments
// of Y). For each 128-input tile it issues one coalesced 128-bit load per
// lane and fragment (lane l holds row l & 15, chunk l >> 4: 32 codes), forms
// exact (q - zp) float16 pairs with the 1024-offset trick and multiplies by
// the block scale with one rounding (the same helper as mnb_dequant, so the
// MFMA operands are exactly the dequantized weights). Those 32 values are
// the lane's B operands for the four MFMAs of the tile: MFMA t uses inputs
// t*8 .. t*8+7 of the lane's chunk. The sum over K does not care which
// inputs an MFMA groups together as long as A and B agree, so A is laid out
// with the same grouping and no lane shuffles are needed on either side.
//
// Activation side: the 128-input tile is split in two LDS stages of 64
// inputs (stage h feeds MFMAs t = 2h, 2h+1). A stage is a list of 1 KB
// lines, one per (16-row fragment, t): line byte 16*l holds the 8 inputs
// lane l passes to that MFMA, so every A read is one conflict-free
// ds_read_b128 of a contiguous kilobyte. The lines are filled by
// buffer_load_dwordx4 ... lds, whose 64 lanes write 64 consecutive 16-byte
// slots: each lane simply loads the piece its slot needs. Rows past M and
// inputs past K fall outside the buffer's range and read as zero. Stages are
// double buffered with one barrier per stage.
#include "mnb_internal.h"

namespace mnb {

typedef __attribute__((address_space(3))) void lds_void;

template <int MF, int NF, int WM, int WN>
struct GemmCfg {
    static constexpr int kMT = WM * MF * 16;
    static constexpr int kNT = WN * NF * 16;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kLines = WM * MF * 2;                       // 1 KB lines per stage
    static constexpr int kLinesPerWave = (kLines + kWaves - 1) / kWaves;
    static constexpr int kStageBytes = kLines * 1024;
    // as many stage buffers as fit in the CU's 160 KB (at most 3)
    static constexpr int kBufs = 3 * kStageBytes <= 160 * 1024 ? 3 : 2;
};

constexpr uint32_t kOob = 0x7FFFFFF0u;  // a buffer offset past any range we build

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2. Renumbering so that XCD x runs a contiguous
// range of logical workgroups puts all N-tiles of one product - which read
// the same activation rows - on one XCD, where they share its L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_logical_wg(int64_t b, int64_t n) {
    const int64_t q = n / kXcds, rem = n % kXcds;
    const int64_t x = b % kXcds, i = b / kXcds;
    return x * q + (x < rem ? x : rem) + i;
}

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int NF>
struct BRaw {
    u32x4 codes[NF];
    u32x4 smeta[NF];    // float16 scales of 8 consecutive tiles
    uint32_t zmeta[NF]; // zero points of the same 8 tiles
};

template <int MF, int NF, int WM, int WN>
__device__ __forceinline__ void gemm_workgroup(const Problem &p, int64_t wg, uint8_t *lds) {
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

    // ---- activation lines: this wave fills lines wave, wave + kWaves, ... --
    const int64_t rows_here = (p.m - m0) < C::kMT ? (p.m - m0) : C::kMT;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(static_cast<const _Float16 *>(p.x) + m0 * p.k), 0,
        (int)(rows_here * p.k * 2), 0x00020000);
    uint32_t voff[C::kLinesPerWave];
#pragma unroll
    for (int i = 0; i < C::kLinesPerWave; ++i) {
        const int L = wave + i * C::kWaves;
        const int a = L >> 1, tt = L & 1;
        voff[i] = (uint32_t)(((a * 16 + r) * p.k + j * kChunk + tt * 8) * 2);
    }
    const bool k_tail = (p.k % kTileK) != 0;
    auto issue_a = [&](int64_t stage) {
        const int64_t c = stage >> 1;
        const int h = (int)(stage & 1);
        const uint32_t soff = (uint32_t)((c * kTileK + h * 16) * 2);
        uint8_t *buf = lds + (int)(stage % C::kBufs) * C::kStageBytes;
        const bool last = k_tail && c == p.kg - 1;
#pragma unroll
        for (int i = 0; i < C::kLinesPerWave; ++i) {
            const int L = wave + i * C::kWaves;
            if (L < C::kLines) {
                uint32_t vo = voff[i];
                if (last && c * kTileK + j * kChunk + (2 * h + (L & 1)) * 8 >= p.k) vo = kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(buf + L * 1024), 16, vo, soff, 0, 0);
            }
        }
    };

    // ---- weight tiles -------------------------------------------------------
    auto load_b = [&](int64_t c, BRaw<NF> &R) {
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const int64_t g = g0 + wn * NF + b;
            if (g < p.rg) {
                R.codes[b] = *(reinterpret_cast<const u32x4 *>(p.packed + (g * p.kg + c) * kTileCodeBytes) + lane);
                if ((c & (kMetaGroup - 1)) == 0) {
                    const int64_t mi = meta_index(g, p.nbt, p.kgp, e, c);
                    R.smeta[b] = *reinterpret_cast<const u32x4 *>(p.packed + p.scales_off + mi * 2);
                    R.zmeta[b] = *reinterpret_cast<const uint32_t *>(p.packed + p.zp_off + (mi >> 1));
                }
            } else {
                R.codes[b] = u32x4{0u, 0u, 0u, 0u};
                R.smeta[b] = u32x4{0u, 0u, 0u, 0u};
                R.zmeta[b] = 0u;
            }
        }
    };
    // dequantize MFMA operands t = 2h, 2h+1 of tile c into out[b][0..1]
    auto dequant_half = [&](int64_t c, int h, const BRaw<NF> &R, h8 (&out)[NF][2]) {
        const int u = (int)(c & (kMetaGroup - 1));
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const u32x4 sm = R.smeta[b];
            const uint32_t sw = sm[u >> 1];
            const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(sw >> (16 * (u & 1))));
            const h2 zm = zp_magic((R.zmeta[b] >> (4 * u)) & 15u);
            const h2 s2 = {s, s};
            const u32x4 w = R.codes[b];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint32_t word = w[2 * h + tt];
                h8 v;
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const h2 d = dequant_pair_f16(word, hh, zm, s2);
                    v[2 * hh] = d.x;
                    v[2 * hh + 1] = d.y;
                }
                out[b][tt] = v;
            }
        }
    };

    f4 acc[MF][NF];
#pragma unroll
    for (int a = 0; a < MF; ++a)
#pragma unroll
        for (int b = 0; b < NF; ++b) acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    auto mfma_stage = [&](int64_t stage, const h8 (&bw)[NF][2]) {
        const uint8_t *As = lds + (int)(stage % C::kBufs) * C::kStageBytes + (wm * MF * 2) * 1024 + lane * 16;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int a = 0; a < MF; ++a) {
                const h8 av = *reinterpret_cast<const h8 *>(As + (a * 2 + tt) * 1024);
#pragma unroll
                for (int b = 0; b < NF; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bw[b][tt], acc[a][b], 0, 0, 0);
            }
        }
    };
    // end of a stage: the next stage's lines (issued one stage earlier) must
    // be in LDS for every wave; the lines two stages ahead may stay in flight
    auto stage_sync = [&](int64_t stage, int64_t n_stages) {
        if (C::kBufs == 3 && stage + 2 < n_stages) wait_vmem<C::kLinesPerWave>();
        else wait_vmem<0>();
        __syncthreads();
    };

    const int64_t n_stages = 2 * p.kg;
    BRaw<NF> rc, rn;   // raw weights of the current and the next tile
    h8 bw0[NF][2], bw1[NF][2];
    load_b(0, rc);
    issue_a(0);
    if (C::kBufs == 3 && n_stages > 1) issue_a(1);
    dequant_half(0, 0, rc, bw0);
    if (C::kBufs == 3 && n_stages > 1) wait_vmem<C::kLinesPerWave>();
    else wait_vmem<0>();
    __syncthreads();

    for (int64_t c = 0; c < p.kg; ++c) {
        // stage 2c: MFMAs on bw0 (t = 0, 1); meanwhile prepare t = 2, 3
        {
            const int64_t s = 2 * c;
            // weights first: at the stage end everything issued before the
            // lines two stages ahead must have landed
            if (c + 1 < p.kg) {
                rn = rc;  // keep the metadata group unless a new one is loaded
                load_b(c + 1, rn);
            }
            if (C::kBufs == 3) {
                if (s + 2 < n_stages) issue_a(s + 2);
            } else {
                issue_a(s + 1);
            }
            mfma_stage(s, bw0);
            dequant_half(c, 1, rc, bw1);
            stage_sync(s, n_stages);
        }
        // stage 2c+1: MFMAs on bw1 (t = 2, 3); meanwhile prepare tile c+1
        {
            const int64_t s = 2 * c + 1;
            if (C::kBufs == 3) {
                if (s + 2 < n_stages) issue_a(s + 2);
            } else if (s + 1 < n_stages) {
                issue_a(s + 1);
            }
            mfma_stage(s, bw1);
            if (c + 1 < p.kg) {
                dequant_half(c + 1, 0, rn, bw0);
                rc = rn;
            }
            stage_sync(s, n_stages);
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
    __shared__ __align__(1024) uint8_t lds[GemmCfg<MF, NF, WM, WN>::kBufs * GemmCfg<MF, NF, WM, WN>::kStageBytes];
    gemm_workgroup<MF, NF, WM, WN>(p, xcd_logical_wg(blockIdx.x, gridDim.x), lds);
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
    __shared__ __align__(1024) uint8_t lds[GemmCfg<MF, NF, WM, WN>::kBufs * GemmCfg<MF, NF, WM, WN>::kStageBytes];
    const int64_t wg = xcd_logical_wg(blockIdx.x, gridDim.x);
    const int i = find_gemm_problem(entries, count, wg);
    const Problem p = entries[i];
    gemm_workgroup<MF, NF, WM, WN>(p, wg - p.wg_begin, lds);
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

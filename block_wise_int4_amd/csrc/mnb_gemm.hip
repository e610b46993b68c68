// Prefill kernel (float16, M >= 2): int4 weight tiles dequantized in
// registers feed v_mfma_f32_16x16x32_f16; activations reach LDS by direct
// buffer-to-LDS loads.
//
// Workgroup = WM x WN waves; wave (wm, wn) computes an (MF * 16) x (NF * 16)
// block of Y, so the workgroup tile is (WM * MF * 16) x (WN * NF * 16). The
// large-M tiles are 208 (or 192) rows by 256 columns, 8 waves of 208 x 32:
// the accumulators (104 registers) leave room for two waves per SIMD, so one
// wave's MFMAs overlap the other's loads and dequantization. Up to 64 rows
// the tiles are 16, 32 or 64 rows by 256 columns, 4 waves of 64 columns
// each: every wave reads all of the workgroup's activation rows from LDS,
// so wide waves halve that traffic per weight and halve the number of
// workgroups (each of which pays a prologue of roughly one memory latency).
//
// Weight side: a wave owns NF 16-row groups of W (= NF 16-column fragments
// of Y). For each 128-input tile it issues one coalesced 128-bit load per
// lane and fragment (lane l holds row l & 15, chunk l >> 4: 32 codes). The
// scales and zero points of its row groups reach LDS once per 8 tiles by
// direct buffer-to-LDS loads (one contiguous span per row group and tile
// group), and each tile's values are read from there. MFMA k-slice t
// (t = 0..3) uses inputs t*8 .. t*8+7 of the lane's chunk: the lane turns
// that word into exact (q - zp) float16 pairs with the 1024- and 64-offset
// tricks and multiplies them by the scale with one rounding, in the shared
// helper dequant_pair_f16 that mnb_dequant also runs, so the MFMA operands
// are exactly the dequantized weights mnb_dequant returns. The sum over K does not
// care which inputs an MFMA groups together as long as A and B agree, so A
// is laid out with the same grouping and no lane shuffles are needed on
// either side. Two operand slots alternate: slice t is multiplied from one
// while slice t + 1 is dequantized into the other.
//
// Instruction order. A stage runs as one fixed sequence (pinned with
// scheduling barriers): each step issues a fragment's MFMAs, the LDS read of
// the fragment kPipe steps later into a small register ring, and one or two
// float16 pairs of the next slice's weights. The compiler's own order, under
// this kernel's register pressure, left each read one step ahead and waited
// for every read. A wave's issue priority is raised while it runs a stage and
// lowered at the stage barrier, so that a workgroup in its start or end does
// not take issue slots from one in its K-loop.
//
// Activation side: an LDS stage holds one whole 128-input tile of the
// workgroup's rows. A stage is a list of 1 KB lines, one per (16-row
// fragment, slice): byte 16*l of a line holds the 8 inputs lane l passes to
// that MFMA, so every A read is one conflict-free ds_read_b128 of a
// contiguous kilobyte. The lines are filled by buffer_load_dwordx4 ... lds,
// whose 64 lanes write 64 consecutive 16-byte slots: each lane loads the
// piece its slot needs; the lines of the stage ahead are issued one per step
// from inside the current stage's MFMA steps.
// Rows past M and inputs past K fall outside the buffer's range and read as
// zero. Two stage buffers (three where they fit) let the loads run one
// stage (two) ahead, with one barrier per stage.
//
// Epilogue: the weight fragment is each MFMA's first operand and the
// activation fragment its second, so a fragment's accumulators are a block
// of Y transposed: a lane holds four consecutive columns of one row. Each
// wave rounds them to float16, writes them to its own LDS area as 8-byte
// pieces (rows padded by 16 bytes) and writes Y back as 16-byte row pieces,
// 64 contiguous bytes per row and store instruction. (Storing the 8-byte
// pieces straight from registers leaves 32-byte row segments per store and
// measured 4-10% slower.)
#include <algorithm>
#include <type_traits>
#include <vector>

#include "mnb_internal.h"

namespace mnb {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPipe = 5;  // A-fragment reads kept in flight ahead of the MFMAs that use them

template <int MF, int NF, int WM, int WN, int MaxBufs>
struct GemmCfg {
    static constexpr int kMT = WM * MF * 16;
    static constexpr int kNT = WN * NF * 16;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kSlices = 4;  // MFMA k-slices (8 inputs per lane) per stage: a whole 128-input tile
    static constexpr int kLines = WM * MF * kSlices;  // 1 KB lines per stage
    static constexpr int kLinesPerWave = (kLines + kWaves - 1) / kWaves;
    // every wave issues kLinesPerWave lines; those past kLines load zeros
    // into padding, so that each wave's count of loads in flight is fixed
    static constexpr int kStageBytes = kLinesPerWave * kWaves * 1024;
    // per wave, two tile groups' metadata of its NF row groups: float16
    // scales (up to 64 entries x 8 tiles = 1 KB) and zero points (256 B)
    static constexpr int kMetaScaleBytes = 1024, kMetaZpBytes = 256;
    static constexpr int kMetaBytes = kWaves * 2 * NF * (kMetaScaleBytes + kMetaZpBytes);
    // as many stage buffers as fit in the CU's 160 KB next to the metadata
    // (at most MaxBufs: 2 or 3)
    static constexpr int kBufs = MaxBufs >= 3 && 3 * kStageBytes + kMetaBytes <= 160 * 1024 ? 3 : 2;
    // a stage's steps 1, 2, ... issue the lines of the stage ahead, one each
    static_assert(kLinesPerWave < kSlices * MF || kSlices * MF == 1, "a step for every line");
    static constexpr int kMetaOff = kBufs * kStageBytes;
    // epilogue staging: each wave's (MF * 16) x (NF * 16) float16 block
    static constexpr int kOutStride = NF * 32 + 16;
    static constexpr int kOutWaveBytes = MF * 16 * kOutStride;
    static constexpr int kLdsBytes = kMetaOff + kMetaBytes > kWaves * kOutWaveBytes ? kMetaOff + kMetaBytes
                                                                                     : kWaves * kOutWaveBytes;
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

constexpr uint32_t kOob = 0x7FFFFFF0u;  // a buffer offset past any range we build

// A value made wave-uniform (kept in a scalar register, so branches on it
// stay scalar branches).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_readfirstlane(v);
#else
    return v;
#endif
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2. Renumbering so that XCD x runs a contiguous
// range of logical workgroups puts all N-tiles of one product - which read
// the same activation rows - on one XCD, where they share its L2.
constexpr int kXcds = kXcdCount;
__device__ __forceinline__ int64_t xcd_logical_wg(int64_t b, int64_t n) {
    const int64_t q = n / kXcds, rem = n % kXcds;
    const int64_t x = b % kXcds, i = b / kXcds;
    return x * q + (x < rem ? x : rem) + i;
}

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#endif
}

// Where a stage's activation lines go and how many of its inputs lie before K.
struct LineDst {
    uint8_t *buf;
    uint32_t soff;  // byte offset of the stage's first input in a row
    int32_t lim;    // K minus the stage's first input (large when no tail)
};

template <int NF>
struct BRaw {
    u32x4 codes[NF];
    uint32_t s[NF];  // float16 scale bits of the lane's block
    uint32_t z[NF];  // the byte holding its zero point
    uint32_t zsh;    // the zero point's shift in that byte (0 or 4; the same for every lane)
    __device__ __forceinline__ uint32_t zp(int b) const { return (z[b] >> zsh) & 15u; }
};

template <int MF, int NF, int WM, int WN, int MaxBufs, bool kSplit>
__device__ __forceinline__ void gemm_workgroup(const Problem &p, int64_t wg_, uint8_t *lds) {
    using C = GemmCfg<MF, NF, WM, WN, MaxBufs>;
    // split K (kSplit): workgroup = (part, output tile); part q covers
    // K-tiles [q * kg / S, (q + 1) * kg / S) and writes float32 partial sums
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int64_t S = kSplit ? p.ksplit : 1;
    const int64_t part = kSplit ? wg_ / tiles : 0;
    const int64_t wg = kSplit ? wg_ - part * tiles : wg_;
    const int64_t c_begin = kSplit ? part * p.kg / S : 0;
    const int64_t c_end = kSplit ? (part + 1) * p.kg / S : p.kg;
    // inputs of this part end at k_end; it reads metadata groups below g_end
    const int64_t k_end = kSplit && c_end * kTileK < p.k ? c_end * kTileK : p.k;
    const int64_t g_end = (c_end + kMetaGroup - 1) / kMetaGroup;
    const int64_t tn = wg % p.tiles_n;
    const int64_t tm = wg / p.tiles_n;
    const int64_t m0 = tm * C::kMT;
    const int64_t g0 = tn * (WN * NF);
    const int tid = threadIdx.x;
    const int wave = (int)uniform_u32((uint32_t)tid >> 6);
    const int lane = tid & 63;
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
        const int a = L / C::kSlices, tt = L % C::kSlices;
        voff[i] = (uint32_t)(((a * 16 + r) * p.k + j * kChunk + tt * 8) * 2);
    }
    // A line piece starting at input (stage's first) + j * 32 + slice * 8
    // reads zeros when that input is at or past K (only in the last K-tile).
    const int jk = j * kChunk;
    auto line_dst = [&](int64_t stage) {  // stage = K-tile
        const int64_t first = stage * kTileK;
        const int64_t left = k_end - first;
        return LineDst{lds + (int)((uint32_t)stage % (uint32_t)C::kBufs) * C::kStageBytes, (uint32_t)(first * 2),
                       (int32_t)(left < kTileK ? left : 0x40000000)};
    };
    auto issue_line = [&](const LineDst &d, int i) {
        const int L = wave + i * C::kWaves;
        const uint32_t vo = L >= C::kLines || jk >= d.lim - (L % C::kSlices) * 8 ? kOob : voff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(d.buf + L * 1024), 16, vo, d.soff, 0, 0);
    };
    auto issue_a = [&](int64_t stage) {
        const LineDst d = line_dst(stage);
#pragma unroll
        for (int i = 0; i < C::kLinesPerWave; ++i) issue_line(d, i);
    };

    // ---- weight metadata: tile group G of this wave's row groups -> LDS ----
    const int E = p.nbt * kTileRows;  // metadata entries per tile
    uint8_t *meta_lds = lds + C::kMetaOff + wave * (2 * NF * (C::kMetaScaleBytes + C::kMetaZpBytes));
    auto meta_s = [&](int slot, int b) { return meta_lds + (slot * NF + b) * C::kMetaScaleBytes; };
    auto meta_z = [&](int slot, int b) {
        return meta_lds + 2 * NF * C::kMetaScaleBytes + (slot * NF + b) * C::kMetaZpBytes;
    };
    auto issue_meta = [&](int64_t G) {
        const int slot = (int)(G & 1);
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const int64_t g = g0 + wn * NF + b;
            const bool in = g < p.rg;
            const int64_t mi = meta_index(in ? g : 0, p.nbt, p.kgp, 0, G * kMetaGroup);
            const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(p.packed + p.scales_off + mi * 2), 0, in ? E * kMetaGroup * 2 : 0, 0x00020000);
            const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(p.packed + p.zp_off + mi / 2), 0, in ? E * kMetaGroup / 2 : 0, 0x00020000);
            const uint32_t so = (uint32_t)lane * 16u, zo = (uint32_t)lane * 4u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void *)meta_s(slot, b), 16, so, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(zr, (lds_void *)meta_z(slot, b), 4, zo, 0, 0, 0);
        }
    };

    // ---- weight tiles -------------------------------------------------------
    // (a row group past N has an empty range: its codes read as zero)
    __amdgpu_buffer_rsrc_t code_rsrc[NF];
#pragma unroll
    for (int b = 0; b < NF; ++b) {
        const int64_t g = g0 + wn * NF + b;
        const bool in = g < p.rg;
        code_rsrc[b] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(p.packed + (in ? g : 0) * p.kg * kTileCodeBytes), 0,
            in ? (int)(p.kg * kTileCodeBytes) : 0, 0x00020000);
    }
    auto load_codes = [&](int64_t c, BRaw<NF> &R) {
#pragma unroll
        for (int b = 0; b < NF; ++b)
            R.codes[b] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc[b], (int)(c * kTileCodeBytes) + lane * 16, 0, 0));
    };
    // (the nibble is taken out where it is used, so that nothing waits for
    // these reads until then)
    auto read_meta = [&](int64_t c, BRaw<NF> &R) {
        const int slot = (int)((c / kMetaGroup) & 1), u = (int)(c % kMetaGroup);
        R.zsh = 4u * (uint32_t)(u & 1);
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const bool in = g0 + wn * NF + b < p.rg;
            const uint32_t sv = *reinterpret_cast<const uint16_t *>(meta_s(slot, b) + e * 16 + u * 2);
            const uint32_t zv = meta_z(slot, b)[e * 4 + (u >> 1)];
            R.s[b] = in ? sv : 0u;
            R.z[b] = in ? zv : 0u;
        }
    };
    f4 acc[MF][NF];
#pragma unroll
    for (int a = 0; a < MF; ++a)
#pragma unroll
        for (int b = 0; b < NF; ++b) acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t n_stages = c_end - c_begin;
    // the next stage's lines must have landed; those two stages ahead may
    // still be in flight (each wave waits for its own loads, then the barrier)
    auto stage_sync = [&](int64_t stage) {
        if (C::kBufs == 3 && stage + 2 < c_end) {
            wait_vmem<C::kLinesPerWave>();
        } else {
            wait_vmem<0>();
        }
        __syncthreads();
    };

    // Tile c: slices 0..3 in one stage. Weights of tile c + 1 are loaded
    // first, so that at the stage end only the newest lines may be pending.
    // A stage runs in a fixed order: its A fragments (slice by slice)
    // stream through a ring of kPipe registers, each read
    // issued that many MFMA groups before its use, and each step forms one
    // float16 pair of the next slice's B operands into the free slot (slice t
    // multiplies from slot t & 1).
    h8 s0[NF], s1[NF];
    // B operands: float16 pairs in the shared dequant pair form, whose masks
    // and offsets are held in registers (literal constants cannot go into
    // the three-operand form), so that masking a pair and adding the offset
    // is one v_and_or_b32.
    PairForm pf = pair_form_literal();
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(pf.mask_lo));
    asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(pf.mask_hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(pf.magic_lo));
    asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(pf.magic_hi));
#endif
    auto put_pair = [&](const BRaw<NF> &R, int t, int b, int hh, h8 &dst) {
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)R.s[b]);
        const h2 s2 = {s, s};
        const h2 d = dequant_pair_f16(R.codes[b][t], hh, R.zp(b), s2, pf);
        dst[2 * hh] = d.x;
        dst[2 * hh + 1] = d.y;
    };
    // B operands of slice t (inputs t*8 .. t*8+7 of the lane's chunk)
    auto dequant_t = [&](const BRaw<NF> &R, int t, h8 (&out)[NF]) {
#pragma unroll
        for (int b = 0; b < NF; ++b)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) put_pair(R, t, b, hh, out[b]);
    };
    // Stage `stage` (K-tile `stage`, slices 0..3): each step forms one pair
    // of the next slice's B operands, from Rc, or from Rn (the next tile's
    // slice 0) after the tile's last slice.
    auto run_stage = [&](int64_t stage, const BRaw<NF> &Rc, const BRaw<NF> &Rn, auto &&step_hook) {
        constexpr int S = C::kSlices;
        constexpr int R = kPipe < S * MF ? kPipe : S * MF;
        constexpr int kPieces = NF * 4;
        const uint8_t *base = lds + (int)((uint32_t)stage % (uint32_t)C::kBufs) * C::kStageBytes +
                              (wm * MF * S) * 1024 + lane * 16;
        auto frag = [&](int q) { return *reinterpret_cast<const h8 *>(base + ((q % MF) * S + q / MF) * 1024); };
        auto piece = [&](int t, int k) {  // pair k of slice t + 1's operands
            h8 &dst = ((t + 1) & 1) ? s1[k / 4] : s0[k / 4];
            if (t + 1 < 4) put_pair(Rc, t + 1, k / 4, k % 4, dst);
            else put_pair(Rn, 0, k / 4, k % 4, dst);
        };
        h8 ring[R];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < R; ++i) ring[i] = frag(i);
#pragma unroll
        for (int q = 0; q < S * MF; ++q) {
            const int t = q / MF, a = q % MF;
            const h8 av = ring[q % R];
#pragma unroll
            for (int b = 0; b < NF; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16((t & 1) ? s1[b] : s0[b], av, acc[a][b], 0, 0, 0);
            if (q + R < S * MF) ring[q % R] = frag(q + R);
            step_hook(q);
            // pairs per step: 2 for the small-M tiles (16 pairs per slice
            // over 1-4 steps), 1 for the tall ones (8 pairs over 12-13 steps)
            constexpr int P = NF >= 4 ? 2 : 1;
#pragma unroll
            for (int u = 0; u < P; ++u)
                if (a * P + u < kPieces) piece(t, a * P + u);
            if (a == MF - 1) {  // pieces the slice had no step left for
#pragma unroll
                for (int k = MF * P; k < kPieces; ++k) piece(t, k);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // Each stage's steps 1, 2, ... issue one activation line each of the
    // stage ahead, where the MFMAs around them cover their issue. Every wave
    // issues the same loads in every tile (past the last stage the lines
    // read zeros into the free buffer), so the compiler's count of the loads
    // in flight is exact wherever it waits for the next tile's codes and
    // never falls back to waiting for all of them.
    // (after the last K-tile Rn holds no weights; its slice is formed and never used)
    auto tile = [&](int64_t c, const BRaw<NF> &Rc, BRaw<NF> &Rn) {
        const int64_t st = c;
        if (c % kMetaGroup == 0 && c / kMetaGroup + 1 < g_end) issue_meta(c / kMetaGroup + 1);
        if (c + 1 < c_end) {
            load_codes(c + 1, Rn);
            read_meta(c + 1, Rn);
        }
        const LineDst d = line_dst(st + (C::kBufs == 3 ? 2 : 1));
        run_stage(st, Rc, Rn, [&](int q) {
            if (q >= 1 && q <= C::kLinesPerWave) issue_line(d, q - 1);
        });
        stage_sync(st);
    };

    BRaw<NF> R0, R1;
#pragma unroll
    for (int b = 0; b < NF; ++b) {
        R1.codes[b] = u32x4{0u, 0u, 0u, 0u};
        R1.s[b] = 0u;
        R1.z[b] = 0u;
    }
    R1.zsh = 0u;
    // metadata, codes and lines of the first K-tile all in flight at once;
    // the metadata is issued first (pinned by a scheduling barrier), since
    // the wait below counts the loads issued after it
    // (a part that starts inside a metadata group also needs the next group
    // before its first group boundary, where the loop issues the one after)
    const bool two = C::kBufs == 3 && n_stages > 1;
    issue_meta(c_begin / kMetaGroup);
    if (c_begin % kMetaGroup != 0 && c_begin / kMetaGroup + 1 < g_end) issue_meta(c_begin / kMetaGroup + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(c_begin, R0);
    issue_a(c_begin);
    if (two) issue_a(c_begin + 1);
    // tile group 0's metadata has landed once at most the codes and the
    // lines are pending
    if (two) wait_vmem<NF + 2 * C::kLinesPerWave>();
    else wait_vmem<NF + C::kLinesPerWave>();
    read_meta(c_begin, R0);
    dequant_t(R0, 0, s0);
    if (two) {
        wait_vmem<C::kLinesPerWave>();
    } else {
        wait_vmem<0>();
    }
    __syncthreads();

    int64_t c = c_begin;
    for (; c + 2 <= c_end; c += 2) {
        tile(c, R0, R1);
        tile(c + 1, R1, R0);
    }
    if (c < c_end) tile(c, R0, R1);

    // ---- epilogue: lane holds row r, columns 4 j .. 4 j + 3 of each fragment
    // (every wave is past the last barrier, so the stage buffers and the
    // metadata area are free)
    _Float16 *y = static_cast<_Float16 *>(p.y);
    const int64_t n_base = (g0 + wn * NF) * kTileRows;
    const int64_t m_base = m0 + wm * MF * 16;
    if (kSplit) {  // float32 partial sums of this K part; a second launch adds the parts
        float *dst = p.part + part * p.m * p.n;
#pragma unroll
        for (int a = 0; a < MF; ++a) {
            const int64_t m = m_base + a * 16 + r;
            if (m >= p.m) continue;
#pragma unroll
            for (int b = 0; b < NF; ++b) {
                const int64_t n = n_base + b * kTileRows + 4 * j;
                if (p.n % 4 == 0) {
                    if (n < p.n) *reinterpret_cast<f4 *>(dst + m * p.n + n) = acc[a][b];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n + i < p.n) dst[m * p.n + n + i] = acc[a][b][i];
                }
            }
        }
        return;
    }
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    if (p.n % 8 == 0) {
        uint8_t *ob = lds + wave * C::kOutWaveBytes;
#pragma unroll
        for (int a = 0; a < MF; ++a)
#pragma unroll
            for (int b = 0; b < NF; ++b)
                *reinterpret_cast<h4 *>(ob + (a * 16 + r) * C::kOutStride + (b * 16 + 4 * j) * 2) =
                    h4{(_Float16)acc[a][b][0], (_Float16)acc[a][b][1], (_Float16)acc[a][b][2], (_Float16)acc[a][b][3]};
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // 16-byte pieces: row q / (2 NF), columns (q % (2 NF)) * 8 .. + 7
        constexpr int kPieces = MF * 16 * NF * 2;
#pragma unroll
        for (int q0 = 0; q0 < kPieces; q0 += 64) {
            const int q = q0 + lane;
            if (kPieces % 64 == 0 || q < kPieces) {
                const int row = q / (NF * 2), piece = q % (NF * 2);
                const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + row * C::kOutStride + piece * 16);
                const int64_t m = m_base + row, n = n_base + piece * 8;
                if (m < p.m && n < p.n) *reinterpret_cast<u32x4 *>(y + m * p.n + n) = v;
            }
        }
        return;
    }
#pragma unroll
    for (int a = 0; a < MF; ++a) {
        const int64_t m = m_base + a * 16 + r;
        if (m >= p.m) continue;
#pragma unroll
        for (int b = 0; b < NF; ++b) {
            const int64_t n = n_base + b * kTileRows + 4 * j;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < p.n) y[m * p.n + n + i] = (_Float16)acc[a][b][i];
        }
    }
}

template <int MF, int NF, int WM, int WN, int MaxBufs, bool kSplit>
__global__ __launch_bounds__(64 * WM *WN) void gemm_kernel(Problem p) {
    __shared__ __align__(1024) uint8_t lds[GemmCfg<MF, NF, WM, WN, MaxBufs>::kLdsBytes];
    gemm_workgroup<MF, NF, WM, WN, MaxBufs, kSplit>(p, xcd_logical_wg(blockIdx.x, gridDim.x), lds);
}

// The product of entries[first, last) (tiles in increasing wg_begin order)
// that holds tile wg: each lane reads one product's first tile, so a range
// of up to 64 products costs one round trip, and a ballot counts the
// products that start at or before wg. Wave-uniform; all 64 lanes active.
__device__ __forceinline__ int find_gemm_problem(const Problem *entries, int first, int last, int64_t wg) {
    const int lane = (int)(threadIdx.x & 63);
    int found = first;
    for (int base = first; base < last; base += 64) {
        const int q = base + lane;
        const int64_t wb = q < last ? entries[q].wg_begin : INT64_MAX;
        const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(wb <= wg));
        if (k == 0) break;
        found = base + k - 1;
        if (k < 64) break;
    }
    return found;
}

// Grouped launches: XCD x (blocks b with b % 8 == x) runs its own tile range
// (products and runs of a product's tiles, balanced by work on the host,
// longest K first); blocks past the end of their XCD's range exit at once.
template <int MF, int NF, int WM, int WN, int MaxBufs>
__global__ __launch_bounds__(64 * WM *WN) void gemm_grouped_kernel(const Problem *entries, int count,
                                                                   XcdSplit split) {
    __shared__ __align__(1024) uint8_t lds[GemmCfg<MF, NF, WM, WN, MaxBufs>::kLdsBytes];
    const int x = (int)(blockIdx.x % kXcds);
    const int64_t wg = split.begin[x] + (int64_t)(blockIdx.x / kXcds);
    if (wg >= split.begin[x + 1]) return;
    const int i = find_gemm_problem(entries, split.first[x], split.first[x + 1], wg);
    const Problem p = entries[i];
    gemm_workgroup<MF, NF, WM, WN, MaxBufs, false>(p, wg - p.wg_begin + p.tile_off, lds);
}

// Split-K: y = float16(part[0] + part[1] + ... + part[S - 1]), the parts
// added in that fixed order, 4 outputs per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int S, int64_t mn,
                                                            _Float16 *__restrict__ y) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    if (mn % 4 == 0) {
        float4 v = *reinterpret_cast<const float4 *>(part + i);
        for (int s = 1; s < S; ++s) {
            const float4 w = *reinterpret_cast<const float4 *>(part + s * mn + i);
            v.x += w.x;
            v.y += w.y;
            v.z += w.z;
            v.w += w.w;
        }
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<h4 *>(y + i) = h4{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        return;
    }
    for (int64_t q = i; q < i + 4 && q < mn; ++q) {
        float v = part[q];
        for (int s = 1; s < S; ++s) v += part[s * mn + q];
        y[q] = (_Float16)v;
    }
}

// ---------------------------------------------------------------------------
// Variants and their selection.
// ---------------------------------------------------------------------------
struct VariantInfo {
    int mt, nt;
};
static const VariantInfo kVariants[] = {
    {16, 256},                // 0: MF 1,  NF 4, 1x4 waves
    {32, 256},                // 1: MF 2,  NF 4, 1x4 waves
    {64, 256},                // 2: MF 4,  NF 4, 1x4 waves
    {208, 256},               // 3: MF 13, NF 2, 1x8 waves
    {192, 256},               // 4: MF 12, NF 2, 1x8 waves
};
constexpr int kNumVariants = 5;

int gemm_variant(int64_t m) {
    if (m <= 16) return 0;
    if (m <= 32) return 1;
    if (m <= 64) return 2;
    // the tall tile that pads M with fewer rows (the 208-row one on a tie)
    int best = 3;
    int64_t best_rows = -1;
    for (int v = 3; v < kNumVariants; ++v) {
        const int64_t mt = kVariants[v].mt;
        const int64_t rows = (m + mt - 1) / mt * mt;
        if (best_rows < 0 || rows < best_rows) {
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

// (variant, MF, NF, WM, WN, stage buffers at most)
#define MNB_GEMM_VARIANTS(X) \
    X(0, 1, 4, 1, 4, 3)      \
    X(1, 2, 4, 1, 4, 3)      \
    X(2, 4, 4, 1, 4, 2)      \
    X(3, 13, 2, 1, 8, 3)                              \
    X(4, 12, 2, 1, 8, 3)

// Workgroups one CU holds at once, per variant (LDS-bound).
static int wgs_per_cu(int variant) { return variant <= 2 ? 2 : 1; }
constexpr int kCus = 256;

// Estimated time (microseconds) of one product on its own at tile variant
// v, split S ways, from a cost model fitted to single-product timings on
// MI355X: a workgroup takes (its K-tiles + 2) steps (its start and end cost
// about two K-tiles); a step takes t0 with the chip lightly loaded (0.95,
// 1.05 and 1.2 us for the 16-, 32- and 64-row tiles, 2.0 us for the tall
// ones) and (1 + a) t0 with every workgroup slot busy (a = 1.0, 1.25, 1.1
// and 0.45, from the grouped launches, whose slots are all busy), in
// between in proportion to the slots in use; workgroups beyond one round of
// slots run in further rounds; and a split adds its float32 partial sums
// (written once, read once) at about 6 TB/s plus about 6 us for the
// partial-sum epilogue and the second launch (the adding kernel alone takes
// 3 to 4 us).
static double gemm_single_us(const Problem &p, int variant, int64_t s) {
    static const double kT0[kNumVariants] = {0.95, 1.05, 1.2, 2.0, 2.0};
    static const double kFull[kNumVariants] = {1.0, 1.25, 1.1, 0.45, 0.45};
    const double t0 = kT0[variant], a = kFull[variant];
    int32_t tm = 0, tn = 0;
    gemm_tiles(p, variant, &tm, &tn);
    const int64_t wgs = (int64_t)tm * tn * s;
    const int64_t slots = (int64_t)kCus * wgs_per_cu(variant);
    const int64_t rounds = (wgs + slots - 1) / slots;
    const double fill = wgs < slots ? (double)wgs / (double)slots : 1.0;
    const int64_t steps = (p.kg + s - 1) / s + 2;
    double t = (double)rounds * (double)steps * t0 * (1.0 + a * fill);
    if (s > 1) t += (2.0 * (double)s + 0.5) * (double)p.m * (double)p.n * 4.0 / 6.0e6 + 6.0;
    return t;
}

// A single product's tile variant and K split (1 = none) by the model
// above. The candidates are the grouped launches' tile for M's row count
// and shorter ones whose extra workgroups fill more of the chip when one
// product runs alone: past 64 rows the 64-row tile (measured per call at
// M = 410 and M = 1500: 16-34% faster than the tall tiles for every
// Qwen3-1.7B and Whisper-small linear, split or not), up to 64 rows the
// 32- and 16-row tiles (at M = 62 the 16-row tile was 15-20% faster than
// the 64-row one for every Qwen3-0.6B linear). With `max_split` 1 nothing
// is split; with `force_split` the split is that (capped at the product's
// K-tiles). A larger split must be 3% better, and so must a shorter tile.
GemmChoice gemm_single_choice(const Problem &p, int max_split, int force_split) {
    const int tall = gemm_variant(p.m);
    int cands[3] = {tall, 2, 2};
    int nc = 1;
    if (p.m > 64) {
        nc = 2;
    } else {
        for (int v = tall - 1; v >= 0; --v) cands[nc++] = v;
    }
    GemmChoice best{tall, 1};
    double best_t = 0.0;
    for (int c = 0; c < nc; ++c) {
        const int v = cands[c];
        int64_t lo = 1, hi = max_split < p.kg ? max_split : p.kg;
        if (force_split > 0) lo = hi = force_split < p.kg ? force_split : p.kg;
        if (hi < 1) lo = hi = 1;
        double vt = 0.0;
        int64_t vs = lo;
        int32_t tm = 0, tn = 0;
        gemm_tiles(p, v, &tm, &tn);
        if ((int64_t)tm * tn * hi > 0x7FFFFFFFLL) continue;  // past a launch's grid
        for (int64_t s = lo; s <= hi; ++s) {
            const double t = gemm_single_us(p, v, s);
            if (s == lo || t < 0.97 * vt) {
                vt = t;
                vs = s;
            }
        }
        if (best_t == 0.0 || vt < 0.97 * best_t) {
            best_t = vt;
            best = GemmChoice{v, (int)vs};
        }
    }
    return best;
}

int64_t gemm_part_bytes(const Problem &p, int ksplit) {
    return ksplit > 1 ? align_up((int64_t)ksplit * p.m * p.n * 4, kAlign) : 0;
}

hipError_t launch_gemm(const Problem &p, int variant, hipStream_t st) {
    const unsigned grid = (unsigned)((int64_t)p.tiles_m * p.tiles_n * (p.ksplit > 1 ? p.ksplit : 1));
    switch (variant) {
#define X(V, MF, NF, WM, WN, B)                                                           \
    case V:                                                                                \
        if (p.ksplit > 1) gemm_kernel<MF, NF, WM, WN, B, true><<<grid, 64 * WM * WN, 0, st>>>(p); \
        else gemm_kernel<MF, NF, WM, WN, B, false><<<grid, 64 * WM * WN, 0, st>>>(p);             \
        break;
        MNB_GEMM_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ksplit <= 1) return e;
    const int64_t mn = p.m * p.n;
    splitk_reduce_kernel<<<(unsigned)((mn + 1023) / 1024), 256, 0, st>>>(p.part, p.ksplit, mn,
                                                                         static_cast<_Float16 *>(p.y));
    return hipGetLastError();
}

int64_t gemm_xcd_schedule(Problem *entries, int count, XcdSplit *split, int *out_count) {
    // A workgroup costs its K-tiles plus 2: its start and end take about as
    // long as two K-tiles.
    auto tile_cost = [&](int i) { return (int64_t)entries[i].kg + 2; };
    struct Piece {
        int prod;
        int64_t t0, t1;  // tiles [t0, t1) of the product
    };
    // whole products to XCDs, largest first, each to the least loaded XCD
    std::vector<int> idx(count);
    for (int i = 0; i < count; ++i) idx[i] = i;
    auto cost = [&](int i) { return (int64_t)entries[i].tiles_m * entries[i].tiles_n * tile_cost(i); };
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return cost(a) > cost(b); });
    std::vector<Piece> pieces[kXcds];
    int64_t load[kXcds] = {0}, total = 0;
    for (int i : idx) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
            if (load[x] < load[best]) best = x;
        pieces[best].push_back(Piece{i, 0, (int64_t)entries[i].tiles_m * entries[i].tiles_n});
        load[best] += cost(i);
        total += cost(i);
    }
    // Whole products leave the XCDs up to one product apart. Where that is
    // more than 2% of an XCD's share, move the last tiles of the shortest-K
    // product of the most loaded XCD to the least loaded one, at most
    // kXcdMoves times; each move adds one entry. The moved tiles are the
    // product's last ones (its last output rows), so its other tiles keep
    // sharing their activation rows in one L2. (Below 2% the moves measured
    // slower: the XCDs' own speeds differ by about that much, and a moved
    // run of tiles reads its weights into a second L2.)
    for (int mv = 0; mv < kXcdMoves; ++mv) {
        int h = 0, l = 0;
        for (int x = 1; x < kXcds; ++x) {
            if (load[x] > load[h]) h = x;
            if (load[x] < load[l]) l = x;
        }
        const int64_t target = (total + kXcds - 1) / kXcds;
        if (50 * (load[h] - load[l]) <= target) break;
        const int64_t want = std::min(load[h] - target, target - load[l]);
        int pick = -1;
        for (int q = 0; q < (int)pieces[h].size(); ++q) {
            const Piece &c = pieces[h][q];
            if (c.t1 - c.t0 >= 2 && (pick < 0 || entries[c.prod].kg <= entries[pieces[h][pick].prod].kg)) pick = q;
        }
        if (pick < 0) break;
        Piece &c = pieces[h][pick];
        const int64_t tc = tile_cost(c.prod);
        int64_t n = (want + tc / 2) / tc;
        if (n > c.t1 - c.t0 - 1) n = c.t1 - c.t0 - 1;
        if (n <= 0) break;
        const Piece moved{c.prod, c.t1 - n, c.t1};
        c.t1 -= n;
        load[h] -= n * tc;
        load[l] += n * tc;
        pieces[l].push_back(moved);
    }
    // entries grouped by XCD; inside a group the pieces with more K-tiles
    // come first, so that each XCD ends on short workgroups
    std::vector<Problem> out;
    out.reserve((size_t)count + kXcdMoves);
    int64_t tiles = 0, widest = 0;
    for (int x = 0; x < kXcds; ++x) {
        std::vector<Piece> &mine = pieces[x];
        std::stable_sort(mine.begin(), mine.end(),
                         [&](const Piece &a, const Piece &b) { return entries[a.prod].kg > entries[b.prod].kg; });
        split->begin[x] = (int32_t)tiles;
        split->first[x] = (int32_t)out.size();
        const int64_t t0 = tiles;
        for (const Piece &c : mine) {
            Problem p = entries[c.prod];
            p.wg_begin = tiles;
            p.tile_off = (int32_t)c.t0;
            tiles += c.t1 - c.t0;
            out.push_back(p);
        }
        if (tiles - t0 > widest) widest = tiles - t0;
    }
    split->begin[kXcds] = (int32_t)tiles;
    split->first[kXcds] = (int32_t)out.size();
    for (size_t i = 0; i < out.size(); ++i) entries[i] = out[i];
    *out_count = (int)out.size();
    return widest * kXcds;
}

hipError_t launch_gemm_grouped(const Problem *dev_entries, int count, const XcdSplit &split, int variant,
                               hipStream_t st) {
    int64_t widest = 0;
    for (int x = 0; x < kXcds; ++x)
        if (split.begin[x + 1] - split.begin[x] > widest) widest = split.begin[x + 1] - split.begin[x];
    const int64_t wgs = widest * kXcds;
    switch (variant) {
#define X(V, MF, NF, WM, WN, B)                                                                            \
    case V:                                                                                                \
        gemm_grouped_kernel<MF, NF, WM, WN, B><<<(unsigned)wgs, 64 * WM * WN, 0, st>>>(dev_entries, count, split); \
        break;
        MNB_GEMM_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mnb

// Device layout of a packed MatMulNBits weight (what mnb_pack writes and the
// compute kernels read). Shared by host and device code of the library.
//
// The weight is cut into tiles of 16 rows x 128 inputs. One tile's codes are
// 1024 contiguous bytes: slot l = j * 16 + r (j = 32-input chunk 0..3,
// r = row 0..15) holds the 32 codes of row r, chunk j in 16 bytes, so one
// wave (64 lanes) reads a whole tile with one fully coalesced 128-bit load
// per lane and lane l owns row (l & 15), chunk (l >> 4).
//
// Inside each 32-bit word (8 consecutive inputs k0..k7) the nibbles are
// ordered k0 k2 k4 k6 k1 k3 k5 k7 (bits 0-3 first), so that
// (word >> 4h) & 0x000F000F puts inputs (2h, 2h+1) into the two 16-bit
// halves: one AND-OR with 0x64006400 then yields the float16 pair
// (1024 + q_2h, 1024 + q_2h+1) with no further shuffling.
//
// Scales and zero points are stored tile by tile in the same tile order:
// per tile, nbt = 128 / block_size blocks per row, entry jb * 16 + r for
// block jb of row r; zero points are 4-bit, two per byte, even entry in the
// low nibble. Rows are padded to a multiple of 16 and inputs to a multiple
// of 128 with zero codes, zero scales and zero zero-points, which dequantize
// to exact zeros.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define MNB_HD __host__ __device__ __forceinline__
#else
#define MNB_HD inline
#endif

namespace mnb {

constexpr int kTileRows = 16;
constexpr int kTileK = 128;
constexpr int kTileCodeBytes = kTileRows * kTileK / 2;  // 1024
constexpr int kChunk = 32;                              // inputs per 16-byte lane chunk
constexpr int64_t kAlign = 256;

MNB_HD int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct Layout {
    int64_t n, k;        // logical shape
    int64_t rg, kg;      // tile rows (N_pad / 16), tile columns (K_pad / 128)
    int bs;              // block size (32 or 64)
    int nbt;             // blocks per row per tile: 128 / bs
    int scale_bytes;     // 2 or 4
    int64_t scales_off;  // byte offsets inside the packed buffer
    int64_t zp_off;
    int64_t total;
};

MNB_HD Layout make_layout(int64_t n, int64_t k, int bs, int scale_bytes) {
    Layout L;
    L.n = n;
    L.k = k;
    L.rg = (n + kTileRows - 1) / kTileRows;
    L.kg = (k + kTileK - 1) / kTileK;
    L.bs = bs;
    L.nbt = kTileK / bs;
    L.scale_bytes = scale_bytes;
    const int64_t tiles = L.rg * L.kg;
    L.scales_off = align_up(tiles * kTileCodeBytes, kAlign);
    L.zp_off = align_up(L.scales_off + tiles * L.nbt * kTileRows * scale_bytes, kAlign);
    L.total = align_up(L.zp_off + tiles * L.nbt * kTileRows / 2, kAlign);
    return L;
}

// Byte offset of tile (row group g, input group c) inside a section.
MNB_HD int64_t tile_index(const Layout &L, int64_t g, int64_t c) { return g * L.kg + c; }

}  // namespace mnb

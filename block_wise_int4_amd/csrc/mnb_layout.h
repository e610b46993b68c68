// Device layout of a packed MatMulNBits weight (what mnb_pack writes and the
// compute kernels read). Shared by host and device code of the library.
//
// Codes. The weight is cut into tiles of 16 rows x 128 inputs. One tile's
// codes are 1024 contiguous bytes: slot l = j * 16 + r (j = 32-input chunk
// 0..3, r = row 0..15) holds the 32 codes of row r, chunk j in 16 bytes, so
// one wave (64 lanes) reads a whole tile with one fully coalesced 128-bit
// load per lane, and lane l owns row (l & 15), chunk (l >> 4). Tiles are
// stored row group by row group, each row group's tiles in input order.
//
// Inside each 32-bit word (8 consecutive inputs k0..k7) the nibbles are
// ordered k0 k2 k4 k6 k1 k3 k5 k7 (bits 0-3 first), so that
// (word >> 4h) & 0x000F000F puts inputs (2h, 2h+1) into the two 16-bit
// halves with one shift and one mask.
//
// Scales and zero points. Within a tile, row r has nbt = 128 / block_size
// blocks; entry e = jb * 16 + r names block jb of row r (lane l reads entry
// (j / (block_size / 32)) * 16 + r). A 256-input block spans two tiles:
// nbt is 1 and both tiles' entries hold that block's scale and zero point. Tiles are taken in groups of 8 (kgp =
// kg rounded up to 8), and for each (row group, tile group) the metadata is
// one contiguous block, entry-major: entry e holds its 8 tiles' values in
// tile order. A lane therefore reads the scales of 8 consecutive tiles with
// one 16-byte load (float16) and their zero points with one 4-byte load, and
// a whole wave reads a tile group's metadata as one contiguous span (1 KB of
// float16 scales for block 32). Zero points are 4-bit, two per byte, even
// tile in the low nibble.
//
// Rows are padded to a multiple of 16 and inputs to a multiple of 128 with
// zero codes, zero scales and zero zero-points, which dequantize to exact
// zeros; metadata padding (tiles kg..kgp) is zero too.
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
constexpr int kMetaGroup = 8;                           // tiles per metadata vector load
constexpr int64_t kAlign = 256;

MNB_HD int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct Layout {
    int64_t n, k;        // logical shape
    int64_t rg, kg;      // tile rows (N_pad / 16), tile columns (K_pad / 128)
    int64_t kgp;         // kg rounded up to a multiple of 8 (metadata stride)
    int bs;              // block size (32, 64, 128 or 256)
    int nbt;             // metadata entries per row per tile: 128 / bs, at least 1
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
    L.kgp = align_up(L.kg, kMetaGroup);
    L.bs = bs;
    L.nbt = bs >= kTileK ? 1 : kTileK / bs;
    L.scale_bytes = scale_bytes;
    const int64_t entries = L.rg * L.nbt * kTileRows;  // metadata entries over all row groups
    L.scales_off = align_up(L.rg * L.kg * kTileCodeBytes, kAlign);
    L.zp_off = align_up(L.scales_off + entries * L.kgp * scale_bytes, kAlign);
    L.total = align_up(L.zp_off + entries * L.kgp / 2, kAlign);
    return L;
}

// Metadata index (in elements for scales, in nibbles for zero points) of
// entry e of row group g, tile c: block (g, c / 8) of nbt * 16 entries of 8.
MNB_HD int64_t meta_index(int64_t g, int nbt, int64_t kgp, int e, int64_t c) {
    return ((g * (kgp / kMetaGroup) + c / kMetaGroup) * (nbt * kTileRows) + e) * kMetaGroup + c % kMetaGroup;
}

}  // namespace mnb

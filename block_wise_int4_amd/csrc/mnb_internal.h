// Library-internal declarations: problem descriptors, the grouped-plan
// image, and the host launchers each kernel file provides.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb_device.h"
#include "mnb_layout.h"

namespace mnb {

constexpr int kF32 = 0;
constexpr int kF16 = 1;

// One product as the kernels see it (single launches pass it by value;
// grouped launches read an array of them from the plan in device memory).
struct Problem {
    const void *x;
    const uint8_t *packed;
    void *y;
    int64_t m, n, k;
    int64_t rg, kg, kgp;     // tile grid of the packed weight, metadata stride
    int64_t scales_off, zp_off;
    int64_t wg_begin;        // first workgroup of this problem inside its launch
    int64_t batch_begin;     // decode kernel: first 4-row-group batch in its launch
    int64_t batch_end;
    int32_t bs, nbt;
    int32_t variant;         // kernel variant index (see mnb_gemm.hip / mnb_gemv.hip)
    int32_t tiles_m, tiles_n;
    int32_t ksplit;          // prefill kernel: K parts per output tile (1 = none)
    int32_t tile_off;        // prefill grouped launches: first output tile of this entry
    float *part;             // with ksplit > 1: float32 partial sums [ksplit][m][n]
};

// Kernel classes a plan can launch.
enum Kind : int32_t { kKindGemv = 0, kKindGemm = 1, kKindGemvI8 = 2 };

// Prefill launches: the output tiles of XCD x (blocks b with b % 8 == x)
// are tiles [begin[x], begin[x + 1]) of the launch, and they belong to
// entries [first[x], first[x + 1]) of the launch (an entry is a whole
// product or a run of its tiles, from tile_off on).
constexpr int kXcdCount = 8;
struct XcdSplit {
    int32_t begin[kXcdCount + 1];
    int32_t first[kXcdCount + 1];
};

struct PlanLaunch {
    int32_t kind;
    int32_t variant;
    int32_t first;           // first problem (index into the plan's entries)
    int32_t count;
    int64_t wgs;             // workgroups of this launch
    int64_t lds;             // dynamic LDS bytes (gemv launches)
    int64_t sched_off;       // decode launches: byte offset of the workgroup table
    XcdSplit split;          // prefill launches
};

// Decode kernel schedule: workgroup w runs batches [b0, b1) (a batch is 4
// row groups of one problem, one per wave), starting in problem p.
struct GemvWg {
    int32_t b0, b1, p, pad_;
};
constexpr int kGemvMaxWgs = 768;  // resident workgroups (3 per CU on 256 CUs)
constexpr int kGemvMaxLaunches = 3;

constexpr uint32_t kPlanMagic = 0x4D4E4250u;  // "PBNM"
constexpr int kMaxPlanLaunches = 16;
constexpr int kMaxPlanProblems = 65536;
// Prefill launches may split a product's tiles over two XCDs: each split
// adds one entry, at most kXcdMoves per launch and 5 prefill launches (one
// per tile shape) per plan.
constexpr int kXcdMoves = kXcdCount - 1;
constexpr int kPlanExtraEntries = 5 * kXcdMoves;

struct PlanHeader {
    uint32_t magic;
    uint32_t version;
    int32_t count;
    int32_t bits, bs, dtype;
    int32_t n_launch;
    int32_t pad_;
    uint64_t bytes;          // total plan bytes
    PlanLaunch launches[kMaxPlanLaunches];
};

inline Problem make_problem(const void *x, const void *packed, void *y, int64_t m, int64_t n, int64_t k, int bs,
                            int scale_bytes) {
    const Layout L = make_layout(n, k, bs, scale_bytes);
    Problem p{};
    p.x = x;
    p.packed = static_cast<const uint8_t *>(packed);
    p.y = y;
    p.m = m;
    p.n = n;
    p.k = k;
    p.rg = L.rg;
    p.kg = L.kg;
    p.kgp = L.kgp;
    p.scales_off = L.scales_off;
    p.zp_off = L.zp_off;
    p.bs = bs;
    p.nbt = L.nbt;
    p.ksplit = 1;
    return p;
}

// Launchers (each returns hipGetLastError() after its launches).
hipError_t launch_quantize_rtn(const float *w, int64_t n, int64_t k, int bs, int dtype, uint8_t *qweight,
                               void *scales, uint8_t *zps, hipStream_t st);
hipError_t launch_pack(const uint8_t *qweight, const void *scales, const uint8_t *zps, const Layout &L,
                       int dtype, uint8_t *packed, hipStream_t st);
hipError_t launch_unpack(const uint8_t *packed, const Layout &L, uint8_t *q, uint8_t *zp, hipStream_t st);
hipError_t launch_dequant(const uint8_t *packed, const Layout &L, int dtype, void *w, hipStream_t st);

// Decode kernel (M = 1, fp16 and fp32) and the fp32 multi-row vector kernel
// (fp32, M >= 2). Variants: 0 = fp16 decode, 1 = fp32 decode, 2 = fp32 rows.
int gemv_variant(int dtype, int64_t m);
int64_t gemv_workgroups(const Problem &p, int variant);   // the fp32 rows variants (2, 3)
bool gemv_lds_fits(const Problem &p, int variant);  // its staged activations fit the LDS of a CU
size_t gemv_lds_bytes(const Problem &p, int variant);
// Decode schedule for a list of problems (host): fills batch_begin/end of
// each problem and the workgroup table; returns the workgroup count.
int64_t gemv_schedule(Problem *entries, int count, GemvWg *table, int max_wgs);
hipError_t launch_gemv(const Problem &p, int dtype, int variant, hipStream_t st);
// int8 embedding rows times their float32 scale, rounded once to dtype.
hipError_t launch_embed_gather(const int8_t *table, const float *scales, const int64_t *ids, int64_t rows,
                               int64_t vocab, int64_t h, int dtype, void *out, hipStream_t st);
// Decode product (variants 0 and 1) fused with a greedy argmax of y.
hipError_t launch_gemv_argmax(const Problem &p, int variant, void *workspace, int64_t *index, hipStream_t st);
// Workspace slots the argmax launch of p writes (one per workgroup), and
// the same count for an LM head of n rows.
int64_t gemv_argmax_slots(const Problem &p);
int64_t argmax_slot_count(int64_t n);
// The embedding row of the argmax that a product's slots name (and the
// index itself, where index is not NULL).
hipError_t launch_embed_gather_argmax(const int8_t *table, const float *scales, const void *slots, int64_t count,
                                      int64_t *index, int64_t vocab, int64_t h, int dtype, void *out,
                                      hipStream_t st);
// This device's library-held argmax slots (device address and slot count),
// looked up once per device.
hipError_t argmax_scratch(void **slots, int64_t *n_slots);
hipError_t launch_gemv_grouped(const Problem *dev_entries, int count, const GemvWg *dev_table, int64_t wgs,
                               int variant, size_t lds, hipStream_t st);

// Int8 compute mode: activations quantized per block to int8 (the caller's
// workspace holds them), integer dot products with the 4-bit codes.
int64_t a8_workspace_bytes(int64_t m, int64_t k, int bs);
int64_t gemm_i8_workgroups(const Problem &p);
bool gemm_i8_fits(const Problem &p);  // the problem's offsets fit the kernels' 32-bit addressing
hipError_t launch_quantize_act(const void *x, int64_t m, int64_t k, int bs, int dtype, int8_t *qa, float *scales,
                               hipStream_t st);
hipError_t launch_gemm_i8(const Problem &p, int dtype, void *workspace, hipStream_t st);
// M = 1 in the int8 mode: one launch that quantizes x in LDS (single
// products, and grouped plans through the decode schedule).
size_t gemv_i8_lds_bytes(const Problem &p);
hipError_t launch_gemv_i8(const Problem &p, int dtype, hipStream_t st);
hipError_t launch_gemv_i8_grouped(const Problem *dev_entries, const GemvWg *dev_table, int64_t wgs, int dtype,
                                  size_t lds, hipStream_t st);

// MFMA kernel: fp16 with M >= 2.
int gemm_variant(int64_t m);
void gemm_tiles(const Problem &p, int variant, int32_t *tiles_m, int32_t *tiles_n);
// A single product's tile variant and K split (1 = none), from a cost model
// of one product running alone: at most max_split parts, or exactly
// force_split (> 0) parts, never more than the product's K-tiles.
struct GemmChoice {
    int variant;
    int ksplit;
};
GemmChoice gemm_single_choice(const Problem &p, int max_split, int force_split);
// Bytes of float32 partial sums a product split into `ksplit` parts needs.
int64_t gemm_part_bytes(const Problem &p, int ksplit);
hipError_t launch_gemm(const Problem &p, int variant, hipStream_t st);
hipError_t launch_gemm_grouped(const Problem *dev_entries, int count, const XcdSplit &split, int variant,
                               hipStream_t st);
// Host: order and split the problems of one prefill launch across the XCDs
// (fills wg_begin and tile_off of each entry). entries has room for
// count + kXcdMoves entries; *out_count receives the number written.
// Returns the launch's workgroup count.
int64_t gemm_xcd_schedule(Problem *entries, int count, XcdSplit *split, int *out_count);

}  // namespace mnb

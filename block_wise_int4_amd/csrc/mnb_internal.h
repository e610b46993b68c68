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
    int64_t rg, kg;          // tile grid of the packed weight
    int64_t scales_off, zp_off;
    int64_t wg_begin;        // first workgroup of this problem inside its launch
    int32_t bs, nbt;
    int32_t variant;         // kernel variant index (see mnb_gemm.hip / mnb_gemv.hip)
    int32_t tiles_m, tiles_n;
    int32_t pad_;
};

// Kernel classes a plan can launch.
enum Kind : int32_t { kKindGemv = 0, kKindGemm = 1 };

struct PlanLaunch {
    int32_t kind;
    int32_t variant;
    int32_t first;           // first problem (index into the plan's entries)
    int32_t count;
    int64_t wgs;             // workgroups of this launch
    int64_t lds;             // dynamic LDS bytes (gemv launches)
};

constexpr uint32_t kPlanMagic = 0x4D4E4250u;  // "PBNM"
constexpr int kMaxPlanLaunches = 16;
constexpr int kMaxPlanProblems = 65536;

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
    p.scales_off = L.scales_off;
    p.zp_off = L.zp_off;
    p.bs = bs;
    p.nbt = L.nbt;
    return p;
}

// Launchers (each returns hipGetLastError() after its launches).
hipError_t launch_quantize_rtn(const float *w, int64_t n, int64_t k, int bs, int dtype, uint8_t *qweight,
                               void *scales, uint8_t *zps, hipStream_t st);
hipError_t launch_pack(const uint8_t *qweight, const void *scales, const uint8_t *zps, const Layout &L,
                       int dtype, uint8_t *packed, hipStream_t st);
hipError_t launch_unpack(const uint8_t *packed, const Layout &L, uint8_t *q, uint8_t *zp, hipStream_t st);
hipError_t launch_dequant(const uint8_t *packed, const Layout &L, int dtype, void *w, hipStream_t st);

// GEMV / vector kernel: M = 1 (fp16, fp32) and fp32 with M >= 2.
int gemv_variant(int dtype, int64_t m);
int64_t gemv_workgroups(const Problem &p, int variant);
int64_t gemv_max_kpad(int variant);
size_t gemv_lds_bytes(const Problem &p, int variant);
hipError_t launch_gemv(const Problem &p, int dtype, int variant, hipStream_t st);
hipError_t launch_gemv_grouped(const Problem *dev_entries, int count, int64_t wgs, int variant, size_t lds,
                               hipStream_t st);

// MFMA kernel: fp16 with M >= 2.
int gemm_variant(int64_t m);
void gemm_tiles(const Problem &p, int variant, int32_t *tiles_m, int32_t *tiles_n);
hipError_t launch_gemm(const Problem &p, int variant, hipStream_t st);
hipError_t launch_gemm_grouped(const Problem *dev_entries, int count, int64_t wgs, int variant, hipStream_t st);

}  // namespace mnb

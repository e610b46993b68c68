// The C ABI (include/mnb.h): argument checks on the host, launch geometry,
// status mapping. Nothing here allocates or synchronizes.
#include <string.h>

#include <algorithm>
#include <new>

#include "../../include/mnb.h"
#include "mnb_internal.h"

using namespace mnb;

namespace {

inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int dtype_bytes(int dtype) { return dtype == MNB_F16 ? 2 : 4; }

// Format and shape checks common to every entry point.
int check_format(int64_t n, int64_t k, int bits, int bs, int dtype) {
    if (bits != 4) return MNB_ERR_BITS;
    if (bs != 32 && bs != 64 && bs != 128 && bs != 256) return MNB_ERR_BLOCK;
    if (dtype != MNB_F32 && dtype != MNB_F16) return MNB_ERR_DTYPE;
    if (n <= 0 || k <= 0 || k % bs != 0) return MNB_ERR_SHAPE;
    if (n > MNB_MAX_ROWS || k > MNB_MAX_K) return MNB_ERR_SHAPE;
    return MNB_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MNB_OK : MNB_ERR_HIP; }

// Checks for one product; fills `variant` and the problem's launch fields.
int prepare_product(const void *x, const void *packed, const void *y, int64_t m, int64_t n, int64_t k, int bits,
                    int bs, int dtype, Problem *out, int *kind, int *variant) {
    if (!x || !packed || !y) return MNB_ERR_NULL;
    int st = check_format(n, k, bits, bs, dtype);
    if (st) return st;
    if (m <= 0 || m > MNB_MAX_ROWS) return MNB_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(y)) return MNB_ERR_ALIGN;
    Problem p = make_problem(x, packed, const_cast<void *>(y), m, n, k, bs, dtype_bytes(dtype));
    // (a launch's workgroup count must fit the 32-bit grid, and stays below 2^31)
    if (dtype == MNB_F16 && m >= 2) {
        *kind = kKindGemm;
        *variant = gemm_variant(m);
        gemm_tiles(p, *variant, &p.tiles_m, &p.tiles_n);
        if ((int64_t)p.tiles_m * p.tiles_n > 0x7FFFFFFFLL) return MNB_ERR_SHAPE;
    } else {
        *kind = kKindGemv;
        *variant = gemv_variant(dtype, m);
        if (*variant == 2 && !gemv_lds_fits(p, 2)) *variant = 3;
        if (!gemv_lds_fits(p, *variant)) return MNB_ERR_SHAPE;
        if (*variant >= 2 && gemv_workgroups(p, *variant) > 0x7FFFFFFFLL) return MNB_ERR_SHAPE;
    }
    *out = p;
    return MNB_OK;
}

// A single matrix-core product (a call of its own, not a plan): its tile
// variant and K split by the library's cost model, at most max_split parts
// or exactly force_split (> 0); sets p's tiles and ksplit and returns the
// variant. Grouped plans keep the tall tiles of prepare_product.
int single_gemm(Problem &p, int max_split, int force_split) {
    const GemmChoice c = gemm_single_choice(p, max_split, force_split);
    gemm_tiles(p, c.variant, &p.tiles_m, &p.tiles_n);
    p.ksplit = c.ksplit;
    return c.variant;
}

}  // namespace

extern "C" {

int mnb_abi_version(void) { return MNB_ABI_VERSION; }

const char *mnb_status_string(int status) {
    switch (status) {
    case MNB_OK: return "ok";
    case MNB_ERR_NULL: return "a required pointer is NULL";
    case MNB_ERR_BITS: return "bits must be 4";
    case MNB_ERR_BLOCK: return "block_size must be 32, 64, 128 or 256";
    case MNB_ERR_SHAPE: return "invalid shape (M, N, K > 0, K a multiple of block_size, within limits)";
    case MNB_ERR_DTYPE: return "unsupported dtype";
    case MNB_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MNB_ERR_HIP: return "HIP runtime error";
    case MNB_ERR_PLAN: return "invalid grouped plan";
    case MNB_ERR_INVALID: return "invalid argument";
    default: return "unknown status";
    }
}

size_t mnb_packed_bytes(int64_t N, int64_t K, int bits, int block_size, int dtype) {
    if (check_format(N, K, bits, block_size, dtype) != MNB_OK) return 0;
    return (size_t)make_layout(N, K, block_size, dtype_bytes(dtype)).total;
}

int mnb_quantize_rtn(const float *w, int64_t N, int64_t K, int bits, int block_size, int dtype, uint8_t *qweight,
                     void *scales, uint8_t *zero_points, void *stream) {
    if (!w || !qweight || !scales) return MNB_ERR_NULL;
    int st = check_format(N, K, bits, block_size, dtype);
    if (st) return st;
    if (!aligned16(w) || !aligned16(qweight) || !aligned16(scales) || (zero_points && !aligned16(zero_points)))
        return MNB_ERR_ALIGN;
    return hip_status(launch_quantize_rtn(w, N, K, block_size, dtype, qweight, scales, zero_points, as_stream(stream)));
}

int mnb_pack(const uint8_t *qweight, const void *scales, const uint8_t *zero_points, int64_t N, int64_t K, int bits,
             int block_size, int dtype, void *packed, void *stream) {
    if (!qweight || !scales || !packed) return MNB_ERR_NULL;
    int st = check_format(N, K, bits, block_size, dtype);
    if (st) return st;
    if (!aligned16(qweight) || !aligned16(packed)) return MNB_ERR_ALIGN;
    const Layout L = make_layout(N, K, block_size, dtype_bytes(dtype));
    return hip_status(launch_pack(qweight, scales, zero_points, L, dtype, static_cast<uint8_t *>(packed),
                                  as_stream(stream)));
}

int mnb_unpack(const void *packed, int64_t N, int64_t K, int bits, int block_size, int dtype, uint8_t *q, uint8_t *zp,
               void *stream) {
    if (!packed || !q || !zp) return MNB_ERR_NULL;
    int st = check_format(N, K, bits, block_size, dtype);
    if (st) return st;
    if (!aligned16(packed)) return MNB_ERR_ALIGN;
    const Layout L = make_layout(N, K, block_size, dtype_bytes(dtype));
    return hip_status(launch_unpack(static_cast<const uint8_t *>(packed), L, q, zp, as_stream(stream)));
}

int mnb_dequant(const void *packed, int64_t N, int64_t K, int bits, int block_size, int dtype, void *w, void *stream) {
    if (!packed || !w) return MNB_ERR_NULL;
    int st = check_format(N, K, bits, block_size, dtype);
    if (st) return st;
    if (!aligned16(packed) || !aligned16(w)) return MNB_ERR_ALIGN;
    const Layout L = make_layout(N, K, block_size, dtype_bytes(dtype));
    return hip_status(launch_dequant(static_cast<const uint8_t *>(packed), L, dtype, w, as_stream(stream)));
}

int mnb_gemm(const void *x, const void *packed, void *y, int64_t M, int64_t N, int64_t K, int bits, int block_size,
             int dtype, void *stream) {
    Problem p;
    int kind = 0, variant = 0;
    int st = prepare_product(x, packed, y, M, N, K, bits, block_size, dtype, &p, &kind, &variant);
    if (st) return st;
    if (kind == kKindGemm) {
        variant = single_gemm(p, 1, 1);
        return hip_status(launch_gemm(p, variant, as_stream(stream)));
    }
    return hip_status(launch_gemv(p, dtype, variant, as_stream(stream)));
}

size_t mnb_gemm_i8_workspace_bytes(int64_t M, int64_t K, int block_size) {
    if (check_format(1, K, 4, block_size, MNB_F32) != MNB_OK) return 0;
    if (M <= 1 || M > MNB_MAX_ROWS) return 0;  // M = 1 quantizes in LDS and needs none
    return (size_t)a8_workspace_bytes(M, K, block_size);
}

int mnb_quantize_act_i8(const void *x, int64_t M, int64_t K, int block_size, int dtype, int8_t *qa, float *scales,
                        void *stream) {
    if (!x || !qa || !scales) return MNB_ERR_NULL;
    int st = check_format(1, K, 4, block_size, dtype);
    if (st) return st;
    if (M <= 0 || M > MNB_MAX_ROWS) return MNB_ERR_SHAPE;
    if ((M * (K / 8) + 255) / 256 > 0x7FFFFFFFLL) return MNB_ERR_SHAPE;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(qa) & 7) || (reinterpret_cast<uintptr_t>(scales) & 3))
        return MNB_ERR_ALIGN;
    return hip_status(launch_quantize_act(x, M, K, block_size, dtype, qa, scales, as_stream(stream)));
}

int mnb_gemm_i8(const void *x, const void *packed, void *y, void *workspace, size_t workspace_bytes, int64_t M,
                int64_t N, int64_t K, int bits, int block_size, int dtype, void *stream) {
    if (!x || !packed || !y) return MNB_ERR_NULL;
    int st = check_format(N, K, bits, block_size, dtype);
    if (st) return st;
    if (M <= 0 || M > MNB_MAX_ROWS) return MNB_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(y)) return MNB_ERR_ALIGN;
    if (M == 1) {
        const Problem p = make_problem(x, packed, y, 1, N, K, block_size, dtype_bytes(dtype));
        return hip_status(launch_gemv_i8(p, dtype, as_stream(stream)));
    }
    if (!workspace) return MNB_ERR_NULL;
    if (!aligned16(workspace)) return MNB_ERR_ALIGN;
    if (workspace_bytes < (size_t)a8_workspace_bytes(M, K, block_size)) return MNB_ERR_INVALID;
    const Problem p = make_problem(x, packed, y, M, N, K, block_size, dtype_bytes(dtype));
    if ((M * (K / 8) + 255) / 256 > 0x7FFFFFFFLL || gemm_i8_workgroups(p) > 0x7FFFFFFFLL || !gemm_i8_fits(p))
        return MNB_ERR_SHAPE;
    return hip_status(launch_gemm_i8(p, dtype, workspace, as_stream(stream)));
}



size_t mnb_gemm_split_k_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits, int block_size, int dtype,
                                        int ksplit) {
    if (ksplit < 0 || ksplit > MNB_MAX_KSPLIT) return 0;
    Problem p;
    int kind = 0, variant = 0;
    // shape checks only: stand-in pointers, never dereferenced
    static const uint8_t probe[16] __attribute__((aligned(16))) = {0};
    if (prepare_product(probe, probe, probe, M, N, K, bits, block_size, dtype, &p, &kind, &variant) != MNB_OK)
        return 0;
    if (kind != kKindGemm) return 0;
    single_gemm(p, MNB_MAX_KSPLIT, ksplit);
    return (size_t)gemm_part_bytes(p, p.ksplit);
}

int mnb_gemm_split_k(const void *x, const void *packed, void *y, void *workspace, size_t workspace_bytes,
                     int64_t M, int64_t N, int64_t K, int bits, int block_size, int dtype, int ksplit,
                     void *stream) {
    if (ksplit < 0 || ksplit > MNB_MAX_KSPLIT) return MNB_ERR_INVALID;
    Problem p;
    int kind = 0, variant = 0;
    int st = prepare_product(x, packed, y, M, N, K, bits, block_size, dtype, &p, &kind, &variant);
    if (st) return st;
    if (kind != kKindGemm) return hip_status(launch_gemv(p, dtype, variant, as_stream(stream)));
    variant = single_gemm(p, MNB_MAX_KSPLIT, ksplit);
    if (p.ksplit > 1) {
        const int64_t need = gemm_part_bytes(p, p.ksplit);
        if (!workspace) return MNB_ERR_NULL;
        if (!aligned16(workspace)) return MNB_ERR_ALIGN;
        if (workspace_bytes < (size_t)need) return MNB_ERR_INVALID;
        if ((int64_t)p.tiles_m * p.tiles_n * p.ksplit > 0x7FFFFFFFLL || (p.m * p.n + 1023) / 1024 > 0x7FFFFFFFLL)
            return MNB_ERR_SHAPE;
        p.part = static_cast<float *>(workspace);
    }
    return hip_status(launch_gemm(p, variant, as_stream(stream)));
}

int mnb_embed_gather(const int8_t *table, const float *row_scales, const int64_t *ids, int64_t T, int64_t V,
                     int64_t H, int dtype, void *out, void *stream) {
    if (!table || !row_scales || !ids || !out) return MNB_ERR_NULL;
    if (dtype != MNB_F16 && dtype != MNB_F32) return MNB_ERR_DTYPE;
    if (T < 0 || V <= 0 || H <= 0 || H % 16 != 0 || T > MNB_MAX_ROWS || V > MNB_MAX_ROWS) return MNB_ERR_SHAPE;
    if (!aligned16(table) || !aligned16(out) || (reinterpret_cast<uintptr_t>(ids) & 7) ||
        (reinterpret_cast<uintptr_t>(row_scales) & 3))
        return MNB_ERR_ALIGN;
    if (T == 0) return MNB_OK;
    return hip_status(launch_embed_gather(table, row_scales, ids, T, V, H, dtype, out, as_stream(stream)));
}

int mnb_gemv_argmax(const void *x, const void *packed, void *y, int64_t *index, void *workspace, int64_t N,
                    int64_t K, int bits, int block_size, int dtype, void *stream) {
    if (!workspace) return MNB_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(index) & 7) || !aligned16(workspace)) return MNB_ERR_ALIGN;
    Problem p;
    int kind = 0, variant = 0;
    // y is optional here: validate with x standing in for it
    int st = prepare_product(x, packed, y ? y : x, 1, N, K, bits, block_size, dtype, &p, &kind, &variant);
    if (st) return st;
    p.y = y;
    return hip_status(launch_gemv_argmax(p, variant, workspace, index, as_stream(stream)));
}

int mnb_embed_gather_argmax(const int8_t *table, const float *row_scales, const void *workspace, int64_t *index,
                            int64_t V, int64_t H, int dtype, void *out, void *stream) {
    if (!table || !row_scales || !workspace || !out) return MNB_ERR_NULL;
    if (dtype != MNB_F16 && dtype != MNB_F32) return MNB_ERR_DTYPE;
    if (V <= 0 || H <= 0 || H % 16 != 0 || V > MNB_MAX_ROWS) return MNB_ERR_SHAPE;
    if (!aligned16(table) || !aligned16(out) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(index) & 7) ||
        (reinterpret_cast<uintptr_t>(row_scales) & 3))
        return MNB_ERR_ALIGN;
    return hip_status(launch_embed_gather_argmax(table, row_scales, workspace, argmax_slot_count(V), index, V, H,
                                                 dtype, out, as_stream(stream)));
}

int mnb_gemv_argmax_noalloc(const void *x, const void *packed, void *y, int64_t *index, int64_t N, int64_t K,
                            int bits, int block_size, int dtype, void *stream) {
    if (!index) return MNB_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(index) & 7) return MNB_ERR_ALIGN;
    Problem p;
    int kind = 0, variant = 0;
    int st = prepare_product(x, packed, y ? y : x, 1, N, K, bits, block_size, dtype, &p, &kind, &variant);
    if (st) return st;
    p.y = y;
    void *slots = nullptr;
    int64_t n_slots = 0;
    if (argmax_scratch(&slots, &n_slots) != hipSuccess) return MNB_ERR_HIP;
    if (gemv_argmax_slots(p) > n_slots) return MNB_ERR_SHAPE;
    return hip_status(launch_gemv_argmax(p, variant, slots, index, as_stream(stream)));
}

int mnb_gemv(const void *x, const void *packed, void *y, int64_t N, int64_t K, int bits, int block_size, int dtype,
             void *stream) {
    return mnb_gemm(x, packed, y, 1, N, K, bits, block_size, dtype, stream);
}

size_t mnb_plan_bytes(int count) {
    if (count < 1 || count > kMaxPlanProblems) return 0;
    return sizeof(PlanHeader) + sizeof(Problem) * ((size_t)count + kPlanExtraEntries) +
           sizeof(GemvWg) * (size_t)kGemvMaxWgs * kGemvMaxLaunches;
}

namespace {
int plan_grouped(const mnb_problem *problems, int count, int bits, int block_size, int dtype, bool int8, void *plan,
                 size_t plan_bytes) {
    if (!problems || !plan) return MNB_ERR_NULL;
    const size_t need = mnb_plan_bytes(count);
    if (need == 0 || plan_bytes < need) return MNB_ERR_PLAN;
    int st = check_format(1, block_size, bits, block_size, dtype);
    if (st) return st;

    // Classify every problem, then lay the entries out launch by launch.
    Problem *tmp = new (std::nothrow) Problem[count];
    int *kinds = new (std::nothrow) int[count];
    int *variants = new (std::nothrow) int[count];
    int *order = new (std::nothrow) int[count];
    if (!tmp || !kinds || !variants || !order) {
        delete[] tmp;
        delete[] kinds;
        delete[] variants;
        delete[] order;
        return MNB_ERR_INVALID;
    }
    for (int i = 0; i < count && st == MNB_OK; ++i) {
        const mnb_problem &q = problems[i];
        st = prepare_product(q.x, q.packed, q.y, q.M, q.N, q.K, bits, block_size, dtype, &tmp[i], &kinds[i],
                             &variants[i]);
        if (st == MNB_OK && int8) {  // the int8 mode takes decode products: one kernel, variant = dtype
            if (q.M != 1) st = MNB_ERR_SHAPE;
            kinds[i] = kKindGemvI8;
            variants[i] = dtype == MNB_F16 ? 0 : 1;
        }
    }
    if (st == MNB_OK) {
        PlanHeader *hdr = static_cast<PlanHeader *>(plan);
        Problem *entries = reinterpret_cast<Problem *>(hdr + 1);
        GemvWg *tables = reinterpret_cast<GemvWg *>(entries + count + kPlanExtraEntries);
        memset(hdr, 0, sizeof(PlanHeader));
        hdr->magic = kPlanMagic;
        hdr->version = MNB_ABI_VERSION;
        hdr->count = count;
        hdr->bits = bits;
        hdr->bs = block_size;
        hdr->dtype = dtype;
        int out = 0, decode_tables = 0;
        // one launch per (kind, variant) present
        for (int kind = kKindGemv; kind <= kKindGemvI8 && st == MNB_OK; ++kind) {
            for (int v = 0; v < 16 && st == MNB_OK; ++v) {
                PlanLaunch L{};
                L.kind = kind;
                L.variant = v;
                L.first = out;
                int64_t wgs = 0;
                size_t lds = 0;
                int n_sel = 0;
                for (int i = 0; i < count; ++i)
                    if (kinds[i] == kind && variants[i] == v) order[n_sel++] = i;
                for (int s = 0; s < n_sel; ++s) {
                    const int i = order[s];
                    Problem p = tmp[i];
                    p.variant = v;
                    p.wg_begin = wgs;
                    if (kind == kKindGemm) wgs += (int64_t)p.tiles_m * p.tiles_n;
                    else if (v >= 2) wgs += gemv_workgroups(p, v);
                    if (kind == kKindGemv && gemv_lds_bytes(p, v) > lds) lds = gemv_lds_bytes(p, v);
                    if (kind == kKindGemvI8 && gemv_i8_lds_bytes(p) > lds) lds = gemv_i8_lds_bytes(p);
                    entries[out++] = p;
                }
                L.count = out - L.first;
                if (L.count == 0) continue;
                if (kind == kKindGemm) {
                    if (wgs > 0x7FFFFFFFLL) {
                        st = MNB_ERR_PLAN;
                        break;
                    }
                    // (the entries after this launch's are free: launches are laid out in order;
                    // the schedule may add up to kXcdMoves of them)
                    if ((int64_t)out + kXcdMoves > (int64_t)count + kPlanExtraEntries) {
                        st = MNB_ERR_PLAN;
                        break;
                    }
                    int n_out = L.count;
                    wgs = gemm_xcd_schedule(entries + L.first, L.count, &L.split, &n_out);
                    out = L.first + n_out;
                    L.count = n_out;
                }
                if ((kind == kKindGemv && v < 2) || kind == kKindGemvI8) {
                    if (decode_tables >= kGemvMaxLaunches) {
                        st = MNB_ERR_PLAN;
                        break;
                    }
                    GemvWg *table = tables + (size_t)decode_tables * kGemvMaxWgs;
                    wgs = gemv_schedule(entries + L.first, L.count, table, kGemvMaxWgs);
                    L.sched_off = reinterpret_cast<uint8_t *>(table) - reinterpret_cast<uint8_t *>(hdr);
                    ++decode_tables;
                }
                if (wgs > 0x7FFFFFFFLL || hdr->n_launch >= kMaxPlanLaunches) {
                    st = MNB_ERR_PLAN;
                    break;
                }
                L.wgs = wgs;
                L.lds = (int64_t)lds;
                hdr->launches[hdr->n_launch++] = L;
            }
        }
        hdr->bytes = need;
    }
    delete[] tmp;
    delete[] kinds;
    delete[] variants;
    delete[] order;
    return st;
}
}  // namespace

int mnb_plan_grouped(const mnb_problem *problems, int count, int bits, int block_size, int dtype, void *plan,
                     size_t plan_bytes) {
    return plan_grouped(problems, count, bits, block_size, dtype, false, plan, plan_bytes);
}

int mnb_plan_grouped_i8(const mnb_problem *problems, int count, int bits, int block_size, int dtype, void *plan,
                        size_t plan_bytes) {
    return plan_grouped(problems, count, bits, block_size, dtype, true, plan, plan_bytes);
}

int mnb_plan_launches(const void *plan_host) {
    if (!plan_host) return -1;
    const PlanHeader *hdr = static_cast<const PlanHeader *>(plan_host);
    if (hdr->magic != kPlanMagic || hdr->version != MNB_ABI_VERSION || hdr->n_launch < 1 ||
        hdr->n_launch > kMaxPlanLaunches)
        return -1;
    return hdr->n_launch;
}

int mnb_gemm_grouped(const void *plan_host, const void *plan_device, void *stream) {
    if (!plan_host || !plan_device) return MNB_ERR_NULL;
    if (!aligned16(plan_device)) return MNB_ERR_ALIGN;
    const PlanHeader *hdr = static_cast<const PlanHeader *>(plan_host);
    if (hdr->magic != kPlanMagic || hdr->version != MNB_ABI_VERSION || hdr->count < 1 ||
        hdr->count > kMaxPlanProblems || hdr->n_launch < 1 || hdr->n_launch > kMaxPlanLaunches ||
        hdr->bytes != mnb_plan_bytes(hdr->count))
        return MNB_ERR_PLAN;
    const Problem *dev = reinterpret_cast<const Problem *>(static_cast<const PlanHeader *>(plan_device) + 1);
    for (int i = 0; i < hdr->n_launch; ++i) {
        const PlanLaunch &L = hdr->launches[i];
        if (L.first < 0 || L.count < 1 || L.first + L.count > hdr->count + kPlanExtraEntries) return MNB_ERR_PLAN;
        hipError_t e;
        if (L.kind == kKindGemm) {
            e = launch_gemm_grouped(dev + L.first, L.count, L.split, L.variant, as_stream(stream));
        } else if (L.kind == kKindGemvI8) {
            const GemvWg *table = reinterpret_cast<const GemvWg *>(static_cast<const uint8_t *>(plan_device) +
                                                                   L.sched_off);
            e = launch_gemv_i8_grouped(dev + L.first, table, L.wgs, L.variant == 0 ? kF16 : kF32, (size_t)L.lds,
                                       as_stream(stream));
        } else {
            const GemvWg *table = reinterpret_cast<const GemvWg *>(static_cast<const uint8_t *>(plan_device) +
                                                                   L.sched_off);
            e = launch_gemv_grouped(dev + L.first, L.count, table, L.wgs, L.variant, (size_t)L.lds,
                                    as_stream(stream));
        }
        if (e != hipSuccess) return MNB_ERR_HIP;
    }
    return MNB_OK;
}

}  // extern "C"

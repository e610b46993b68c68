/*
 * mnb.h - MatMulNBits for AMD Instinct MI355X (gfx950): weight-only,
 * block-wise, asymmetric 4-bit quantized matrix multiplication.
 *
 *   Y[M, N] = X[M, K] * D[N, K]^T,   D[n, k] = (q[n, k] - zp[n, b]) * s[n, b],
 *   b = k / block_size.
 *
 * The operator is the one the int4 ONNX model cards call MatMulNBits:
 * 4-bit codes, blocks of 32 inputs, asymmetric ("Mega-ASR INT4 ONNX",
 * section "Conversion details"); round-to-nearest, block 32, fp16 float
 * tensors in the q4f16 variant ("Qwen3-ASR-0.6B ONNX for the browser",
 * section "Pick a variant" and section "Graph contracts"); block 64
 * ("sherpa-onnx STT int4", section "whisper-small"; "qwen3-asr-0.6b-onnx-
 * int4-merged", section "Provenance"); only the weights are quantized and
 * activations enter as they are ("sherpa-onnx STT int4", section "Why int4
 * rather than the usual int8").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named x, y, w, qweight, scales, zero_points, packed, q, zp are
 *    DEVICE pointers. The caller owns all memory; the library allocates,
 *    frees and synchronizes nothing and keeps no state between calls (beyond
 *    raising a kernel's LDS limit, once per device and to its maximum, the
 *    first time a long K needs it), so calls are reentrant. Calls on one
 *    stream run in order.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call that touches device memory is asynchronous on it.
 *  - bits must be 4, block_size 32, 64, 128 or 256, K a positive multiple of
 *    block_size, M and N positive. The pages use 32 and 64; 128 and 256 are
 *    format variants (a 256-input block spans two of the layout's 128-input
 *    tiles), with the same formula.
 *  - dtype is the activation dtype, which is also the scale dtype and the
 *    output dtype: MNB_F32 or MNB_F16. Accumulation is float32.
 *  - Every argument is checked on the host before anything is enqueued; on
 *    error nothing is enqueued and a nonzero mnb_status is returned. A launch
 *    failure reported by the HIP runtime returns MNB_ERR_HIP.
 *  - Device pointers must be 16-byte aligned (MNB_ERR_ALIGN otherwise);
 *    outputs must not overlap inputs.
 *  - The packed buffer carries no header: pack and use must be given the
 *    same (N, K, block_size, dtype). This is documented, not checked.
 *
 * Canonical (interchange) weight format, as produced by mnb_quantize_rtn and
 * consumed by mnb_pack:
 *  - qweight     uint8 [N][K/2]: byte j of row n holds code k = 2j in bits
 *                0-3 and k = 2j+1 in bits 4-7 (low nibble first).
 *  - scales      dtype [N][K/block_size].
 *  - zero_points uint8 [N][ceil(K/block_size/2)]: byte i of row n holds the
 *                zero point of block 2i in bits 0-3 and of block 2i+1 in bits
 *                4-7; an odd block count leaves a zero pad nibble.
 */
#ifndef MNB_H
#define MNB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MNB_ABI_VERSION 2

typedef enum mnb_dtype {
    MNB_F32 = 0, /* float32 activations, scales and outputs */
    MNB_F16 = 1  /* float16 activations, scales and outputs */
} mnb_dtype;

typedef enum mnb_status {
    MNB_OK = 0,
    MNB_ERR_NULL = 1,      /* a required pointer is NULL                     */
    MNB_ERR_BITS = 2,      /* bits != 4                                      */
    MNB_ERR_BLOCK = 3,     /* block_size not 32, 64, 128 or 256              */
    MNB_ERR_SHAPE = 4,     /* M, N, K <= 0, K % block_size != 0, or a size
                              beyond the documented limits                    */
    MNB_ERR_DTYPE = 5,     /* dtype not MNB_F32 / MNB_F16, or not supported
                              by this entry point                             */
    MNB_ERR_ALIGN = 6,     /* a device pointer is not 16-byte aligned        */
    MNB_ERR_HIP = 7,       /* the HIP runtime reported a launch error        */
    MNB_ERR_PLAN = 8,      /* grouped plan: bad count, size or contents      */
    MNB_ERR_INVALID = 9    /* any other invalid argument                     */
} mnb_status;

/* Limits checked by the entry points (MNB_ERR_SHAPE beyond them). A product
 * is also rejected when its kernel would need more than 2^31 - 1
 * workgroups (an M x N output beyond about 2^44 elements). */
#define MNB_MAX_K 32768            /* inputs per row                         */
#define MNB_MAX_ROWS 0x7FFFFFF0LL  /* M and N                                */

/* ABI version of the loaded library (MNB_ABI_VERSION it was built with). */
int mnb_abi_version(void);

/* Static description of a status code; never NULL, "unknown status" for
 * values outside the enum. */
const char *mnb_status_string(int status);

/* Bytes of device memory mnb_pack writes for one weight, or 0 if the
 * arguments are invalid. Host only. Padding rounds N up to 16 and K up to
 * 128 and is filled with zero codes, zero scales and zero zero-points. */
size_t mnb_packed_bytes(int64_t N, int64_t K, int bits, int block_size, int dtype);

/*
 * Round-to-nearest block quantization of a float32 weight W[N][K] into the
 * canonical format. The pages name the quantizer (RTN, blocks along K,
 * asymmetric; "Qwen3-ASR-0.6B ONNX for the browser", section "Pick a
 * variant"; "Mega-ASR INT4 ONNX", section "Conversion details") but print no
 * formula; per block this computes, in float64:
 *   lo = min(0, min w), hi = max(0, max w),
 *   s  = (hi - lo) / 15 rounded once (half to even) to dtype,
 *   zp = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + zp, 0, 15),
 * and zp = q = 0 for a block whose stored scale is 0. rint rounds half to
 * even. w: device float32 [N][K]. Outputs: qweight [N][K/2], scales
 * [N][K/bs] of dtype, zero_points [N][ceil(K/bs/2)] (canonical layout).
 *
 * zero_points NULL selects the symmetric format (the is_symmetric setting of
 * the same conversion, "Mega-ASR INT4 ONNX", section "Conversion details"):
 * no zero points are stored, every block uses the fixed zero point 8 (the
 * middle of the 4-bit range), and s = max|w| / 7 rounded once to dtype, so
 * that q = clamp(rint(w / s) + 8, 0, 15) never clips; q = 8 where s is 0.
 * Weights must be finite. Not a hot-path call (offline tooling).
 */
int mnb_quantize_rtn(const float *w, int64_t N, int64_t K, int bits, int block_size, int dtype,
                     uint8_t *qweight, void *scales, uint8_t *zero_points, void *stream);

/*
 * Canonical format -> the device layout the compute kernels read, written to
 * `packed` (mnb_packed_bytes(...) bytes, device). Runs once per weight.
 * The canonical format is the one the conversion writes: 4-bit codes in
 * blocks of block_size along K with one scale and one 4-bit zero point per
 * block ("Mega-ASR INT4 ONNX", section "Conversion details"), low nibble
 * first. Inputs: qweight [N][K/2], scales [N][K/bs] of dtype, zero_points
 * [N][ceil(K/bs/2)], all device, all read only; the device layout is
 * described with the library's sources and is not an interface.
 * zero_points NULL: the symmetric format, stored as zero point 8 for every
 * block (the compute kernels then run unchanged).
 */
int mnb_pack(const uint8_t *qweight, const void *scales, const uint8_t *zero_points,
             int64_t N, int64_t K, int bits, int block_size, int dtype,
             void *packed, void *stream);

/*
 * Test export: the unpacked codes q uint8 [N][K] (values 0..15) and zero
 * points zp uint8 [N][K/bs] of the format in "Mega-ASR INT4 ONNX", section
 * "Conversion details", read back from `packed` (device, read only) into
 * device buffers the caller owns. Each code is read through the pair form
 * the float16 decode kernel feeds its dot products (the codes as exact
 * float16 subnormals), and must agree with the reader the float32 kernels
 * use; a code where the two disagree reads 0xFF. Bit-exact with the
 * canonical input.
 */
int mnb_unpack(const void *packed, int64_t N, int64_t K, int bits, int block_size, int dtype,
               uint8_t *q, uint8_t *zp, void *stream);

/*
 * Test export: dequantized weights w [N][K] in dtype (device, caller-owned),
 * D = (q - zp) * s per block ("Mega-ASR INT4 ONNX", section "Conversion
 * details": asymmetric codes with a zero point), each (q - zp) formed
 * exactly and multiplied by s with one round-half-to-even rounding. Float16
 * weights come from the same pair helper that forms the matrix-core
 * kernel's operands, so they are bitwise the values that kernel multiplies.
 * Bit-exact.
 */
int mnb_dequant(const void *packed, int64_t N, int64_t K, int bits, int block_size, int dtype,
                void *w, void *stream);

/*
 * Decode-step product, M = 1: y[N] = x[K] * D^T, the step graph's one new
 * position ("Qwen3-ASR-0.6B ONNX for the browser", section "Graph
 * contracts"). x [K] and y [N] are device buffers of dtype; packed is the
 * mnb_pack output for (N, K, block_size, dtype). Accumulates in float32 and
 * rounds y once to dtype.
 */
int mnb_gemv(const void *x, const void *packed, void *y,
             int64_t N, int64_t K, int bits, int block_size, int dtype, void *stream);

/*
 * Decode-step product fused with a greedy argmax, for the LM head: the
 * decoder emits logits for the last position only and decoding picks the
 * largest one until an end token ("Qwen3-ASR-0.6B ONNX for the browser",
 * sections "Graph contracts" and "Validation"; "Qwen3-ASR-1.7B ONNX", section
 * "Inference Pipeline"). Computes the same y as mnb_gemv (rounded to dtype)
 * and writes to *index (device int64) the n of its largest value, the lowest
 * such n on ties (-0 counts as +0; y is taken to be finite). y may be NULL:
 * then the logits are not written at all.
 *
 * workspace: device buffer of MNB_ARGMAX_WORKSPACE_BYTES bytes, 16-byte
 * aligned, any contents: it receives one partial result per workgroup,
 * which a second launch on the same stream reduces to the index. Calls that
 * run one after another may share it; calls that may overlap (different
 * streams) need workspaces of their own. index must be 8-byte aligned.
 * index may be NULL: then only the partial results are written (one launch),
 * for mnb_embed_gather_argmax to reduce.
 */
#define MNB_ARGMAX_WORKSPACE_BYTES 8192
int mnb_gemv_argmax(const void *x, const void *packed, void *y, int64_t *index, void *workspace,
                    int64_t N, int64_t K, int bits, int block_size, int dtype, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the same
 * product and argmax as mnb_gemv_argmax, with the per-workgroup partial
 * results kept in a device array the library holds instead of a caller
 * workspace. The array holds 768 slots (6 KB) per device, the most any
 * argmax launch uses, so no N or K within the documented limits is
 * rejected for its sake; a launch that would need more slots returns
 * MNB_ERR_SHAPE. The array is looked up once per device, on the first call
 * on that device; nothing is allocated or freed, and each device keeps its
 * copy until the process ends. Every call on a device shares that device's
 * array: calls that may overlap on one device (different streams) race and
 * must not be issued; calls one after another on one stream are safe. The
 * array needs no clearing: each call writes every slot whose value it
 * uses. Arguments, results and errors otherwise as mnb_gemv_argmax.
 */
int mnb_gemv_argmax_noalloc(const void *x, const void *packed, void *y, int64_t *index,
                            int64_t N, int64_t K, int bits, int block_size, int dtype, void *stream);

/*
 * The step before the product in decode: the next input embeddings, as
 * int8 rows of the token table times each row's float32 scale ("Qwen3-ASR-
 * 0.6B ONNX for the browser", section "Building the prompt": an int8 row
 * times its embed scale, in float32 or float16).
 *   out[t][h] = table[ids[t]][h] * row_scales[ids[t]], t < T, h < H,
 * the exact product rounded once (to nearest even) to dtype.
 * table: device int8 [V][H]; row_scales: device float32 [V]; ids: device
 * int64 [T]; out: device dtype [T][H]. H must be a positive multiple of 16
 * (MNB_ERR_SHAPE otherwise); T = 0 enqueues nothing. An id outside [0, V)
 * gives a row of zeros. Pointers 16-byte aligned (ids: 8).
 */
int mnb_embed_gather(const int8_t *table, const float *row_scales, const int64_t *ids, int64_t T, int64_t V,
                     int64_t H, int dtype, void *out, void *stream);

/*
 * One greedy decoding step's hand-over from the LM head to the next input
 * embedding (the token the largest logit names, "Qwen3-ASR-1.7B ONNX",
 * section "Inference Pipeline", and its int8 row times its embed scale,
 * "Qwen3-ASR-0.6B ONNX for the browser", section "Building the prompt"):
 * reduces the partial results that mnb_gemv_argmax left in `workspace`
 * (called with index NULL and N = V, earlier on the same stream) to the
 * index of the largest logit, the lowest on ties, writes it to *index
 * (device int64, 8-byte aligned) unless index is NULL, and writes that
 * token's embedding to out [H] exactly as mnb_embed_gather with one id.
 * One launch: the argmax's own reducing launch moves into this one.
 * table, row_scales, H, dtype and alignment as mnb_embed_gather; workspace
 * as mnb_gemv_argmax (not modified here).
 */
int mnb_embed_gather_argmax(const int8_t *table, const float *row_scales, const void *workspace, int64_t *index,
                            int64_t V, int64_t H, int dtype, void *out, void *stream);

/*
 * General product for any M >= 1: Y[M][N] = X[M][K] * D^T, X and Y
 * row-major device buffers in dtype; only the weights are quantized and the
 * activations enter as they are ("sherpa-onnx STT int4", section "Why int4
 * rather than the usual int8"). M = 1 runs the decode kernel; float16 with
 * M >= 2 runs the matrix-core (MFMA) kernel that dequantizes weight tiles
 * and feeds fp16 MFMA with float32 accumulation; float32 with M >= 2 runs a
 * vector kernel. A single matrix-core call picks its output tile from a
 * cost model of one product running alone: the tall tiles that grouped
 * plans use, or 64-row tiles when M spans several of them and the tall
 * tiles would leave much of the GPU idle. The tile does not change the
 * float32 sum any output element is built from, so the result is the same
 * either way.
 */
int mnb_gemm(const void *x, const void *packed, void *y,
             int64_t M, int64_t N, int64_t K, int bits, int block_size, int dtype, void *stream);

/*
 * Split-K form of mnb_gemm, for a product too small to fill the GPU by its
 * output tiles alone (a single linear of a prefill). Same product, same
 * arguments as mnb_gemm, plus a caller workspace: the matrix-core kernel
 * (float16, M >= 2) splits K into `ksplit` contiguous ranges of whole
 * 128-input tiles, each workgroup writes the float32 partial sums of one
 * range into the workspace, and a second launch adds the ranges in a fixed
 * order (range 0 first) and rounds once to float16. The result is
 * deterministic (the same bits on every call with the same arguments); it
 * can differ from mnb_gemm's in the last bit, since the float32 sums are
 * grouped differently. Other calls (M = 1, float32) run exactly as
 * mnb_gemm and ignore the workspace.
 *
 * ksplit: 0 = the library's choice (the split, and the output tile as in
 * mnb_gemm, with the lowest time in a cost model of one product running
 * alone; none when the output tiles already fill the GPU); 1 = no split
 * (one launch, as mnb_gemm);
 * 2..MNB_MAX_KSPLIT = that many ranges, capped at the number of 128-input
 * tiles. Anything else: MNB_ERR_INVALID.
 *
 * mnb_gemm_split_k_workspace_bytes: the workspace bytes a call with these
 * arguments needs (0 when it splits nothing, or when the arguments are
 * invalid). workspace: device, 16-byte aligned, at least that many bytes
 * (MNB_ERR_INVALID if workspace_bytes is smaller; may be NULL when 0 is
 * needed); its contents are overwritten, and calls that may overlap must
 * not share it.
 */
#define MNB_MAX_KSPLIT 16
size_t mnb_gemm_split_k_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits, int block_size, int dtype,
                                        int ksplit);
int mnb_gemm_split_k(const void *x, const void *packed, void *y, void *workspace, size_t workspace_bytes,
                     int64_t M, int64_t N, int64_t K, int bits, int block_size, int dtype, int ksplit,
                     void *stream);

/*
 * Int8 compute mode. The published int4 exports set an accuracy level of 4
 * ("Qwen3-ASR-0.6B ONNX for the browser", section "Pick a variant";
 * "sherpa-onnx STT int4", section "whisper-small"), read here as
 * MatMulNBits' int8 compute setting: the activations are quantized per
 * (row, block of block_size inputs) to symmetric int8, in float32,
 *   a_s = amax / 127,  qa = clamp(rint(x / a_s), -127, 127)
 * (round to nearest even; a block of zeros gets a_s = 0, qa = 0), and
 *   Y[m][n] = sum_b s[n][b] * a_s[m][b] * sum_{k in b} (q[n][k] - zp[n][b]) * qa[m][k],
 * the block sums exact in integers, the scaling and the sum over blocks in
 * float32, rounded once to dtype.
 *
 * mnb_gemm_i8_workspace_bytes: device workspace mnb_gemm_i8 needs for M
 * rows of K inputs (quantized activations, their scales and chunk sums);
 * 0 if the arguments are invalid.
 *
 * mnb_quantize_act_i8: the quantizer alone (for tests and for callers that
 * keep quantized activations). x: device [M][K] dtype; qa: device int8
 * [M][K] (8-byte aligned); scales: device float32 [M][K / block_size].
 *
 * mnb_gemm_i8: the product, any M >= 1. x, y: device row-major [M][K],
 * [M][N] dtype; packed: mnb_pack output. M >= 2: workspace is device
 * memory, 16-byte aligned, at least mnb_gemm_i8_workspace_bytes(M, K,
 * block_size) bytes (MNB_ERR_INVALID if workspace_bytes is smaller); its
 * contents are overwritten and it must not be shared by calls that may
 * overlap; two launches on `stream` (quantize, product). M = 1 (decode):
 * one launch whose workgroups quantize x in their own LDS, with the
 * quantizer's arithmetic (same codes and scales); workspace is not used
 * (may be NULL; mnb_gemm_i8_workspace_bytes returns 0). Nothing is
 * allocated.
 *
 * mnb_plan_grouped_i8 (declared with the grouped plans below):
 * mnb_plan_grouped for the int8 mode. Every problem
 * must have M = 1 (MNB_ERR_SHAPE otherwise): the whole decode step runs as
 * one launch of the decode schedule, each workgroup quantizing the vector
 * of the product it is in. Run the plan with mnb_gemm_grouped; the outputs
 * equal single mnb_gemm_i8 calls bit for bit.
 */
size_t mnb_gemm_i8_workspace_bytes(int64_t M, int64_t K, int block_size);
int mnb_quantize_act_i8(const void *x, int64_t M, int64_t K, int block_size, int dtype, int8_t *qa, float *scales,
                        void *stream);
int mnb_gemm_i8(const void *x, const void *packed, void *y, void *workspace, size_t workspace_bytes,
                int64_t M, int64_t N, int64_t K, int bits, int block_size, int dtype, void *stream);

/*
 * Grouped execution: many independent products in one launch per kernel
 * class (one for the M = 1 problems, one for the M >= 2 problems). All
 * problems of a plan share bits, block_size and dtype.
 */
typedef struct mnb_problem {
    const void *x;      /* device, [M][K] dtype                          */
    const void *packed; /* device, mnb_pack output for (N, K)            */
    void *y;            /* device, [M][N] dtype                          */
    int64_t M, N, K;
} mnb_problem;

/* Bytes of a plan for `count` problems (0 if count is out of range 1..65536). */
size_t mnb_plan_bytes(int count);

/*
 * Host only: validate `problems[0..count)` and write a plan (a position-
 * independent byte image of mnb_plan_bytes(count) bytes) into the HOST
 * buffer `plan`. The caller copies that image to device memory unchanged.
 */
int mnb_plan_grouped(const mnb_problem *problems, int count, int bits, int block_size, int dtype,
                     void *plan, size_t plan_bytes);

/* The int8 compute mode's plan (decode products only; described with
 * mnb_gemm_i8 above). Same arguments and plan image as mnb_plan_grouped. */
int mnb_plan_grouped_i8(const mnb_problem *problems, int count, int bits, int block_size, int dtype,
                        void *plan, size_t plan_bytes);

/* Kernel launches mnb_gemm_grouped issues for a plan (one per kernel class
 * and tile variant present), or -1 if `plan_host` is not a valid plan. Host only. */
int mnb_plan_launches(const void *plan_host);

/*
 * Run a plan. plan_host: the host image written by mnb_plan_grouped (read
 * for launch geometry); plan_device: a device copy of the same bytes (read
 * by the kernels). The two must be identical; the host copy is re-checked.
 */
int mnb_gemm_grouped(const void *plan_host, const void *plan_device, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MNB_H */

"""MatMulNBits oracle: RTN block quantization, nibble packing, exact
dequantization and a float64 matmul.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain NumPy; no
blocking, fusion or reordering beyond what each definition states.

Notation, following the model-card pages ("Mega-ASR INT4 ONNX", section
"Conversion details"; "Qwen3-ASR-0.6B ONNX for the browser", section "Pick a
variant"): a weight W has N output rows and K inputs; blocks of `bs` (32, 64,
128 or 256) consecutive inputs of one row share one scale `s` and one 4-bit zero
point `zp`; codes `q` are 4-bit unsigned. MatMulNBits computes
Y[M, N] = X[M, K] @ D[N, K]^T with D = (q - zp) * s.

Readings where the pages are silent (each one is listed in the design notes):
  * the block extent includes zero: lo = min(0, min w), hi = max(0, max w);
  * s = (hi - lo) / 15 computed in float64, then rounded once (round half to
    even) to the scale dtype; zp and q are computed from that stored scale;
  * zp = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + zp, 0, 15),
    rint = round half to even;
  * a scale that rounds to zero gives zp = 0 and q = 0 for its block;
  * packing is low nibble first: byte j of a row holds element 2j in bits
    0-3 and element 2j+1 in bits 4-7; zero points of a row are packed the
    same way, an odd block count padded with a zero nibble.
"""

import math

import numpy as np

BITS = 4
QMAX = (1 << BITS) - 1  # 15: largest 4-bit unsigned code


def _blocks(shape_k, block_size):
    if block_size <= 0 or shape_k % block_size != 0:
        raise ValueError(f"K={shape_k} is not a positive multiple of block_size={block_size}")
    return shape_k // block_size


# ---------------------------------------------------------------------------
# Quantization (RTN), per row and per block along K.
# ---------------------------------------------------------------------------

def rtn_quantize(w, block_size, scale_dtype):
    """Round-to-nearest asymmetric 4-bit quantization of W[N, K].

    The pages name the quantizer (round-to-nearest at block 32 on the
    Qwen3-ASR-0.6B page, section "Pick a variant"; at block 64 on the
    merged-decoder page, section "Provenance") and say it is asymmetric
    ("Mega-ASR INT4 ONNX", section "Conversion details"). Per block:

      1. lo = min(0, min w), hi = max(0, max w)
      2. s  = round_to_scale_dtype((hi - lo) / 15)          (float64 divide)
      3. zp = clamp(rint(-lo / s), 0, 15)
      4. q  = clamp(rint(w / s) + zp, 0, 15)
    A block whose stored scale is zero gets zp = 0 and q = 0.

    Returns (q uint8 [N, K] in 0..15, scales [N, K/bs] of scale_dtype,
    zero_points uint8 [N, K/bs] in 0..15), all unpacked.
    """
    w = np.asarray(w)
    if w.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    n_rows, k = w.shape
    nb = _blocks(k, block_size)
    blocks = w.astype(np.float64).reshape(n_rows, nb, block_size)

    lo = np.minimum(blocks.min(axis=2), 0.0)
    hi = np.maximum(blocks.max(axis=2), 0.0)
    scale = ((hi - lo) / QMAX).astype(scale_dtype)  # one rounding to the stored dtype
    s = scale.astype(np.float64)

    live = s != 0.0
    s_div = np.where(live, s, 1.0)
    zp = np.clip(np.rint(-lo / s_div), 0, QMAX)
    zp = np.where(live, zp, 0.0)
    q = np.clip(np.rint(blocks / s_div[:, :, None]) + zp[:, :, None], 0, QMAX)
    q = np.where(live[:, :, None], q, 0.0)

    return (q.reshape(n_rows, k).astype(np.uint8),
            scale,
            zp.astype(np.uint8))


SYM_ZP = 1 << (BITS - 1)  # 8: the zero point of the symmetric format
SYM_QMAX = SYM_ZP - 1      # 7: largest magnitude the symmetric scale maps to


def rtn_quantize_symmetric(w, block_size, scale_dtype):
    """Round-to-nearest symmetric 4-bit quantization of W[N, K] (the
    is_symmetric setting of the conversion, "Mega-ASR INT4 ONNX", section
    "Conversion details"; the pages use it off, and define nothing more, so
    this follows the usual symmetric form). Per block:

      1. a = max |w|
      2. s = round_to_scale_dtype(a / 7)                     (float64 divide)
      3. q = clamp(rint(w / s) + 8, 0, 15)    (the zero point is fixed at 8)
    A block whose stored scale is zero gets q = 8.

    Returns (q uint8 [N, K], scales [N, K/bs], zero_points uint8 [N, K/bs]
    all equal to 8), so that dequantize() and matmul_nbits() apply as they are.
    """
    w = np.asarray(w)
    if w.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    n_rows, k = w.shape
    nb = _blocks(k, block_size)
    blocks = w.astype(np.float64).reshape(n_rows, nb, block_size)

    amax = np.abs(blocks).max(axis=2)
    scale = (amax / SYM_QMAX).astype(scale_dtype)  # one rounding to the stored dtype
    s = scale.astype(np.float64)

    live = s != 0.0
    s_div = np.where(live, s, 1.0)
    q = np.clip(np.rint(blocks / s_div[:, :, None]) + SYM_ZP, 0, QMAX)
    q = np.where(live[:, :, None], q, float(SYM_ZP))
    zp = np.full((n_rows, nb), SYM_ZP, dtype=np.uint8)
    return q.reshape(n_rows, k).astype(np.uint8), scale, zp


# ---------------------------------------------------------------------------
# Packing: two 4-bit values per byte, low nibble first.
# ---------------------------------------------------------------------------

def pack_nibbles(vals):
    """Pack 4-bit values along the last axis: out[..., j] = v[2j] | v[2j+1] << 4.

    An odd count is padded with a zero nibble.
    """
    v = np.asarray(vals, dtype=np.uint8)
    if np.any(v > QMAX):
        raise ValueError("values must be 4-bit")
    if v.shape[-1] % 2:
        pad = np.zeros(v.shape[:-1] + (1,), dtype=np.uint8)
        v = np.concatenate([v, pad], axis=-1)
    return (v[..., 0::2] | (v[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed, count):
    """Inverse of pack_nibbles: the first `count` 4-bit values along the last axis."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0x0F
    hi = p >> 4
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out[..., :count]


def pack_weight(q, zero_points):
    """Canonical stored form: (qweight [N, K/2], zero_points [N, ceil(nb/2)])."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[1] % 2:
        raise ValueError("K must be even")
    return pack_nibbles(q), pack_nibbles(zero_points)


def unpack_weight(qweight, packed_zp, k, block_size):
    """Canonical stored form back to (q [N, K], zp [N, K/bs]), both uint8."""
    nb = _blocks(k, block_size)
    return unpack_nibbles(qweight, k), unpack_nibbles(packed_zp, nb)


# ---------------------------------------------------------------------------
# Dequantization and the matmul.
# ---------------------------------------------------------------------------

def dequantize_exact(q, zero_points, scales, block_size):
    """D[n, k] = (q[n, k] - zp[n, k // bs]) * s[n, k // bs], exactly, as float64.

    The integer difference lies in [-15, 15] and the scale has at most 24
    significant bits, so the float64 product carries no rounding.
    """
    q = np.asarray(q).astype(np.int64)
    zp = np.repeat(np.asarray(zero_points).astype(np.int64), block_size, axis=1)
    s = np.repeat(np.asarray(scales).astype(np.float64), block_size, axis=1)
    return (q - zp).astype(np.float64) * s


def round_to(values, dtype):
    """Round float64 values once, half to even, to float32 or float16."""
    return np.asarray(values, dtype=np.float64).astype(dtype)


def dequantize(q, zero_points, scales, block_size, dtype=None):
    """Dequantized weights in `dtype` (default: the scale dtype), one rounding."""
    scales = np.asarray(scales)
    out_dtype = scales.dtype if dtype is None else dtype
    return round_to(dequantize_exact(q, zero_points, scales, block_size), out_dtype)


def matmul_nbits(x, q, zero_points, scales, block_size):
    """Y = X @ D^T in float64 (X [M, K] in any float dtype, converted exactly).

    Activations enter unquantized; only the weights are block-quantized
    ("sherpa-onnx STT int4", section "Why int4 rather than the usual int8").
    """
    x64 = np.asarray(x).astype(np.float64)
    d = dequantize_exact(q, zero_points, scales, block_size)
    return x64 @ d.T


def matmul_nbits_rows(x, q_rows, zp_rows, scale_rows, block_size):
    """Y[:, rows] for a subset of weight rows (the arrays hold only those rows)."""
    return matmul_nbits(x, q_rows, zp_rows, scale_rows, block_size)


def within_tolerance(y, y_ref, tol):
    """max |y - y_ref| <= tol * max |y_ref| over one call's whole output."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = float(np.max(np.abs(y - y_ref))) if y.size else 0.0
    ref = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    return err <= tol * ref, err, ref


# ---------------------------------------------------------------------------
# Int8 compute mode: activations quantized per block, integer dot products.
# ---------------------------------------------------------------------------

A8_QMAX = 127  # largest magnitude of a symmetric int8 activation code


def quantize_activations_i8(x, block_size):
    """Activations X[M, K] as symmetric int8 per (row, block of bs inputs).

    The conversions set an accuracy level of 4 ("Qwen3-ASR-0.6B ONNX for the
    browser", section "Pick a variant"; "sherpa-onnx STT int4", section
    "whisper-small") and the pages never say what it computes. Read as the
    int8 compute setting of MatMulNBits: each activation block is quantized
    symmetrically with the weights' block size, and the dot products run on
    integers. Per block, in float32 arithmetic (the precision the kernel
    takes these decisions in):

      1. amax = max |x| over the block            (exact in float32)
      2. a_s  = amax / 127                        (one float32 division, RNE)
      3. qa   = clamp(rint(x / a_s), -127, 127)   (x / a_s one float32 division)
    A block with amax = 0 gets a_s = 0 and qa = 0.

    Returns (qa int8 [M, K], a_s float32 [M, K/bs]).
    """
    x32 = np.asarray(x).astype(np.float32)
    m, k = x32.shape
    nb = _blocks(k, block_size)
    xb = x32.reshape(m, nb, block_size)
    amax = np.max(np.abs(xb), axis=2)
    a_s = (amax / np.float32(A8_QMAX)).astype(np.float32)
    safe = np.where(a_s > 0, a_s, np.float32(1))
    ratio = (xb / safe[:, :, None]).astype(np.float32)   # float32 operands: a float32 division
    qa = np.where(a_s[:, :, None] > 0, np.rint(ratio), 0.0)
    qa = np.clip(qa, -A8_QMAX, A8_QMAX).astype(np.int8).reshape(m, k)
    return qa, a_s


def matmul_nbits_i8(x, q, zero_points, scales, block_size):
    """Y[M, N] in the int8 compute mode:

      Y[m, n] = sum_b s[n, b] * a_s[m, b] * sum_{k in b} (q[n, k] - zp[n, b]) * qa[m, k]

    with (qa, a_s) = quantize_activations_i8(X). The integer block sums are
    exact (int64); scaling and the sum over blocks are float64.
    """
    qa, a_s = quantize_activations_i8(x, block_size)
    m, k = qa.shape
    n = np.asarray(q).shape[0]
    nb = _blocks(k, block_size)
    w = np.asarray(q).astype(np.int64) - np.repeat(np.asarray(zero_points).astype(np.int64), block_size, axis=1)
    isum = np.einsum("mbk,nbk->mnb", qa.astype(np.int64).reshape(m, nb, block_size),
                     w.reshape(n, nb, block_size))
    s = np.asarray(scales).astype(np.float64)
    return np.sum(isum.astype(np.float64) * a_s.astype(np.float64)[:, None, :] * s[None, :, :], axis=2)


# ---------------------------------------------------------------------------
# Storage accounting.
# ---------------------------------------------------------------------------

def packed_nbytes(n_rows, k, block_size, scale_bytes):
    """Bytes of one stored weight: codes + scales + packed zero points."""
    nb = _blocks(k, block_size)
    return n_rows * (k // 2) + n_rows * nb * scale_bytes + n_rows * math.ceil(nb / 2)


# ---------------------------------------------------------------------------
# Decode-step neighbours of the op.
# ---------------------------------------------------------------------------

def greedy_argmax(logits):
    """Greedy next token: index of the largest logit in each row, lowest index
    on ties ("Qwen3-ASR-0.6B ONNX for the browser", section "Building the
    prompt", step 5; the prefill and step graphs emit last-position logits,
    section "Graph contracts")."""
    a = np.asarray(logits, dtype=np.float64)
    return np.argmax(a, axis=-1)


def embedding_dequant(table_i8, row_scales, ids, dtype):
    """Rows of an int8 embedding table times their per-row scale, rounded
    once to `dtype` ("Qwen3-ASR-0.6B ONNX for the browser", section "Building
    the prompt", step 4: int8 row times embed_scales[id], fp32 or fp16).

    The int8 value times a float32 scale needs at most 32 significant bits,
    so the float64 product is exact and the single rounding is to `dtype`.
    """
    t = np.asarray(table_i8, dtype=np.int8)
    s = np.asarray(row_scales, dtype=np.float32)
    ids = np.asarray(ids, dtype=np.int64)
    exact = t[ids].astype(np.float64) * s[ids].astype(np.float64)[:, None]
    return round_to(exact, dtype)

"""CPU oracle for MatMulNBits, the weight-only block-wise 4-bit matmul.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark may import this package. The
GPU library never calls it, and it shares no code, table or constant with the
HIP sources.

Everything here is plain NumPy in float64 (integers for the codes), written
to be read against the model-card pages that describe the format:

* "Mega-ASR INT4 ONNX" (VidraAI/mega-asr-onnx), section "Conversion details":
  4-bit, asymmetric, block size 32 along the reduction axis.
* "Qwen3-ASR-0.6B ONNX for the browser", section "Pick a variant": RTN
  (round-to-nearest) quantization of MatMul weights, block 32; fp16 float
  tensors in the q4f16 variant.
* "sherpa-onnx STT int4", section "Why int4 rather than the usual int8":
  only the weights are quantized, block by block; activations stay as they are.
* "qwen3-asr-0.6b-onnx-int4-merged", section "Provenance": RTN, block 64.

The pages name the format but print no formula and no worked example, so the
plainest reading is written out and every reading is listed in the design
notes. The functions and what pins each one (tests/test_oracle_pins.py):

  rtn_quantize        pinned: nearest-grid-point brute force, on-grid blocks,
                      RNE tie block, single-signed and all-zero blocks,
                      round-trip error bound
  rtn_quantize_symmetric
                      pinned: on-grid blocks, RNE tie, all-zero block,
                      nearest-grid-point brute force, no clipping
  pack_nibbles /
  unpack_nibbles      pinned: all 256 byte values against divmod, round trip
  dequantize_exact    pinned: Fraction arithmetic, integrality of D/s
  round_to            pinned: an independent integer RNE routine
  matmul_nbits        pinned: Fraction-exact tiny shapes, int64 special case,
                      pure-Python triple loop
  packed_nbytes       pinned: the 340 MB decoder-weights size printed on the
                      merged-decoder page
  greedy_argmax,
  embedding_dequant   pinned: brute force and closed forms (see the module)
  quantize_activations_i8
                      pinned: exact-rational division with an independent
                      float32 rounding routine, ties, extreme and all-zero
                      blocks, round-trip bound
  matmul_nbits_i8     pinned: equality with matmul_nbits where the int8
                      activations are exact, Fraction-exact tiny shapes
"""

from .mnb_oracle import (  # noqa: F401
    QMAX,
    rtn_quantize,
    rtn_quantize_symmetric,
    SYM_ZP,
    pack_nibbles,
    unpack_nibbles,
    pack_weight,
    unpack_weight,
    dequantize_exact,
    round_to,
    dequantize,
    matmul_nbits,
    matmul_nbits_rows,
    within_tolerance,
    packed_nbytes,
    greedy_argmax,
    embedding_dequant,
    A8_QMAX,
    quantize_activations_i8,
    matmul_nbits_i8,
)

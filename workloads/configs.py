"""Shapes of the MatMulNBits workloads: which linears, at which M, block size
and activation dtype. Data only: no quantization or matmul arithmetic.

Linear shapes are (N outputs, K inputs), i.e. W is [N, K] and Y = X @ W^T.

* Qwen3-ASR 0.6B decoder: hidden 1024, 28 layers, 8 KV heads of 128
  ("Qwen3-ASR-0.6B ONNX for the browser", section "Graph contracts": the
  [28, 1, 8, S, 128] KV tensors and the 1024-wide embeddings).
* Qwen3-ASR 1.7B decoder: hidden 2048 ("qwen3-asr-1.7b-onnx", section
  "Files": the [151936, 2048] embedding table), 28 layers ("Mega-ASR INT4
  ONNX", section "GPTQ calibration": 56 per-layer key/value tensors).
* LM head: vocabulary 151936, last position only ("Qwen3-ASR-0.6B ONNX for
  the browser", section "Graph contracts": logits [1, 1, 151936]).
* Whisper-small encoder: width 768, MLP 3072, 12 layers, block 64
  ("sherpa-onnx STT int4", section "whisper-small").
* Prefill M = 410: audio tokens for 30 s (3000 mel frames) by the formula in
  "Qwen3-ASR-0.6B ONNX for the browser", section "Building the prompt", step
  2, gives 390; plus about 20 prompt rows (steps 3 and 6).
* Mid-M chunk M = 62: a 3.2 s command gives 42 audio rows by the same
  formula, plus about 20 prompt rows; the decoder that takes such chunks
  after a cached prefix is the merged one, quantized at block 64
  ("qwen3-asr-0.6b-onnx-int4-merged", sections "Why" and "Provenance").
* Format variants: the same decode step at block 128, and with symmetric
  codes (the is_symmetric setting, "Mega-ASR INT4 ONNX", section
  "Conversion details", which those exports leave off).
"""

from dataclasses import dataclass, field

VOCAB = 151936

QWEN3_06B_LAYER = (
    ("q", 2048, 1024), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 1024, 2048),
    ("gate", 3072, 1024), ("up", 3072, 1024), ("down", 1024, 3072),
)
QWEN3_17B_LAYER = (
    ("q", 2048, 2048), ("k", 1024, 2048), ("v", 1024, 2048), ("o", 2048, 2048),
    ("gate", 6144, 2048), ("up", 6144, 2048), ("down", 2048, 6144),
)
WHISPER_SMALL_LAYER = (
    ("q", 768, 768), ("k", 768, 768), ("v", 768, 768), ("o", 768, 768),
    ("fc1", 3072, 768), ("fc2", 768, 3072),
)


def audio_tokens(mel_frames):
    """Audio-token count for T mel frames ("Qwen3-ASR-0.6B ONNX for the
    browser", section "Building the prompt", step 2): three stride-2 halvings
    of T mod 100 plus 13 tokens per full 100 frames."""
    def conv(t):
        return (t + 1) // 2
    return conv(conv(conv(mel_frames % 100))) + 13 * (mel_frames // 100)


@dataclass(frozen=True)
class Linear:
    layer: int      # -1 for the LM head
    proj: str
    n: int
    k: int


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    m: int
    block_size: int
    dtype: str              # activation dtype == scale dtype: "f32" or "f16"
    linears: tuple = field(default_factory=tuple)
    symmetric: bool = False  # no zero points (fixed zero point 8)

    @property
    def kind(self):
        return "decode" if self.m == 1 else "prefill"


def _stack(layer_shapes, n_layers, lm_head_k=None):
    out = [Linear(layer, p, n, k) for layer in range(n_layers) for (p, n, k) in layer_shapes]
    if lm_head_k is not None:
        out.append(Linear(-1, "lm_head", VOCAB, lm_head_k))
    return tuple(out)


CONFIGS = (
    Config(0, "gemv-1024x3072-bs32-f32", 1, 32, "f32", (Linear(0, "single", 3072, 1024),)),
    Config(1, "qwen3-0.6b-decode-step", 1, 32, "f16", _stack(QWEN3_06B_LAYER, 28, 1024)),
    Config(2, "qwen3-1.7b-decode-step", 1, 32, "f16", _stack(QWEN3_17B_LAYER, 28, 2048)),
    Config(3, "qwen3-1.7b-prefill-m410", 410, 32, "f16", _stack(QWEN3_17B_LAYER, 28)),
    Config(4, "whisper-small-encoder-m1500-bs64", 1500, 64, "f16", _stack(WHISPER_SMALL_LAYER, 12)),
    Config(5, "qwen3-0.6b-chunk-m62-bs64", 62, 64, "f16", _stack(QWEN3_06B_LAYER, 28)),
    # format variants of the 0.6B decode step: block 128, and symmetric codes
    Config(6, "qwen3-0.6b-decode-step-bs128", 1, 128, "f16", _stack(QWEN3_06B_LAYER, 28, 1024)),
    Config(7, "qwen3-0.6b-decode-step-symmetric", 1, 32, "f16", _stack(QWEN3_06B_LAYER, 28, 1024), True),
)

PROJ_INDEX = {p: i for i, p in enumerate(
    ("q", "k", "v", "o", "gate", "up", "down", "fc1", "fc2", "lm_head", "single"))}


def by_name(name):
    for c in CONFIGS:
        if c.name == name or str(c.index) == str(name):
            return c
    raise KeyError(name)

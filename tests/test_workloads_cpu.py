"""The benchmark's workloads have the sizes their definitions state: the
algorithmic bytes and FLOPs per step of each configuration (to the precision
they are quoted at), the linear counts, and the prefill M from the pages'
audio-token formula. A wrong shape, block size or dtype in a workload would
change what the benchmark measures; these pins catch it without a GPU."""

import pytest

from block_wise_int4_amd import workload as wl
from workloads import configs

# (name, linears, algorithmic bytes, relative precision of the quoted bytes, FLOPs, precision)
QUOTED = [
    ("gemv-1024x3072-bs32-f32", 1, 2_031_616, 0.0, 6.29e6, 1e-3),
    ("qwen3-0.6b-decode-step", 197, 346.12e6, 2e-5, 1.192e9, 1e-3),
    ("qwen3-1.7b-decode-step", 197, 997.12e6, 1e-5, 3.441e9, 1e-3),
    ("qwen3-1.7b-prefill-m410", 196, 1708e6, 1e-3, 1.1556e12, 1e-4),
    ("whisper-small-encoder-m1500-bs64", 72, 543.4e6, 1e-3, 254.8e9, 1e-3),
]


@pytest.mark.parametrize("name,count,nbytes,bprec,flops,fprec", QUOTED)
def test_workload_sizes(name, count, nbytes, bprec, flops, fprec):
    cfg = configs.by_name(name)
    assert len(cfg.linears) == count
    b = wl.algorithmic_bytes(cfg)
    f = wl.flops(cfg)
    assert abs(b - nbytes) <= bprec * nbytes + 0.5, b
    assert abs(f - flops) <= fprec * flops, f


def test_decode_step_bytes_by_hand():
    # 28 layers of q 2048x1024, k/v 1024x1024, o 1024x2048, gate/up 3072x1024,
    # down 1024x3072, plus the 151936x1024 LM head; block 32, fp16 scales,
    # packed 4-bit zero points, fp16 x and y
    shapes = [(2048, 1024), (1024, 1024), (1024, 1024), (1024, 2048), (3072, 1024), (3072, 1024), (1024, 3072)]
    lin = shapes * 28 + [(151936, 1024)]
    total = 0
    for n, k in lin:
        blocks = k // 32
        total += n * k // 2 + n * blocks * 2 + n * ((blocks + 1) // 2) + k * 2 + n * 2
    assert wl.algorithmic_bytes(configs.by_name("qwen3-0.6b-decode-step")) == total


def test_prefill_rows_follow_the_audio_token_formula():
    # 30 s of audio = 3000 mel frames -> 390 audio rows, plus about 20 prompt rows
    assert configs.audio_tokens(3000) == 390
    assert configs.by_name("qwen3-1.7b-prefill-m410").m == 390 + 20
    # a 3.2 s command: 320 frames -> 42 audio rows, plus about 20 prompt rows
    assert configs.audio_tokens(320) == 42
    assert configs.by_name("qwen3-0.6b-chunk-m62-bs64").m == 42 + 20


def test_format_variants_change_only_the_format():
    base = configs.by_name("qwen3-0.6b-decode-step")
    for name, bs, sym in (("qwen3-0.6b-decode-step-bs128", 128, False),
                          ("qwen3-0.6b-decode-step-symmetric", 32, True)):
        v = configs.by_name(name)
        assert v.linears == base.linears and v.m == base.m and v.dtype == base.dtype
        assert (v.block_size, v.symmetric) == (bs, sym)

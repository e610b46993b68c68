"""The argmax entry point that allocates nothing (mnb_gemv_argmax_noalloc,
partial results in the library's per-device array) against the one that
takes a caller workspace (mnb_gemv_argmax), through the C ABI: two calls in
a row, the second on a smaller input, so that the second call would read
the first call's leftover slots if it read more than its own."""

import pytest
import torch

from block_wise_int4_amd import mnb
from workloads import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {"f16": torch.float16, "f32": torch.float32}


def packed_case(n, k, bs, dt, seed):
    w, x = synth.random_case(seed, 1, n, k, dt)
    gq, gs, gz = mnb.mnb_quantize_rtn(torch.from_numpy(w).to(DEV), bs, TD[dt])
    pw = mnb.mnb_pack(gq, gs, gz, n, k, bs)
    return torch.from_numpy(x).to(DEV).reshape(-1), pw


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_noalloc_argmax_matches_workspace_call(dt):
    ws = mnb.argmax_workspace(DEV)
    # 151936 rows use all 768 slots; the next call uses 47, then 3
    for n, k, bs, seed in ((151936, 1024, 32, 11), (3000, 512, 64, 12), (200, 2048, 32, 13)):
        print(f"noalloc argmax {dt} N={n} K={k} bs={bs}", flush=True)
        x, pw = packed_case(n, k, bs, dt, seed)
        i_ref, y_ref = mnb.mnb_gemv_argmax(x, pw, ws, logits=True)
        i_na, y_na = mnb.mnb_gemv_argmax_noalloc(x, pw, logits=True)
        i_nl = mnb.mnb_gemv_argmax_noalloc(x, pw)
        torch.cuda.synchronize()
        assert i_na.item() == i_ref.item(), (n, i_na.item(), i_ref.item())
        assert i_nl.item() == i_ref.item(), (n, i_nl.item(), i_ref.item())
        assert torch.equal(y_na, y_ref)
        # the index names a largest logit, the lowest such index
        top = y_ref.float().max()
        assert y_ref[i_ref.item()].float() == top
        assert not bool((y_ref[: i_ref.item()].float() == top).any())


def test_noalloc_argmax_rejects_bad_arguments_and_enqueues_nothing():
    x, pw = packed_case(64, 128, 32, "f16", 3)
    idx = torch.full((1,), -7, dtype=torch.int64, device=DEV)
    bad = mnb.PackedWeight(pw.packed, 64, 96, 64, torch.float16)      # K % bs != 0
    with pytest.raises(mnb.MnbError) as ei:
        mnb.mnb_gemv_argmax_noalloc(torch.zeros(96, dtype=torch.float16, device=DEV), bad, index=idx)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert idx.item() == -7

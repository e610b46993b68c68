"""GPU: the LM-head product fused with a greedy argmax (mnb_gemv_argmax).

The index is unique given the logits, so it is checked exactly against the
first maximum of the logits the same call writes (which must equal
mnb_gemv's bit for bit). Against the oracle the logits agree only to the
output tolerance, so there the check is that the chosen row's exact logit
is within that tolerance of the largest exact logit. A planted tie pins the
lowest-index rule.
"""

import numpy as np
import pytest
import torch

import oracle
from block_wise_int4_amd import mnb
from workloads import configs, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {np.float16: 2e-3, np.float32: 1e-5}


def _packed(w, bs, dt):
    q, s, zp = oracle.rtn_quantize(w, bs, dt)
    qw, pz = oracle.pack_weight(q, zp)
    n, k = w.shape
    pw = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(pz).to(DEV),
                      n, k, bs)
    return pw, (q, s, zp)


def _check(x, pw, oracle_parts, bs, dt, expect=None):
    xd = torch.from_numpy(x.reshape(-1)).to(DEV)
    ws = mnb.argmax_workspace(DEV)
    y_plain = mnb.mnb_gemv(xd, pw)
    idx, y = mnb.mnb_gemv_argmax(xd, pw, ws, logits=True)
    idx_only = mnb.mnb_gemv_argmax(xd, pw, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_plain), "fused logits differ from mnb_gemv"
    logits = y.float().cpu().numpy()
    i = int(idx.item())
    assert i == int(np.argmax(logits)), "index is not the first maximum of the logits"
    assert int(idx_only.item()) == i
    q, s, zp = oracle_parts
    ref = oracle.matmul_nbits(x.reshape(1, -1), q, zp, s, bs)[0]
    assert ref[i] >= ref.max() - TOL[dt] * np.abs(ref).max()
    if expect is not None:
        assert i == expect
    return i


@pytest.mark.parametrize("n,k,bs,dt", [(3000, 1024, 32, np.float16), (20011, 2048, 32, np.float16),
                                       (4099, 512, 64, np.float32), (17, 128, 32, np.float16),
                                       (1, 32, 32, np.float16), (777, 4160, 32, np.float32)])
def test_argmax_matches_logits_and_oracle(n, k, bs, dt):
    w, x = synth.random_case(n * 7 + k, 1, n, k, "f16" if dt == np.float16 else "f32")
    pw, parts = _packed(w, bs, dt)
    _check(x, pw, parts, bs, dt)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_argmax_tie_takes_lowest_index(dt):
    n, k, bs = 2500, 1024, 32
    w, x = synth.random_case(4242, 1, n, k, "f16" if dt == np.float16 else "f32")
    # row 1700 points along x (far the largest logit); row 9 is an identical copy
    w[1700] = (x[0].astype(np.float32) / np.abs(x[0]).max() * 0.05).astype(np.float32)
    w[9] = w[1700]
    pw, parts = _packed(w, bs, dt)
    _check(x, pw, parts, bs, dt, expect=9)


@pytest.mark.parametrize("n", [5000, 151936])
def test_argmax_workspace_serves_consecutive_calls(n):
    k, bs, dt = 1024, 32, np.float16
    w, _ = synth.random_case(77, 1, n, k, "f16")
    pw, parts = _packed(w, bs, dt)
    ws = mnb.argmax_workspace(DEV)
    picks = []
    for seed in range(4):
        _, x = synth.random_case(1000 + seed, 1, n, k, "f16")
        xd = torch.from_numpy(x.reshape(-1)).to(DEV)
        picks.append(mnb.mnb_gemv_argmax(xd, pw, ws))
        y = mnb.mnb_gemv(xd, pw)
        torch.cuda.synchronize()
        assert int(picks[-1].item()) == int(np.argmax(y.float().cpu().numpy()))


def test_argmax_full_size_lm_head():
    cfg = configs.CONFIGS[1]
    lin = [l for l in cfg.linears if l.proj == "lm_head"][0]
    print(f"LM head {lin.n}x{lin.k}", flush=True)
    w, x = synth.linear_inputs(cfg, lin)
    pw, parts = _packed(w, cfg.block_size, np.float16)
    _check(x, pw, parts, cfg.block_size, np.float16)


def test_argmax_graph_replays():
    """The fused call captured in a HIP graph and replayed with new inputs
    copied into the captured buffer: every replay's index matches the eager
    product's argmax (both launches captured; nothing needs clearing between
    replays: every slot the finishing launch reads is written first)."""
    n, k, bs = 151936, 1024, 32
    w, _ = synth.random_case(600, 1, n, k, "f16")
    pw, parts = _packed(w, bs, np.float16)
    ws = mnb.argmax_workspace(DEV)
    xin = torch.empty(k, dtype=torch.float16, device=DEV)
    idx = torch.empty(1, dtype=torch.int64, device=DEV)
    _, x0 = synth.random_case(601, 1, n, k, "f16")
    xin.copy_(torch.from_numpy(x0.reshape(-1)))
    mnb.mnb_gemv_argmax(xin, pw, ws, index=idx)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mnb.mnb_gemv_argmax(xin, pw, ws, index=idx)
    torch.cuda.synchronize()
    for seed in range(4):
        _, x = synth.random_case(610 + seed, 1, n, k, "f16")
        xin.copy_(torch.from_numpy(x.reshape(-1)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y = mnb.mnb_gemv(xin, pw)
        torch.cuda.synchronize()
        assert int(idx.item()) == int(np.argmax(y.float().cpu().numpy())), f"replay {seed}"

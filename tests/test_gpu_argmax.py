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


@pytest.mark.parametrize("n,k,bs,dt,hidden", [(151936, 1024, 32, np.float16, 1024), (3000, 1024, 32, np.float16, 64),
                                              (4099, 512, 64, np.float32, 2048), (17, 128, 32, np.float16, 16),
                                              (1, 32, 32, np.float32, 32)])
def test_gather_of_the_argmax_equals_the_two_step_form(n, k, bs, dt, hidden):
    """The LM head's partial results (one launch) handed to the gather, which
    reduces them itself: the same index as the two-launch argmax, and the
    same embedding row as mnb_embed_gather of that index, bit for bit; the
    index is also the first maximum of the call's own logits."""
    w, x = synth.random_case(n * 3 + k, 1, n, k, "f16" if dt == np.float16 else "f32")
    pw, _ = _packed(w, bs, dt)
    table, scales, _ = synth.embedding_inputs(n + hidden, n, hidden, 1)
    td, sd = torch.from_numpy(table).to(DEV), torch.from_numpy(scales).to(DEV)
    tdt = torch.float16 if dt == np.float16 else torch.float32
    xd = torch.from_numpy(x.reshape(-1)).to(DEV)
    ws = mnb.argmax_workspace(DEV)
    idx_ref = mnb.mnb_gemv_argmax(xd, pw, ws)
    row_ref = mnb.mnb_embed_gather(td, sd, idx_ref, dtype=tdt)
    y = torch.empty(n, dtype=tdt, device=DEV)
    none, _ = mnb.mnb_gemv_argmax(xd, pw, ws, y=y, partial=True)
    assert none is None
    row, idx = mnb.mnb_embed_gather_argmax(td, sd, ws, dtype=tdt)
    torch.cuda.synchronize()
    assert int(idx.item()) == int(idx_ref.item()) == int(np.argmax(y.float().cpu().numpy()))
    assert torch.equal(row, row_ref)


def test_gather_of_the_argmax_tie_and_consecutive_steps():
    """Planted tie (lowest index wins) and two greedy steps in a row on one
    workspace, the second with a smaller LM head: each step's row and index
    come from its own product."""
    n, k, bs, hidden = 2500, 1024, 32, 128
    w, x = synth.random_case(777, 1, n, k, "f16")
    w[1700] = (x[0].astype(np.float32) / np.abs(x[0]).max() * 0.05).astype(np.float32)
    w[9] = w[1700]
    pw, _ = _packed(w, bs, np.float16)
    w2, x2 = synth.random_case(778, 1, 300, k, "f16")
    pw2, _ = _packed(w2, bs, np.float16)
    table, scales, _ = synth.embedding_inputs(31, n, hidden, 1)
    td, sd = torch.from_numpy(table).to(DEV), torch.from_numpy(scales).to(DEV)
    ws = mnb.argmax_workspace(DEV)
    mnb.mnb_gemv_argmax(torch.from_numpy(x.reshape(-1)).to(DEV), pw, ws, partial=True)
    row1, idx1 = mnb.mnb_embed_gather_argmax(td, sd, ws)
    x2d = torch.from_numpy(x2.reshape(-1)).to(DEV)
    mnb.mnb_gemv_argmax(x2d, pw2, ws, partial=True)
    row2, idx2 = mnb.mnb_embed_gather_argmax(td[:300].contiguous(), sd[:300].contiguous(), ws)
    idx2_ref = mnb.mnb_gemv_argmax(x2d, pw2, mnb.argmax_workspace(DEV))
    torch.cuda.synchronize()
    assert int(idx1.item()) == 9
    assert torch.equal(row1, mnb.mnb_embed_gather(td, sd, idx1))
    assert int(idx2.item()) == int(idx2_ref.item())
    assert torch.equal(row2, mnb.mnb_embed_gather(td, sd, idx2))


def test_gather_of_the_argmax_graph_replays():
    """The greedy hand-over (partial argmax, then the gather that reduces it)
    captured in a HIP graph and replayed with new inputs, with eager calls on
    the same workspace between replays: every replay's index and row equal
    the eager two-step form's."""
    n, k, bs, hidden = 151936, 1024, 32, 1024
    w, _ = synth.random_case(620, 1, n, k, "f16")
    pw, _ = _packed(w, bs, np.float16)
    table, scales, _ = synth.embedding_inputs(41, n, hidden, 1)
    td, sd = torch.from_numpy(table).to(DEV), torch.from_numpy(scales).to(DEV)
    ws = mnb.argmax_workspace(DEV)
    xin = torch.empty(k, dtype=torch.float16, device=DEV)
    idx = torch.empty(1, dtype=torch.int64, device=DEV)
    row = torch.empty((1, hidden), dtype=torch.float16, device=DEV)
    _, x0 = synth.random_case(621, 1, n, k, "f16")
    xin.copy_(torch.from_numpy(x0.reshape(-1)))
    mnb.mnb_gemv_argmax(xin, pw, ws, partial=True)
    mnb.mnb_embed_gather_argmax(td, sd, ws, out=row, index=idx)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mnb.mnb_gemv_argmax(xin, pw, ws, partial=True)
        mnb.mnb_embed_gather_argmax(td, sd, ws, out=row, index=idx)
    torch.cuda.synchronize()
    for seed in range(4):
        _, x = synth.random_case(630 + seed, 1, n, k, "f16")
        xin.copy_(torch.from_numpy(x.reshape(-1)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_idx, got_row = int(idx.item()), row.clone()
        ref_idx = mnb.mnb_gemv_argmax(xin, pw, ws)  # eager, on the same workspace
        ref_row = mnb.mnb_embed_gather(td, sd, ref_idx)
        torch.cuda.synchronize()
        assert got_idx == int(ref_idx.item()), f"replay {seed}"
        assert torch.equal(got_row, ref_row), f"replay {seed}"

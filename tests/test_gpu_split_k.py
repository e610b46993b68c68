"""GPU tests of the split-K product (mnb_gemm_split_k): K split into ranges
over workgroups, float32 partial sums added in a fixed order.

Parity: within the product tolerance (max |y - y_ref| <= 2e-3 * max |y_ref|)
of the oracle on small cases and of a float32 product of the call's own
dequantized weights (mnb_dequant, pinned bit-exact to the oracle elsewhere)
at full size. Determinism: repeated calls give the same bits; ksplit = 1 is
bitwise mnb_gemm. Ranges that start inside a metadata group of 8 tiles, a
ragged K tail and every block size are covered."""

import numpy as np
import pytest
import torch

import oracle
from block_wise_int4_amd import mnb
from workloads import configs, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3


def packed_case(m, n, k, bs, seed):
    w, x = synth.random_case(seed, m, n, k, "f16")
    q, s, zp = oracle.rtn_quantize(w, bs, np.float16)
    qw, pz = oracle.pack_weight(q, zp)
    pw = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(pz).to(DEV),
                      n, k, bs)
    return x, q, s, zp, pw


CASES = [  # (M, N, K, bs, ksplit)
    (2, 48, 1024, 32, 2),
    (17, 64, 2048, 64, 3),      # ranges 5 and 10 start inside a metadata group
    (40, 130, 4160, 32, 5),     # ragged K (33 tiles, the last half full)
    (64, 256, 1536, 128, 4),
    (65, 96, 2048, 256, 7),
    (200, 272, 3072, 32, 16),
    (410, 300, 2048, 64, 0),
]


@pytest.mark.parametrize("m,n,k,bs,ksplit", CASES)
def test_split_k_against_oracle(m, n, k, bs, ksplit):
    x, q, s, zp, pw = packed_case(m, n, k, bs, seed=m + n + k)
    ref = oracle.matmul_nbits(x, q, zp, s, bs)
    xt = torch.from_numpy(x).to(DEV)
    y = mnb.mnb_gemm_split_k(xt, pw, ksplit=ksplit)
    y2 = mnb.mnb_gemm_split_k(xt, pw, ksplit=ksplit)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "repeated split-K calls differ"
    ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), ref, TOL)
    assert ok, f"err {err:.3e} vs {TOL} * {mx:.3e}"


def test_split_k_one_is_mnb_gemm_bitwise():
    x, q, s, zp, pw = packed_case(100, 96, 2048, 32, seed=5)
    xt = torch.from_numpy(x).to(DEV)
    assert mnb.mnb_gemm_split_k_workspace_bytes(100, pw, 1) == 0
    y1 = mnb.mnb_gemm_split_k(xt, pw, ksplit=1)
    y0 = mnb.mnb_gemm(xt, pw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_split_k_decode_and_float32_run_as_mnb_gemm():
    """M = 1 and float32 products do not split: no workspace, mnb_gemm's bits."""
    x, q, s, zp, pw = packed_case(1, 64, 1024, 32, seed=6)
    assert mnb.mnb_gemm_split_k_workspace_bytes(1, pw, 0) == 0
    xt = torch.from_numpy(x).to(DEV)
    assert torch.equal(mnb.mnb_gemm_split_k(xt, pw, ksplit=4), mnb.mnb_gemm(xt, pw))
    w, x32 = synth.random_case(7, 5, 64, 1024, "f32")
    q, s, zp = oracle.rtn_quantize(w, 32, np.float32)
    qw, pz = oracle.pack_weight(q, zp)
    pw32 = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(pz).to(DEV),
                        64, 1024, 32)
    assert mnb.mnb_gemm_split_k_workspace_bytes(5, pw32, 4) == 0
    x32t = torch.from_numpy(x32).to(DEV)
    assert torch.equal(mnb.mnb_gemm_split_k(x32t, pw32, ksplit=4), mnb.mnb_gemm(x32t, pw32))


def test_split_k_workspace_too_small_is_refused():
    x, q, s, zp, pw = packed_case(64, 64, 2048, 32, seed=8)
    need = mnb.mnb_gemm_split_k_workspace_bytes(64, pw, 4)
    assert need >= 4 * 64 * 64 * 4
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(mnb.MnbError):
        mnb.mnb_gemm_split_k(torch.from_numpy(x).to(DEV), pw, workspace=ws, ksplit=4)


@pytest.mark.parametrize("ci", [3, 4, 5])
def test_split_k_full_size_linears(ci):
    """Every linear of a full-size prefill workload through the split-K call
    with the library's own choice of split (the per-linear schedule's
    launches): within tolerance of a float32 product of mnb_dequant's weights,
    and bitwise repeatable."""
    from block_wise_int4_amd import workload
    cfg = configs.CONFIGS[ci]
    print(f"config {cfg.name}: {len(cfg.linears)} linears", flush=True)
    data = workload.build_config(cfg, DEV, linears=cfg.linears[:7])
    ws = None
    for ld in data.linears:  # one layer: every projection shape of the workload
        need = mnb.mnb_gemm_split_k_workspace_bytes(cfg.m, ld.pw, 0)
        if need and (ws is None or ws.numel() < need):
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        y = mnb.mnb_gemm_split_k(ld.x, ld.pw, workspace=ws if need else None)
        y2 = mnb.mnb_gemm_split_k(ld.x, ld.pw, workspace=ws if need else None)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"{ld.lin}: repeated calls differ"
        d = mnb.mnb_dequant(ld.pw).float()
        ref = (ld.x.float() @ d.t()).double()
        err = (y.double() - ref).abs().max().item()
        mx = ref.abs().max().item()
        assert err <= TOL * mx, f"{ld.lin}: err {err:.3e} vs {TOL} * {mx:.3e}"
    del data
    torch.cuda.empty_cache()

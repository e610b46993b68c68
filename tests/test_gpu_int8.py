"""GPU parity of the int8 compute mode (the exports' accuracy level 4)
against the oracle: the activation quantizer bit-exact (codes and float32
scales), the product within tolerance of the oracle's exact-integer product
(max |y - y_ref| <= tol * max |y_ref|; tol = 2e-3 for float16 outputs, 1e-5
for float32: the block sums are exact on both sides, and what differs is the
float32 scaling and accumulation over K / block_size blocks plus the final
rounding to the output dtype)."""

import numpy as np
import pytest
import torch

import oracle
from block_wise_int4_amd import mnb
from workloads import configs, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {np.float16: 2e-3, np.float32: 1e-5}
TD = {np.float16: torch.float16, np.float32: torch.float32}


def planted_activations(m, k, bs, dt, seed):
    """N(0, 1) rows with planted blocks: all zero, an exact rounding tie in
    every position (a_s a power of two, x = (n + 1/2) a_s), both extremes of
    the range, one large-magnitude block and one tiny block."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    nb = k // bs
    if m >= 2 and nb >= 2:
        x[0, :bs] = 0.0
        a = np.float32(2.0 ** -6)
        ties = (rng.integers(-126, 126, size=bs) + 0.5).astype(np.float32) * a
        ties[0] = 127 * a                       # amax = 127 a_s: a_s = 2^-6 exactly
        x[1, bs:2 * bs] = ties
        x[1, :bs] = rng.choice([-1.0, 1.0], size=bs) * np.float32(3.0)  # codes +-127 only
    if m >= 3 and nb >= 2:
        x[2, :bs] *= np.float32(2000.0 if dt == np.float16 else 1e6)
        x[2, bs:2 * bs] *= np.float32(1e-3)
    return x.astype(dt)


def packed_case(w, bs, dt, symmetric=False):
    quant = oracle.rtn_quantize_symmetric if symmetric else oracle.rtn_quantize
    q, s, zp = quant(w, bs, dt)
    qw, pz = oracle.pack_weight(q, zp)
    n, k = w.shape
    pw = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(pz).to(DEV),
                      n, k, bs)
    return q, s, zp, pw


QSHAPES = [(1, 32, 32), (3, 256, 64), (17, 384, 128), (5, 512, 256), (64, 1024, 32), (2, 4160, 32)]


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("m,k,bs", QSHAPES)
def test_activation_quantizer_bit_exact(m, k, bs, dt):
    x = planted_activations(m, k, bs, dt, seed=m * 13 + k)
    qa_ref, as_ref = oracle.quantize_activations_i8(x, bs)
    qa, a_s = mnb.mnb_quantize_act_i8(torch.from_numpy(x).to(DEV), bs)
    torch.cuda.synchronize()
    assert np.array_equal(a_s.cpu().numpy().view(np.uint32), as_ref.view(np.uint32))
    assert np.array_equal(qa.cpu().numpy(), qa_ref)


PSHAPES = [(1, 64, 256, 32), (1, 40, 4160, 32), (2, 17, 96, 32), (3, 33, 192, 64), (4, 64, 512, 128),
           (7, 50, 512, 256), (16, 130, 640, 64), (62, 96, 1024, 32), (410, 48, 2048, 64)]


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("m,n,k,bs", PSHAPES)
def test_int8_product_against_oracle(m, n, k, bs, dt):
    rng = np.random.default_rng(m * 1000 + n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = planted_activations(m, k, bs, dt, seed=n + k)
    q, s, zp, pw = packed_case(w, bs, dt)
    ref = oracle.matmul_nbits_i8(x, q, zp, s, bs)
    y = mnb.mnb_gemm_i8(torch.from_numpy(x).to(DEV), pw)
    torch.cuda.synchronize()
    ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), ref, TOL[dt])
    assert ok, f"err {err:.3e} vs {TOL[dt]} * {mx:.3e}"


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_int8_product_symmetric_weights(dt):
    m, n, k, bs = 5, 48, 512, 32
    w, x = synth.random_case(41, m, n, k, "f16" if dt == np.float16 else "f32")
    q, s, zp, pw = packed_case(w, bs, dt, symmetric=True)
    ref = oracle.matmul_nbits_i8(x, q, zp, s, bs)
    y = mnb.mnb_gemm_i8(torch.from_numpy(x).to(DEV), pw)
    torch.cuda.synchronize()
    ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), ref, TOL[dt])
    assert ok, f"err {err:.3e} vs {TOL[dt]} * {mx:.3e}"


def test_int8_workspace_reuse_and_smaller_call():
    """One workspace serves a call and then a smaller one; both match the
    calls made with workspaces of their own."""
    dt = np.float16
    w, x = synth.random_case(42, 40, 80, 1024, "f16")
    _, _, _, pw = packed_case(w, 64, dt)
    xt = torch.from_numpy(x).to(DEV)
    ws = mnb.i8_workspace(40, 1024, 64, DEV)
    y1 = mnb.mnb_gemm_i8(xt, pw, ws)
    y2 = mnb.mnb_gemm_i8(xt[:9].contiguous(), pw, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, mnb.mnb_gemm_i8(xt, pw))
    assert torch.equal(y2, mnb.mnb_gemm_i8(xt[:9].contiguous(), pw))
    assert torch.equal(y2, y1[:9])


@pytest.mark.parametrize("ci,lin_index", [(0, 0), (1, 3), (3, 6), (4, 1)])
def test_int8_full_size_linears_sampled(ci, lin_index):
    """A linear of a full-size workload at its real shape and M (the launch
    the product issues), checked on sampled outputs: 8 activation rows by 64
    weight rows computed by the oracle (rows are independent in both the
    quantizer and the product)."""
    cfg = configs.CONFIGS[ci]
    lin = cfg.linears[lin_index]
    dt = synth.np_dtype(cfg.dtype)
    w, x = synth.linear_inputs(cfg, lin)
    print(f"config {cfg.name}: {lin.layer}.{lin.proj} M={cfg.m} N={lin.n} K={lin.k}", flush=True)
    q, s, zp, pw = packed_case(w, cfg.block_size, dt)
    y = mnb.mnb_gemm_i8(torch.from_numpy(x).to(DEV), pw).cpu().numpy()
    rng = np.random.default_rng(ci)
    rows = np.unique(np.concatenate([[0, cfg.m - 1], rng.integers(0, cfg.m, 6)]))
    cols = np.unique(np.concatenate([[0, lin.n - 1], rng.integers(0, lin.n, 62)]))
    ref = oracle.matmul_nbits_i8(x[rows], q[cols], zp[cols], s[cols], cfg.block_size)
    ok, err, mx = oracle.within_tolerance(y[np.ix_(rows, cols)], ref, TOL[dt])
    assert ok, f"err {err:.3e} vs {TOL[dt]} * {mx:.3e}"

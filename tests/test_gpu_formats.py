"""GPU: the format variants - symmetric weights (no zero points, fixed zero
point 8) and block sizes 128 and 256 (a block spanning two 128-input tiles) -
through quantize, pack, unpack, dequant and the products, against the oracle (bit-exact for codes, scales, zero points
and dequantized weights; outputs within the usual tolerance)."""

import numpy as np
import pytest
import torch

import oracle
from block_wise_int4_amd import mnb
from workloads import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {np.float16: 2e-3, np.float32: 1e-5}
TD = {np.float16: torch.float16, np.float32: torch.float32}


def _weight(n, k, bs, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    if n >= 3:
        w[0, :bs] = 0.0                                   # all-zero block
        w[1, :bs] = np.abs(w[1, :bs]) + 0.001             # single-signed block
        w[2, :4] = np.array([7.0, 2.5, -1.5, 0.5]) * 2.0 ** -7
        w[2, 4:bs] = 0.0                                  # symmetric ties at block 0 of row 2
    return w


def _oracle(w, bs, dt, symmetric):
    return (oracle.rtn_quantize_symmetric if symmetric else oracle.rtn_quantize)(w, bs, dt)


FORMATS = [(True, 32), (True, 64), (True, 128), (False, 128), (False, 256), (True, 256)]
# (9, 768): an odd number of 256-blocks per row, so the last zero-point byte is half padding
SHAPES = [(64, 256), (17, 384), (1, 128), (40, 4224), (9, 768), (33, 2560)]


def _valid(shapes, formats):
    """(shape, format) pairs whose K is a whole number of blocks."""
    return [(*sh, sym, bs) for sh in shapes for sym, bs in formats if sh[-1] % bs == 0]


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("n,k,symmetric,bs", _valid(SHAPES, FORMATS))
def test_quantize_pack_unpack_dequant_bit_exact(n, k, symmetric, bs, dt):
    w = _weight(n, k, bs, seed=n + k + bs)
    q, s, zp = _oracle(w, bs, dt, symmetric)
    qw, pz = oracle.pack_weight(q, zp)
    gq, gs, gz = mnb.mnb_quantize_rtn(torch.from_numpy(w).to(DEV), bs, TD[dt], symmetric=symmetric)
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), qw)
    assert np.array_equal(gs.cpu().numpy().view(np.uint8), s.view(np.uint8))
    if symmetric:
        assert gz is None
    else:
        assert np.array_equal(gz.cpu().numpy(), pz)
    pw = mnb.mnb_pack(gq, gs, gz, n, k, bs)
    uq, uz = mnb.mnb_unpack(pw)
    d = mnb.mnb_dequant(pw)
    torch.cuda.synchronize()
    assert np.array_equal(uq.cpu().numpy(), q)
    assert np.array_equal(uz.cpu().numpy(), zp)
    ref = oracle.dequantize(q, zp, s, bs, dt)
    assert np.array_equal(d.cpu().numpy().view(np.uint8), ref.view(np.uint8))


PRODUCTS = [(1, 3072, 1024), (1, 100, 4224), (2, 64, 512), (62, 1024, 3072), (410, 512, 2048), (1500, 256, 768)]


@pytest.mark.parametrize("m,n,k,symmetric,bs", _valid(PRODUCTS, FORMATS))
def test_products_within_tolerance(m, n, k, symmetric, bs):
    dt = np.float16
    w, x = synth.random_case(m * 13 + n + k + bs, m, n, k, "f16")
    q, s, zp = _oracle(w, bs, dt, symmetric)
    qw, pz = oracle.pack_weight(q, zp)
    pw = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV),
                      None if symmetric else torch.from_numpy(pz).to(DEV), n, k, bs)
    xd = torch.from_numpy(x).to(DEV)
    y = mnb.mnb_gemv(xd.reshape(-1), pw) if m == 1 else mnb.mnb_gemm(xd, pw)
    torch.cuda.synchronize()
    ref = oracle.matmul_nbits(x, q, zp, s, bs)
    ok, err, mx = oracle.within_tolerance(y.cpu().numpy().reshape(m, n), ref, TOL[dt])
    assert ok, f"max err {err:.3e} vs 2e-3 * {mx:.3e}"


@pytest.mark.parametrize("bs", [32, 128])
def test_fp32_products_block_128_and_symmetric(bs):
    m, n, k = 3, 200, 1024
    w, x = synth.random_case(555 + bs, m, n, k, "f32")
    for symmetric in (False, True):
        q, s, zp = _oracle(w, bs, np.float32, symmetric)
        qw, pz = oracle.pack_weight(q, zp)
        pw = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV),
                          None if symmetric else torch.from_numpy(pz).to(DEV), n, k, bs)
        y = mnb.mnb_gemm(torch.from_numpy(x).to(DEV), pw)
        torch.cuda.synchronize()
        ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), oracle.matmul_nbits(x, q, zp, s, bs), 1e-5)
        assert ok, f"max err {err:.3e} vs 1e-5 * {mx:.3e}"

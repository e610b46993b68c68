"""GPU: a seeded random sweep of product shapes against the oracle.

The fixed cases elsewhere pin the tile shapes and edges one by one; this
sweep crosses them at random: M from 1 (decode kernel) through the 16-, 32-,
64-row and 192/208-row GEMM tiles, N with partial last tiles, K with ragged
128-input tails, every block size, float16 and float32 activations. Outputs
within the usual tolerance of the oracle's float64 product.
"""

import numpy as np
import pytest
import torch

import oracle
from block_wise_int4_amd import mnb
from workloads import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {np.float16: 2e-3, np.float32: 1e-5}


def _cases(count=48, seed=2024, max_macs=1.2e9):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        bs = int(rng.choice([32, 64, 128, 256]))
        k = bs * int(rng.integers(1, 8192 // bs + 1))
        band = rng.random()
        if band < 0.3:
            m = 1
        elif band < 0.65:
            m = int(rng.integers(2, 65))
        else:
            m = int(rng.integers(65, 601))
        n = int(rng.integers(1, 701))
        dt = np.float32 if (m <= 8 and rng.random() < 0.4) else np.float16
        if m * n * k > max_macs:
            continue
        out.append((m, n, k, bs, dt, len(out)))
    return out


@pytest.mark.parametrize("m,n,k,bs,dt,i", _cases())
def test_random_shape(m, n, k, bs, dt, i):
    w, x = synth.random_case(5000 + i, m, n, k, "f16" if dt == np.float16 else "f32")
    q, s, zp = oracle.rtn_quantize(w, bs, dt)
    qw, pz = oracle.pack_weight(q, zp)
    pw = mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(pz).to(DEV),
                      n, k, bs)
    xd = torch.from_numpy(x).to(DEV)
    y = mnb.mnb_gemv(xd.reshape(-1), pw) if m == 1 else mnb.mnb_gemm(xd, pw)
    torch.cuda.synchronize()
    ref = oracle.matmul_nbits(x, q, zp, s, bs)
    ok, err, mx = oracle.within_tolerance(y.cpu().numpy().reshape(m, n), ref, TOL[dt])
    assert ok, f"M={m} N={n} K={k} bs={bs} {dt.__name__}: max err {err:.3e} vs {TOL[dt]} * {mx:.3e}"

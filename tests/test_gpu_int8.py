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
           (7, 50, 512, 256), (15, 40, 256, 32),
           # M >= 16: the matrix-core kernel (ragged M and N, K tails, blocks spanning two tiles)
           (16, 130, 640, 64), (17, 16, 128, 128), (40, 70, 4160, 32), (62, 96, 1024, 32), (64, 33, 512, 256),
           (100, 200, 1536, 128), (410, 48, 2048, 64)]


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
    """One workspace serves a call and then smaller ones (the matrix-core
    kernel at M = 40 and 20, the vector kernel at M = 9); each matches the
    call made with a workspace of its own, and a row's bits do not depend on
    how many rows the call has (within one kernel)."""
    dt = np.float16
    w, x = synth.random_case(42, 40, 80, 1024, "f16")
    _, _, _, pw = packed_case(w, 64, dt)
    xt = torch.from_numpy(x).to(DEV)
    ws = mnb.i8_workspace(40, 1024, 64, DEV)
    assert mnb.mnb_gemm_i8_workspace_bytes(1, 1024, 64) == 0
    y1 = mnb.mnb_gemm_i8(xt, pw, ws)
    y2 = mnb.mnb_gemm_i8(xt[:20].contiguous(), pw, ws)
    y3 = mnb.mnb_gemm_i8(xt[:9].contiguous(), pw, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, mnb.mnb_gemm_i8(xt, pw))
    assert torch.equal(y2, mnb.mnb_gemm_i8(xt[:20].contiguous(), pw))
    assert torch.equal(y3, mnb.mnb_gemm_i8(xt[:9].contiguous(), pw))
    assert torch.equal(y2, y1[:20])
    y4 = mnb.mnb_gemm_i8(xt[:5].contiguous(), pw, ws)
    torch.cuda.synchronize()
    assert torch.equal(y4, y3[:5])
    ok, err, mx = oracle.within_tolerance(y3.float().cpu().numpy(), y1[:9].float().cpu().numpy(), TOL[dt])
    assert ok, f"vector and matrix-core kernels differ by {err:.3e} (max {mx:.3e})"


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


DECODE_SHAPES = [(64, 256, 32), (40, 4160, 32), (17, 96, 32), (33, 192, 64), (50, 512, 128), (70, 1024, 256),
                 (3000, 1024, 32), (1000, 32768, 64)]


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("n,k,bs", DECODE_SHAPES)
def test_int8_decode_one_launch_equals_two_launch_form(n, k, bs, dt):
    """M = 1 runs one launch that quantizes x in LDS; its outputs equal, bit
    for bit, row 0 of a two-row call (quantize launch + product launch) on
    [x; x], and are within tolerance of the oracle."""
    w, x = synth.random_case(n + 3 * k, 1, n, k, "f16" if dt == np.float16 else "f32")
    q, s, zp, pw = packed_case(w, bs, dt)
    xt = torch.from_numpy(x).to(DEV)
    y1 = mnb.mnb_gemm_i8(xt, pw)
    y2 = mnb.mnb_gemm_i8(torch.cat([xt, xt]).contiguous(), pw)
    torch.cuda.synchronize()
    assert torch.equal(y1[0], y2[0]) and torch.equal(y2[0], y2[1])
    ref = oracle.matmul_nbits_i8(x, q, zp, s, bs)
    ok, err, mx = oracle.within_tolerance(y1.cpu().numpy(), ref, TOL[dt])
    assert ok, f"err {err:.3e} vs {TOL[dt]} * {mx:.3e}"


def test_int8_decode_planted_activations():
    """Zero blocks, ties and extremes through the one-launch decode path."""
    n, k, bs, dt = 48, 1024, 32, np.float16
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x3 = planted_activations(3, k, bs, dt, seed=11)
    q, s, zp, pw = packed_case(w, bs, dt)
    for row in range(3):
        x = x3[row:row + 1]
        y = mnb.mnb_gemm_i8(torch.from_numpy(x).to(DEV), pw)
        torch.cuda.synchronize()
        ref = oracle.matmul_nbits_i8(x, q, zp, s, bs)
        ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), ref, TOL[dt])
        assert ok, f"row {row}: err {err:.3e} vs {TOL[dt]} * {mx:.3e}"


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_int8_grouped_plan_equals_single_calls(dt):
    """A plan of decode products of mixed shapes (one launch): every output
    bitwise equal to its single mnb_gemm_i8 call; products past the first of
    a workgroup's range re-quantize their own vector."""
    rng = np.random.default_rng(21)
    problems, singles = [], []
    for i in range(23):
        n = int(rng.integers(1, 3000))
        k = int(rng.choice([256, 1024, 2048, 4160 if dt == np.float32 else 3072]))
        w, x = synth.random_case(700 + i, 1, n, k, "f16" if dt == np.float16 else "f32")
        _, _, _, pw = packed_case(w, 32, dt)
        xt = torch.from_numpy(x.reshape(-1)).to(DEV)
        problems.append((xt, pw, None))
        singles.append(mnb.mnb_gemm_i8(xt.reshape(1, -1), pw))
    plan = mnb.mnb_plan_grouped(problems, 32, TD[dt], int8=True)
    assert mnb.mnb_plan_launches(plan) == 1
    mnb.mnb_gemm_grouped(plan)
    torch.cuda.synchronize()
    for i, (y, ys) in enumerate(zip(plan.outputs, singles)):
        assert torch.equal(y.reshape(-1), ys.reshape(-1)), f"problem {i}"


def test_int8_plan_refuses_prefill_products():
    w, x = synth.random_case(5, 4, 32, 256, "f16")
    _, _, _, pw = packed_case(w, 32, np.float16)
    with pytest.raises(mnb.MnbError):
        mnb.mnb_plan_grouped([(torch.from_numpy(x).to(DEV), pw, None)], 32, torch.float16, int8=True)


def test_int8_full_size_decode_step_grouped():
    """The 0.6B decode step in the int8 mode as one grouped launch (the
    launch bench.py times): every output bitwise equal to single calls, and
    sampled outputs of three linears (the LM head among them) within
    tolerance of the oracle."""
    from block_wise_int4_amd import workload
    cfg = configs.CONFIGS[1]
    data = workload.build_config(cfg, DEV)
    plan = mnb.mnb_plan_grouped([(ld.x.reshape(-1), ld.pw, ld.y) for ld in data.linears], cfg.block_size,
                                torch.float16, int8=True)
    mnb.mnb_gemm_grouped(plan)
    torch.cuda.synchronize()
    for ld in data.linears:
        single = mnb.mnb_gemm_i8(ld.x.reshape(1, -1), ld.pw)
        assert torch.equal(single.reshape(-1), ld.y.reshape(-1)), f"{ld.lin}"
    for ld in (data.linears[0], data.linears[6], data.linears[-1]):
        w, x = synth.linear_inputs(cfg, ld.lin)
        rows = np.random.default_rng(ld.lin.n).integers(0, ld.lin.n, 64)
        q, s, zp = oracle.rtn_quantize(w[rows], cfg.block_size, np.float16)
        ref = oracle.matmul_nbits_i8(x, q, zp, s, cfg.block_size)
        got = ld.y.reshape(-1).cpu().numpy()[rows][None, :]
        ok, err, mx = oracle.within_tolerance(got, ref, TOL[np.float16])
        assert ok, f"{ld.lin}: err {err:.3e} vs {TOL[np.float16]} * {mx:.3e}"

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: RTN codes, scales and zero points; unpacked codes; dequantized
weights. Within tolerance (max |y - y_ref| <= tol * max |y_ref| per call):
outputs, tol = 2e-3 for float16 activations and 1e-5 for float32.
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
NP = {torch.float16: np.float16, torch.float32: np.float32}
TD = {np.float16: torch.float16, np.float32: torch.float32}


def special_weight(n, k, bs, seed):
    """N(0, 0.02) rows with edge blocks planted: all zero, single-signed
    (both signs), an exact RNE tie for the zero point, a tiny block whose
    float16 scale underflows, and a wide-range block."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    nb = k // bs
    if n >= 6 and nb >= 1:
        w[0, :bs] = 0.0
        w[1, :bs] = np.abs(w[1, :bs]) + 0.001
        w[2, :bs] = -np.abs(w[2, :bs]) - 0.001
        sc = 2.0 ** -7
        t = np.zeros(bs)
        t[:4] = np.array([-2.5, 12.5, 0.5, 1.5]) * sc
        w[3, :bs] = t
        w[4, :bs] = rng.standard_normal(bs) * 1e-9
        w[5, :bs] = rng.standard_normal(bs) * 30.0
    return w


def quantize_oracle(w, bs, dt):
    q, s, zp = oracle.rtn_quantize(w, bs, dt)
    qw, pz = oracle.pack_weight(q, zp)
    return q, s, zp, qw, pz


def upload_packed(qw, s, pz, n, k, bs):
    return mnb.mnb_pack(torch.from_numpy(qw).to(DEV), torch.from_numpy(s).to(DEV),
                        torch.from_numpy(pz).to(DEV), n, k, bs)


SHAPES = [(64, 256, 32), (17, 96, 32), (33, 192, 64), (6, 64, 64), (40, 4160, 32), (1, 32, 32)]


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("n,k,bs", SHAPES)
def test_quantize_rtn_bit_exact(n, k, bs, dt):
    w = special_weight(n, k, bs, seed=n * 31 + k)
    q, s, zp, qw, pz = quantize_oracle(w, bs, dt)
    gq, gs, gz = mnb.mnb_quantize_rtn(torch.from_numpy(w).to(DEV), bs, TD[dt])
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), qw)
    assert np.array_equal(gs.cpu().numpy().view(np.uint8), s.view(np.uint8))
    assert np.array_equal(gz.cpu().numpy(), pz)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("n,k,bs", SHAPES)
def test_unpack_and_dequant_bit_exact(n, k, bs, dt):
    w = special_weight(n, k, bs, seed=n + 7 * k)
    q, s, zp, qw, pz = quantize_oracle(w, bs, dt)
    pw = upload_packed(qw, s, pz, n, k, bs)
    gq, gz = mnb.mnb_unpack(pw)
    d = mnb.mnb_dequant(pw)
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), q)
    assert np.array_equal(gz.cpu().numpy(), zp)
    ref = oracle.dequantize(q, zp, s, bs, dt)
    assert np.array_equal(d.cpu().numpy().view(np.uint8), ref.view(np.uint8))


def run_product(m, n, k, bs, dt, seed, std=0.02):
    w, x = synth.random_case(seed, m, n, k, "f16" if dt == np.float16 else "f32", std)
    q, s, zp, qw, pz = quantize_oracle(w, bs, dt)
    pw = upload_packed(qw, s, pz, n, k, bs)
    xd = torch.from_numpy(x).to(DEV)
    y = mnb.mnb_gemv(xd.reshape(-1), pw) if m == 1 else mnb.mnb_gemm(xd, pw)
    torch.cuda.synchronize()
    ref = oracle.matmul_nbits(x, q, zp, s, bs)
    return y.cpu().numpy().reshape(m, n), ref


GEMV_CASES = [(3072, 1024, 32, np.float32), (1, 32, 32, np.float16), (17, 96, 32, np.float16),
              (100, 192, 64, np.float16), (64, 2048, 32, np.float16), (300, 4160, 32, np.float16),
              (33, 8192, 32, np.float32), (2048, 1024, 32, np.float16), (5, 32768, 32, np.float16),
              (250, 736, 32, np.float32), (96, 768, 64, np.float32), (7, 32768, 32, np.float32),
              (3072, 1024, 32, np.float16), (1024, 6144, 64, np.float16)]


@pytest.mark.parametrize("n,k,bs,dt", GEMV_CASES)
def test_gemv_parity(n, k, bs, dt):
    y, ref = run_product(1, n, k, bs, dt, seed=n + k)
    ok, err, mx = oracle.within_tolerance(y, ref, TOL[dt])
    assert ok, f"max err {err:.3e} vs {TOL[dt]} * {mx:.3e}"


GEMM_CASES = [(2, 64, 64, 32), (7, 200, 256, 32), (16, 1024, 2048, 32), (17, 96, 96, 32), (31, 130, 512, 64),
              (33, 64, 1024, 32), (64, 300, 4160, 32), (65, 512, 768, 64), (100, 256, 2048, 32),
              (130, 1024, 768, 64), (257, 384, 1024, 32), (410, 1024, 2048, 32), (500, 200, 3072, 64),
              (1500, 768, 768, 64),
              # one K-tile (with and without a ragged tail) and K-loops shorter or a little longer than
              # each tile shape's ring of prefetched code tiles
              (40, 64, 128, 32), (48, 200, 96, 32), (70, 100, 128, 32), (60, 130, 384, 64), (64, 256, 640, 32),
              (12, 100, 896, 32), (16, 64, 2176, 32), (30, 70, 1152, 64), (62, 3072, 1024, 64),
              # the 208- and 192-row tiles with a ragged K tail and a partial last N-tile
              (200, 130, 2112, 64), (300, 520, 1184, 32), (100, 300, 4160, 32), (250, 130, 96, 32)]


@pytest.mark.parametrize("m,n,k,bs", GEMM_CASES)
def test_gemm_fp16_parity(m, n, k, bs):
    y, ref = run_product(m, n, k, bs, np.float16, seed=m * 1000 + n + k)
    ok, err, mx = oracle.within_tolerance(y, ref, TOL[np.float16])
    assert ok, f"max err {err:.3e} vs 2e-3 * {mx:.3e}"


@pytest.mark.parametrize("m,n,k,bs", [(2, 64, 1024, 32), (5, 100, 4096, 32), (3, 40, 8192, 64), (9, 17, 96, 32),
                                      (3, 40, 16384, 32), (6, 20, 32768, 64)])
def test_gemm_fp32_parity(m, n, k, bs):
    y, ref = run_product(m, n, k, bs, np.float32, seed=m + n + k)
    ok, err, mx = oracle.within_tolerance(y, ref, TOL[np.float32])
    assert ok, f"max err {err:.3e} vs 1e-5 * {mx:.3e}"


@pytest.mark.parametrize("bs", [32, 256])
def test_grouped_plan_matches_single_calls_bitwise(bs):
    specs = [(1, 256, 1024, 1), (1, 17, 96, 2), (410, 128, 256, 3), (33, 64, 512, 4), (1, 2048, 2048, 5),
             (1500, 64, 768, 6)]
    problems, singles, refs = [], [], []
    for m, n, k, seed in specs:
        k = k if k % bs == 0 else bs
        w, x = synth.random_case(seed, m, n, k, "f16")
        q, s, zp, qw, pz = quantize_oracle(w, bs, np.float16)
        pw = upload_packed(qw, s, pz, n, k, bs)
        xd = torch.from_numpy(x).to(DEV)
        problems.append((xd, pw, None))
        singles.append(mnb.mnb_gemm(xd, pw))
        refs.append((x, q, zp, s))
    plan = mnb.mnb_plan_grouped(problems, bs, torch.float16)
    outs = mnb.mnb_gemm_grouped(plan)
    torch.cuda.synchronize()
    for y, ys, (x, q, zp, s) in zip(outs, singles, refs):
        assert torch.equal(y, ys)
        ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), oracle.matmul_nbits(x, q, zp, s, bs), 2e-3)
        assert ok, (err, mx)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_single_decode_split_matches_grouped_bitwise(dt):
    """Single M = 1 products of one round of workgroups (the split kernel:
    one, two or four waves share a row group's load groups of 1024 inputs)
    against the grouped kernel (one wave walks a row group's load groups in
    order) bit for bit, and against the oracle: K from one to nine load
    groups with ragged K tails, N that leaves the last workgroup partly or
    wholly past N, the largest staged K in float32, and shapes on both
    sides of each switch (768 workgroups of 4 row groups, of 1 row group with
    four waves each, and past them)."""
    specs = [(1024, 1024), (1024, 2048), (1024, 3072), (2048, 4096), (100, 5120), (70, 6144), (33, 7168),
             (16, 2176), (48, 8320), (200, 96), (768 * 64, 256), (769 * 64, 256), (12288, 3072),
             (12304, 3072)] + ([(40, 32768)] if dt == np.float32 else [])
    for i, (n, k) in enumerate(specs):
        w, x = synth.random_case(300 + i, 1, n, k, "f16" if dt == np.float16 else "f32")
        q, s, zp, qw, pz = quantize_oracle(w, 32, dt)
        pw = upload_packed(qw, s, pz, n, k, 32)
        xd = torch.from_numpy(x).to(DEV)
        single = mnb.mnb_gemv(xd.reshape(-1), pw)
        plan = mnb.mnb_plan_grouped([(xd, pw, None)], 32, TD[dt])
        (grouped,) = mnb.mnb_gemm_grouped(plan)
        torch.cuda.synchronize()
        assert torch.equal(single.reshape(1, n), grouped.reshape(1, n)), (n, k)
        ok, err, mx = oracle.within_tolerance(single.cpu().numpy().reshape(1, n),
                                              oracle.matmul_nbits(x, q, zp, s, 32), TOL[dt])
        assert ok, (n, k, err, mx)


@pytest.mark.parametrize("band,bs", [((65, 208), 32), ((65, 208), 64), ((2, 16), 32), ((17, 64), 64),
                                     ((209, 420), 32)])
def test_grouped_tiles_across_products(band, bs):
    """Many products of one tile shape in one plan, so that each XCD's range
    holds several and a workgroup's consecutive tiles cross from one product
    to the next (different K, N not always a multiple of 8, odd tile
    counts): bit-equal to single calls and within tolerance of the oracle."""
    rng = np.random.default_rng(band[0] * 7 + bs)
    ks = [128, 384, 640, 1024, 2176, 96 if bs == 32 else 192]
    specs = []
    for i in range(30):
        m = int(rng.integers(band[0], band[1] + 1))
        n = int(rng.choice([64, 100, 200, 256, 520, 777]))
        k = int(ks[i % len(ks)])
        specs.append((m, n, k, 1000 + i))
    _grouped_vs_single(specs, bs)


def _grouped_vs_single(specs, bs):
    """One grouped plan over specs [(m, n, k, seed)], outputs filled with NaN
    beforehand (so a tile the launch skips shows), against single calls
    (bitwise) and the oracle (tolerance)."""
    problems, singles, refs = [], [], []
    for m, n, k, seed in specs:
        w, x = synth.random_case(seed, m, n, k, "f16")
        q, s, zp, qw, pz = quantize_oracle(w, bs, np.float16)
        pw = upload_packed(qw, s, pz, n, k, bs)
        xd = torch.from_numpy(x).to(DEV)
        problems.append((xd, pw, torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)))
        singles.append(mnb.mnb_gemm(xd, pw))
        refs.append((x, q, zp, s))
    plan = mnb.mnb_plan_grouped(problems, bs, torch.float16)
    outs = mnb.mnb_gemm_grouped(plan)
    torch.cuda.synchronize()
    for (m, n, k, _), y, ys, (x, q, zp, s) in zip(specs, outs, singles, refs):
        assert torch.equal(y, ys), (m, n, k)
        ok, err, mx = oracle.within_tolerance(y.cpu().numpy(), oracle.matmul_nbits(x, q, zp, s, bs), 2e-3)
        assert ok, (m, n, k, err, mx)


@pytest.mark.parametrize("layers", [1, 3, 12])
def test_grouped_tiles_moved_between_xcds(layers):
    """Encoder-shaped products (q/k/v/o, fc1, fc2 of a 768-wide layer at 400
    rows, block 64) whose whole-product split leaves the XCDs unequal, so
    that the schedule moves the last tiles of short-K products to other
    XCDs: every output still written once, bit-equal to single calls."""
    specs = []
    for li in range(layers):
        for j, (n, k) in enumerate([(768, 768)] * 4 + [(3072, 768), (768, 3072)]):
            specs.append((400, n, k, 5000 + 10 * li + j))
    _grouped_vs_single(specs, 64)


def test_calls_run_on_the_current_stream():
    """Products issued under a side stream run there: after that stream alone
    is synchronized, their outputs equal the default stream's bit for bit."""
    m, n, k = 410, 512, 2048
    w, x = synth.random_case(31, m, n, k, "f16")
    q, s, zp, qw, pz = quantize_oracle(w, 32, np.float16)
    pw = upload_packed(qw, s, pz, n, k, 32)
    xd = torch.from_numpy(x).to(DEV)
    ref_mm = mnb.mnb_gemm(xd, pw)
    ref_mv = mnb.mnb_gemv(xd[0].contiguous(), pw)
    plan = mnb.mnb_plan_grouped([(xd, pw, None), (xd[:1].contiguous(), pw, None)], 32, torch.float16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y_mm = mnb.mnb_gemm(xd, pw)
        y_mv = mnb.mnb_gemv(xd[0].contiguous(), pw)
        outs = mnb.mnb_gemm_grouped(plan)
    side.synchronize()
    assert torch.equal(y_mm, ref_mm)
    assert torch.equal(y_mv, ref_mv)
    assert torch.equal(outs[0], ref_mm)
    assert torch.equal(outs[1].reshape(-1), ref_mv)


def test_repeated_calls_are_deterministic():
    w, x = synth.random_case(3, 410, 512, 2048, "f16")
    q, s, zp, qw, pz = quantize_oracle(w, 32, np.float16)
    pw = upload_packed(qw, s, pz, 512, 2048, 32)
    xd = torch.from_numpy(x).to(DEV)
    a = mnb.mnb_gemm(xd, pw)
    b = mnb.mnb_gemm(xd, pw)
    g1 = mnb.mnb_gemv(xd[0].contiguous(), pw)
    g2 = mnb.mnb_gemv(xd[0].contiguous(), pw)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(g1, g2)


def test_errors_raise_and_enqueue_nothing():
    w, x = synth.random_case(1, 4, 64, 128, "f16")
    q, s, zp, qw, pz = quantize_oracle(w, 32, np.float16)
    pw = upload_packed(qw, s, pz, 64, 128, 32)
    y = torch.full((64,), 7.0, dtype=torch.float16, device=DEV)
    bad = mnb.PackedWeight(pw.packed, 64, 96, 64, torch.float16)        # K % bs != 0
    with pytest.raises(mnb.MnbError) as ei:
        mnb.mnb_gemv(torch.zeros(96, dtype=torch.float16, device=DEV), bad, y)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------------------
# Full-size configurations, in the launch configuration the benchmark times
# (one grouped plan over the config's linears), checked on sampled rows.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4, 5, 6, 7])
def test_full_size_config_sampled(ci):
    from block_wise_int4_amd import workload
    cfg = configs.CONFIGS[ci]
    print(f"config {cfg.name}: {len(cfg.linears)} linears", flush=True)
    data = workload.build_config(cfg, DEV, sample_rows=12)
    plan = workload.make_plan(cfg, data.linears)
    assert mnb.mnb_plan_launches(plan) == 1
    mnb.mnb_gemm_grouped(plan)
    torch.cuda.synchronize()
    dt = np.float16 if cfg.dtype == "f16" else np.float32
    for ld in data.linears:
        rows = ld.sample_rows
        quantize = oracle.rtn_quantize_symmetric if cfg.symmetric else oracle.rtn_quantize
        q, s, zp = quantize(ld.w_rows, cfg.block_size, dt)
        gq, gs, gz = ld.canonical
        qw, pz = oracle.pack_weight(q, zp)
        assert np.array_equal(gq, qw) and (gz is None if cfg.symmetric else np.array_equal(gz, pz))
        assert np.array_equal(gs.view(np.uint8), s.view(np.uint8))
        x = ld.x.cpu().numpy()
        mrows = np.unique(np.linspace(0, cfg.m - 1, min(cfg.m, 6)).astype(int))
        ref = oracle.matmul_nbits(x[mrows], q, zp, s, cfg.block_size)
        got = ld.y.cpu().numpy()[np.ix_(mrows, rows)]
        ok, err, mx = oracle.within_tolerance(got, ref, TOL[dt])
        assert ok, f"{ld.lin}: err {err:.3e} vs {TOL[dt]} * {mx:.3e}"


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4, 5, 6, 7])
def test_full_size_config_every_output(ci):
    """Every output of the full-size grouped launch: bitwise equal to the
    same product issued as a single call, and within the tolerance of a
    float32 product of the call's own dequantized weights (mnb_dequant, which
    the bit-exact tests pin to the oracle) computed with PyTorch."""
    from block_wise_int4_amd import workload
    cfg = configs.CONFIGS[ci]
    print(f"config {cfg.name}: {len(cfg.linears)} linears", flush=True)
    data = workload.build_config(cfg, DEV)
    plan = workload.make_plan(cfg, data.linears)
    mnb.mnb_gemm_grouped(plan)
    torch.cuda.synchronize()
    dt = np.float16 if cfg.dtype == "f16" else np.float32
    for ld in data.linears:
        single = mnb.mnb_gemv(ld.x.reshape(-1), ld.pw) if cfg.m == 1 else mnb.mnb_gemm(ld.x, ld.pw)
        assert torch.equal(single.reshape(ld.y.shape), ld.y), f"{ld.lin}: grouped differs from the single call"
        d = mnb.mnb_dequant(ld.pw).float()
        ref = (ld.x.float() @ d.t()).double()
        err = (ld.y.double() - ref).abs().max().item()
        mx = ref.abs().max().item()
        assert err <= TOL[dt] * mx, f"{ld.lin}: err {err:.3e} vs {TOL[dt]} * {mx:.3e}"
    del data, plan
    torch.cuda.empty_cache()

"""Pins for the CPU oracle: checks against closed forms, exact rational
arithmetic, brute force and the sizes printed on the pages, never against a
re-typed copy of the oracle's own formulas.

Which plausible mistake each group catches:
  unpack / pack       swapped nibble order, wrong mask or shift, odd padding
  dequant (Fraction)  wrong sign of zp, zp added instead of subtracted, wrong
                      block index (k // bs), scale/zp swapped
  rounding            double rounding, round-half-away instead of half-even
  RTN                 extent without zero, rint vs round-half-away, q = w/s - zp,
                      scale computed from unrounded value, degenerate blocks
  matmul              transposed operand, dropped term, wrong row/column
  sizes               wrong bytes-per-weight accounting
"""

import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Independent helpers (exact rational arithmetic, no NumPy rounding).
# ---------------------------------------------------------------------------

FMT = {np.float16: (10, -14, 15), np.float32: (23, -126, 127)}


def rne(fr, dtype):
    """Round a Fraction to the nearest float16/float32 value, ties to even,
    by integer arithmetic (subnormals included, overflow to inf)."""
    mant, emin, emax = FMT[dtype]
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * ulp
    if val >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * val


def frac(x):
    return Fraction(float(x))


def nibbles_by_divmod(byte):
    hi, lo = divmod(int(byte), 16)
    return lo, hi


# ---------------------------------------------------------------------------
# Packing.
# ---------------------------------------------------------------------------

def test_unpack_every_byte_value():
    allbytes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    out = oracle.unpack_nibbles(allbytes, 512)
    for b in range(256):
        assert tuple(out[0, 2 * b: 2 * b + 2]) == nibbles_by_divmod(b)


@pytest.mark.parametrize("count", [2, 9, 64, 65])
def test_pack_is_base16_digits_and_round_trips(count):
    rng = np.random.default_rng(count)
    v = rng.integers(0, 16, size=(3, count), dtype=np.uint8)
    p = oracle.pack_nibbles(v)
    assert p.shape == (3, (count + 1) // 2)
    for r in range(3):
        for j in range(p.shape[1]):
            lo = int(v[r, 2 * j])
            hi = int(v[r, 2 * j + 1]) if 2 * j + 1 < count else 0
            assert int(p[r, j]) == lo + 16 * hi
    assert np.array_equal(oracle.unpack_nibbles(p, count), v)


def test_pack_rejects_wide_values():
    with pytest.raises(ValueError):
        oracle.pack_nibbles(np.array([[16, 0]], dtype=np.uint8))


# ---------------------------------------------------------------------------
# Dequantization and rounding.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,bs", [(np.float16, 32), (np.float32, 32), (np.float16, 64)])
def test_dequant_exact_against_fractions(dtype, bs):
    rng = np.random.default_rng(7)
    n, k = 3, 2 * bs
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zp = rng.integers(0, 16, size=(n, k // bs), dtype=np.uint8)
    s = (rng.random((n, k // bs)) * 0.01 + 1e-4).astype(dtype)
    d = oracle.dequantize_exact(q, zp, s, bs)
    for i in range(n):
        for j in range(k):
            blk = j // bs
            exact = (int(q[i, j]) - int(zp[i, blk])) * frac(s[i, blk])
            assert frac(d[i, j]) == exact
            ratio = exact / frac(s[i, blk])
            assert ratio.denominator == 1 and -15 <= ratio <= 15


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_round_to_matches_integer_rne(dtype):
    rng = np.random.default_rng(11)
    mant, _, _ = FMT[dtype]
    vals = list(rng.standard_normal(200) * 0.01)
    # exact ties between neighbours, both parities, and subnormal / huge ones
    for base in (1.0, 1.0 + 2.0 ** -mant, 0.75, 2.0 ** -20, -3.0):
        vals.append(base + 2.0 ** (np.floor(np.log2(abs(base))) - mant - 1))
    vals += [2.0 ** -24 * 1.5, 2.0 ** -24 * 2.5, 65520.0, -65519.0, 0.0]
    out = oracle.round_to(np.array(vals, dtype=np.float64), dtype)
    for v, o in zip(vals, out):
        ref = rne(Fraction(v), dtype)
        if isinstance(ref, float):
            assert np.isinf(o) and np.sign(o) == np.sign(ref)
        else:
            assert frac(o) == ref, (v, o, ref)


def test_dequantize_rounds_once_from_exact():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(4, 64), dtype=np.uint8)
    zp = rng.integers(0, 16, size=(4, 2), dtype=np.uint8)
    s32 = (rng.random((4, 2)) * 0.01).astype(np.float32)
    d = oracle.dequantize(q, zp, s32, 32)
    assert d.dtype == np.float32
    for i in range(4):
        for j in range(64):
            exact = (int(q[i, j]) - int(zp[i, j // 32])) * frac(s32[i, j // 32])
            assert frac(d[i, j]) == rne(exact, np.float32)
    d16 = oracle.dequantize(q, zp, s32.astype(np.float16), 32)
    assert d16.dtype == np.float16


# ---------------------------------------------------------------------------
# RTN quantization.
# ---------------------------------------------------------------------------

def test_on_grid_blocks_quantize_exactly():
    bs = 32
    rng = np.random.default_rng(5)
    rows, want_q, want_z, want_e = [], [], [], []
    for z in range(16):
        e = 3 + z % 7
        c = np.concatenate([np.arange(16), rng.integers(0, 16, size=bs - 16)])
        rng.shuffle(c)
        rows.append((c.astype(np.float64) - z) * 2.0 ** -e)
        want_q.append(c)
        want_z.append(z)
        want_e.append(e)
    w = np.array(rows, dtype=np.float32)
    for dtype in (np.float16, np.float32):
        q, s, zp = oracle.rtn_quantize(w, bs, dtype)
        assert np.array_equal(q, np.array(want_q, dtype=np.uint8))
        assert np.array_equal(zp[:, 0], np.array(want_z, dtype=np.uint8))
        assert np.array_equal(s[:, 0].astype(np.float64), 2.0 ** -np.array(want_e, dtype=np.float64))
        d = oracle.dequantize_exact(q, zp, s, bs)
        assert np.array_equal(d, w.astype(np.float64))


def test_tie_block_rounds_half_to_even():
    sc = 2.0 ** -6
    w = np.zeros((1, 32), dtype=np.float64)
    w[0, :6] = np.array([-2.5, 12.5, 0.5, 1.5, -0.5, 2.5]) * sc
    q, s, zp = oracle.rtn_quantize(w.astype(np.float32), 32, np.float16)
    assert float(s[0, 0]) == sc
    assert int(zp[0, 0]) == 2              # rint(2.5) = 2, not 3
    # w/s = 0.5 -> 0, 1.5 -> 2, -0.5 -> -0, 2.5 -> 2 (then + zp)
    assert [int(v) for v in q[0, 2:6]] == [2, 4, 2, 4]
    assert int(q[0, 0]) == 0               # -2.5 -> -2, + 2 = 0
    assert int(q[0, 1]) == 14              # 12.5 -> 12, + 2 = 14


def test_single_signed_blocks_extend_to_zero():
    rng = np.random.default_rng(9)
    pos = (rng.random((1, 32)) + 1.0) * 0.01          # all in [0.01, 0.02)
    neg = -pos
    for w, want_zp in ((pos, 0), (neg, 15)):
        w = w.astype(np.float32)
        q, s, zp = oracle.rtn_quantize(w, 32, np.float32)
        assert int(zp[0, 0]) == want_zp
        extent = Fraction(float(np.abs(w).max()))
        assert frac(s[0, 0]) == rne(extent / 15, np.float32)


def test_all_zero_and_underflowing_blocks():
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 32:] = 1e-9                       # fp16 scale rounds to 0
    q, s, zp = oracle.rtn_quantize(w, 32, np.float16)
    assert np.all(s == 0) and np.all(zp == 0) and np.all(q == 0)
    assert np.all(oracle.dequantize_exact(q, zp, s, 32) == 0)
    q32, s32, zp32 = oracle.rtn_quantize(w, 32, np.float32)
    assert float(s32[1, 1]) > 0 and int(zp32[1, 1]) == 0


def _check_nearest_grid(w, q, s, zp, bs):
    """Brute force: every code is the nearest of the 16 grid points (ties to
    an even offset from zp), zp is the integer nearest -lo/s (ties even)."""
    n, k = w.shape
    for i in range(n):
        for b in range(k // bs):
            sb = frac(s[i, b])
            if sb == 0:
                assert int(zp[i, b]) == 0 and not q[i, b * bs:(b + 1) * bs].any()
                continue
            blk = [frac(v) for v in w[i, b * bs:(b + 1) * bs]]
            lo = min(min(blk), Fraction(0))
            t = -lo / sb
            dz = [abs(t - z) for z in range(16)]
            best = min(dz)
            cands = [z for z in range(16) if dz[z] == best]
            z = int(zp[i, b])
            assert z in cands and (len(cands) == 1 or z % 2 == 0)
            for j, v in enumerate(blk):
                dist = [abs(v - (c - z) * sb) for c in range(16)]
                best = min(dist)
                cands = [c for c in range(16) if dist[c] == best]
                c = int(q[i, b * bs + j])
                assert c in cands, (i, b, j)
                if len(cands) == 2:
                    assert (c - z) % 2 == 0


@pytest.mark.parametrize("dtype,bs", [(np.float16, 32), (np.float32, 32), (np.float16, 64), (np.float32, 64),
                                      (np.float16, 256)])
def test_rtn_codes_are_nearest_grid_points(dtype, bs):
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((4, 2 * bs)) * 0.02).astype(np.float32)
    q, s, zp = oracle.rtn_quantize(w, bs, dtype)
    _check_nearest_grid(w, q, s, zp, bs)


@pytest.mark.parametrize("dtype,bs", [(np.float16, 32), (np.float32, 32), (np.float16, 64), (np.float32, 256)])
def test_rtn_round_trip_bound(dtype, bs):
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((64, 8 * bs)) * 0.02).astype(np.float32)
    q, s, zp = oracle.rtn_quantize(w, bs, dtype)
    d = oracle.dequantize_exact(q, zp, s, bs)
    blocks = w.astype(np.float64).reshape(64, 8, bs)
    extent = np.maximum(blocks.max(2), 0) - np.minimum(blocks.min(2), 0)
    s64 = s.astype(np.float64)
    # |w - D| <= s/2 + 15 |s - (hi - lo)/15|: the half-step of the grid, plus
    # the shift of the grid's top end caused by storing a rounded scale.
    bound = s64 / 2 + np.abs(15 * s64 - extent)
    err = np.abs(w.astype(np.float64) - d).reshape(64, 8, bs).max(2)
    assert np.all(err <= bound * (1 + 1e-12))
    # and the plain half-step bound holds wherever the clamp did not engage
    inner = (q > 0) & (q < 15)
    assert np.all(np.abs(w - d)[inner] <= np.repeat(s64, bs, 1)[inner] / 2 * (1 + 1e-12))


@settings(max_examples=40, deadline=None)
@given(n=st.integers(1, 4), nb=st.integers(1, 3), bs=st.sampled_from([32, 64]),
       f16=st.booleans(), seed=st.integers(0, 2 ** 31 - 1),
       spread=st.sampled_from([1e-3, 0.02, 1.0]))
def test_rtn_nearest_grid_random(n, nb, bs, f16, seed, spread):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, nb * bs)) * spread).astype(np.float32)
    dtype = np.float16 if f16 else np.float32
    q, s, zp = oracle.rtn_quantize(w, bs, dtype)
    _check_nearest_grid(w, q, s, zp, bs)


# ---------------------------------------------------------------------------
# The matmul.
# ---------------------------------------------------------------------------

def _small_case(rng, m, n, k, bs, dtype):
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32).astype(dtype)
    q, s, zp = oracle.rtn_quantize(w, bs, dtype)
    return x, q, s, zp


@pytest.mark.parametrize("dtype,bs,m,n,k", [(np.float16, 32, 2, 3, 64), (np.float32, 32, 3, 5, 128),
                                            (np.float16, 64, 1, 4, 128)])
def test_matmul_against_exact_rationals(dtype, bs, m, n, k):
    rng = np.random.default_rng(m * 100 + n)
    x, q, s, zp = _small_case(rng, m, n, k, bs, dtype)
    y = oracle.matmul_nbits(x, q, zp, s, bs)
    assert y.shape == (m, n)
    u = Fraction(1, 2 ** 53)
    for i in range(m):
        for j in range(n):
            terms = [frac(x[i, t]) * (int(q[j, t]) - int(zp[j, t // bs])) * frac(s[j, t // bs])
                     for t in range(k)]
            exact = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(frac(y[i, j]) - exact) <= k * u * mag * Fraction(11, 10)


def test_matmul_integer_special_case():
    rng = np.random.default_rng(21)
    m, n, k, bs = 4, 6, 96, 32
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zp = np.zeros((n, k // bs), dtype=np.uint8)
    s = np.ones((n, k // bs), dtype=np.float16)
    xi = rng.integers(-8, 9, size=(m, k))
    y = oracle.matmul_nbits(xi.astype(np.float16), q, zp, s, bs)
    assert np.array_equal(y, (xi.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64))


def _triple_loop_from_packed(x, qweight, packed_zp, scales, bs):
    """Pure-Python MatMulNBits straight from the stored bytes."""
    m, k = x.shape
    n = qweight.shape[0]
    y = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                code = nibbles_by_divmod(qweight[j, t // 2])[t % 2]
                z = nibbles_by_divmod(packed_zp[j, (t // bs) // 2])[(t // bs) % 2]
                acc += float(x[i, t]) * (code - z) * float(scales[j, t // bs])
            y[i][j] = acc
    return np.array(y)


@settings(max_examples=25, deadline=None)
@given(m=st.integers(1, 3), n=st.integers(1, 4), nb=st.integers(1, 3),
       bs=st.sampled_from([32, 64]), f16=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_matmul_triple_loop_random(m, n, nb, bs, f16, seed):
    rng = np.random.default_rng(seed)
    dtype = np.float16 if f16 else np.float32
    x, q, s, zp = _small_case(rng, m, n, nb * bs, bs, dtype)
    qweight, pzp = oracle.pack_weight(q, zp)
    assert np.array_equal(oracle.unpack_weight(qweight, pzp, nb * bs, bs)[0], q)
    y_loop = _triple_loop_from_packed(x, qweight, pzp, s, bs)
    y = oracle.matmul_nbits(x, q, zp, s, bs)
    ok, err, ref = oracle.within_tolerance(y, y_loop, 1e-12)
    assert ok, (err, ref)


def test_within_tolerance_is_relative_to_max():
    ok, err, ref = oracle.within_tolerance([1.0, 2.001], [1.0, 2.0], 1e-3)
    assert ok and abs(err - 0.001) < 1e-12 and ref == 2.0
    assert not oracle.within_tolerance([1.0, 2.01], [1.0, 2.0], 1e-3)[0]


# ---------------------------------------------------------------------------
# Storage accounting and workload pins from the pages.
# ---------------------------------------------------------------------------

def _golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if line and not line.startswith("#"):
                key, val, *_ = line.split()
                rows[key] = float(val)
    return rows


def test_packed_bytes_match_the_printed_decoder_size():
    sizes = _golden("page_sizes.txt")
    cfg = configs.CONFIGS[1]                      # 0.6B linears + LM head
    total = sum(oracle.packed_nbytes(l.n, l.k, 64, 4) for l in cfg.linears)
    assert abs(total / 1e6 - sizes["merged_decoder_weights_int4_block64"]) < 0.5
    # the difference to the 962 MB package is the fp32 embedding table
    emb = configs.VOCAB * 1024 * 4 / 1e6
    assert abs(sizes["decoder_weights_with_embedding"] - total / 1e6 - emb) < 1.0
    # int8 table and fp32 row scales of the 0.6B
    assert abs(configs.VOCAB * 1024 / 1e6 - sizes["int8_embedding_table"]) < 0.05
    assert abs(configs.VOCAB * 4 / 1e6 - sizes["embedding_row_scales"]) < 0.05


def test_packed_bytes_closed_form():
    # 4 bits per code, plus per block a scale and half a byte of zero point
    assert oracle.packed_nbytes(1, 64, 32, 2) == 32 + 4 + 1
    assert oracle.packed_nbytes(3, 96, 32, 4) == 3 * (48 + 12 + 2)
    with pytest.raises(ValueError):
        oracle.packed_nbytes(1, 48, 32, 2)


def test_audio_token_formula_and_prefill_rows():
    for frames, tokens in _golden("audio_tokens.txt").items():
        assert configs.audio_tokens(int(frames)) == int(tokens)
    assert configs.CONFIGS[3].m == configs.audio_tokens(3000) + 20
    assert configs.CONFIGS[5].m == configs.audio_tokens(320) + 20


# ---------------------------------------------------------------------------
# Decode-step neighbours.
# ---------------------------------------------------------------------------

def test_greedy_argmax_brute_force():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((5, 300)).astype(np.float16)
    logits[2, 17] = logits[2, 200] = 100.0        # tie -> lowest index
    idx = oracle.greedy_argmax(logits)
    for r in range(5):
        row = [float(v) for v in logits[r]]
        best = max(row)
        assert idx[r] == min(i for i, v in enumerate(row) if v == best)
    assert idx[2] == 17


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_embedding_dequant_exact(dtype):
    rng = np.random.default_rng(4)
    table = rng.integers(-128, 128, size=(50, 16), dtype=np.int8)
    scales = (rng.random(50) * 0.02).astype(np.float32)
    ids = np.array([3, 0, 49, 3])
    out = oracle.embedding_dequant(table, scales, ids, dtype)
    assert out.dtype == dtype and out.shape == (4, 16)
    for r, i in enumerate(ids):
        for c in range(16):
            assert frac(out[r, c]) == rne(int(table[i, c]) * frac(scales[i]), dtype)


# ---------------------------------------------------------------------------
# Symmetric format (fixed zero point 8, s = max|w| / 7)
# ---------------------------------------------------------------------------

def test_symmetric_on_grid_blocks_quantize_exactly():
    bs = 32
    rng = np.random.default_rng(15)
    rows, want_q, want_e = [], [], []
    for i in range(12):
        e = 2 + i % 9
        c = rng.integers(1, 16, size=bs)
        c[rng.integers(0, bs)] = 1 if i % 2 else 15   # |c - 8| = 7 is present
        rows.append((c.astype(np.float64) - 8) * 2.0 ** -e)
        want_q.append(c)
        want_e.append(e)
    w = np.array(rows, dtype=np.float32)
    for dtype in (np.float16, np.float32):
        q, s, zp = oracle.rtn_quantize_symmetric(w, bs, dtype)
        assert np.array_equal(q, np.array(want_q, dtype=np.uint8))
        assert (zp == 8).all()
        assert np.array_equal(s[:, 0].astype(np.float64), 2.0 ** -np.array(want_e, dtype=np.float64))
        assert np.array_equal(oracle.dequantize_exact(q, zp, s, bs), w.astype(np.float64))


def test_symmetric_tie_rounds_half_to_even_and_zero_block():
    sc = 2.0 ** -7
    blk = np.zeros(32)
    blk[:5] = np.array([7.0, 2.5, -1.5, 0.5, -7.0]) * sc
    w = np.stack([blk, np.zeros(32)]).astype(np.float32)
    q, s, zp = oracle.rtn_quantize_symmetric(w, 32, np.float16)
    assert float(s[0, 0]) == sc
    assert list(q[0, :5]) == [15, 10, 6, 8, 1]   # 7, rint(2.5) = 2, rint(-1.5) = -2, rint(0.5) = 0, -7
    assert float(s[1, 0]) == 0.0 and (q[1] == 8).all()


@pytest.mark.parametrize("dtype,bs", [(np.float16, 32), (np.float32, 64), (np.float16, 128), (np.float16, 256)])
def test_symmetric_codes_are_nearest_grid_points(dtype, bs):
    rng = np.random.default_rng(bs)
    w = (rng.standard_normal((6, 2 * bs)) * 0.02).astype(np.float32)
    q, s, zp = oracle.rtn_quantize_symmetric(w, bs, dtype)
    assert q.min() >= 1   # max|w| / s <= 7: the code 0 (offset -8) is never needed
    for i in range(w.shape[0]):
        for b in range(w.shape[1] // bs):
            sb = frac(s[i, b])
            for j in range(bs):
                v = frac(w[i, b * bs + j])
                dist = [abs(v - (c - 8) * sb) for c in range(16)]
                best = min(dist)
                cands = [c for c in range(16) if dist[c] == best]
                c = int(q[i, b * bs + j])
                assert c in cands
                if len(cands) == 2:
                    assert (c - 8) % 2 == 0


@pytest.mark.parametrize("dtype,u", [(np.float16, 2.0 ** -11), (np.float32, 2.0 ** -24)])
def test_symmetric_round_trip_bound(dtype, u):
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    q, s, zp = oracle.rtn_quantize_symmetric(w, 64, dtype)
    d = oracle.dequantize_exact(q, zp, s, 64)
    err = np.abs(w.astype(np.float64) - d).reshape(40, 4, 64).max(axis=2)
    assert (err <= s.astype(np.float64) * (0.5 + 7 * u)).all()


# ---------------------------------------------------------------------------
# Int8 compute mode: activation quantizer and the integer-dot product.
# ---------------------------------------------------------------------------

def rint_half_even(fr):
    """Nearest integer to a Fraction, ties to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def a8_reference(block):
    """One block of float32 activations -> (scale, codes), from exact
    rationals and the integer float32 rounding routine above."""
    vals = [frac(v) for v in block]
    amax = max(abs(v) for v in vals)
    scale = rne(amax / 127, np.float32)
    if scale == 0:
        return Fraction(0), [0] * len(vals)
    codes = [max(-127, min(127, rint_half_even(rne(v / scale, np.float32)))) for v in vals]
    return scale, codes


@pytest.mark.parametrize("f16,bs", [(True, 32), (False, 32), (True, 64), (False, 128)])
def test_a8_quantizer_against_exact_rationals(f16, bs):
    rng = np.random.default_rng(bs + 3 * f16)
    x = rng.standard_normal((3, 2 * bs)).astype(np.float16 if f16 else np.float32)
    x[1, :bs] *= 1e-3           # a small-magnitude block
    x[2, bs:] = 0.0             # an all-zero block
    qa, a_s = oracle.quantize_activations_i8(x, bs)
    assert qa.dtype == np.int8 and a_s.dtype == np.float32 and a_s.shape == (3, 2)
    for m in range(3):
        for b in range(2):
            scale, codes = a8_reference(x[m, b * bs:(b + 1) * bs])
            assert frac(a_s[m, b]) == scale
            assert [int(c) for c in qa[m, b * bs:(b + 1) * bs]] == codes


def test_a8_extremes_ties_and_zero_block():
    bs = 32
    x = np.zeros((2, 2 * bs), dtype=np.float32)
    # amax = 127/8 gives the exact scale 1/8: the extremes are +-127 and
    # quotients k + 1/2 round to even
    x[0, 0] = 127 / 8
    x[0, 1] = -127 / 8
    x[0, 2] = 2.5 / 8
    x[0, 3] = 3.5 / 8
    x[0, 4] = -2.5 / 8
    x[0, 5] = 0.5 / 8
    qa, a_s = oracle.quantize_activations_i8(x, bs)
    assert a_s[0, 0] == np.float32(1 / 8)
    assert list(qa[0, :6]) == [127, -127, 2, 4, -2, 0]
    assert a_s[0, 1] == 0 and a_s[1, 0] == 0 and not qa[1].any() and not qa[0, bs:].any()


@pytest.mark.parametrize("bs", [32, 64])
def test_a8_round_trip_bound(bs):
    rng = np.random.default_rng(40 + bs)
    x = (rng.standard_normal((8, 4 * bs)) * rng.choice([1e-3, 1.0, 30.0], size=(8, 1))).astype(np.float32)
    qa, a_s = oracle.quantize_activations_i8(x, bs)
    s = np.repeat(a_s.astype(np.float64), bs, axis=1)
    err = np.abs(x.astype(np.float64) - qa.astype(np.float64) * s)
    # half a step, plus the float32 roundings of the scale and of the quotient
    assert np.all(err <= s * (0.5 + 127 * 2.0 ** -22))
    assert np.all(np.abs(qa.astype(np.int64)) <= 127)


def test_a8_product_equals_plain_product_when_activations_are_exact():
    """Blocks whose largest magnitude is 127 * 2^-e and whose values are
    multiples of 2^-e quantize exactly, so the int8 product is the plain
    product (pinned on its own) computed another way."""
    rng = np.random.default_rng(9)
    m, n, bs, nb = 3, 5, 32, 4
    k = bs * nb
    codes = rng.integers(-127, 128, size=(m, k))
    codes[:, ::bs] = 127                      # every block reaches 127
    e = rng.integers(2, 9, size=(m, nb))
    x = (codes * np.repeat(2.0 ** -e, bs, axis=1)).astype(np.float32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s, zp = oracle.rtn_quantize(w, bs, np.float16)
    y8 = oracle.matmul_nbits_i8(x, q, zp, s, bs)
    y = oracle.matmul_nbits(x, q, zp, s, bs)
    assert np.array_equal(y8, y)


@pytest.mark.parametrize("bs", [32, 64])
def test_a8_product_against_fractions(bs):
    rng = np.random.default_rng(77 + bs)
    m, n, k = 2, 3, 2 * bs
    x = rng.standard_normal((m, k)).astype(np.float16)
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zp = rng.integers(0, 16, size=(n, k // bs), dtype=np.uint8)
    s = (rng.random((n, k // bs)) * 0.01 + 1e-4).astype(np.float16)
    y = oracle.matmul_nbits_i8(x, q, zp, s, bs)
    for i in range(m):
        blocks = [a8_reference(x[i, b * bs:(b + 1) * bs]) for b in range(k // bs)]
        for jn in range(n):
            exact = Fraction(0)
            for b, (scale, codes) in enumerate(blocks):
                isum = sum((int(q[jn, b * bs + t]) - int(zp[jn, b])) * codes[t] for t in range(bs))
                exact += frac(s[jn, b]) * scale * isum
            # float64 scaling and sum over two blocks: within a few roundings
            assert abs(frac(y[i, jn]) - exact) <= abs(exact) * 2 ** -50 + Fraction(1, 2 ** 80)

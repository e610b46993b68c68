"""GPU: int8 embedding-row gather (mnb_embed_gather) against the oracle,
bit for bit: every output is the exact int8 x float32 product rounded once
to the output dtype. Float16 outputs include products whose float32
rounding lands exactly on a float16 midpoint, where a plain float32 ->
float16 conversion would round twice."""

import numpy as np
import pytest
import torch

import oracle
from block_wise_int4_amd import mnb
from workloads import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {np.float16: torch.float16, np.float32: torch.float32}


def _gather(table, scales, ids, dt):
    out = mnb.mnb_embed_gather(torch.from_numpy(table).to(DEV), torch.from_numpy(scales).to(DEV),
                               torch.from_numpy(ids).to(DEV), TD[dt])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _expected(table, scales, ids, dt):
    ok = (ids >= 0) & (ids < table.shape[0])
    ref = np.zeros((ids.size, table.shape[1]), dtype=dt)
    if ok.any():
        ref[ok] = oracle.embedding_dequant(table, scales, ids[ok], dt)
    return ref


@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("vocab,hidden,tokens", [(5000, 1024, 64), (3000, 2048, 410), (77, 16, 5), (100, 48, 1)])
def test_gather_bit_exact(vocab, hidden, tokens, dt):
    table, scales, ids = synth.embedding_inputs(vocab + hidden, vocab, hidden, tokens)
    ids[0] = ids[-1]  # a repeated id
    got = _gather(table, scales, ids, dt)
    assert np.array_equal(got.view(np.uint8), _expected(table, scales, ids, dt).view(np.uint8))


def test_gather_out_of_range_ids_give_zero_rows():
    table, scales, ids = synth.embedding_inputs(5, 200, 64, 6)
    ids[:] = [3, -1, 200, 199, 2 ** 40, 0]
    got = _gather(table, scales, ids, np.float16)
    assert np.array_equal(got.view(np.uint16), _expected(table, scales, ids, np.float16).view(np.uint16))
    assert not got[1].any() and not got[2].any() and not got[4].any()


def test_gather_float16_midpoints_round_once():
    # scales s with q * s just above or below a float16 midpoint m, close
    # enough that the float32 product is m itself
    rng = np.random.default_rng(11)
    mids, qs = [], []
    for _ in range(400):
        e = int(rng.integers(-12, 4))
        mant = int(rng.integers(1024, 2048))
        m = (mant + 0.5) * 2.0 ** (e - 10)             # a float16 midpoint
        q = int(rng.choice([3, 5, 7, 9, 11, 13, 25, 51, 101, 127]))
        for sgn in (-1, 1):
            s = np.float32((m + sgn * m * 2.0 ** -30) / q)
            if np.float32(q) * s == np.float32(m) and float(q) * float(s) != m:
                mids.append(s)
                qs.append(q)
    assert len(mids) > 50
    vocab = len(mids)
    table = np.zeros((vocab, 16), dtype=np.int8)
    table[:, 0] = qs
    table[:, 1] = -np.array(qs)
    scales = np.array(mids, dtype=np.float32)
    ids = np.arange(vocab, dtype=np.int64)
    got = _gather(table, scales, ids, np.float16)
    ref = _expected(table, scales, ids, np.float16)
    naive = (table[:, :2].astype(np.float32) * scales[:, None]).astype(np.float16)
    assert (naive != ref[:, :2]).any(), "the cases do not exercise double rounding"
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_gather_full_size_table():
    table, scales, ids = synth.embedding_inputs(7, 151936, 2048, 410)
    got = _gather(table, scales, ids, np.float16)
    assert np.array_equal(got.view(np.uint16), _expected(table, scales, ids, np.float16).view(np.uint16))

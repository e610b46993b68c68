"""Seeded synthetic inputs shared by the tests, the oracle checks and the
benchmark. Random numbers only: no quantization or matmul arithmetic.

Recipe (one generator per linear, so any linear can be regenerated alone):
  stream = PCG64(SeedSequence(SEED, spawn_key=(config, layer + 1, proj)))
  W = standard_normal((N, K), float32) * 0.02        (std 0.02)
  X = standard_normal((M, K), float32), cast to the activation dtype
W is drawn first, then X, from the same stream.
"""

import concurrent.futures as _cf
import os

import numpy as np

from .configs import PROJ_INDEX

SEED = 0
WEIGHT_STD = np.float32(0.02)

_NP_DTYPES = {"f32": np.float32, "f16": np.float16}


def np_dtype(name):
    return _NP_DTYPES[name]


def stream(config_index, layer, proj):
    key = (int(config_index), int(layer) + 1, PROJ_INDEX[proj])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=key)))


def weight(rng, n, k):
    return rng.standard_normal((n, k), dtype=np.float32) * WEIGHT_STD


def activation(rng, m, k, dtype):
    return rng.standard_normal((m, k), dtype=np.float32).astype(np_dtype(dtype))


def linear_inputs(cfg, lin, m=None):
    """(W float32 [N, K], X [M, K] in the config's activation dtype)."""
    rng = stream(cfg.index, lin.layer, lin.proj)
    w = weight(rng, lin.n, lin.k)
    x = activation(rng, cfg.m if m is None else m, lin.k, cfg.dtype)
    return w, x


def all_linear_inputs(cfg, linears=None, m=None, workers=None):
    """linear_inputs for many linears, generated on a thread pool (each
    linear has its own stream, so the result does not depend on the pool)."""
    linears = cfg.linears if linears is None else linears
    workers = workers or min(16, len(os.sched_getaffinity(0)))
    with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda lin: linear_inputs(cfg, lin, m), linears))


def random_case(seed, m, n, k, dtype, weight_std=0.02):
    """A small free-standing case for shape sweeps: (W float32, X)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(99, seed))))
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(weight_std)
    x = rng.standard_normal((m, k), dtype=np.float32).astype(np_dtype(dtype))
    return w, x


def embedding_inputs(seed, vocab, hidden, tokens):
    """A synthetic int8 embedding table with per-row float32 scales and token
    ids: table uniform in [-127, 127], scales |N(0, 0.02)| / 127 (rows of
    about the spread of the float weights), ids uniform over the vocabulary."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(98, seed))))
    table = rng.integers(-127, 128, size=(vocab, hidden), dtype=np.int8)
    scales = (np.abs(rng.standard_normal(vocab)) * 0.02 / 127).astype(np.float32)
    ids = rng.integers(0, vocab, size=tokens, dtype=np.int64)
    return table, scales, ids

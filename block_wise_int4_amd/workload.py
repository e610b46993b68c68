"""Device-resident workloads for the benchmark and the full-size tests: every
linear of a configuration quantized (RTN, on the GPU) and packed, with its
activations and an output buffer, and grouped plans over them.

Weights and activations come from the seeded generators in `workloads`
(float32 W on the host, one stream per linear); quantization and packing run
in the library's kernels.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

from workloads import synth

from . import mnb

_TORCH = {"f32": torch.float32, "f16": torch.float16}


def torch_dtype(name):
    return _TORCH[name]


@dataclass
class LinearData:
    lin: object                 # workloads.configs.Linear
    pw: mnb.PackedWeight
    x: torch.Tensor             # [M, K]
    y: torch.Tensor             # [M, N]
    canonical: tuple = None     # (qweight, scales, zero_points) if kept
    sample_rows: np.ndarray = None
    w_rows: np.ndarray = None   # float32 W[sample_rows] for the oracle


@dataclass
class ConfigData:
    cfg: object
    linears: list
    plan: mnb.Plan = None
    replicas: list = field(default_factory=list)   # extra (linears, plan) copies


def build_linear(cfg, lin, device, m=None, keep_canonical=False, sample_rows=0, rng_rows=None):
    w, x = synth.linear_inputs(cfg, lin, m)
    dt = torch_dtype(cfg.dtype)
    wd = torch.from_numpy(w).to(device)
    q, s, z = mnb.mnb_quantize_rtn(wd, cfg.block_size, dt, symmetric=cfg.symmetric)
    pw = mnb.mnb_pack(q, s, z, lin.n, lin.k, cfg.block_size)
    xd = torch.from_numpy(x).to(device)
    y = torch.empty((x.shape[0], lin.n), dtype=dt, device=device)
    ld = LinearData(lin, pw, xd, y)
    if keep_canonical:
        ld.canonical = (q, s, z)
    if sample_rows:
        rng = rng_rows or np.random.default_rng(lin.n * 7 + lin.k + max(lin.layer, 0))
        rows = np.sort(rng.choice(lin.n, size=min(sample_rows, lin.n), replace=False))
        ld.sample_rows = rows
        ld.w_rows = w[rows].copy()
        ld.canonical = (q[rows.tolist()].cpu().numpy(), s[rows.tolist()].cpu().numpy(),
                        None if z is None else z[rows.tolist()].cpu().numpy())
    del wd
    return ld


def build_config(cfg, device, linears=None, m=None, keep_canonical=False, sample_rows=0):
    """Quantize and pack `linears` (default: all of the config) on `device`."""
    linears = cfg.linears if linears is None else linears
    out = [build_linear(cfg, lin, device, m, keep_canonical, sample_rows) for lin in linears]
    return ConfigData(cfg, out)


def make_plan(cfg, linears):
    problems = [(ld.x, ld.pw, ld.y) for ld in linears]
    return mnb.mnb_plan_grouped(problems, cfg.block_size, torch_dtype(cfg.dtype))


def replicate(cfg, linears):
    """A copy of every packed weight, activation and output at new addresses."""
    out = []
    for ld in linears:
        pw = mnb.PackedWeight(ld.pw.packed.clone(), ld.pw.N, ld.pw.K, ld.pw.block_size, ld.pw.dtype, ld.pw.bits)
        out.append(LinearData(ld.lin, pw, ld.x.clone(), torch.empty_like(ld.y)))
    return out


def algorithmic_bytes(cfg, linears=None):
    """Bytes the method must move per step: codes + scales + packed zero
    points (none in the symmetric format) + activations + outputs, each
    counted once."""
    linears = cfg.linears if linears is None else linears
    a = 2 if cfg.dtype == "f16" else 4
    total = 0
    for lin in linears:
        nb = lin.k // cfg.block_size
        total += lin.n * lin.k // 2 + lin.n * nb * a + (0 if cfg.symmetric else lin.n * ((nb + 1) // 2))
        total += cfg.m * lin.k * a + cfg.m * lin.n * a
    return total


def flops(cfg, linears=None):
    linears = cfg.linears if linears is None else linears
    return sum(2 * cfg.m * lin.n * lin.k for lin in linears)

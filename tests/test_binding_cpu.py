"""Argument checks of the Python binding that need no GPU: a caller-provided
output or input buffer of the wrong dtype, size or device is refused before
anything reaches the library. CPU tensors stand in for device tensors; every
call below raises before a device address is taken."""

import pytest
import torch

from block_wise_int4_amd import mnb

N, K, BS = 64, 256, 32
F16 = torch.float16


def _pw(dtype=F16, bs=BS, device="cpu"):
    return mnb.PackedWeight(torch.zeros(4096, dtype=torch.uint8, device=device), N, K, bs, dtype)


def _x(m=None, dtype=F16):
    return torch.zeros(K if m is None else (m, K), dtype=dtype)


@pytest.mark.parametrize("y, msg", [
    (torch.zeros(N - 1, dtype=F16), "elements"),
    (torch.zeros(N, dtype=torch.float32), "must be"),
    (torch.zeros(2 * N, dtype=F16), "elements"),
])
def test_gemv_output_checked(y, msg):
    with pytest.raises(ValueError, match=msg):
        mnb.mnb_gemv(_x(), _pw(), y)


@pytest.mark.parametrize("m, y, msg", [
    (5, torch.zeros((4, N), dtype=F16), "elements"),
    (5, torch.zeros((5, N - 16), dtype=F16), "elements"),
    (5, torch.zeros((5, N), dtype=torch.float32), "must be"),
])
def test_gemm_output_checked(m, y, msg):
    with pytest.raises(ValueError, match=msg):
        mnb.mnb_gemm(_x(m), _pw(), y)


def test_weight_and_activation_on_one_device():
    meta = mnb.PackedWeight(torch.zeros(16, dtype=torch.uint8, device="meta"), N, K, BS, F16)
    with pytest.raises(ValueError, match="weight is on"):
        mnb.mnb_gemm(_x(3), meta)


def test_argmax_buffers_checked():
    ws = torch.zeros(mnb.ARGMAX_WORKSPACE_BYTES // 8, dtype=torch.int64)
    with pytest.raises(ValueError, match="elements"):
        mnb.mnb_gemv_argmax(_x(), _pw(), ws, y=torch.zeros(N - 1, dtype=F16))
    with pytest.raises(ValueError, match="must be"):
        mnb.mnb_gemv_argmax(_x(), _pw(), ws, index=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="elements"):
        mnb.mnb_gemv_argmax(_x(), _pw(), ws, index=torch.zeros(0, dtype=torch.int64))
    with pytest.raises(ValueError, match="workspace"):
        mnb.mnb_gemv_argmax(_x(), _pw(), ws[:10])


def test_plan_checks_each_problem():
    good = (_x(2), _pw(), None)
    with pytest.raises(ValueError, match=r"y\[1\]"):
        mnb.mnb_plan_grouped([good, (_x(2), _pw(), torch.zeros((3, N), dtype=F16))], BS, F16)
    with pytest.raises(ValueError, match="format differs"):
        mnb.mnb_plan_grouped([good, (_x(2), _pw(bs=64), None)], BS, F16)
    with pytest.raises(ValueError, match="format differs"):
        mnb.mnb_plan_grouped([good], BS, torch.float32)


def test_embed_gather_output_checked():
    table = torch.zeros((10, 8), dtype=torch.int8)
    rs = torch.zeros(10, dtype=torch.float32)
    ids = torch.zeros(3, dtype=torch.int64)
    with pytest.raises(ValueError, match="elements"):
        mnb.mnb_embed_gather(table, rs, ids, out=torch.zeros((2, 8), dtype=F16))
    with pytest.raises(ValueError, match="one device"):
        mnb.mnb_embed_gather(table, rs, ids.to("meta"))


def test_quantize_outputs_checked():
    w = torch.zeros((N, K), dtype=torch.float32)
    nb = K // BS
    q = torch.zeros((N, K // 2), dtype=torch.uint8)
    s = torch.zeros((N, nb), dtype=F16)
    z = torch.zeros((N, nb // 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="qweight"):
        mnb.mnb_quantize_rtn(w, BS, F16, out=(q[:-1], s, z))
    with pytest.raises(ValueError, match="scales"):
        mnb.mnb_quantize_rtn(w, BS, F16, out=(q, s.float(), z))
    with pytest.raises(ValueError, match="zero_points"):
        mnb.mnb_quantize_rtn(w, BS, F16, out=(q, s, z[:, :1]))


def test_pack_inputs_checked():
    nb = K // BS
    q = torch.zeros((N, K // 2), dtype=torch.uint8)
    s = torch.zeros((N, nb), dtype=F16)
    z = torch.zeros((N, (nb + 1) // 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="qweight"):
        mnb.mnb_pack(q[:, :-1], s, z, N, K, BS)
    with pytest.raises(ValueError, match="scales"):
        mnb.mnb_pack(q, s[:-1], z, N, K, BS)
    with pytest.raises(ValueError, match="zero_points"):
        mnb.mnb_pack(q, s, z[:-1], N, K, BS)
    with pytest.raises(ValueError, match="qweight"):
        mnb.mnb_pack(q.view(torch.int8), s, z, N, K, BS)

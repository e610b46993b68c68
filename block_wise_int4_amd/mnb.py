"""Python binding for libmnb.so (include/mnb.h), through ctypes.

Argument marshalling only: every function here checks Python-side types,
takes device pointers and torch's current HIP stream, and calls the C entry
point of the same name. PyTorch only provides device memory and streams.
The library must be built (block_wise_int4_amd.build); nothing falls back
to another implementation when it is missing.
"""

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmnb.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "mnb.h")

MNB_F32 = 0
MNB_F16 = 1
_DTYPES = {torch.float32: MNB_F32, torch.float16: MNB_F16}
_TORCH_DTYPES = {MNB_F32: torch.float32, MNB_F16: torch.float16}

STATUS = {
    0: "MNB_OK", 1: "MNB_ERR_NULL", 2: "MNB_ERR_BITS", 3: "MNB_ERR_BLOCK", 4: "MNB_ERR_SHAPE",
    5: "MNB_ERR_DTYPE", 6: "MNB_ERR_ALIGN", 7: "MNB_ERR_HIP", 8: "MNB_ERR_PLAN", 9: "MNB_ERR_INVALID",
}

_lib = None


class MnbError(RuntimeError):
    def __init__(self, fn, status, message):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({message})")
        self.status = status


class mnb_problem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_SIGNATURES = {
    "mnb_abi_version": (_int, []),
    "mnb_status_string": (ctypes.c_char_p, [_int]),
    "mnb_packed_bytes": (_sz, [_i64, _i64, _int, _int, _int]),
    "mnb_quantize_rtn": (_int, [_vp, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp]),
    "mnb_pack": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp, _vp]),
    "mnb_unpack": (_int, [_vp, _i64, _i64, _int, _int, _int, _vp, _vp, _vp]),
    "mnb_dequant": (_int, [_vp, _i64, _i64, _int, _int, _int, _vp, _vp]),
    "mnb_gemv": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "mnb_gemv_argmax": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "mnb_gemv_argmax_noalloc": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "mnb_embed_gather": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _vp]),
    "mnb_embed_gather_argmax": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _vp, _vp]),
    "mnb_gemm": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _vp]),
    "mnb_gemm_split_k_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int, _int, _int]),
    "mnb_gemm_split_k": (_int, [_vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _int, _int, _int, _int, _vp]),
    "mnb_gemm_i8_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "mnb_quantize_act_i8": (_int, [_vp, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "mnb_gemm_i8": (_int, [_vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _int, _int, _int, _vp]),
    "mnb_plan_bytes": (_sz, [_int]),
    "mnb_plan_grouped": (_int, [ctypes.POINTER(mnb_problem), _int, _int, _int, _int, _vp, _sz]),
    "mnb_plan_grouped_i8": (_int, [ctypes.POINTER(mnb_problem), _int, _int, _int, _int, _vp, _sz]),
    "mnb_plan_launches": (_int, [_vp]),
    "mnb_gemm_grouped": (_int, [_vp, _vp, _vp]),
}


def header_functions():
    """Names of the functions include/mnb.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mnb_[a-z0-9_]+)\s*\(", text)))


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_wise_int4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise MnbError(fn, status, lib().mnb_status_string(status).decode())


def _dev(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check_buf(t, name, dtype, numel, device):
    """A caller-provided buffer the kernels read or write whole: its dtype,
    size and device must match (contiguity is checked by _dev)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, {numel} expected")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, not {device}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def dtype_code(dtype):
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    return _DTYPES[dtype]


def mnb_abi_version():
    return lib().mnb_abi_version()


def mnb_status_string(status):
    return lib().mnb_status_string(status).decode()


def mnb_packed_bytes(N, K, block_size, dtype, bits=4):
    return lib().mnb_packed_bytes(N, K, bits, block_size, dtype_code(dtype))


@dataclass
class PackedWeight:
    """A packed weight in device memory plus the shape it was packed for."""
    packed: torch.Tensor
    N: int
    K: int
    block_size: int
    dtype: torch.dtype
    bits: int = 4


def mnb_quantize_rtn(w, block_size, dtype, bits=4, out=None, symmetric=False):
    """RTN-quantize float32 W[N, K] on the GPU -> (qweight, scales, zero_points),
    canonical layout; symmetric=True: no zero points (None), fixed zero point 8."""
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    N, K = w.shape
    nb = K // block_size if block_size else 0
    if out is None:
        out = (torch.empty((N, K // 2), dtype=torch.uint8, device=w.device),
               torch.empty((N, max(nb, 1)), dtype=dtype, device=w.device),
               None if symmetric else torch.empty((N, max((nb + 1) // 2, 1)), dtype=torch.uint8, device=w.device))
    q, s, z = out
    if block_size in (32, 64, 128, 256) and K % block_size == 0 and K % 2 == 0:
        _check_buf(q, "qweight", torch.uint8, N * K // 2, w.device)
        _check_buf(s, "scales", dtype, N * nb, w.device)
        if z is not None:
            _check_buf(z, "zero_points", torch.uint8, N * ((nb + 1) // 2), w.device)
    _check("mnb_quantize_rtn", lib().mnb_quantize_rtn(
        _dev(w, "w"), N, K, bits, block_size, dtype_code(dtype),
        _dev(q, "qweight"), _dev(s, "scales"), None if z is None else _dev(z, "zero_points"), _stream(w.device)))
    return q, s, z


def mnb_pack(qweight, scales, zero_points, N, K, block_size, bits=4, packed=None):
    """Canonical format -> PackedWeight (device layout of the compute kernels).
    zero_points None: the symmetric format (zero point 8 in every block)."""
    dtype = scales.dtype
    zp_arg = (lambda: None) if zero_points is None else (lambda: _dev(zero_points, "zero_points"))
    nbytes = mnb_packed_bytes(N, K, block_size, dtype, bits)
    if nbytes:
        nb = K // block_size
        _check_buf(qweight, "qweight", torch.uint8, N * K // 2, qweight.device)
        _check_buf(scales, "scales", dtype, N * nb, qweight.device)
        if zero_points is not None:
            _check_buf(zero_points, "zero_points", torch.uint8, N * ((nb + 1) // 2), qweight.device)
    if nbytes == 0:
        # invalid format: let the library name the error (it returns before
        # touching the GPU, so a placeholder output address is never used)
        _check("mnb_pack", lib().mnb_pack(
            _dev(qweight, "qweight"), _dev(scales, "scales"), zp_arg(),
            N, K, bits, block_size, dtype_code(dtype), ctypes.c_void_p(256), None))
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=qweight.device)
    elif packed.numel() * packed.element_size() < nbytes:
        raise ValueError("packed buffer too small")
    _check("mnb_pack", lib().mnb_pack(
        _dev(qweight, "qweight"), _dev(scales, "scales"), zp_arg(),
        N, K, bits, block_size, dtype_code(dtype), _dev(packed, "packed"), _stream(qweight.device)))
    return PackedWeight(packed, N, K, block_size, dtype, bits)


def mnb_unpack(pw):
    """Read back (q uint8 [N, K], zp uint8 [N, K/bs]) from a PackedWeight."""
    dev = pw.packed.device
    q = torch.empty((pw.N, pw.K), dtype=torch.uint8, device=dev)
    zp = torch.empty((pw.N, pw.K // pw.block_size), dtype=torch.uint8, device=dev)
    _check("mnb_unpack", lib().mnb_unpack(
        _dev(pw.packed, "packed"), pw.N, pw.K, pw.bits, pw.block_size, dtype_code(pw.dtype),
        _dev(q, "q"), _dev(zp, "zp"), _stream(dev)))
    return q, zp


def mnb_dequant(pw):
    """Dequantized weights [N, K] in the scale dtype."""
    dev = pw.packed.device
    w = torch.empty((pw.N, pw.K), dtype=pw.dtype, device=dev)
    _check("mnb_dequant", lib().mnb_dequant(
        _dev(pw.packed, "packed"), pw.N, pw.K, pw.bits, pw.block_size, dtype_code(pw.dtype),
        _dev(w, "w"), _stream(dev)))
    return w


def _check_x(x, pw, name="x"):
    if x.dtype != pw.dtype:
        raise ValueError(f"{name} dtype {x.dtype} differs from the weight's {pw.dtype}")
    if x.shape[-1] != pw.K:
        raise ValueError(f"{name} has {x.shape[-1]} inputs, the weight {pw.K}")
    if pw.packed.device != x.device:
        raise ValueError(f"the weight is on {pw.packed.device}, {name} on {x.device}")


def mnb_gemv(x, pw, y=None):
    """y[N] = x[K] @ dequant(W)^T."""
    _check_x(x, pw)
    if x.numel() != pw.K:
        raise ValueError("mnb_gemv takes one activation row")
    if y is None:
        y = torch.empty(pw.N, dtype=pw.dtype, device=x.device)
    _check_buf(y, "y", pw.dtype, pw.N, x.device)
    _check("mnb_gemv", lib().mnb_gemv(
        _dev(x, "x"), _dev(pw.packed, "packed"), _dev(y, "y"), pw.N, pw.K, pw.bits, pw.block_size,
        dtype_code(pw.dtype), _stream(x.device)))
    return y


ARGMAX_WORKSPACE_BYTES = 8192


def argmax_workspace(device):
    """A workspace for mnb_gemv_argmax (reusable by calls that run one after
    another on one stream)."""
    return torch.empty(ARGMAX_WORKSPACE_BYTES // 8, dtype=torch.int64, device=device)


def mnb_gemv_argmax(x, pw, workspace, y=None, index=None, logits=False, partial=False):
    """Greedy argmax of y = x @ dequant(W)^T, fused into the decode product.
    Returns the index as a device int64 tensor of one element (and y, when
    logits=True or y is given). With partial=True only the per-workgroup
    partial results are written to workspace (one launch), for
    mnb_embed_gather_argmax; then the index is None."""
    _check_x(x, pw)
    if x.numel() != pw.K:
        raise ValueError("mnb_gemv_argmax takes one activation row")
    if workspace.numel() * workspace.element_size() < ARGMAX_WORKSPACE_BYTES or workspace.device != x.device:
        raise ValueError("workspace: a device buffer from argmax_workspace()")
    if y is None and logits:
        y = torch.empty(pw.N, dtype=pw.dtype, device=x.device)
    if y is not None:
        _check_buf(y, "y", pw.dtype, pw.N, x.device)
    if partial:
        index = None
    else:
        if index is None:
            index = torch.empty(1, dtype=torch.int64, device=x.device)
        _check_buf(index, "index", torch.int64, 1, x.device)
    _check("mnb_gemv_argmax", lib().mnb_gemv_argmax(
        _dev(x, "x"), _dev(pw.packed, "packed"), None if y is None else _dev(y, "y"),
        None if index is None else _dev(index, "index"), _dev(workspace, "workspace"), pw.N, pw.K, pw.bits,
        pw.block_size, dtype_code(pw.dtype), _stream(x.device)))
    return (index, y) if y is not None else index


def mnb_gemv_argmax_noalloc(x, pw, y=None, index=None, logits=False):
    """mnb_gemv_argmax with the library's own per-device partial-result
    slots instead of a workspace (for callers that cannot allocate); calls
    that may overlap on one device race."""
    _check_x(x, pw)
    if x.numel() != pw.K:
        raise ValueError("mnb_gemv_argmax_noalloc takes one activation row")
    if y is None and logits:
        y = torch.empty(pw.N, dtype=pw.dtype, device=x.device)
    if y is not None:
        _check_buf(y, "y", pw.dtype, pw.N, x.device)
    if index is None:
        index = torch.empty(1, dtype=torch.int64, device=x.device)
    _check_buf(index, "index", torch.int64, 1, x.device)
    _check("mnb_gemv_argmax_noalloc", lib().mnb_gemv_argmax_noalloc(
        _dev(x, "x"), _dev(pw.packed, "packed"), None if y is None else _dev(y, "y"), _dev(index, "index"),
        pw.N, pw.K, pw.bits, pw.block_size, dtype_code(pw.dtype), _stream(x.device)))
    return (index, y) if y is not None else index


def mnb_embed_gather(table, row_scales, ids, dtype=torch.float16, out=None):
    """out[t] = table[ids[t]] (int8 [V, H]) * row_scales[ids[t]] (float32 [V]),
    rounded once to dtype; ids outside [0, V) give zero rows."""
    if table.dtype != torch.int8 or table.dim() != 2:
        raise TypeError("table must be int8 [V, H]")
    if row_scales.dtype != torch.float32 or row_scales.numel() != table.shape[0]:
        raise TypeError("row_scales must be float32 [V]")
    if ids.dtype != torch.int64:
        raise TypeError("ids must be int64")
    V, H = table.shape
    T = ids.numel()
    if out is None:
        out = torch.empty((T, H), dtype=dtype, device=table.device)
    _check_buf(out, "out", out.dtype, T * H, table.device)
    if row_scales.device != table.device or ids.device != table.device:
        raise ValueError("table, row_scales and ids must be on one device")
    _check("mnb_embed_gather", lib().mnb_embed_gather(
        _dev(table, "table"), _dev(row_scales, "row_scales"), _dev(ids, "ids"), T, V, H, dtype_code(out.dtype),
        _dev(out, "out"), _stream(table.device)))
    return out


def mnb_embed_gather_argmax(table, row_scales, workspace, dtype=torch.float16, out=None, index=None):
    """The embedding row (int8 table [V, H] times row_scales [V], rounded once
    to dtype) of the greedy argmax whose partial results a preceding
    mnb_gemv_argmax(..., partial=True) on an LM head of V rows left in
    workspace, on the same stream. Returns (out [1, H], index [1])."""
    if table.dtype != torch.int8 or table.dim() != 2:
        raise TypeError("table must be int8 [V, H]")
    if row_scales.dtype != torch.float32 or row_scales.numel() != table.shape[0]:
        raise TypeError("row_scales must be float32 [V]")
    if workspace.numel() * workspace.element_size() < ARGMAX_WORKSPACE_BYTES or workspace.device != table.device:
        raise ValueError("workspace: the argmax workspace the LM head's partial call wrote")
    V, H = table.shape
    if out is None:
        out = torch.empty((1, H), dtype=dtype, device=table.device)
    _check_buf(out, "out", out.dtype, H, table.device)
    if index is None:
        index = torch.empty(1, dtype=torch.int64, device=table.device)
    _check_buf(index, "index", torch.int64, 1, table.device)
    if row_scales.device != table.device:
        raise ValueError("table and row_scales must be on one device")
    _check("mnb_embed_gather_argmax", lib().mnb_embed_gather_argmax(
        _dev(table, "table"), _dev(row_scales, "row_scales"), _dev(workspace, "workspace"), _dev(index, "index"),
        V, H, dtype_code(out.dtype), _dev(out, "out"), _stream(table.device)))
    return out, index


def mnb_gemm(x, pw, y=None):
    """Y[M, N] = X[M, K] @ dequant(W)^T for any M >= 1."""
    _check_x(x, pw)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, pw.N), dtype=pw.dtype, device=x.device)
    _check_buf(y, "y", pw.dtype, M * pw.N, x.device)
    _check("mnb_gemm", lib().mnb_gemm(
        _dev(x, "x"), _dev(pw.packed, "packed"), _dev(y, "y"), M, pw.N, pw.K, pw.bits, pw.block_size,
        dtype_code(pw.dtype), _stream(x.device)))
    return y


@dataclass
class Plan:
    host: torch.Tensor       # uint8 image written by mnb_plan_grouped (CPU)
    device: torch.Tensor     # the same bytes in device memory
    outputs: list            # the y tensors, in problem order (kept alive)
    inputs: list             # the x tensors and packed weights (kept alive)


def mnb_plan_grouped(problems, block_size, dtype, device=None, bits=4, int8=False):
    """problems: list of (x [M, K], PackedWeight, y [M, N] or None). Returns a Plan.
    int8=True plans the int8 compute mode (decode products, M = 1, only)."""
    count = len(problems)
    nbytes = lib().mnb_plan_bytes(count)
    if nbytes == 0:
        raise MnbError("mnb_plan_bytes", 8, "count out of range")
    arr = (mnb_problem * count)()
    outs, keep = [], []
    device = torch.device(device) if device is not None else problems[0][0].device
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    for i, (x, pw, y) in enumerate(problems):      # every problem checked before any is marshalled
        _check_x(x, pw)
        if (pw.block_size, pw.dtype, pw.bits) != (block_size, dtype, bits):
            raise ValueError(f"problem {i}: the weight's format differs from the plan's")
        if x.device != device:
            raise ValueError(f"problem {i}: x is on {x.device}, the plan on {device}")
        if y is not None:
            _check_buf(y, f"y[{i}]", pw.dtype, (1 if x.dim() == 1 else x.shape[0]) * pw.N, x.device)
    for i, (x, pw, y) in enumerate(problems):
        M = 1 if x.dim() == 1 else x.shape[0]
        if y is None:
            y = torch.empty((M, pw.N), dtype=pw.dtype, device=x.device)
        arr[i] = mnb_problem(_dev(x, "x").value, _dev(pw.packed, "packed").value, _dev(y, "y").value,
                             M, pw.N, pw.K)
        outs.append(y)
        keep.append((x, pw))
    host = torch.empty(nbytes, dtype=torch.uint8)
    fn = "mnb_plan_grouped_i8" if int8 else "mnb_plan_grouped"
    _check(fn, getattr(lib(), fn)(arr, count, bits, block_size, dtype_code(dtype), ctypes.c_void_p(host.data_ptr()),
                                  nbytes))
    dev = host.to(device)
    return Plan(host, dev, outs, keep)


def mnb_plan_launches(plan):
    """Kernel launches one mnb_gemm_grouped(plan) call issues."""
    return lib().mnb_plan_launches(ctypes.c_void_p(plan.host.data_ptr()))


def mnb_gemm_grouped(plan):
    """Run every product of a plan (one launch per kernel class present)."""
    _check("mnb_gemm_grouped", lib().mnb_gemm_grouped(
        ctypes.c_void_p(plan.host.data_ptr()), _dev(plan.device, "plan_device"), _stream(plan.device.device)))
    return plan.outputs


MAX_KSPLIT = 16


def mnb_gemm_split_k_workspace_bytes(M, pw, ksplit=0):
    """Workspace bytes mnb_gemm_split_k needs for M rows times this weight."""
    return lib().mnb_gemm_split_k_workspace_bytes(M, pw.N, pw.K, pw.bits, pw.block_size, dtype_code(pw.dtype),
                                                  ksplit)


def split_k_workspace(M, pw, ksplit=0, device=None):
    """A workspace for mnb_gemm_split_k (None when the call splits nothing)."""
    nbytes = mnb_gemm_split_k_workspace_bytes(M, pw, ksplit)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device or pw.packed.device)


def mnb_gemm_split_k(x, pw, workspace=None, y=None, ksplit=0):
    """Y = X @ dequant(W)^T with K split over workgroups (float32 partial
    sums in `workspace`, added in a fixed order by a second launch)."""
    _check_x(x, pw)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    if workspace is None:
        workspace = split_k_workspace(M, pw, ksplit, x.device)
    if workspace is not None and workspace.device != x.device:
        raise ValueError(f"workspace is on {workspace.device}, not {x.device}")
    if y is None:
        y = torch.empty((M, pw.N), dtype=pw.dtype, device=x.device)
    _check_buf(y, "y", pw.dtype, M * pw.N, x.device)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mnb_gemm_split_k", lib().mnb_gemm_split_k(
        _dev(x, "x"), _dev(pw.packed, "packed"), _dev(y, "y"), ws_ptr, ws_bytes, M, pw.N, pw.K, pw.bits,
        pw.block_size, dtype_code(pw.dtype), ksplit, _stream(x.device)))
    return y


def mnb_gemm_i8_workspace_bytes(M, K, block_size):
    return lib().mnb_gemm_i8_workspace_bytes(M, K, block_size)


def i8_workspace(M, K, block_size, device):
    """A workspace for mnb_gemm_i8 with M rows of K inputs (reusable by calls
    of at most that size that run one after another on one stream; None for
    M = 1, which needs none)."""
    if M == 1:
        return None
    nbytes = mnb_gemm_i8_workspace_bytes(M, K, block_size)
    if nbytes == 0:
        raise ValueError(f"no int8 workspace for M={M}, K={K}, block_size={block_size}")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def mnb_quantize_act_i8(x, block_size):
    """(qa int8 [M, K], a_s float32 [M, K/bs]): the int8 compute mode's
    per-block symmetric activation quantizer."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    qa = torch.empty((M, K), dtype=torch.int8, device=x.device)
    a_s = torch.empty((M, K // block_size), dtype=torch.float32, device=x.device)
    _check("mnb_quantize_act_i8", lib().mnb_quantize_act_i8(
        _dev(x, "x"), M, K, block_size, dtype_code(x.dtype), _dev(qa, "qa"), _dev(a_s, "scales"),
        _stream(x.device)))
    return qa, a_s


def mnb_gemm_i8(x, pw, workspace=None, y=None):
    """Y[M, N] in the int8 compute mode: X quantized per block to int8, then
    integer dot products with the 4-bit codes (any M >= 1)."""
    _check_x(x, pw)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    if workspace is None and M > 1:
        workspace = i8_workspace(M, pw.K, pw.block_size, x.device)
    if workspace is not None and workspace.device != x.device:
        raise ValueError(f"workspace is on {workspace.device}, not {x.device}")
    if y is None:
        y = torch.empty((M, pw.N), dtype=pw.dtype, device=x.device)
    _check_buf(y, "y", pw.dtype, M * pw.N, x.device)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mnb_gemm_i8", lib().mnb_gemm_i8(
        _dev(x, "x"), _dev(pw.packed, "packed"), _dev(y, "y"), ws_ptr, ws_bytes, M, pw.N, pw.K, pw.bits,
        pw.block_size, dtype_code(pw.dtype), _stream(x.device)))
    return y

"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every function the header declares, and the host-only entry points
(status strings, sizes, plans, argument validation) behave as documented.
No kernel is launched here: every call below returns before reaching HIP."""

import ctypes
import math

import pytest

from block_wise_int4_amd import mnb

MNB_OK, NULL, BITS, BLOCK, SHAPE, DTYPE, ALIGN, HIP, PLAN, INVALID = range(10)


@pytest.fixture(scope="module")
def L():
    return mnb.lib()


def test_exports_every_declared_function(L):
    names = mnb.header_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
        assert name in mnb._SIGNATURES, f"binding lacks {name}"


def test_abi_version(L):
    assert L.mnb_abi_version() == 2


def test_status_strings_cover_every_code(L):
    seen = set()
    for code in range(10):
        s = L.mnb_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 10
    assert L.mnb_status_string(99).decode() == "unknown status"
    assert L.mnb_status_string(-1).decode() == "unknown status"


def _expected_bytes(n, k, bs, sb):
    def up(v, a=256):
        return (v + a - 1) // a * a
    rg, kg = math.ceil(n / 16), math.ceil(k / 128)
    kgp = math.ceil(kg / 8) * 8           # per-entry metadata padded to 8 tiles
    entries = rg * max(1, 128 // bs) * 16   # a 256-input block: one entry per tile
    codes = up(rg * kg * 1024)
    scales = up(codes + entries * kgp * sb)
    return up(scales + entries * kgp // 2)


@pytest.mark.parametrize("n,k,bs,dt", [(3072, 1024, 32, 0), (151936, 1024, 32, 1), (768, 3072, 64, 1),
                                       (17, 96, 32, 1), (1, 32, 32, 0), (5, 64, 64, 1), (2048, 1024, 128, 1),
                                       (33, 384, 128, 0), (100, 512, 256, 1), (16, 256, 256, 0)])
def test_packed_bytes(L, n, k, bs, dt):
    assert L.mnb_packed_bytes(n, k, 4, bs, dt) == _expected_bytes(n, k, bs, 4 if dt == 0 else 2)


def test_packed_bytes_equal_algorithmic_bytes_on_whole_tiles(L):
    # no padding when N % 16 == 0 and K % 128 == 0: codes + scales + zero points
    n, k = 2048, 6144
    algo = n * k // 2 + n * (k // 32) * 2 + n * (k // 32) // 2
    assert L.mnb_packed_bytes(n, k, 4, 32, 1) == algo


@pytest.mark.parametrize("args", [(0, 64, 4, 32, 1), (4, 0, 4, 32, 1), (4, 48, 4, 32, 1), (4, 64, 3, 32, 1),
                                  (4, 64, 4, 16, 1), (4, 64, 4, 32, 2), (4, 65536, 4, 32, 1), (4, 128, 4, 256, 1),
                                  (4, 512, 4, 512, 1)])
def test_packed_bytes_invalid_is_zero(L, args):
    assert L.mnb_packed_bytes(*args) == 0


FAKE = ctypes.c_void_p(1 << 20)   # aligned placeholders: never dereferenced
FAKE2 = ctypes.c_void_p(2 << 20)
FAKE3 = ctypes.c_void_p(3 << 20)
ODD = ctypes.c_void_p((1 << 20) + 8)


@pytest.mark.parametrize("call,status", [
    (lambda L: L.mnb_gemv(None, FAKE2, FAKE3, 64, 64, 4, 32, 1, None), NULL),
    (lambda L: L.mnb_gemv(FAKE, FAKE2, FAKE3, 64, 64, 8, 32, 1, None), BITS),
    (lambda L: L.mnb_gemv(FAKE, FAKE2, FAKE3, 64, 64, 4, 96, 1, None), BLOCK),
    (lambda L: L.mnb_gemv(FAKE, FAKE2, FAKE3, 64, 64, 4, 32, 7, None), DTYPE),
    (lambda L: L.mnb_gemv(FAKE, FAKE2, FAKE3, 64, 48, 4, 32, 1, None), SHAPE),
    (lambda L: L.mnb_gemv(FAKE, FAKE2, FAKE3, -1, 64, 4, 32, 1, None), SHAPE),
    (lambda L: L.mnb_gemv(ODD, FAKE2, FAKE3, 64, 64, 4, 32, 1, None), ALIGN),
    (lambda L: L.mnb_gemm(FAKE, FAKE2, FAKE3, 0, 64, 64, 4, 32, 1, None), SHAPE),
    (lambda L: L.mnb_gemm(FAKE, FAKE2, ODD, 8, 64, 64, 4, 32, 1, None), ALIGN),
    (lambda L: L.mnb_gemm(FAKE, FAKE2, FAKE3, 8, 64, 40000, 4, 32, 1, None), SHAPE),
    (lambda L: L.mnb_pack(None, FAKE2, None, 64, 64, 4, 32, 1, FAKE3, None), NULL),
    (lambda L: L.mnb_pack(FAKE, FAKE2, None, 64, 512, 4, 512, 1, FAKE3, None), BLOCK),
    (lambda L: L.mnb_pack(FAKE, FAKE2, None, 64, 384, 4, 256, 1, FAKE3, None), SHAPE),
    (lambda L: L.mnb_pack(FAKE, FAKE2, None, 64, 64, 4, 16, 1, FAKE3, None), BLOCK),
    (lambda L: L.mnb_quantize_rtn(FAKE, 64, 64, 4, 32, 1, FAKE2, None, None, None), NULL),
    (lambda L: L.mnb_gemv(FAKE, FAKE2, FAKE3, 64, 192, 4, 128, 1, None), SHAPE),
    (lambda L: L.mnb_pack(FAKE, FAKE2, FAKE3, 64, 64, 4, 64, 1, ODD, None), ALIGN),
    (lambda L: L.mnb_unpack(FAKE, 64, 64, 4, 32, 1, None, FAKE3, None), NULL),
    (lambda L: L.mnb_dequant(FAKE, 64, 65, 4, 32, 1, FAKE2, None), SHAPE),
    (lambda L: L.mnb_quantize_rtn(FAKE, 64, 64, 4, 32, 3, FAKE2, FAKE3, FAKE, None), DTYPE),
    (lambda L: L.mnb_quantize_rtn(FAKE, 64, 64, 5, 32, 1, FAKE2, FAKE3, FAKE, None), BITS),
    # index NULL asks for the partial results only: accepted, so this fails on bits
    (lambda L: L.mnb_gemv_argmax(FAKE, FAKE2, None, None, FAKE3, 64, 64, 3, 32, 1, None), BITS),
    (lambda L: L.mnb_gemv_argmax(FAKE, FAKE2, None, FAKE3, None, 64, 64, 4, 32, 1, None), NULL),
    (lambda L: L.mnb_gemv_argmax(FAKE, FAKE2, None, ctypes.c_void_p((3 << 20) + 4), FAKE, 64, 64, 4, 32, 1,
                                 None), ALIGN),
    (lambda L: L.mnb_gemv_argmax(FAKE, FAKE2, None, FAKE3, FAKE, 64, 64, 8, 32, 1, None), BITS),
    (lambda L: L.mnb_gemv_argmax(None, FAKE2, None, FAKE3, FAKE, 64, 64, 4, 32, 1, None), NULL),
    (lambda L: L.mnb_embed_gather(FAKE, FAKE2, None, 4, 100, 64, 1, FAKE3, None), NULL),
    (lambda L: L.mnb_embed_gather(FAKE, FAKE2, FAKE, 4, 100, 40, 1, FAKE3, None), SHAPE),
    (lambda L: L.mnb_embed_gather(FAKE, FAKE2, FAKE, 4, 0, 64, 1, FAKE3, None), SHAPE),
    (lambda L: L.mnb_embed_gather(FAKE, FAKE2, FAKE, 4, 100, 64, 5, FAKE3, None), DTYPE),
    (lambda L: L.mnb_embed_gather(FAKE, FAKE2, FAKE, 4, 100, 64, 1, ODD, None), ALIGN),
    (lambda L: L.mnb_embed_gather(FAKE, FAKE2, FAKE, 0, 100, 64, 1, FAKE3, None), MNB_OK),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, None, FAKE3, 100, 64, 1, FAKE, None), NULL),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, FAKE3, None, 100, 64, 1, None, None), NULL),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, FAKE3, None, 100, 40, 1, FAKE, None), SHAPE),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, FAKE3, None, 0, 64, 1, FAKE, None), SHAPE),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, FAKE3, None, 100, 64, 5, FAKE, None), DTYPE),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, FAKE3, ctypes.c_void_p((3 << 20) + 4), 100, 64, 1, FAKE,
                                         None), ALIGN),
    (lambda L: L.mnb_embed_gather_argmax(FAKE, FAKE2, ODD, None, 100, 64, 1, FAKE, None), ALIGN),
])
def test_invalid_arguments_are_rejected_before_launch(L, call, status):
    assert call(L) == status


def test_k_limit(L):
    # a product whose tile grid would not fit a launch is rejected, not wrapped
    assert L.mnb_gemm(FAKE, FAKE2, FAKE3, 0x7FFFFFF0, 0x7FFFFFF0, 64, 4, 32, 1, None) == SHAPE
    assert L.mnb_gemm(FAKE, FAKE2, FAKE3, 0x7FFFFFF0, 0x7FFFFFF0, 64, 4, 32, 0, None) == SHAPE
    # K up to MNB_MAX_K = 32768 inputs for both dtypes
    assert L.mnb_gemv(FAKE, FAKE2, FAKE3, 64, 32768 + 32, 4, 32, 0, None) == SHAPE
    assert L.mnb_gemm(FAKE, FAKE2, FAKE3, 4, 64, 32768 + 64, 4, 64, 1, None) == SHAPE


def _problems(specs):
    arr = (mnb.mnb_problem * len(specs))()
    base = 1 << 24
    for i, (m, n, k) in enumerate(specs):
        arr[i] = mnb.mnb_problem(base + i * 4096, base + i * 4096 + 1024, base + i * 4096 + 2048, m, n, k)
    return arr


def test_plan_bytes(L):
    assert L.mnb_plan_bytes(0) == 0
    assert L.mnb_plan_bytes(65537) == 0
    assert L.mnb_plan_bytes(2) > L.mnb_plan_bytes(1) > 0


def test_plan_groups_launches_by_kernel_class(L):
    specs = [(1, 2048, 1024), (410, 1024, 2048), (1, 151936, 1024), (1500, 768, 768), (410, 2048, 2048)]
    arr = _problems(specs)
    nbytes = L.mnb_plan_bytes(len(specs))
    buf = ctypes.create_string_buffer(nbytes)
    assert L.mnb_plan_grouped(arr, len(specs), 4, 32, 1, buf, nbytes) == MNB_OK
    hdr = ctypes.cast(buf, ctypes.POINTER(ctypes.c_int32))
    assert hdr[0] == 0x4D4E4250 and hdr[2] == len(specs)
    n_launch = hdr[6]
    assert n_launch == 3        # gemv fp16, gemm M=410 tiles, gemm M=1500 tiles
    assert L.mnb_plan_launches(buf) == 3
    assert L.mnb_plan_launches(ctypes.create_string_buffer(64)) == -1


def test_plan_rejects_bad_problems(L):
    arr = _problems([(1, 64, 64), (1, 64, 48)])
    nbytes = L.mnb_plan_bytes(2)
    buf = ctypes.create_string_buffer(nbytes)
    assert L.mnb_plan_grouped(arr, 2, 4, 32, 1, buf, nbytes) == SHAPE
    assert L.mnb_plan_grouped(arr, 2, 4, 32, 1, buf, nbytes - 1) == PLAN
    assert L.mnb_plan_grouped(arr, 0, 4, 32, 1, buf, nbytes) == PLAN


def test_grouped_rejects_a_foreign_plan(L):
    junk = ctypes.create_string_buffer(4096)
    assert L.mnb_gemm_grouped(junk, FAKE, None) == PLAN
    assert L.mnb_gemm_grouped(None, FAKE, None) == NULL

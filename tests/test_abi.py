"""C-ABI contract tests that run without a GPU.

The library must load, export every function include/fp8bs.h declares, and
reject bad arguments with the documented status before touching the HIP
runtime (so fake, never-dereferenced pointers are enough here).  With valid
arguments and no GPU the device check answers FP8BS_ERR_DEVICE.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, NULL, SHAPE, ALIGN, FLAGS, DEVICE, LAUNCH = range(7)
P = ctypes.c_void_p
I64, I32, U32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
FAKE = 0x10000          # 16-byte aligned, never dereferenced
MIS = 0x10008           # 8-byte aligned only


def _no_device() -> bool:
    # A call with valid arguments and fake pointers reaches the device check;
    # with a HIP device present it would launch on those pointers, so such
    # calls are made only where no device is visible (counting devices does
    # not initialise the runtime).
    import torch
    return torch.cuda.device_count() == 0


NO_DEVICE = _no_device()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fp8bs_status|const char\*|int32_t)\s+(fp8bs_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib(lib_path):
    return ctypes.CDLL(lib_path)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in fp8bs.h but not exported"


def test_abi_version_matches_header(lib):
    want = int(re.search(r"#define FP8BS_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    lib.fp8bs_abi_version.restype = ctypes.c_int32
    assert lib.fp8bs_abi_version() == want


def test_status_strings(lib):
    lib.fp8bs_status_str.restype = ctypes.c_char_p
    lib.fp8bs_status_str.argtypes = [ctypes.c_int]
    seen = {lib.fp8bs_status_str(i).decode() for i in range(7)}
    assert len(seen) == 7 and lib.fp8bs_status_str(99).decode() == "unknown status"


def fn(lib, name, args):
    f = getattr(lib, name)
    f.argtypes = args
    f.restype = ctypes.c_int
    return f


def test_quantize_1x128_validation(lib):
    f = fn(lib, "fp8bs_quantize_1x128", [P, I64, I64, P, P, U32, P])
    assert f(FAKE, 4, 100, FAKE, FAKE, 0, None) == SHAPE       # K % 128
    assert f(FAKE, -1, 128, FAKE, FAKE, 0, None) == SHAPE
    assert f(FAKE, 4, 0, FAKE, FAKE, 0, None) == SHAPE
    assert f(FAKE, 4, 128, FAKE, FAKE, 2, None) == FLAGS
    assert f(None, 0, 128, None, None, 0, None) == OK          # empty: nothing launched
    assert f(None, 4, 128, FAKE, FAKE, 0, None) == NULL
    assert f(FAKE, 4, 128, MIS, FAKE, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, 4, 128, FAKE, FAKE, 1, None) == DEVICE      # no device


def test_transpose_validation(lib):
    f = fn(lib, "fp8bs_quantize_transpose_128x1", [P, P, I64, I64, P, P, U32, P])
    assert f(FAKE, FAKE, 100, 128, FAKE, FAKE, 0, None) == SHAPE   # M % 128
    assert f(FAKE, FAKE, 128, 64, FAKE, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, 128, 128, FAKE, FAKE, 4, None) == FLAGS
    assert f(None, None, 0, 128, None, None, 0, None) == OK
    assert f(FAKE, None, 128, 128, FAKE, FAKE, 0, None) == NULL
    assert f(FAKE, FAKE, 128, 128, FAKE, MIS, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, FAKE, 128, 128, FAKE, FAKE, 0, None) == DEVICE


def test_quantize_128x128_validation(lib):
    f = fn(lib, "fp8bs_quantize_128x128", [P, I64, I64, I64, P, P, U32, P])
    assert f(FAKE, 1, 64, 96, FAKE, FAKE, 0, None) == SHAPE
    assert f(FAKE, -2, 64, 128, FAKE, FAKE, 0, None) == SHAPE
    assert f(FAKE, 1, 64, 128, FAKE, FAKE, 8, None) == FLAGS
    assert f(None, 0, 64, 128, None, None, 0, None) == OK
    assert f(FAKE, 1, 64, 128, None, FAKE, 0, None) == NULL
    assert f(MIS, 1, 64, 128, FAKE, FAKE, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, 1, 200, 128, FAKE, FAKE, 0, None) == DEVICE


def test_gemm_validation(lib):
    f = fn(lib, "fp8bs_gemm_fp8_blockscaled", [P, P, P, P, P, I64, I64, I64, I32, U32, P])
    args = [FAKE] * 5
    assert f(*args, 128, 100, 256, 0, 0, None) == SHAPE          # N % 16
    assert f(*args, 128, 256, 200, 0, 0, None) == SHAPE          # K % 128
    assert f(*args, -1, 256, 256, 0, 0, None) == SHAPE
    assert f(*args, 128, 256, 256, 2, 0, None) == FLAGS          # unknown out dtype
    assert f(*args, 128, 256, 256, 0, 2, None) == FLAGS          # unknown flag bit
    assert f(None, None, None, None, None, 0, 256, 256, 0, 0, None) == OK
    assert f(FAKE, FAKE, FAKE, None, FAKE, 128, 256, 256, 0, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, MIS, 128, 256, 256, 1, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(*args, 128, 2112, 7168, 0, 0, None) == DEVICE
        assert f(*args, 128, 2112, 7168, 0, 1, None) == DEVICE   # power-of-two scales accepted


def test_grouped_validation(lib):
    fc = fn(lib, "fp8bs_grouped_gemm_fp8_contiguous", [P, P, P, P, P, P, I32, I64, I64, I64, I32, U32, P])
    fm = fn(lib, "fp8bs_grouped_gemm_fp8_masked", [P, P, P, P, P, P, I32, I64, I64, I64, I32, U32, P])
    six = [FAKE] * 6
    assert fc(*six, 8, 100, 256, 256, 0, 0, None) == SHAPE        # Mt % 128
    assert fc(*six, -1, 128, 256, 256, 0, 0, None) == SHAPE
    assert fc(*six, 8, 128, 256, 256, 7, 0, None) == FLAGS
    assert fc(*six, 8, 128, 256, 256, 0, 4, None) == FLAGS
    assert fc(*([None] * 6), 0, 128, 256, 256, 0, 0, None) == OK
    assert fc(FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, 128, 256, 256, 0, 0, None) == NULL
    assert fc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 8, 128, 256, 256, 0, 0, None) == ALIGN
    if NO_DEVICE:
        assert fc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 8, 128, 256, 256, 0, 0, None) == DEVICE
    assert fm(*six, 4, 256, 100, 256, 0, 0, None) == SHAPE
    assert fm(*six, 4, -5, 128, 256, 0, 0, None) == SHAPE
    assert fm(*six, 4, 256, 128, 256, -1, 0, None) == FLAGS
    assert fm(*six, 4, 256, 128, 256, 0, 3, None) == FLAGS
    assert fm(*([None] * 6), 4, 0, 128, 256, 0, 0, None) == OK
    assert fm(FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, 256, 128, 256, 0, 0, None) == NULL
    assert fm(FAKE, FAKE, FAKE, MIS, FAKE, FAKE, 4, 256, 128, 256, 0, 0, None) == ALIGN
    if NO_DEVICE:
        assert fm(*six, 32, 256, 7168, 2048, 0, 0, None) == DEVICE


def test_cast_validation(lib):
    f = fn(lib, "fp8bs_cast_f32_to_e4m3", [P, I64, P, P])
    assert f(FAKE, -1, FAKE, None) == SHAPE
    assert f(None, 0, None, None) == OK
    assert f(FAKE, 5, None, None) == NULL
    assert f(MIS, 5, FAKE, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, 5, FAKE, None) == DEVICE


def test_binding_imports_and_reports_its_library(lib_path):
    from fp8_block_scaled_04_amd import fp8bs
    assert fp8bs.library() == lib_path
    assert fp8bs.abi_version() == 2


def test_wgrad_validation(lib):
    f = fn(lib, "fp8bs_gemm_fp8_wgrad", [P, P, P, P, P, I64, I64, I64, I32, P])
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 24, 128, 0, None) == SHAPE     # N % 16
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 100, 0, None) == SHAPE     # K % 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 32, 128, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 2, None) == FLAGS     # accumulate in {0, 1}
    assert f(None, None, None, None, None, 0, 32, 128, 0, None) == OK        # empty
    assert f(FAKE, FAKE, None, FAKE, FAKE, 4, 32, 128, 1, None) == NULL
    assert f(FAKE, FAKE, FAKE, MIS, FAKE, 4, 32, 128, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 1, None) == DEVICE


def test_transpose_weight_validation(lib):
    f = fn(lib, "fp8bs_transpose_128x128", [P, P, I64, I64, I64, P, P, P])
    assert f(FAKE, FAKE, 1, 100, 256, FAKE, FAKE, None) == SHAPE      # N % 16
    assert f(FAKE, FAKE, 1, 128, 200, FAKE, FAKE, None) == SHAPE      # K % 128
    assert f(FAKE, FAKE, -1, 128, 256, FAKE, FAKE, None) == SHAPE
    assert f(None, None, 0, 128, 256, None, None, None) == OK          # empty
    assert f(None, None, 1, 0, 256, None, None, None) == OK
    assert f(FAKE, None, 1, 128, 256, FAKE, FAKE, None) == NULL
    assert f(MIS, FAKE, 1, 128, 256, FAKE, FAKE, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, FAKE, 1, 144, 256, FAKE, FAKE, None) == DEVICE


def test_quantize_dual_validation(lib):
    f = fn(lib, "fp8bs_quantize_dual", [P, I64, I64, P, P, P, P, U32, P])
    assert f(FAKE, 100, 128, FAKE, FAKE, FAKE, FAKE, 0, None) == SHAPE      # M % 128
    assert f(FAKE, 128, 200, FAKE, FAKE, FAKE, FAKE, 0, None) == SHAPE      # K % 128
    assert f(FAKE, 128, 128, FAKE, FAKE, FAKE, FAKE, 2, None) == FLAGS
    assert f(None, 0, 128, None, None, None, None, 0, None) == OK          # empty
    assert f(FAKE, 128, 128, FAKE, FAKE, None, FAKE, 1, None) == NULL
    assert f(FAKE, 128, 128, FAKE, FAKE, FAKE, MIS, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, 128, 128, FAKE, FAKE, FAKE, FAKE, 0, None) == DEVICE


def test_gemm_rejects_sizes_beyond_32bit_addressing(lib):
    # Operand panels (256 rows of K bytes) and scale arrays are addressed with
    # 32-bit offsets in the kernels; larger problems are refused up front.
    # (Only where no GPU is visible: a case that wrongly passed the checks
    # would otherwise launch on the fake pointers.)
    if not NO_DEVICE:
        pytest.skip("argument-only checks run where no GPU is visible")
    g = fn(lib, "fp8bs_gemm_fp8_blockscaled", [P] * 5 + [I64] * 3 + [I32, U32, P])
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 256, (1 << 23), 0, 0, None) == SHAPE      # 256*K = 2^31
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 22, 256, 1 << 17, 0, 0, None) == SHAPE    # 4*(K/128)*M = 2^32
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 1 << 28, 1 << 16, 0, 0, None) == SHAPE    # weight block scales
    w = fn(lib, "fp8bs_gemm_fp8_wgrad", [P] * 5 + [I64] * 3 + [I32, P])
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 1 << 22, 1 << 17, 0, None) == SHAPE     # per-row weight scales
    c = fn(lib, "fp8bs_grouped_gemm_fp8_contiguous", [P] * 6 + [I32, I64, I64, I64, I32, U32, P])
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1 << 22, 256, 1 << 17, 0, 0, None) == SHAPE
    m = fn(lib, "fp8bs_grouped_gemm_fp8_masked", [P] * 6 + [I32, I64, I64, I64, I32, U32, P])
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 256, 256, (1 << 23), 0, 0, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 256, (1 << 23) - 128, 0, 0, None) == SHAPE  # 4*(K/128)*M >= 2^31
    # inside the limits: the arguments pass and the device check answers
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 17, 256, 1 << 17, 0, 0, None) == DEVICE   # 4*(K/128)*M = 2^29
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 2112, 7168, 0, 0, None) == DEVICE

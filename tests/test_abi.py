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
    assert len(names) == 18, names
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


def test_quantize_1x128_grid_bound(lib):
    # one workgroup row per 2 tiles of 128 columns, at most 65535 of them:
    # K/128 = 131070 is the largest width, one tile more is refused up front
    f = fn(lib, "fp8bs_quantize_1x128", [P, I64, I64, P, P, U32, P])
    assert f(FAKE, 1, 128 * 131071, FAKE, FAKE, 0, None) == SHAPE
    assert f(FAKE, 1, 128 * 131072, FAKE, FAKE, 0, None) == SHAPE
    if NO_DEVICE:
        assert f(FAKE, 1, 128 * 131070, FAKE, FAKE, 0, None) == DEVICE


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


def test_splitk_workspace_query(lib):
    q = fn(lib, "fp8bs_gemm_splitk_workspace", [I64, I64, I64, P])
    out = ctypes.c_int64(-1)
    # the pages' decode-sized rows: 33 tiles of 64x64 -> 7 splits
    assert q(64, 2112, 7168, ctypes.byref(out)) == OK and out.value == 33 * 7 * 64 * 64 * 4
    # at most 128 rows on 64x64 split tiles, more on 128x96: 66 tiles -> 3
    # splits; 44 tiles -> 5 splits
    assert q(128, 2112, 7168, ctypes.byref(out)) == OK and out.value == 66 * 3 * 64 * 64 * 4
    assert q(129, 2112, 7168, ctypes.byref(out)) == OK and out.value == 44 * 5 * 128 * 96 * 4
    assert q(256, 2112, 7168, ctypes.byref(out)) == OK and out.value == 44 * 5 * 128 * 96 * 4
    # enough tiles already, or fewer than 32 chunks: no split, no workspace
    assert q(4096, 2112, 7168, ctypes.byref(out)) == OK and out.value == 0
    assert q(128, 7168, 2048, ctypes.byref(out)) == OK and out.value == 0
    assert q(64, 2112, 128, ctypes.byref(out)) == OK and out.value == 0
    assert q(0, 2112, 7168, ctypes.byref(out)) == OK and out.value == 0
    assert q(64, 100, 7168, ctypes.byref(out)) == SHAPE                # N % 16
    assert q(64, 2112, 200, ctypes.byref(out)) == SHAPE                # K % 128
    assert q(-1, 2112, 7168, ctypes.byref(out)) == SHAPE
    assert q(64, 2112, 7168, None) == NULL


def test_splitk_validation(lib):
    f = fn(lib, "fp8bs_gemm_fp8_blockscaled_splitk", [P, P, P, P, P, I64, I64, I64, I32, U32, P, I64, P])
    ws = 33 * 7 * 64 * 64 * 4
    args = [FAKE] * 5
    assert f(*args, 64, 100, 7168, 0, 0, FAKE, ws, None) == SHAPE            # N % 16
    assert f(*args, 64, 2112, 7168, 0, 0, FAKE, ws - 1, None) == SHAPE       # workspace too small
    assert f(*args, 64, 2112, 7168, 2, 0, FAKE, ws, None) == FLAGS           # unknown out dtype
    assert f(*args, 64, 2112, 7168, 0, 2, FAKE, ws, None) == FLAGS           # unknown flag bit
    assert f(None, None, None, None, None, 0, 2112, 7168, 0, 0, None, 0, None) == OK
    assert f(*args, 64, 2112, 7168, 0, 0, None, ws, None) == NULL            # workspace needed
    assert f(*args, 64, 2112, 7168, 0, 0, MIS, ws, None) == ALIGN
    assert f(FAKE, FAKE, None, FAKE, FAKE, 64, 2112, 7168, 0, 0, FAKE, ws, None) == NULL
    if NO_DEVICE:
        assert f(*args, 64, 2112, 7168, 0, 0, FAKE, ws, None) == DEVICE
        assert f(*args, 4096, 2112, 7168, 0, 1, None, 0, None) == DEVICE     # no split: no workspace


def test_splitk_noalloc_validation(lib):
    f = fn(lib, "fp8bs_gemm_fp8_blockscaled_splitk_noalloc", [P, P, P, P, P, I64, I64, I64, I32, U32, P])
    args = [FAKE] * 5
    assert f(*args, 64, 100, 7168, 0, 0, None) == SHAPE            # N % 16
    assert f(*args, 64, 2112, 7168, 2, 0, None) == FLAGS           # unknown out dtype
    assert f(*args, 64, 2112, 7168, 0, 2, None) == FLAGS           # unknown flag bit
    assert f(None, None, None, None, None, 0, 2112, 7168, 0, 0, None) == OK
    assert f(FAKE, FAKE, None, FAKE, FAKE, 64, 2112, 7168, 0, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, MIS, 64, 2112, 7168, 0, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(*args, 64, 2112, 7168, 0, 0, None) == DEVICE


def test_splitk_workspace_never_exceeds_the_static_scratch(lib):
    # the allocation-free variant's fixed array (12 MiB) covers every split:
    # splits * tiles <= 256 partial tiles of at most 128 x 96 FP32
    q = fn(lib, "fp8bs_gemm_splitk_workspace", [I64, I64, I64, P])
    out = ctypes.c_int64(-1)
    worst = 0
    for M in (1, 64, 128, 129, 256, 384, 1000):
        for N in (16, 96, 112, 208, 2112, 4096, 7168, 12288):
            for K in (4096, 4224, 7168, 16384, 65536):
                assert q(M, N, K, ctypes.byref(out)) == OK
                worst = max(worst, out.value)
    assert 0 < worst <= 256 * 128 * 96 * 4


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
    assert fp8bs.abi_version() == 9


def test_package_exports_every_binding_function(lib_path):
    # every public function of the binding is reachable from the package
    import inspect

    import fp8_block_scaled_04_amd as pkg
    from fp8_block_scaled_04_amd import fp8bs
    public = {n for n, v in vars(fp8bs).items()
              if not n.startswith("_") and (inspect.isfunction(v) or inspect.isclass(v))
              and getattr(v, "__module__", "") == fp8bs.__name__}
    assert public == set(pkg.__all__), public ^ set(pkg.__all__)
    for n in pkg.__all__:
        assert getattr(pkg, n) is getattr(fp8bs, n)


def test_fused_quantize_validation(lib):
    f = fn(lib, "fp8bs_gemm_fused_quantize", [P, P, P, P, I64, I64, I64, I32, U32, P])
    four = [FAKE] * 4
    assert f(*four, 64, 24, 128, 0, 0, None) == SHAPE             # N % 16
    assert f(*four, 64, 32, 100, 0, 0, None) == SHAPE             # K % 128
    assert f(*four, -1, 32, 128, 0, 0, None) == SHAPE
    assert f(*four, 64, 32, 1 << 24, 0, 0, None) == SHAPE         # 256 * K >= 2^31
    assert f(*four, 64, 32, 128, 2, 0, None) == FLAGS             # unknown out dtype
    assert f(*four, 64, 32, 128, 0, 2, None) == FLAGS             # unknown flag
    assert f(None, None, None, None, 0, 32, 128, 0, 1, None) == OK   # empty
    assert f(FAKE, None, FAKE, FAKE, 64, 32, 128, 0, 0, None) == NULL
    assert f(MIS, FAKE, FAKE, FAKE, 64, 32, 128, 1, 0, None) == ALIGN
    if NO_DEVICE:
        assert f(*four, 64, 32, 128, 1, 1, None) == DEVICE


def test_wgrad_validation(lib):
    f = fn(lib, "fp8bs_gemm_fp8_wgrad", [P, P, P, P, P, I64, I64, I64, I32, U32, P])
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 24, 128, 0, 0, None) == SHAPE     # N % 16
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 100, 0, 0, None) == SHAPE     # K % 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 32, 128, 0, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 2, 0, None) == FLAGS     # accumulate in {0, 1}
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 0, 2, None) == FLAGS     # unknown flag
    assert f(None, None, None, None, None, 0, 32, 128, 0, 1, None) == OK        # empty
    assert f(FAKE, FAKE, None, FAKE, FAKE, 4, 32, 128, 1, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, MIS, FAKE, 4, 32, 128, 0, 1, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 1, 1, None) == DEVICE


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
    w = fn(lib, "fp8bs_gemm_fp8_wgrad", [P] * 5 + [I64] * 3 + [I32, U32, P])
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 1 << 22, 1 << 17, 0, 0, None) == SHAPE     # per-row weight scales
    c = fn(lib, "fp8bs_grouped_gemm_fp8_contiguous", [P] * 6 + [I32, I64, I64, I64, I32, U32, P])
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1 << 22, 256, 1 << 17, 0, 0, None) == SHAPE
    m = fn(lib, "fp8bs_grouped_gemm_fp8_masked", [P] * 6 + [I32, I64, I64, I64, I32, U32, P])
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 256, 256, (1 << 23), 0, 0, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 256, (1 << 23) - 128, 0, 0, None) == SHAPE  # 4*(K/128)*M >= 2^31
    # inside the limits: the arguments pass and the device check answers
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 17, 256, 1 << 17, 0, 0, None) == DEVICE   # 4*(K/128)*M = 2^29
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 2112, 7168, 0, 0, None) == DEVICE


def test_gemm_tile_query_validation(lib):
    f = fn(lib, "fp8bs_gemm_tile", [I32, I64, I64, I64, I32, U32, P, P, P])
    out = (ctypes.c_int32 * 3)()
    o = ctypes.addressof(out)
    assert f(5, 128, 256, 512, 1, 0, o, o + 4, o + 8) == FLAGS          # unknown layout
    assert f(4, 128, 256, 512, 2, 0, o, o + 4, o + 8) == SHAPE          # BF16 activation: G = 1
    assert f(4, 128, 256, 512, 1, 2, o, o + 4, o + 8) == FLAGS
    assert f(4, 128, 256, 512, 1, 1, None, o + 4, o + 8) == NULL
    assert f(0, 128, 24, 512, 1, 0, o, o + 4, o + 8) == SHAPE           # N % 16
    assert f(0, 128, 256, 500, 1, 0, o, o + 4, o + 8) == SHAPE          # K % 128
    assert f(0, 128, 256, 512, 2, 0, o, o + 4, o + 8) == SHAPE          # dense takes G = 1
    assert f(1, 100, 256, 512, 2, 0, o, o + 4, o + 8) == SHAPE          # Mt % 128
    assert f(0, 128, 256, 512, 1, 2, o, o + 4, o + 8) == FLAGS
    assert f(3, 128, 256, 512, 1, 2, o, o + 4, o + 8) == FLAGS          # unknown flag
    assert f(3, 128, 256, 512, 1, 1, o, o + 4, o + 8) == OK             # power-of-two weight gradient
    assert f(0, 128, 256, 512, 1, 0, None, o + 4, o + 8) == NULL
    assert f(0, 128, 256, 512, 1, 0, o, o + 4, o + 8) == OK and tuple(out) == (64, 64, 0)


# The tile each benchmark workload and each labelled parity case runs on
# (host-side dispatch, no GPU): the parity tests' labels cannot drift from
# what the dispatcher does.
TILES = [
    (("dense", 4096, 2112, 7168), (192, 192, 1)),        # training projection: ping-pong loop
    (("dense", 4001, 2112, 7168), (192, 192, 0)),        # rows not a multiple of 4: the other loop
    (("dense", 8192, 4096, 7168), (256, 256, 0)),
    (("dense", 128, 24576, 1536), (128, 96, 0)),         # decode
    (("dense", 128, 7168, 2048), (64, 64, 0)),           # few rows, too few 128x96 tiles
    (("dense", 128, 12288, 1536), (64, 64, 0)),          # 384 tiles of 64x64: the most it takes
    (("dense", 128, 12352, 1536), (128, 96, 0)),         # 386
    (("dense", 100, 13328, 384), (128, 96, 0)),          # ragged rows and columns on 128x96
    (("dense", 37, 208, 1152), (64, 64, 0)),
    (("dense", 256, 2112, 7168), (64, 64, 0)),           # up to 512 rows: 64x64 up to two per CU
    (("dense", 512, 4096, 2048), (64, 64, 0)),           # 512 tiles of 64x64: the most it takes
    (("dense", 512, 4112, 2048), (128, 128, 0)),         # 520
    (("dense", 513, 144, 1152), (128, 128, 0)),          # past 512 rows
    (("dense", 4096, 7168, 2176), (256, 256, 0)),        # data gradient
    (("dense", 4000, 7168, 256), (256, 256, 0)),         # ragged rows on 256x256
    (("dense", 4096, 4096, 256), (256, 256, 0)),
    (("dense", 4000, 4112, 384), (192, 192, 1)),
    (("dense", 2304, 4096, 256), (256, 160, 0)),
    (("dense", 2560, 3584, 384), (256, 160, 0)),
    (("dense", 2450, 3696, 256, 1, True), (256, 160, 0)),     # power-of-two scales
    (("dense", 4096, 2112, 1024, 1, True), (192, 192, 1)),
    (("contiguous", 8192, 4096, 7168, 8), (192, 192, 1)),   # MoE workload: ping-pong loop
    (("contiguous", 1408, 7168, 256, 3), (256, 256, 0)),
    (("contiguous", 1152, 7168, 256, 2), (256, 160, 0)),
    (("contiguous", 2048, 4096, 256, 2), (192, 192, 1)),
    (("contiguous", 4608, 4096, 256, 7), (128, 128, 0)),
    (("masked", 256, 7168, 2048, 32), (128, 256, 0)),
    (("wgrad", 2112, 7168, 4096), (256, 256, 0)),
    (("wgrad", 300, 208, 384), (256, 160, 0)),
    (("fused_quantize", 16384, 256, 7168), (64, 128, 0)),
    (("fused_quantize", 100, 48, 256), (64, 128, 0)),
    (("fused_quantize", 300, 528, 640, 1, True), (64, 128, 0)),
]


@pytest.mark.parametrize("args,tile", TILES)
def test_gemm_tile_choice(lib_path, args, tile):
    from fp8_block_scaled_04_amd import fp8bs
    assert fp8bs.gemm_tile(*args) == tile


def test_stream_reference_validation(lib):
    f = fn(lib, "fp8bs_stream_reference", [P, I64, P, I64, P])
    assert f(FAKE, 32, FAKE, 24, None) == SHAPE           # not a multiple of 16
    assert f(FAKE, 48, FAKE, 16, None) == SHAPE           # 3:1
    assert f(None, 0, None, 0, None) == OK
    assert f(None, 32, FAKE, 16, None) == NULL
    assert f(MIS, 32, FAKE, 16, None) == ALIGN
    if NO_DEVICE:
        assert f(FAKE, 32, FAKE, 16, None) == DEVICE


def test_binding_rejects_host_tensors_before_the_library(lib_path):
    # host (or strided) tensors would hand the kernels pointers they cannot
    # use: the binding refuses them before it calls the library
    import torch
    from fp8_block_scaled_04_amd import fp8bs
    a = torch.zeros((64, 256), dtype=torch.uint8)
    b = torch.zeros((128, 256), dtype=torch.uint8)
    sa, sb = torch.ones((2, 64)), torch.ones((1, 2))
    out = torch.empty((64, 128), dtype=torch.bfloat16)
    calls = {"gemm": lambda: fp8bs.gemm(a, sa, b, sb, out=out),
             "gemm_splitk": lambda: fp8bs.gemm_splitk(a, sa, b, sb, out=out),
             "gemm_splitk_noalloc": lambda: fp8bs.gemm_splitk_noalloc(a, sa, b, sb, out)}
    for name, call in calls.items():
        with pytest.raises(ValueError, match="GPU tensor"):
            call()

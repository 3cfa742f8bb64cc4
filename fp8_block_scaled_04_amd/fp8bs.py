"""ctypes binding of libfp8bs (the C ABI declared in include/fp8bs.h).

Argument marshalling only: tensors are checked, outputs are allocated with
torch on the input's device, and raw device pointers plus torch's current
HIP stream are passed to the library.  Every step of the computation runs in
the library's HIP kernels; there is no CPU fallback.  Importing this module
raises if the library has not been built.

E4M3 codes are torch.float8_e4m3fn tensors (uint8 tensors are accepted as
inputs and viewed as codes); scales are float32; BF16 data is torch.bfloat16.
"""

import ctypes
import os

import torch

from .build import library_path

_PATH = library_path()
if not os.path.exists(_PATH):
    raise ImportError(
        f"{_PATH} is missing: build it with `python -m fp8_block_scaled_04_amd.build` "
        "(the HIP library is required; there is no fallback)")

_lib = ctypes.CDLL(_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32


def _sig(name, args):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = ctypes.c_int
    return f


_q1x128 = _sig("fp8bs_quantize_1x128", [_P, _I64, _I64, _P, _P, _U32, _P])
_qt = _sig("fp8bs_quantize_transpose_128x1", [_P, _P, _I64, _I64, _P, _P, _U32, _P])
_q128 = _sig("fp8bs_quantize_128x128", [_P, _I64, _I64, _I64, _P, _P, _U32, _P])
_gemm = _sig("fp8bs_gemm_fp8_blockscaled", [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _U32, _P])
_wgrad = _sig("fp8bs_gemm_fp8_wgrad", [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _U32, _P])
_gcont = _sig("fp8bs_grouped_gemm_fp8_contiguous",
              [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _U32, _P])
_gmask = _sig("fp8bs_grouped_gemm_fp8_masked",
              [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _U32, _P])
_cast = _sig("fp8bs_cast_f32_to_e4m3", [_P, _I64, _P, _P])
_t128 = _sig("fp8bs_transpose_128x128", [_P, _P, _I64, _I64, _I64, _P, _P, _P])
_qdual = _sig("fp8bs_quantize_dual", [_P, _I64, _I64, _P, _P, _P, _P, _U32, _P])
_gtile = _sig("fp8bs_gemm_tile", [_I32, _I64, _I64, _I64, _I32, _U32, _P, _P, _P])
_sref = _sig("fp8bs_stream_reference", [_P, _I64, _P, _I64, _P])
_gfq = _sig("fp8bs_gemm_fused_quantize", [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _U32, _P])
_gsplit = _sig("fp8bs_gemm_fp8_blockscaled_splitk",
               [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _U32, _P, _I64, _P])
_gsplit_ws = _sig("fp8bs_gemm_splitk_workspace", [_I64, _I64, _I64, _P])
_gsplit_na = _sig("fp8bs_gemm_fp8_blockscaled_splitk_noalloc", [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _U32, _P])
_lib.fp8bs_status_str.argtypes = [ctypes.c_int]
_lib.fp8bs_status_str.restype = ctypes.c_char_p
_lib.fp8bs_abi_version.argtypes = []
_lib.fp8bs_abi_version.restype = ctypes.c_int32

SCALE_POW2 = 1
OUT_BF16, OUT_FP32 = 0, 1


class Fp8bsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.fp8bs_status_str(status).decode()} (status {status})")


def library() -> str:
    """Path of the loaded native library."""
    return _PATH


def abi_version() -> int:
    return int(_lib.fp8bs_abi_version())


def _check(status: int, where: str):
    if status != 0:
        raise Fp8bsError(status, where)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} must be float8_e4m3fn (or uint8 codes), got {t.dtype}")
    return t


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _out_code(out_dtype):
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    if out_dtype == torch.float32:
        return OUT_FP32
    raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")


def quantize_1x128(x: torch.Tensor, pow2: bool = False):
    """BF16 x[M][K] -> (q[M][K] E4M3, s[K/128][M] FP32), one scale per 1x128 tile."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _check(_q1x128(_ptr(x), M, K, _ptr(q), _ptr(s), SCALE_POW2 if pow2 else 0, _stream(x)),
           "quantize_1x128")
    return q, s


def quantize_transpose_128x1(q: torch.Tensor, s: torch.Tensor, pow2: bool = False):
    """1x128-tiled (q[M][K], s[K/128][M]) -> 128x1 tiles stored transposed:
    (qt[K][M] E4M3, st[M/128][K] FP32)."""
    _codes(q, "q")
    _need(q, "q", None, 2)
    _need(s, "s", torch.float32, 2)
    M, K = q.shape
    if tuple(s.shape) != (K // 128, M):
        raise ValueError(f"s must have shape {(K // 128, M)}, got {tuple(s.shape)}")
    qt = torch.empty((K, M), dtype=torch.float8_e4m3fn, device=q.device)
    st = torch.empty((M // 128, K), dtype=torch.float32, device=q.device)
    _check(_qt(_ptr(q), _ptr(s), M, K, _ptr(qt), _ptr(st), SCALE_POW2 if pow2 else 0, _stream(q)),
           "quantize_transpose_128x1")
    return qt, st


def quantize_dual(x: torch.Tensor, pow2: bool = False):
    """BF16 x[M][K] (M, K multiples of 128) -> (q, s, qt, st): 1x128 tiles
    q[M][K], s[K/128][M] and 128x1 tiles stored transposed qt[K][M],
    st[M/128][K], both from one read of x."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    qt = torch.empty((K, M), dtype=torch.float8_e4m3fn, device=x.device)
    st = torch.empty((M // 128, K), dtype=torch.float32, device=x.device)
    _check(_qdual(_ptr(x), M, K, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), SCALE_POW2 if pow2 else 0, _stream(x)),
           "quantize_dual")
    return q, s, qt, st


def quantize_128x128(w: torch.Tensor, pow2: bool = False, out=None):
    """BF16 weights w[N][K] or w[G][N][K] -> (q, s) with one scale per 128x128
    block: s[ceil(N/128)][K/128] (or [G][...]).  out=(q, s) writes into the
    caller's tensors."""
    _need(w, "w", torch.bfloat16)
    if w.dim() not in (2, 3):
        raise ValueError("w must be [N][K] or [G][N][K]")
    G, N, K = (1, *w.shape) if w.dim() == 2 else w.shape
    sshape = ((N + 127) // 128, K // 128) if w.dim() == 2 else (G, (N + 127) // 128, K // 128)
    if out is None:
        q = torch.empty(w.shape, dtype=torch.float8_e4m3fn, device=w.device)
        s = torch.empty(sshape, dtype=torch.float32, device=w.device)
    else:
        q, s = out
        _codes(q, "q")
        _need(q, "q")
        _need(s, "s", torch.float32)
        if tuple(q.shape) != tuple(w.shape) or tuple(s.shape) != sshape:
            raise ValueError("out has the wrong shapes")
    _check(_q128(_ptr(w), G, N, K, _ptr(q), _ptr(s), SCALE_POW2 if pow2 else 0, _stream(w)),
           "quantize_128x128")
    return q, s


def transpose_128x128(q: torch.Tensor, s: torch.Tensor):
    """Block-scaled weight q[N][K] (or [G][N][K]) with s[ceil(N/128)][K/128]
    -> the transposed weight (qt[K][Np], st[K/128][Np/128]), Np =
    128*ceil(N/128), columns past N zero: the B operand of the data gradient
    dX = dY W (dY quantized over the zero-padded width Np)."""
    _codes(q, "q")
    _need(q, "q")
    if q.dim() not in (2, 3):
        raise ValueError("q must be [N][K] or [G][N][K]")
    G, N, K = (1, *q.shape) if q.dim() == 2 else q.shape
    NB = (N + 127) // 128
    sshape = (NB, K // 128) if q.dim() == 2 else (G, NB, K // 128)
    _need(s, "s", torch.float32, len(sshape))
    if tuple(s.shape) != sshape:
        raise ValueError("scale grid does not match the weight")
    qt = torch.empty((K, NB * 128) if q.dim() == 2 else (G, K, NB * 128), dtype=torch.float8_e4m3fn,
                     device=q.device)
    st = torch.empty((K // 128, NB) if q.dim() == 2 else (G, K // 128, NB), dtype=torch.float32, device=q.device)
    _check(_t128(_ptr(q), _ptr(s), G, N, K, _ptr(qt), _ptr(st), _stream(q)), "transpose_128x128")
    return qt, st


def gemm(a, sa, b, sb, out_dtype=torch.bfloat16, out=None, pow2_scales=False):
    """D[M][N] = A * B^T with 1x128 scales sa[K/128][M] and 128x128 block
    scales sb[ceil(N/128)][K/128].  pow2_scales=True: every scale is a power
    of two 2^e, -127 <= e <= 127, and the matrix core applies them (outputs
    that depend on any other scale are NaN)."""
    _codes(a, "a"); _codes(b, "b")
    for t, n in ((a, "a"), (b, "b")):
        _need(t, n, None, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if tuple(sa.shape) != (K // 128, M) or tuple(sb.shape) != ((N + 127) // 128, K // 128):
        raise ValueError("scale shapes do not match the operands")
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    _check(_gemm(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), M, N, K, code,
                 SCALE_POW2 if pow2_scales else 0, _stream(a)),
           "gemm_fp8_blockscaled")
    return out


def splitk_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes gemm_splitk needs for M x N x K (0: it would not split)."""
    out = ctypes.c_int64(0)
    _check(_gsplit_ws(M, N, K, ctypes.byref(out)), "gemm_splitk_workspace")
    return int(out.value)


def gemm_splitk(a, sa, b, sb, out_dtype=torch.bfloat16, out=None, pow2_scales=False, workspace=None):
    """gemm() with the K chunks of each output tile split over several
    workgroups (for few rows and columns); equal to gemm() up to the order of
    FP32 additions.  workspace: a uint8 device tensor of at least
    splitk_workspace_bytes(M, N, K) bytes, allocated here when not given."""
    _codes(a, "a"); _codes(b, "b")
    for t, n in ((a, "a"), (b, "b")):
        _need(t, n, None, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if tuple(sa.shape) != (K // 128, M) or tuple(sb.shape) != ((N + 127) // 128, K // 128):
        raise ValueError("scale shapes do not match the operands")
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    need = splitk_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != a.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the operands' device")
    _check(_gsplit(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), M, N, K, code,
                   SCALE_POW2 if pow2_scales else 0, _ptr(workspace), workspace.numel(), _stream(a)),
           "gemm_fp8_blockscaled_splitk")
    return out


def gemm_splitk_noalloc(a, sa, b, sb, out):
    """gemm_splitk into the caller's `out` (its dtype picks BF16 or FP32)
    with the library's fixed per-GPU scratch instead of a workspace: no
    device memory is allocated.  Calls on one GPU must not overlap in time."""
    _codes(a, "a"); _codes(b, "b")
    for t, n in ((a, "a"), (b, "b")):
        _need(t, n, None, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    _need(out, "out", None, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("operand or output shapes do not match")
    if tuple(sa.shape) != (K // 128, M) or tuple(sb.shape) != ((N + 127) // 128, K // 128):
        raise ValueError("scale shapes do not match the operands")
    _check(_gsplit_na(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), M, N, K, _out_code(out.dtype), 0,
                      _stream(a)), "gemm_fp8_blockscaled_splitk_noalloc")
    return out


def gemm_fused_quantize(x, b, sb, out_dtype=torch.bfloat16, out=None, pow2=False):
    """D[M][N] = Q(x) * B^T for a BF16 activation x[M][K], Q being the 1x128
    quantization of quantize_1x128 (pow2: power-of-two tile scales), done in
    the GEMM's operand load; equal bit for bit to quantize_1x128 then gemm
    with pow2_scales=False.  b: codes [N][K], sb[ceil(N/128)][K/128]."""
    _need(x, "x", torch.bfloat16, 2)
    _codes(b, "b")
    _need(b, "b", None, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = x.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("x and b must share K")
    if tuple(sb.shape) != ((N + 127) // 128, K // 128):
        raise ValueError(f"sb must have shape {((N + 127) // 128, K // 128)}, got {tuple(sb.shape)}")
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _need(out, "out", out_dtype, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    _check(_gfq(_ptr(x), _ptr(b), _ptr(sb), _ptr(out), M, N, K, code, SCALE_POW2 if pow2 else 0, _stream(x)),
           "gemm_fused_quantize")
    return out


def gemm_wgrad(a, sa, b, sb, out=None, accumulate=False, pow2_scales=False):
    """Weight gradient D[M][N] (FP32) = A * B^T, K = tokens, both operands with
    one scale per row per 128 K: sa[K/128][M], sb[K/128][N] (the layout the
    transpose-requantize step produces).  With accumulate=True the product is
    added to `out`.  pow2_scales=True: every scale is a power of two and the
    matrix core applies them (outputs that depend on any other scale are
    NaN)."""
    _codes(a, "a"); _codes(b, "b")
    for t, n in ((a, "a"), (b, "b")):
        _need(t, n, None, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if tuple(sa.shape) != (K // 128, M) or tuple(sb.shape) != (K // 128, N):
        raise ValueError("scale shapes do not match the operands")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out")
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    else:
        _need(out, "out", torch.float32, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    _check(_wgrad(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), M, N, K, 1 if accumulate else 0,
                  SCALE_POW2 if pow2_scales else 0, _stream(a)),
           "gemm_fp8_wgrad")
    return out


def grouped_gemm_contiguous(a, sa, b, sb, m_offsets, out_dtype=torch.bfloat16, out=None, pow2_scales=False):
    """Contiguous MoE layout: group g owns rows [m_offsets[g], m_offsets[g+1])
    of a[Mt][K] and d[Mt][N] and uses b[g], sb[g].  m_offsets is an int32 GPU
    tensor of G+1 entries; rows past m_offsets[G] are not written."""
    _codes(a, "a"); _codes(b, "b")
    _need(a, "a", None, 2)
    _need(b, "b", None, 3)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 3)
    _need(m_offsets, "m_offsets", torch.int32, 1)
    Mt, K = a.shape
    G, N, Kb = b.shape
    if Kb != K or m_offsets.numel() != G + 1:
        raise ValueError("inconsistent shapes")
    if tuple(sa.shape) != (K // 128, Mt) or tuple(sb.shape) != (G, (N + 127) // 128, K // 128):
        raise ValueError("scale shapes do not match the operands")
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((Mt, N), dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype, 2)
        if tuple(out.shape) != (Mt, N):
            raise ValueError("out has the wrong shape")
    _check(_gcont(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), _ptr(m_offsets), G, Mt, N, K, code,
                  SCALE_POW2 if pow2_scales else 0, _stream(a)), "grouped_gemm_fp8_contiguous")
    return out


def grouped_gemm_masked(a, sa, b, sb, masked_m, out_dtype=torch.bfloat16, out=None, pow2_scales=False):
    """Masked MoE layout: a[G][cap][K], sa[G][K/128][cap], b[G][N][K],
    sb[G][ceil(N/128)][K/128]; group g uses its first masked_m[g] rows (int32
    GPU tensor).  Rows past the count keep the previous contents of `out`."""
    _codes(a, "a"); _codes(b, "b")
    _need(a, "a", None, 3)
    _need(b, "b", None, 3)
    _need(sa, "sa", torch.float32, 3)
    _need(sb, "sb", torch.float32, 3)
    _need(masked_m, "masked_m", torch.int32, 1)
    G, cap, K = a.shape
    Gb, N, Kb = b.shape
    if Gb != G or Kb != K or masked_m.numel() != G:
        raise ValueError("inconsistent shapes")
    if tuple(sa.shape) != (G, K // 128, cap) or tuple(sb.shape) != (G, (N + 127) // 128, K // 128):
        raise ValueError("scale shapes do not match the operands")
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((G, cap, N), dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype, 3)
        if tuple(out.shape) != (G, cap, N):
            raise ValueError("out has the wrong shape")
    _check(_gmask(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), _ptr(masked_m), G, cap, N, K, code,
                  SCALE_POW2 if pow2_scales else 0, _stream(a)), "grouped_gemm_fp8_masked")
    return out


def cast_to_e4m3(x: torch.Tensor) -> torch.Tensor:
    """Elementwise FP32 -> E4M3 with the quantizers' encoding (RNE, saturating)."""
    _need(x, "x", torch.float32)
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    _check(_cast(_ptr(x), x.numel(), _ptr(q), _stream(x)), "cast_f32_to_e4m3")
    return q


GEMM_LAYOUTS = {"dense": 0, "contiguous": 1, "masked": 2, "wgrad": 3, "fused_quantize": 4}


def gemm_tile(layout: str, rows: int, N: int, K: int, G: int = 1, pow2_scales: bool = False):
    """(tile_m, tile_n, loop) the GEMM call of `layout` ("dense",
    "contiguous", "masked", "wgrad", "fused_quantize") would run on;
    host-side, no device work.  rows is M, Mt or cap; loop is 1 for the
    ping-pong main loop, else 0."""
    out = (ctypes.c_int32 * 3)()
    base = ctypes.addressof(out)
    _check(_gtile(GEMM_LAYOUTS[layout], rows, N, K, G, SCALE_POW2 if pow2_scales else 0,
                  base, base + 4, base + 8), "gemm_tile")
    return int(out[0]), int(out[1]), int(out[2])


def stream_reference(src: torch.Tensor, dst: torch.Tensor):
    """Bandwidth reference (not part of the method): stream src into dst; src
    holds as many bytes as dst (a copy) or twice as many (2:1 read:write: each
    16-byte piece of src folds into an 8-byte piece of dst)."""
    for t, nm in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous device tensor")
    nb_s = src.numel() * src.element_size()
    nb_d = dst.numel() * dst.element_size()
    _check(_sref(_ptr(src), nb_s, _ptr(dst), nb_d, _stream(src)), "stream_reference")
    return dst

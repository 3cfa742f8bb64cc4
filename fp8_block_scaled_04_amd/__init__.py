"""Block-scaled FP8 GEMM and quantizers for AMD Instinct MI355X (gfx950).

The compute lives in ``libfp8bs.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fp8bs.h``).  This package is a thin ctypes binding over
it: it checks tensor arguments, allocates outputs with torch and passes raw
device pointers plus torch's current HIP stream.  There is no CPU fallback --
if the library is missing, importing the binding raises.

    import fp8_block_scaled_04_amd as fb
    q, s = fb.quantize_1x128(x_bf16)
    d = fb.gemm(q, s, wq, ws)

Sub-modules: ``fp8bs`` (the binding, loaded on first use of a public name),
``synth`` (seeded synthetic workloads), ``build`` (compiles the library).
"""

_PUBLIC = (
    "quantize_1x128", "quantize_transpose_128x1", "quantize_128x128", "quantize_dual",
    "transpose_128x128", "gemm", "gemm_splitk", "gemm_splitk_noalloc", "splitk_workspace_bytes",
    "gemm_fused_quantize", "gemm_wgrad", "grouped_gemm_contiguous", "grouped_gemm_masked",
    "cast_to_e4m3", "gemm_tile", "stream_reference", "abi_version", "Fp8bsError", "library",
)

__all__ = list(_PUBLIC)


def __getattr__(name):
    if name in _PUBLIC:
        from . import fp8bs
        return getattr(fp8bs, name)
    raise AttributeError(name)

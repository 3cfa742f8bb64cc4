"""Helpers for GPU parity tests: host<->device marshalling and the GEMM
tolerance.  Inputs come from the seeded generators and the oracle only."""

import numpy as np
import torch

DEV = "cuda"

# Elementwise GEMM tolerance: |gpu - ref| <= REL * |ref| + ABS_RMS * rms(ref),
# ref = the float64 definition rounded once to the output dtype, rms over all
# outputs compared in the call.
REL = 8e-3
ABS_RMS = 1e-3


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def bf16_dev(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def codes_dev(q) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).view(torch.float8_e4m3fn).to(DEV)


def f32_dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def i32_dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(DEV)


def codes_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def f32_bits_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def out_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_codes_equal(got, ref, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} differences, first at {bad[:5].tolist()}: " \
                          f"gpu {got[tuple(bad[0])]:#x} oracle {ref[tuple(bad[0])]:#x}"


# The matrix core's own accumulation.  One v_mfma_*_16x16x128_f8f6f4 sums
# its 128 products in groups of consecutive K, each group aligned to its
# largest product with about 14 bits kept and the rest truncated
# (tests/test_gpu_mfma_accumulation.py pins this on single-chunk GEMMs,
# against the bound below) -- the limited accumulation page 2 describes for
# Hopper's tensor cores, here inside one 128-wide chunk; the promotion to FP32
# after every chunk keeps it from growing along K.  Where outputs cancel (two
# large chunk partials of opposite sign) this error can exceed the stated
# elementwise tolerance.  Such elements are then held to the stated tolerance
# plus this bound, computed for that element: for each chunk, |sA sB| times,
# for each group of 8 consecutive K, 8 * 2^(E - 13), E the exponent of the
# group's largest |product| (one bit below the measured ~14 as margin).
MFMA_GROUP = 8
MFMA_BITS = 13


def mfma_allowance(arows, ascales, brows, bscales):
    """Per-element bound of the matrix core's truncation.  arows/brows: E4M3
    codes [P][K] of the A and B rows of P outputs; ascales/bscales: their
    per-chunk scales [P][K/128]."""
    from oracle import e4m3
    arows = np.asarray(arows, np.uint8)
    brows = np.asarray(brows, np.uint8)
    P, K = arows.shape
    prod = np.abs(e4m3.decode(arows) * e4m3.decode(brows)).reshape(P, K // 128, 128 // MFMA_GROUP, MFMA_GROUP)
    mx = prod.max(axis=-1)
    _, e = np.frexp(mx)
    lsb = np.where(mx == 0, 0.0, np.ldexp(1.0, (e - 1) - MFMA_BITS))
    per_chunk = np.sum(MFMA_GROUP * lsb, axis=-1)
    s = np.abs(np.asarray(ascales, np.float64) * np.asarray(bscales, np.float64))
    # plus FP32 rounding of the chunk partial and of each promotion step
    chunk_mag = np.sum(prod, axis=(-1, -2)) * s
    return np.sum(per_chunk * s, axis=-1) + 2.0 ** -22 * (K // 128 + 1) * np.sum(chunk_mag, axis=-1)


def dense_allowance(a, sa, b, sb, wgrad=False):
    """Element bound callback for D = A B^T with 1x128-scaled A ([K/128][M]
    scales) and 128x128-scaled B ([N/128][K/128]), or with wgrad=True per-row
    scaled B ([K/128][N])."""
    a = np.asarray(a); b = np.asarray(b); sa = np.asarray(sa); sb = np.asarray(sb)

    def f(idx):
        m, n = idx[:, 0], idx[:, 1]
        bs = sb[:, n].T if wgrad else sb[n // 128, :]
        return mfma_allowance(a[m], sa[:, m].T, b[n], bs)
    return f


def contiguous_allowance(a, sa, b, sb, offsets, rows=None):
    """Element bound callback for the contiguous layout; `rows` maps the
    compared rows to rows of A (default: all rows)."""
    a = np.asarray(a); b = np.asarray(b); sa = np.asarray(sa); sb = np.asarray(sb)
    offs = np.asarray(offsets, np.int64)
    rows = np.arange(a.shape[0]) if rows is None else np.asarray(rows)

    def f(idx):
        m, n = rows[idx[:, 0]], idx[:, 1]
        g = np.searchsorted(offs, m, side="right") - 1
        return mfma_allowance(a[m], sa[:, m].T, b[g, n], sb[g, n // 128, :])
    return f


def masked_allowance(a, sa, b, sb, valid):
    """Element bound callback for the masked layout, outputs compared as
    out[valid] ([G][cap] mask)."""
    a = np.asarray(a); b = np.asarray(b); sa = np.asarray(sa); sb = np.asarray(sb)
    gm = np.argwhere(np.asarray(valid))

    def f(idx):
        g, m, n = gm[idx[:, 0], 0], gm[idx[:, 0], 1], idx[:, 1]
        return mfma_allowance(a[g, m], sa[g, :, m], b[g, n], sb[g, n // 128, :])
    return f


def assert_gemm_close(got64, ref64, what, extra=None):
    """Elementwise |got - ref| <= REL |ref| + ABS_RMS rms(ref) (rms over all
    outputs compared).  With `extra` (a callback returning the matrix core's
    accumulation bound for an array of output indices), elements beyond that
    tolerance are held to the tolerance plus their bound instead."""
    got64 = np.asarray(got64, np.float64)
    ref64 = np.asarray(ref64, np.float64)
    assert got64.shape == ref64.shape
    assert np.isfinite(got64).all(), f"{what}: non-finite outputs"
    rms = float(np.sqrt(np.mean(ref64 ** 2)))
    err = np.abs(got64 - ref64)
    lim = REL * np.abs(ref64) + ABS_RMS * rms
    bad = err > lim
    worst = float(np.max(err / np.maximum(lim, 1e-300)))
    if bad.any() and extra is not None:
        idx = np.argwhere(bad)
        allow = extra(idx)
        beyond = err[bad] > lim[bad] + allow
        assert not beyond.any(), (f"{what}: {int(beyond.sum())} of {bad.size} outside the tolerance plus the "
                                  f"matrix core's accumulation bound (worst {worst:.3g}x the tolerance)")
        print(f"{what}: {int(bad.sum())} of {bad.size} outputs beyond the tolerance (worst {worst:.3g}x), "
              f"all within the matrix core's accumulation bound", flush=True)
        return worst
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance (worst {worst:.3g}x)"
    return worst

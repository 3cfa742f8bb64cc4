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


def assert_gemm_close(got64, ref64, what):
    got64 = np.asarray(got64, np.float64)
    ref64 = np.asarray(ref64, np.float64)
    assert got64.shape == ref64.shape
    assert np.isfinite(got64).all(), f"{what}: non-finite outputs"
    rms = float(np.sqrt(np.mean(ref64 ** 2)))
    err = np.abs(got64 - ref64)
    lim = REL * np.abs(ref64) + ABS_RMS * rms
    bad = err > lim
    worst = float(np.max(err / np.maximum(lim, 1e-300)))
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance (worst {worst:.3g}x)"
    return worst

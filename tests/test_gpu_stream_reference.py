"""The bandwidth reference the benchmark sets the quantizers against: a
1:1 copy and a 2:1 stream whose every 16-byte output piece is the XOR of two
input pieces, checked byte for byte (tails shorter than one grid stride and
sizes that are not a multiple of the unroll included)."""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs
from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 8192 * 256 * 16 * 5 + 16 * 333, 58_720_256])
@pytest.mark.parametrize("ratio", [1, 2])
def test_stream_reference(nbytes, ratio):
    print(f"stream reference {ratio}:1, {nbytes} bytes written", flush=True)
    rng = np.random.default_rng(nbytes + ratio)
    src_h = rng.integers(0, 256, ratio * nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    fp8bs.stream_reference(src, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    if ratio == 1:
        want = src_h
    else:
        pieces = src_h.reshape(-1, 2, 16)
        want = (pieces[:, 0] ^ pieces[:, 1]).reshape(-1)
    assert np.array_equal(got, want)

"""The bandwidth reference the benchmark sets the quantizers against: a
1:1 copy and a 2:1 stream whose 8-byte output piece i holds (w0 ^ w1, w2 ^ w3)
of the 32-bit words of input piece i, checked byte for byte (tails shorter
than one grid stride included)."""

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
        words = src_h.view(np.uint32).reshape(-1, 4)
        want = np.stack([words[:, 0] ^ words[:, 1], words[:, 2] ^ words[:, 3]], axis=1).reshape(-1).view(np.uint8)
    assert np.array_equal(got, want)

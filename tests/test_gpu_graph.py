"""Graph capture of the hot path: the quantizer and the GEMM called inside a
HIP graph (as a serving loop or the benchmark step runs them) give, on every
replay, exactly the eager results.  The library issues kernels only (no
memsets, no allocations); replays are separated by eager work and
synchronizations."""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from tests.gpu_util import bf16_dev, codes_host, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


@pytest.mark.parametrize("M,N,K", [(512, 2112, 1024), (128, 4096, 1536)])
def test_graph_replays_match_eager(M, N, K):
    print(f"graph capture quantize + gemm M={M} N={N} K={K}", flush=True)
    w = synth.dense(M, N, K, seed=M + N)
    x = bf16_dev(w["a"])
    b, sb = fp8bs.quantize_128x128(bf16_dev(w["b"]))
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device="cuda")
    s = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        qq, ss = fp8bs.quantize_1x128(x)
        q.copy_(qq)
        s.copy_(ss)
        fp8bs.gemm(qq, ss, b, sb, out=d)

    step()
    torch.cuda.synchronize()
    want_q, want_s, want_d = codes_host(q), s.cpu().numpy().copy(), d.view(torch.int16).cpu().numpy().copy()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        q.zero_(); s.zero_(); d.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(codes_host(q), want_q), f"replay {rep}: codes"
        assert np.array_equal(s.cpu().numpy(), want_s), f"replay {rep}: scales"
        assert np.array_equal(d.view(torch.int16).cpu().numpy(), want_d), f"replay {rep}: gemm output"
        step()                       # eager work between replays
        torch.cuda.synchronize()


def test_graph_replays_quantizers_and_masked_gemm():
    """The transposing quantizers and the masked grouped GEMM (device-side
    counts) inside one captured graph: every replay equals the eager run."""
    print("graph capture dual / transpose-requant / masked gemm", flush=True)
    M, K = 256, 512
    x = bf16_dev(synth.activation(M, K, seed=11)["a"])
    G, cap, N, Km = 4, 128, 256, 384
    w = synth.masked(G, cap, N, Km, seed=12)
    am, sam = fp8bs.quantize_1x128(bf16_dev(w["a"].reshape(G * cap, Km)))
    am = am.view(G, cap, Km)
    sam = sam.view(Km // 128, G, cap).permute(1, 0, 2).contiguous()
    bm, sbm = fp8bs.quantize_128x128(bf16_dev(w["b"]))
    cnt = torch.tensor([0, 5, 128, 77], dtype=torch.int32, device="cuda")
    outs = {
        "q": torch.empty((M, K), dtype=torch.float8_e4m3fn, device="cuda"),
        "s": torch.empty((K // 128, M), dtype=torch.float32, device="cuda"),
        "qt": torch.empty((K, M), dtype=torch.float8_e4m3fn, device="cuda"),
        "st": torch.empty((M // 128, K), dtype=torch.float32, device="cuda"),
        "qt2": torch.empty((K, M), dtype=torch.float8_e4m3fn, device="cuda"),
        "st2": torch.empty((M // 128, K), dtype=torch.float32, device="cuda"),
        "dm": torch.zeros((G, cap, N), dtype=torch.bfloat16, device="cuda"),
    }

    def step():
        q, s, qt, st = fp8bs.quantize_dual(x)
        qt2, st2 = fp8bs.quantize_transpose_128x1(q, s)
        for k, v in (("q", q), ("s", s), ("qt", qt), ("st", st), ("qt2", qt2), ("st2", st2)):
            outs[k].copy_(v)
        fp8bs.grouped_gemm_masked(am, sam, bm, sbm, cnt, out=outs["dm"])

    def snapshot():
        return {k: (v.view(torch.uint8) if v.dtype == torch.float8_e4m3fn else
                    v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy().copy()
                for k, v in outs.items()}

    step()
    torch.cuda.synchronize()
    want = snapshot()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for k, v in outs.items():
            if k != "dm":       # rows past the counts keep their previous contents
                v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in want:
            assert np.array_equal(got[k], want[k]), f"replay {rep}: {k}"
        step()
        torch.cuda.synchronize()


def test_graph_replays_fused_quantize_gemm():
    """The GEMM that quantizes its BF16 activation in the operand load, inside
    a captured graph: every replay equals the eager call."""
    M, N, K = 320, 256, 1024
    print(f"graph capture fused-quantize gemm M={M} N={N} K={K}", flush=True)
    w = synth.dense(M, N, K, seed=21)
    x = bf16_dev(w["a"])
    b, sb = fp8bs.quantize_128x128(bf16_dev(w["b"]))
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    fp8bs.gemm_fused_quantize(x, b, sb, out=d)
    torch.cuda.synchronize()
    want = d.view(torch.int16).cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fp8bs.gemm_fused_quantize(x, b, sb, out=d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        d.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(d.view(torch.int16).cpu().numpy(), want), f"replay {rep}"
        fp8bs.gemm_fused_quantize(x, b, sb)      # eager work between replays
        torch.cuda.synchronize()


def test_graph_replays_splitk_gemm():
    """The split-K GEMM (partials kernel + reduction kernel, caller workspace)
    and its allocation-free variant captured in one graph: every replay, with
    eager calls of both between replays, equals the eager results."""
    M, N, K = 64, 2112, 7168
    print(f"graph capture split-K gemm M={M} N={N} K={K}", flush=True)
    w = synth.dense(M, N, K, seed=9)
    a, sa = fp8bs.quantize_1x128(bf16_dev(w["a"]))
    b, sb = fp8bs.quantize_128x128(bf16_dev(w["b"]))
    ws = torch.empty(fp8bs.splitk_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    d1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    d2 = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        fp8bs.gemm_splitk(a, sa, b, sb, out=d1, workspace=ws)
        fp8bs.gemm_splitk_noalloc(a, sa, b, sb, d2)

    step()
    torch.cuda.synchronize()
    want1, want2 = d1.view(torch.int16).cpu().numpy().copy(), d2.view(torch.int32).cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        d1.zero_(); d2.zero_(); ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(d1.view(torch.int16).cpu().numpy(), want1), f"replay {rep}: split-K (workspace)"
        assert np.array_equal(d2.view(torch.int32).cpu().numpy(), want2), f"replay {rep}: split-K (no allocation)"
        step()
        torch.cuda.synchronize()

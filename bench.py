"""Benchmark of the block-scaled FP8 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

One step = one pass of the forward hot path of an FP8 linear layer on the
4096 x 2112 x 7168 training-shaped projection: 1x128 quantization of the BF16
activation [4096][7168] followed by the block-scaled FP8 GEMM against the
128x128-quantized weight [2112][7168] (weights are quantized once, before
timing, as a training step would for a resident weight).  `value` is GEMM
TFLOP/s over the whole step (2*M*N*K / step time); inputs are resident in HBM
before the timed region.

Printed as one JSON line, with
  roofline      the GEMM kernel alone, timed with HIP events on the stream it
                runs on, against the MI355X dense FP8 MFMA peak (5.0 PFLOP/s);
  cpu_baseline  the CPU oracle (NumPy, float64) timed on this host on the
                same step, twice;
  kernels       every kernel of the hot path on its own workload (1x128 and
                transpose quantizers on 8192 x 7168, the decode-shaped GEMM
                128 x 24576 x 1536 with its quantizer, the MoE contiguous and
                masked grouped GEMMs), HBM-bound ones over rotating buffers so
                the 256 MB last-level cache does not serve repeats.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
WORKLOAD = dict(name="dense_4096x2112x7168", M=4096, N=2112, K=7168)
# rocprofv3 summary of the dominant kernel on this workload, and the sources it was built from
GEMM_PROFILE = "profiles/k_gemm_dense_4096x2112x7168.md"
GEMM_SOURCES = ["fp8_block_scaled_04_amd/csrc/gemm_pp.hip", "fp8_block_scaled_04_amd/csrc/gemm_common.h",
                "fp8_block_scaled_04_amd/csrc/device_common.h", "fp8_block_scaled_04_amd/csrc/launch.h"]
GEMM_KERNEL = "k_gemm_pp (dense, ping-pong 192x192 tile)"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_events(fn, iters, warmup=3):
    """Average device time of fn() in microseconds, from HIP events recorded on
    torch's current stream (the stream the library launches on)."""
    for _ in range(warmup):
        fn()
    start = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    end = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        start[i].record()
        fn()
        end[i].record()
    torch.cuda.synchronize()
    return float(np.mean([s.elapsed_time(e) for s, e in zip(start, end)])) * 1e3


EAGER = False   # --eager: per-kernel lines from plain launches (for profiler runs)


def time_graph(fn, calls=20, reps=5):
    """Average device time of fn() in microseconds, from a HIP graph of
    `calls` consecutive calls replayed `reps` times between two events (no
    host launch overhead between kernels).  Falls back to per-call events
    if the calls cannot be captured, or with --eager."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    if EAGER:
        return time_events(fn, calls), "events"
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(calls):
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
    except Exception:
        return time_events(fn, calls), "events"
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (calls * reps)
    del g
    return us, "graph"


def rotation(bytes_per_set, min_total=1 << 29):
    return int(max(1, -(-min_total // max(bytes_per_set, 1))))


def stream_rate_on(fb, srcs, ratio):
    """GB/s of the library's streaming reference reading the byte tensors
    `srcs` in turn (ratio 2: writing half as many bytes, 1: as many)."""
    n = srcs[0].numel() // ratio
    dsts = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in srcs]
    it = iter(range(10 ** 9))
    us, _ = time_graph(lambda: (lambda i: fb.stream_reference(srcs[i % len(srcs)], dsts[i % len(srcs)]))(next(it)))
    del dsts
    return (ratio + 1) * n / us / 1e3


def progress(msg):
    """One line on stderr as each part of the run finishes (the JSON record
    stays the only line on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class _Reported(dict):
    """The per-kernel table: reports each entry on stderr as it is measured."""

    def __setitem__(self, key, value):
        super().__setitem__(key, value)
        us = value.get("us") if isinstance(value, dict) else None
        progress(f"{key}: {us:.2f} us" if isinstance(us, float) else f"{key}: done")


def extra_kernels(fb, synth):
    """Per-kernel measurements on each workload of the hot path."""
    out = _Reported()
    # 1x128 quantizer and transpose-requant on the 8192 x 7168 activation
    M, K = 8192, 7168
    x_bits = synth.activation(M, K, seed=0)["a"]
    x0 = dev_bf16(x_bits)
    R = rotation(3 * M * K)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    qs = [fb.quantize_1x128(x) for x in xs]
    it = iter(range(10 ** 9))
    us, how = time_graph(lambda: fb.quantize_1x128(xs[next(it) % R]))
    byt = 2 * M * K + M * K + 4 * M * (K // 128)
    out["quantize_1x128_8192x7168"] = dict(us=us, timing=how, GBs=byt / us / 1e3, frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS,
                                           bytes=byt)
    it = iter(range(10 ** 9))
    us, how = time_graph(lambda: fb.quantize_transpose_128x1(*qs[next(it) % R]))
    byt = 2 * M * K + 4 * (M * K // 128) * 2
    out["quantize_transpose_128x1_8192x7168"] = dict(us=us, timing=how, GBs=byt / us / 1e3,
                                                     frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt)
    it = iter(range(10 ** 9))
    us, how = time_graph(lambda: fb.quantize_dual(xs[next(it) % R]))
    byt = 2 * M * K + 2 * M * K + 8 * (M * K // 128)
    out["quantize_dual_8192x7168"] = dict(us=us, timing=how, GBs=byt / us / 1e3,
                                          frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt)
    # Practical ceilings on this device: the library's streaming reference
    # (nontemporal 16-byte loads, no arithmetic) writing the same M*K bytes
    # while reading twice as many (the 1x128 quantizer's mix, 8-byte stores)
    # or as many (the transpose-requantizer's, 16-byte nontemporal stores).
    # Each quantizer's line carries its fraction of the matching stream's
    # rate.  The streams read the quantizers' own inputs (the BF16 activation
    # for 2:1, its codes for 1:1): on this device the same access pattern
    # moves constant data about 6 % faster than random data.
    dsts = [torch.empty(M * K, dtype=torch.uint8, device="cuda") for _ in range(R)]
    ref_src = {2: [x.view(torch.uint8).reshape(-1) for x in xs], 1: [q.view(torch.uint8).reshape(-1) for q, _ in qs]}
    for ratio in (2, 1):
        it = iter(range(10 ** 9))
        us, how = time_graph(lambda: (lambda i: fb.stream_reference(ref_src[ratio][i % R], dsts[i % R]))(next(it)))
        byt = (ratio + 1) * M * K
        out[f"reference_stream_{ratio}to1_{M * K / 1e6:.1f}MB_written"] = dict(
            us=us, timing=how, GBs=byt / us / 1e3, frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt)
    del ref_src, dsts
    for name, ref in (("quantize_1x128_8192x7168", "2to1"), ("quantize_transpose_128x1_8192x7168", "1to1"),
                      ("quantize_dual_8192x7168", "1to1")):
        r = out[f"reference_stream_{ref}_{M * K / 1e6:.1f}MB_written"]
        out[name]["frac_of_stream_reference"] = out[name]["GBs"] / r["GBs"]
    # The code-only 128x128 block transpose of the same 8192 x 7168 codes
    # (the transpose-requantizer's access pattern, no arithmetic).
    sw = [torch.ones((1, M // 128, K // 128), device="cuda") for _ in range(R)]
    it = iter(range(10 ** 9))

    def code_transpose(i):
        return fb.transpose_128x128(qs[i % R][0].view(1, M, K), sw[i % R])
    us, how = time_graph(lambda: code_transpose(next(it)))
    byt = 2 * M * K
    out["reference_code_transpose_8192x7168"] = dict(us=us, timing=how, GBs=byt / us / 1e3,
                                                     frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt)
    del xs, qs, x0, sw
    torch.cuda.empty_cache()

    # decode-shaped GEMM 128 x 24576 x 1536 (power-of-two scales) + its quantizer
    M, N, K = 128, 24576, 1536
    w = synth.dense(M, N, K, seed=0)
    xa = dev_bf16(w["a"])
    wb = dev_bf16(w["b"])
    a, sa = fb.quantize_1x128(xa, pow2=True)
    R = rotation(N * K)
    bsets = [fb.quantize_128x128(wb, pow2=True) for _ in range(R)]
    it = iter(range(10 ** 9))
    us, how = time_graph(lambda: fb.gemm(a, sa, *bsets[next(it) % R]))
    byt = M * K + N * K + 2 * M * N + 4 * (M * K // 128) + 4 * (N // 128) * (K // 128)
    out["gemm_decode_128x24576x1536_pow2"] = dict(us=us, timing=how, TFLOPs=2 * M * N * K / us / 1e6,
                                                  GBs=byt / us / 1e3, frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS,
                                                  bytes=byt)
    us, how = time_graph(lambda: fb.quantize_1x128(xa, pow2=True))
    out["quantize_1x128_128x1536_pow2"] = dict(us=us, timing=how, GBs=(3 * M * K + 4 * M * K // 128) / us / 1e3)
    del bsets, wb
    torch.cuda.empty_cache()

    # The pages' Table 1 shapes (DeepGEMM on Hopper; their times are context,
    # not targets): the few-row ones on the split-K GEMM, beside the unsplit
    # GEMM on the same operands; weights rotated over >= 512 MB.
    for (M, N, K, pages_us) in ((64, 2112, 7168, 9.41), (128, 7168, 2048, 7.37), (4096, 4096, 7168, 184.45)):
        w = synth.dense(M, N, K, seed=0)
        a, sa = fb.quantize_1x128(dev_bf16(w["a"]))
        wb = dev_bf16(w["b"])
        R = rotation(N * K)
        bsets = [fb.quantize_128x128(wb) for _ in range(R)]
        del wb
        d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(16, fb.splitk_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
        it = iter(range(10 ** 9))
        us_u, how = time_graph(lambda: fb.gemm(a, sa, *bsets[next(it) % R], out=d))
        us, how = time_graph(lambda: fb.gemm_splitk(a, sa, *bsets[next(it) % R], out=d, workspace=ws))
        # split tiles: 64x64 up to 128 rows, else 128x96
        tm, tn = (64, 64) if M <= 128 else (128, 96)
        tiles = ((M + tm - 1) // tm) * ((N + tn - 1) // tn)
        byt = M * K + N * K + 2 * M * N + 4 * (K // 128) * (M + (N + 127) // 128)
        out[f"gemm_pages_table1_{M}x{N}x{K}"] = dict(
            us=us, timing=how, TFLOPs=2 * M * N * K / us / 1e6, GBs=byt / us / 1e3,
            frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, frac_mfma=2 * M * N * K / us / 1e6 / FP8_PEAK_TFLOPS,
            splits=fb.splitk_workspace_bytes(M, N, K) // (tiles * tm * tn * 4) or 1, us_unsplit=us_u,
            tile_unsplit=list(fb.gemm_tile("dense", M, N, K)[:2]), pages_hopper_us=pages_us)
        del bsets, ws, a, sa, d
        torch.cuda.empty_cache()

    # MoE contiguous 8 x (sum M = 8192) x 4096 x 7168
    G, Mt, N, K = 8, 8192, 4096, 7168
    w = synth.contiguous(G, Mt, N, K, seed=0)
    a, sa = fb.quantize_1x128(dev_bf16(w["a"]))
    wb = dev_bf16(w["b"])
    b, sb = fb.quantize_128x128(wb)
    # the experts' 128x128 weight quantization (a 2:1 read:write stream of 705 MB)
    us, how = time_graph(lambda: fb.quantize_128x128(wb, out=(b, sb)))
    byt = 3 * G * N * K + 4 * G * (N // 128) * (K // 128)
    ref = stream_rate_on(fb, [wb.view(torch.uint8).reshape(-1)], 2)
    out[f"quantize_128x128_{G}x{N}x{K}"] = dict(us=us, timing=how, GBs=byt / us / 1e3,
                                                frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt,
                                                stream_reference_GBs=ref, frac_of_stream_reference=byt / us / 1e3 / ref)
    del wb
    offs = torch.from_numpy(w["m_offsets"]).cuda()
    us, how = time_graph(lambda: fb.grouped_gemm_contiguous(a, sa, b, sb, offs))
    out["grouped_contiguous_8x8192x4096x7168"] = dict(us=us, timing=how, TFLOPs=2 * Mt * N * K / us / 1e6,
                                                      frac_mfma=2 * Mt * N * K / us / 1e6 / FP8_PEAK_TFLOPS)
    del a, sa, b, sb
    torch.cuda.empty_cache()

    # MoE masked 32 x 256 x 7168 x 2048 (decode)
    G, cap, N, K = 32, 256, 7168, 2048
    w = synth.masked(G, cap, N, K, seed=0)
    a2, sa2 = fb.quantize_1x128(dev_bf16(w["a"].reshape(G * cap, K)))
    a = a2.view(G, cap, K)
    sa = sa2.view(K // 128, G, cap).permute(1, 0, 2).contiguous()
    wbits = dev_bf16(w["b"])
    b, sb = fb.quantize_128x128(wbits)
    del wbits
    cnt = torch.from_numpy(w["masked_m"]).cuda()
    c = w["masked_m"].astype(np.int64)
    flops = 2 * int(c.sum()) * N * K
    nz = int((c > 0).sum())
    byt = nz * (N * K + 4 * (N // 128) * (K // 128)) + int(c.sum()) * (K + 4 * K // 128 + 2 * N)
    us, how = time_graph(lambda: fb.grouped_gemm_masked(a, sa, b, sb, cnt))
    out["grouped_masked_32x256x7168x2048"] = dict(us=us, timing=how, TFLOPs=flops / us / 1e6, GBs=byt / us / 1e3,
                                                  frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt)

    # power-of-two scales on the training projection and a large square: the
    # matrix core applies the scales (E8M0) vs the FP32 promotion on the VALU
    for (M, N, K) in ((4096, 2112, 7168), (8192, 4096, 7168)):
        w = synth.dense(M, N, K, seed=3)
        a, sa = fb.quantize_1x128(dev_bf16(w["a"]), pow2=True)
        b, sb = fb.quantize_128x128(dev_bf16(w["b"]), pow2=True)
        # the two paths alternate (three rounds, the first path swapped each
        # round; median per path): timed back to back, the second path ran
        # under a different power state than the first
        times = {True: [], False: []}
        for rnd in range(3):
            for hw in ((True, False) if rnd % 2 == 0 else (False, True)):
                us, how = time_graph(lambda: fb.gemm(a, sa, b, sb, pow2_scales=hw))
                times[hw].append(us)
        for hw in (True, False):
            us = float(np.median(times[hw]))
            out[f"gemm_pow2_{'hw' if hw else 'sw'}_{M}x{N}x{K}"] = dict(
                us=us, timing=how + ", alternated", TFLOPs=2 * M * N * K / us / 1e6,
                frac_mfma=2 * M * N * K / us / 1e6 / FP8_PEAK_TFLOPS)
        del a, sa, b, sb
    torch.cuda.empty_cache()

    # backward of the 7168 -> 2112 projection over 4096 tokens: weight
    # transposed for the data gradient, dX = dY W (K padded 2112 -> 2176), and
    # GEMM on a BF16 activation with the 1x128 quantization in its operand
    # load, against the two steps it replaces (quantize_1x128, then the GEMM):
    # one or two 128-column tiles per row block (8192 x 128, 16384 x 256), and
    # the projection shape, whose 17 column tiles each quantize the activation
    # rows again.
    for (M, N, K) in ((8192, 128, 7168), (16384, 256, 7168), (4096, 2112, 7168)):
        w = synth.dense(M, N, K, seed=0)
        b, sb = fb.quantize_128x128(dev_bf16(w["b"]))
        x0 = dev_bf16(w["a"])
        del w
        R = rotation(3 * M * K)
        xs = [x0] + [x0.clone() for _ in range(R - 1)]
        d = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        it = iter(range(10 ** 9))
        us_f, how = time_graph(lambda: fb.gemm_fused_quantize(xs[next(it) % R], b, sb, out=d))
        it = iter(range(10 ** 9))
        us_2, _ = time_graph(lambda: (lambda q: fb.gemm(q[0], q[1], b, sb, out=d))(fb.quantize_1x128(xs[next(it) % R])))
        flop = 2 * M * N * K
        out[f"gemm_fused_quantize_{M}x{N}x{K}"] = dict(
            us=us_f, timing=how, TFLOPs=flop / us_f / 1e6, frac_mfma=flop / us_f / 1e6 / FP8_PEAK_TFLOPS,
            two_step_us=us_2, speedup_vs_two_step=us_2 / us_f)
        del xs, x0, d, b, sb
        torch.cuda.empty_cache()

    # the weight gradient dW = dY^T X from the transposed activations
    T, NO, NI = 4096, 2112, 7168
    w = synth.dense(T, NO, NI, seed=0)
    wbits = dev_bf16(w["b"])
    wq, ws = fb.quantize_128x128(wbits)
    # the projection weight's 128x128 quantization (2:1 read:write)
    R = rotation(3 * NO * NI)
    wsrc = [wbits] + [wbits.clone() for _ in range(R - 1)]
    wdst = [fb.quantize_128x128(x) for x in wsrc]
    it = iter(range(10 ** 9))
    us, how = time_graph(lambda: (lambda i: fb.quantize_128x128(wsrc[i % R], out=wdst[i % R]))(next(it)))
    byt = 3 * NO * NI + 4 * ((NO + 127) // 128) * (NI // 128)
    ref = stream_rate_on(fb, [x.view(torch.uint8).reshape(-1) for x in wsrc], 2)
    out[f"quantize_128x128_{NO}x{NI}"] = dict(us=us, timing=how, GBs=byt / us / 1e3,
                                              frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt,
                                              stream_reference_GBs=ref, frac_of_stream_reference=byt / us / 1e3 / ref)
    del wsrc, wdst, wbits
    R = rotation(2 * NO * NI)
    wsets = [(wq.clone(), ws.clone()) for _ in range(R)]
    it = iter(range(10 ** 9))
    us, how = time_graph(lambda: fb.transpose_128x128(*wsets[next(it) % R]))
    NB = (NO + 127) // 128
    byt = NO * NI + NI * NB * 128 + 2 * 4 * NB * (NI // 128)
    out["transpose_128x128_2112x7168"] = dict(us=us, timing=how, GBs=byt / us / 1e3,
                                              frac_hbm=byt / us / 1e3 / HBM_PEAK_GBS, bytes=byt)
    del wsets
    qt, st = fb.transpose_128x128(wq, ws)
    dy_bits = synth.activation(T, NO, seed=1)["a"]
    pad = np.zeros((T, NB * 128), np.uint16)
    pad[:, :NO] = dy_bits
    a, sa = fb.quantize_1x128(dev_bf16(pad))
    us, how = time_graph(lambda: fb.gemm(a, sa, qt, st))
    out["gemm_dgrad_4096x7168x2112"] = dict(us=us, timing=how, TFLOPs=2 * T * NI * NO / us / 1e6,
                                            frac_mfma=2 * T * NI * NO / us / 1e6 / FP8_PEAK_TFLOPS,
                                            padded_K=NB * 128)
    x_bits = synth.activation(T, NI, seed=2)["a"]
    ayt, sayt = fb.quantize_transpose_128x1(a, sa)               # dY^T [Np][T] (zero rows past 2112)
    axt, saxt = fb.quantize_transpose_128x1(*fb.quantize_1x128(dev_bf16(x_bits)))   # X^T [NI][T]
    # the same operands with power-of-two scales, for the scaled-MFMA weight gradient
    ayt2, sayt2 = fb.quantize_transpose_128x1(*fb.quantize_1x128(dev_bf16(pad), pow2=True), pow2=True)
    axt2, saxt2 = fb.quantize_transpose_128x1(*fb.quantize_1x128(dev_bf16(x_bits), pow2=True), pow2=True)
    del qt, st, a, sa
    dw = torch.empty((ayt.shape[0], NI), dtype=torch.float32, device="cuda")
    us, how = time_graph(lambda: fb.gemm_wgrad(ayt, sayt, axt, saxt, out=dw))
    # flops on the 2112 valid output rows; the kernel also runs the 64 zero
    # rows that pad dY^T to whole 128-row blocks
    out["gemm_wgrad_2112x7168x4096"] = dict(us=us, timing=how, TFLOPs=2 * NO * NI * T / us / 1e6,
                                            frac_mfma=2 * NO * NI * T / us / 1e6 / FP8_PEAK_TFLOPS,
                                            rows_run=int(ayt.shape[0]))
    times = {True: [], False: []}
    for rnd in range(3):   # alternated, as for the dense pair above
        for hw in ((True, False) if rnd % 2 == 0 else (False, True)):
            us2, how2 = time_graph(lambda: (fb.gemm_wgrad(ayt2, sayt2, axt2, saxt2, out=dw, pow2_scales=True) if hw
                                            else fb.gemm_wgrad(ayt2, sayt2, axt2, saxt2, out=dw)))
            times[hw].append(us2)
    for hw in (True, False):
        us2 = float(np.median(times[hw]))
        out[f"gemm_wgrad_pow2_{'hw' if hw else 'sw'}_2112x7168x4096"] = dict(
            us=us2, timing=how2 + ", alternated", TFLOPs=2 * NO * NI * T / us2 / 1e6,
            frac_mfma=2 * NO * NI * T / us2 / 1e6 / FP8_PEAK_TFLOPS)
    return out


def vs_hipblaslt(fb, synth, reps=5, burst=20):
    """Context, not part of the step: the block-scaled GEMM beside hipBLASLt's
    plain FP8 GEMM (torch._scaled_mm with one scale per tensor, and with one
    per row of A and column of B) on the same FP8 operand bytes (the
    quantized synthetic workload).  The library applies no 1x128 / 128x128
    block scales, so per output it does strictly less work.  Interleaved
    bursts of `burst` back-to-back calls between two events; medians in us."""
    out = {}
    for (M, N, K) in [(4096, 2112, 7168), (8192, 4096, 7168)]:
        w = synth.dense(M, N, K, seed=1)
        a, sa = fb.quantize_1x128(dev_bf16(w["a"]))
        b, sb = fb.quantize_128x128(dev_bf16(w["b"]))
        d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        one = torch.ones((), device="cuda")
        ra, rb = torch.ones((M, 1), device="cuda"), torch.ones((1, N), device="cuda")
        bt = b.t()
        fns = {
            "block_scaled_gemm": lambda: fb.gemm(a, sa, b, sb, out=d),
            "hipblaslt_fp8_tensorwise": lambda: torch._scaled_mm(a, bt, scale_a=one, scale_b=one,
                                                                 out_dtype=torch.bfloat16),
            "hipblaslt_fp8_rowwise": lambda: torch._scaled_mm(a, bt, scale_a=ra, scale_b=rb,
                                                              out_dtype=torch.bfloat16),
        }
        times = {k: [] for k in fns}
        for f in fns.values():
            for _ in range(3):
                f()
        torch.cuda.synchronize()
        for _ in range(reps):
            for k, f in fns.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(burst):
                    f()
                e1.record()
                torch.cuda.synchronize()
                times[k].append(e0.elapsed_time(e1) * 1e3 / burst)
        flops = 2.0 * M * N * K
        out[f"{M}x{N}x{K}"] = {k: {"us": round(float(np.median(v)), 2),
                                   "TFLOPs": round(flops / float(np.median(v)) / 1e6, 1)}
                               for k, v in times.items()}
    return out


def cpu_baseline(synth, reps=8):
    """The CPU oracle on the same step: 1x128 quantization of the whole BF16
    activation and its GEMM against the quantized weight, run `reps` times
    (about ten seconds of CPU work on a 16-core host), in TFLOP/s of GEMM work
    per step."""
    from oracle import gemm as og, quantize as oq
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    M, N, K = WORKLOAD["M"], WORKLOAD["N"], WORKLOAD["K"]
    w = synth.dense(M, N, K, seed=0)
    bq, bs = oq.quantize_128x128(w["b"])
    t0 = time.perf_counter()
    for _ in range(reps):
        a, sa = oq.quantize_1x128(w["a"])
        _ = og.gemm_ref(a, sa, bq, bs, "bf16")
    dt = (time.perf_counter() - t0) / reps
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=2 * M * N * K / dt / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle", cpu_model=model,
                sample=f"the whole step ({M}x{K} activation quantized 1x128, then its {M}x{N}x{K} GEMM, "
                       f"{2 * M * N * K / 1e9:.0f} GFLOP) run {reps} times: {dt:.2f} s per step")


def smi_sample():
    """Graphics clock (MHz, mean over the XCDs) and socket power (W) from
    amd-smi, or None where the tool is missing or prints something else."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p"], capture_output=True, text=True, timeout=20)
    except Exception:
        return None
    gfx, power, section = [], None, ""
    for line in r.stdout.splitlines():
        t = line.strip()
        if t.endswith(":") and t[:-1].replace("_", "").isalnum():
            section = t[:-1]
        if t.startswith("SOCKET_POWER:"):
            try:
                power = float(t.split(":", 1)[1].split()[0])
            except ValueError:
                pass
        if t.startswith("CLK:") and section.startswith("GFX_"):
            try:
                gfx.append(float(t.split(":", 1)[1].split()[0]))
            except ValueError:
                pass
    if not gfx and power is None:
        return None
    return {"gfx_clock_mhz": round(sum(gfx) / len(gfx), 0) if gfx else None, "socket_power_w": power}


def sustained_clock(step, seconds=2.0):
    """amd-smi's graphics clock and socket power while the step runs
    continuously for `seconds` (sampled once, after the first second)."""
    import threading
    out = {}
    stop = threading.Event()

    def sampler():
        time.sleep(min(1.0, seconds / 2))
        if not stop.is_set():
            out["s"] = smi_sample()
    th = threading.Thread(target=sampler)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    return out.get("s")


def code_hash(sources):
    """First 16 hex digits of the SHA-256 of the kernel sources with comments,
    trailing blanks and empty lines removed, so that a summary stays valid
    across comment-only edits but not across any change to the code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            for line in fh:
                line = re.sub(r"//.*$", "", line).rstrip()
                if line:
                    h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def profile_traffic(path, sources):
    """HBM-side bytes per launch of the dominant kernel, as recorded in a
    rocprofv3 summary under profiles/, or None when the kernel's code has
    changed since the counters were taken (the summary stores its hash)."""
    try:
        text = open(os.path.join(ROOT, path)).read()
    except OSError:
        return None
    tb = [l.split(":", 1)[1].strip() for l in text.splitlines() if l.startswith("traffic_bytes_per_launch:")]
    hs = [l.split(":", 1)[1].split()[0] for l in text.splitlines() if l.startswith("kernel_source_sha256_16:")]
    if not tb or not hs:
        return None
    return int(tb[0]) if code_hash(sources) == hs[0] else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="skip the per-kernel workload table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true",
                    help="time the per-kernel table call by call instead of replaying HIP graphs (and skip the "
                         "graph-replayed step)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    ap.add_argument("--vs-hipblaslt", action="store_true",
                    help="only time the block-scaled GEMM beside hipBLASLt's plain FP8 GEMM on the same operand "
                         "bytes (context for the roofline fraction) and print that as one JSON line")
    args = ap.parse_args()
    global EAGER
    EAGER = args.eager
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path runs on a single "
              "device: each kernel works on one GPU's share and nothing here communicates)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 5}), flush=True)
        return

    from fp8_block_scaled_04_amd import fp8bs as fb, synth

    if args.vs_hipblaslt:
        print(json.dumps({"vs_hipblaslt": vs_hipblaslt(fb, synth)}), flush=True)
        return

    M, N, K = WORKLOAD["M"], WORKLOAD["N"], WORKLOAD["K"]
    w = synth.dense(M, N, K, seed=0)
    x = dev_bf16(w["a"])
    bq, bs = fb.quantize_128x128(dev_bf16(w["b"]))
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    progress(f"workload {M}x{N}x{K} on the device")

    def step():
        q, s = fb.quantize_1x128(x)
        fb.gemm(q, s, bq, bs, out=d)

    # The GEMM's own duration, second reading: HIP events, on the stream it
    # runs on, around bursts of 10 back-to-back launches right after one of
    # the step's quantizer calls.  (An event between two kernels adds a drain
    # to the interval: one event pair per launch read 88-90 us where the
    # kernel trace shows 78 us.)  A burst of GEMMs alone draws more power than
    # the step, so it runs at a lower clock.
    for _ in range(args.warmup):
        step()
    burst = 10
    spans = []
    for _ in range(max(2, args.steps // burst)):
        q, s = fb.quantize_1x128(x)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(burst):
            fb.gemm(q, s, bq, bs, out=d)
        e1.record()
        spans.append((e0, e1))
    torch.cuda.synchronize()
    gemm_us_burst = float(np.mean([a.elapsed_time(b) for a, b in spans])) * 1e3 / burst
    # The timed steps: plain launches, exactly `steps` of them between two
    # synchronizations (nothing else in flight), bracketed by HIP events on
    # the launch stream as well.
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / args.steps * 1e3
    # The GEMM's duration inside the timed steps (roofline): the events' span
    # of the steps minus that of the same number of quantizer calls alone,
    # per step -- the GEMM under the step's own power state.
    qv0, qv1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qv0.record()
    for _ in range(args.steps):
        fb.quantize_1x128(x)
    qv1.record()
    torch.cuda.synchronize()
    quant_us = qv0.elapsed_time(qv1) * 1e3 / args.steps
    progress(f"{args.steps} timed steps: {ms_per_step * 1e3:.1f} us per step")
    gemm_us = ev0.elapsed_time(ev1) * 1e3 / args.steps - quant_us
    kernel_us_method = "timed steps minus as many quantizer calls, HIP events"
    if not gemm_us > 0:   # the difference of two noisy spans; not expected
        gemm_us, kernel_us_method = gemm_us_burst, "bursts of 10 launches, HIP events"

    # For reference, the same step captured once in a HIP graph and replayed
    # (the library launches kernels only).  On ROCm 7.2 the replays were
    # slower than the eager launches (107 vs 98 us per step), so they are
    # reported beside the value, not used for it.
    ms_graph = None
    if not args.eager:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    step()
            torch.cuda.current_stream().wait_stream(side)
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            ms_graph = (time.perf_counter() - t0) / args.steps * 1e3
        except Exception as exc:
            print(f"graph capture failed ({exc})", file=sys.stderr)
    clocks = None if args.eager else sustained_clock(step)
    flops = 2.0 * M * N * K
    achieved = flops / gemm_us / 1e6
    rec = {
        "metric": "FP8 block-scaled GEMM TFLOPS (% of MI355X FP8 peak); quantizer GB/s",
        "value": flops / (ms_per_step / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "fp8 linear forward: quantize_1x128(A bf16 4096x7168) + block-scaled GEMM "
                               "4096x2112x7168, bf16 out", "M": M, "N": N, "K": K,
                   "ms_per_step_graph_replay": ms_graph,
                   "clocks_sustained_step": clocks},
        # Other hardware, for context only: the pages report DeepGEMM reaching
        # up to 1350 FP8 TFLOP/s on NVIDIA Hopper (page 4, "Deepseek
        # veroeffentlicht Deepgemm", section "Schluesselmerkmale von DeepGemm";
        # no shape given), so it is not a baseline for this workload.
        "context_other_hardware": {"tflops": 1350, "hardware": "NVIDIA Hopper", "shape": "not stated",
                                   "what": "peak FP8 GEMM throughput the surveyed pages report for DeepGEMM"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP8_PEAK_TFLOPS,
                     "traffic": profile_traffic(GEMM_PROFILE, GEMM_SOURCES),
                     "kernel": GEMM_KERNEL, "kernel_us": gemm_us,
                     "kernel_us_method": kernel_us_method,
                     "kernel_us_burst": gemm_us_burst, "quantizer_us_in_step": quant_us},
    }
    if not args.no_extra:
        rec["kernels"] = extra_kernels(fb, synth)
    if not args.no_cpu:
        progress("oracle on the host cores (cpu_baseline)")
        rec["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

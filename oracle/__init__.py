"""CPU oracle for the block-scaled FP8 hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy restatement of what the
hot path computes.  It exists so that the GPU kernels can be checked against
something written independently of them.  It shares no code, headers, tables
or constants with the HIP path, and the HIP path never imports it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in here.  Product code that
routes through this package (or any other CPU fallback) is a bug.

Sources.  The method is described on the surveyed web pages:
  * page 1, the uniondaocoop.com board post that paraphrases DeepSeek's FP8
    mixed-precision training framework (paragraphs on fine-grained 1x128 /
    128x1 tiling, FP8 GEMM outputs in BF16 or FP32, FP8 activation caching and
    promotion of partial sums to FP32 registers);
  * page 2, "A Deadly Mistake Uncovered on Deepseek China Ai ..." (paragraph
    on Hopper's fixed-point accumulation keeping about 14 bits after a
    sign-fill right shift; power-of-two scaling factors; group-scaled MMA);
  * page 4, "Deepseek veroeffentlicht Deepgemm ..." (dense and two MoE
    layouts; section "Was ist fp8?"; Table 1 "DeepGemm Performance
    Benchmarks").
The pages leave the FP8 format, the scale formula, rounding, and the block
shape of weights open; the readings taken here (OCP E4M3 "FN", scale =
amax/448 in FP32, round-to-nearest-even, satfinite, 128x128 weight blocks,
promotion every 128 of K) are listed with their justification in the design
notes at the repository root.

Modules
  e4m3       -- OCP E4M3 encode/decode by bit manipulation.
  bf16       -- BF16 bit helpers (decode, RNE from float64).
  quantize   -- 1x128 row tiles, 1x128 -> 128x1 transpose-requantize,
                128x128 weight blocks.
  gemm       -- dequantize-then-FP64 GEMM reference (dense, contiguous
                grouped, masked grouped) and an exact int64 chunk-sum path.
  accum_emu  -- emulator of a limited-precision fixed-point accumulator, with
                and without per-128 FP32 promotion.

Parity status: every public function here is pinned by ``-m "not gpu"``
tests in ``tests/test_oracle_*.py`` against values fixed by something other
than this package (torch's float8/bfloat16 casts, exact integer or Fraction
arithmetic, closed forms, brute-force searches).
"""

from . import e4m3, bf16, quantize, gemm, accum_emu  # noqa: F401

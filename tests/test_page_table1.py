"""Byte-count convention behind page 4's Table 1 (CPU only).

The benchmark reports achieved bandwidth for GEMMs with the convention that
reproduces the table's bandwidth column from its TFLOPS column: FP8 A and B
read once, BF16 D written once, scales not counted (the benchmark also reports
the figure with scales).  This test pins that reading against the printed
rows.
"""

import json
import os

TABLE = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_claims.json")))["table1"]


def test_table1_bandwidth_is_fp8_inputs_plus_bf16_output():
    for M, N, K, tflops, gbs, _ in TABLE["rows"]:
        seconds = 2.0 * M * N * K / (tflops * 1e12)
        implied = (M * K + N * K + 2 * M * N) / seconds / 1e9
        assert abs(implied - gbs) / gbs < 0.005, (M, N, K, implied, gbs)

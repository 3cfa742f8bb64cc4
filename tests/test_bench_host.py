"""Host logic of bench.py (CPU only): the comment-insensitive source hash that
ties a committed rocprofv3 summary to the kernel code, the traffic lookup that
goes null once the code changes, and the one-GPU guard."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int x = 1;  // one\n\n// a note\nint y;\n")
    b = tmp_path / "b.hip"
    b.write_text("int x = 1;\nint y;   \n")
    c = tmp_path / "c.hip"
    c.write_text("int x = 2;\nint y;\n")
    assert bench.code_hash([str(a)]) == bench.code_hash([str(b)])
    assert bench.code_hash([str(a)]) != bench.code_hash([str(c)])
    assert len(bench.code_hash([str(a)])) == 16


def test_profile_traffic_follows_the_code_hash(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int k;\n")
    prof = tmp_path / "p.md"
    prof.write_text("| figure | value |\n"
                    "traffic_bytes_per_launch: 1234\n"
                    f"kernel_source_sha256_16: {bench.code_hash([str(src)])}  (SHA-256 of k.hip)\n")
    assert bench.profile_traffic(str(prof), [str(src)]) == 1234
    src.write_text("int k;  // a comment only\n")
    assert bench.profile_traffic(str(prof), [str(src)]) == 1234
    src.write_text("int k2;\n")
    assert bench.profile_traffic(str(prof), [str(src)]) is None
    assert bench.profile_traffic(str(tmp_path / "missing.md"), [str(src)]) is None


def test_committed_dense_profile_records_traffic_and_code_hash():
    # The roofline's `traffic` is read from this summary only while the GEMM
    # code hashes to what the summary recorded; after a kernel change it is
    # reported as null until the counters are taken again.
    text = open(os.path.join(ROOT, bench.GEMM_PROFILE)).read()
    lines = text.splitlines()
    tb = [l for l in lines if l.startswith("traffic_bytes_per_launch:")]
    hs = [l for l in lines if l.startswith("kernel_source_sha256_16:")]
    assert tb and hs, f"{bench.GEMM_PROFILE} lacks its traffic or code-hash line"
    matches = hs[0].split(":", 1)[1].split()[0] == bench.code_hash(bench.GEMM_SOURCES)
    want = int(tb[0].split(":", 1)[1].strip()) if matches else None
    assert bench.profile_traffic(bench.GEMM_PROFILE, bench.GEMM_SOURCES) == want


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr

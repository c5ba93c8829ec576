"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, and the byte and flop counts it reports match their closed
forms for the workloads it times."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_bytes_closed_form():
    # packed codes N K / 2 + bf16 scales 2 N K / 32 + X 2 M K + Y 2 M N
    N, K = bench.DECODE_N, bench.DECODE_K
    for M in bench.DECODE_MS:
        assert bench.decode_bytes(M) == N * K // 2 + 2 * N * (K // 32) + 2 * M * K + 2 * M * N
    # zero points add one byte per group
    assert bench.decode_bytes(1, zero_points=True) == bench.decode_bytes(1) + N * (K // 32)
    # the sweep's per-launch figures quoted in the documentation
    assert [bench.decode_bytes(M) for M in (1, 8, 16, 32)] == [28344320, 28573696, 28835840,
                                                               29360128]


def test_gemm_flops():
    assert bench.gemm_flops(4096, 14336, 4096) == 2 * 4096 * 14336 * 4096

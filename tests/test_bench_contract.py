"""bench.py's contract on the CPU: one GPU only, and the algorithmic work per
token-head that its rooflines divide by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_work_per_token_head():
    # flops: 6 dk dv (state products) + 4C dk + 2C dv + C(dk + dv) (chunk
    # Gram, W, U and M terms) with C = 16; bytes: q, k, g, v and beta in bf16,
    # o out in fp32
    assert bench.prefill_units(128, 128) == (114688, 1538)
    assert bench.prefill_units(64, 64) == (32768, 770)


def test_clock_sampler_without_the_driver_file():
    c = bench.ClockSampler()
    c.path = None
    c.start()
    assert c.stop() is None

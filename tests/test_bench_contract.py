"""Host-side parts of bench.py's contract (no GPU): it runs on one GPU only
and says so for any other --gpus, and its roofline helpers price the work
as the metric defines it."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_blended_roofline_of_pure_fp8_and_bf16_work():
    # all work FP8: the peak is the FP8 peak; all bf16: the bf16 peak
    ms = 1.0
    m8 = dict(f_qk8=1e12, f_pv=0.0, f_qk16=0.0, attn_ms=ms)
    m16 = dict(f_qk8=0.0, f_pv=1e12, f_qk16=0.0, attn_ms=ms)
    a8, p8 = bench.roofline_of(m8)
    a16, p16 = bench.roofline_of(m16)
    assert abs(p8 - bench.PEAK_FP8) < 1e-6 * p8 and abs(p16 - bench.PEAK_BF16) < 1e-6 * p16
    assert abs(a8 - 1e15) < 1e3 and abs(a16 - 1e15) < 1e3
    # equal FLOP counts: the harmonic blend
    a, p = bench.roofline_of(dict(f_qk8=1e12, f_pv=1e12, f_qk16=0.0, attn_ms=ms))
    assert abs(p - 2.0 / (1.0 / bench.PEAK_FP8 + 1.0 / bench.PEAK_BF16)) < 1e-6 * p

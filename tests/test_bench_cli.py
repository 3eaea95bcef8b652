"""bench.py on the CPU: it measures one GPU only, and its workload arithmetic
(ranks from the parameter ratio, algorithmic bytes of a decode layer set)
gives the configured figures."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_ranks_from_the_parameter_ratio():
    # r = floor(rho d_in d_out / (d_in + d_out)) at the 7B and 13B shapes
    assert bench.rank(0.6, 4096, 4096) == 1228 and bench.rank(0.6, 4096, 11008) == 1791
    assert bench.rank(0.6, 11008, 4096) == 1791
    assert bench.rank(0.4, 4096, 4096) == 819 and bench.rank(0.4, 4096, 11008) == 1194
    assert bench.rank(0.2, 4096, 4096) == 409 and bench.rank(0.2, 4096, 11008) == 597
    assert bench.rank(0.4, 5120, 5120) == 1024 and bench.rank(0.4, 5120, 13824) == 1494
    for rho, a, b in ((0.6, 4096, 11008), (0.4, 5120, 13824), (0.2, 4096, 4096)):
        r = bench.rank(rho, a, b)   # the largest r whose two factors fit the ratio
        assert r * (a + b) <= rho * a * b < (r + 1) * (a + b)


def test_decode_layer_set_bytes():
    # both factors once, x in, y out (bf16): 242.9 / 244.0 / 247.8 / 252.8 MB
    # per 7-projection layer set at T = 1 / 8 / 32 / 64
    def layer_set(T):
        return sum(bench.decode_bytes(T, a, bench.rank(0.6, a, b), b)
                   for a, b in bench.SHAPES.values())
    got = [round(layer_set(T) / 1e6, 1) for T in bench.TOKENS]
    assert got == [242.9, 244.0, 247.8, 252.8]
    # the dominant launch class: gate and up at T = 64
    gu = sum(bench.decode_bytes(64, 4096, 1791, 11008) for _ in range(2))
    assert gu == 112071680

"""CPU checks of the benchmark's byte accounting and its output contract."""
import os
import subprocess
import sys

import pytest

import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


@pytest.mark.parametrize("cfg", [2, 3, 4])
@pytest.mark.parametrize("b", [1, 4, 8, 32])
def test_algorithmic_bytes_match_the_oracle_accounting(cfg, b):
    """The roofline's numerator (bench.algorithmic_bytes) is the oracle's byte
    accounting, which the page totals pin (7.75 GB INT8 pool, 1.89 GB 3B)."""
    bench = _bench()
    spec = synth.stack_spec(cfg)
    for lin in spec.linears():
        want = (O.algorithmic_bytes_int4o(lin.N, lin.K, b) if spec.fmt == "int4o"
                else O.algorithmic_bytes_int8(lin.N, lin.K, b))
        assert bench.algorithmic_bytes(spec.fmt, lin.N, lin.K, b) == want


def test_per_step_bytes_of_the_benchmark_line():
    """The 3B-shaped step moves 1,498,427,392 algorithmic bytes at b = 1 (the
    figure bench.py reports), 112 products of 13,378,816 bytes on average."""
    bench = _bench()
    spec = synth.stack_spec(2)
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    total = 0
    for names in groups:
        N = sum(spec.linear(n).N for n in names)
        total += bench.algorithmic_bytes("int4o", N, spec.linear(names[0]).K, 1)
    assert spec.layers * total == 1498427392
    assert spec.layers * total // (4 * spec.layers) == 13378816


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

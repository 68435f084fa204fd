"""Host-side checks of bench.py (no GPU): the one-GPU guard, and the
algorithmic work it divides by (useful Phase-1 pairs, decode bytes), pinned
by brute-force counting over (query, key) positions and by the sizes the
workload table states (8B-128K: 4.838e13 FLOP per Phase-1 launch, 537.7 MB
per decode step)."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("L,b,a", [(700, 200, 200), (512, 128, 0), (333, 1000, 1000),
                                   (97, 32, 16), (1, 16, 16)])
def test_phase1_pairs_brute_force(L, b, a):
    """Query q (block i = q // b) sees key k when k is in its own block and
    k <= q, or when i >= 1 and k < a (the anchor)."""
    bench = load_bench()
    q = np.arange(L)[:, None]
    k = np.arange(L)[None, :]
    own = (k // b == q // b) & (k <= q)
    anchor = (q // b >= 1) & (k < a)
    assert bench.phase1_pairs(L, b, a) == int((own | anchor).sum())


def test_workload_work_figures():
    bench = load_bench()
    from workloads import WORKLOADS
    w = WORKLOADS["llama8b-128k"]
    assert bench.phase1_flops(w) == pytest.approx(4.838e13, rel=1e-3)
    assert bench.decode_bytes(w, w.T - 1) == pytest.approx(537.7e6, rel=1e-3)
    w = WORKLOADS["llama8b-1m"]
    assert bench.phase1_flops(w) == pytest.approx(8.268e14, rel=1e-3)
    assert bench.decode_bytes(w, w.T - 1) == pytest.approx(4.295e9, rel=1e-3)


def test_traffic_only_for_the_profiled_kernel(tmp_path, monkeypatch):
    """The HBM traffic figure is reported only while the kernel source is the
    one the counter summary was taken from."""
    bench = load_bench()
    t = bench.pmc_traffic()
    assert t is None or t > 0
    other = tmp_path / "flash2.hip"
    other.write_text("// another kernel\n")
    monkeypatch.setattr(bench, "FLASH_SRC", str(other))
    assert bench.pmc_traffic() is None

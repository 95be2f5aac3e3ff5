"""Host-side pieces of bench.py: the work model, the one-GPU guard and the oracle baseline leg.

The FLOP model is the page's canonical count (page "Write a fast Based (Taylor linear attention) forward
kernel", field flops_src, with C = 64); the byte model counts q, k, v read once and o written once. The
expected numbers below are those two formulas evaluated by hand for the benchmark shapes.
"""
import os
import subprocess
import sys

import numpy as np

import bench
from taylor_feature_map_amd.inputs import Workload, make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_work_model_benchmark_shapes():
    # (B, T, H, K, V, output bytes) -> canonical FLOPs, algorithmic bytes
    cases = [
        ((1, 512, 2, 8, 64, 4), 28_573_696, 425_984),
        ((4, 8192, 16, 16, 64, 2), 42_010_148_864, 167_772_160),
        ((8, 4096, 16, 16, 128, 2), 82_946_555_904, 301_989_888),
        ((1, 65000, 16, 16, 64, 2), 83_333_120_000, 332_800_000),
    ]
    for (B, T, H, K, V, ob), flops, nbytes in cases:
        assert bench.canonical_flops(B, T, H, K, V) == flops
        assert bench.algorithmic_bytes(B, T, H, K, V, ob) == nbytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_only_for_its_workload_and_code(monkeypatch):
    """A traffic figure is read only from its own workload's summary, and only while the device code is the
    one the counters were taken on."""
    assert bench.measured_traffic("no_such_workload") is None
    path = bench.traffic_file("b4_t8192_h16_k16_v64")
    if not os.path.exists(path):
        return
    recorded = None
    for line in open(path):
        if line.strip().startswith("device_code_sha256:"):
            recorded = line.split(":", 1)[1].strip()
    assert recorded is not None
    monkeypatch.setattr(bench, "device_code_digest", lambda lib=None: "0" * 64)
    assert bench.measured_traffic("b4_t8192_h16_k16_v64") is None
    monkeypatch.setattr(bench, "device_code_digest", lambda lib=None: recorded)
    assert bench.measured_traffic("b4_t8192_h16_k16_v64") > bench.algorithmic_bytes(4, 8192, 16, 16, 64, 2)


def test_oracle_baseline_leg():
    w = Workload(name="tiny", B=1, T=96, H=2, K=8, V=16, seed=5, scale=None, out_dtype="bf16")
    qb, kb, vb = make_workload(w)
    r = bench.cpu_baseline(w, qb, kb, vb, budget_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["cores"] >= 1
    assert r["seconds"] >= 0.2 - 1e-9
    assert np.isfinite(r["value"]) and r["value"] > 0
    # at least one (b, h) sequence, and more than one pass over the two pairs in 0.2 s of oracle time
    assert "(b,h) sequences of T=96" in r["sample"]


def test_counter_figures_only_for_the_built_code():
    assert bench.counter_summary("no_such_workload") is None


def test_row_probe_argument_check():
    """The 32-byte-row read probe (counter calibration) refuses a (b, h) count that does not split over the
    8 XCDs, on the host."""
    import ctypes
    path = os.path.join(ROOT, "taylor_feature_map_amd", "libbased_probe.so")
    if not os.path.exists(path):
        import pytest
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(path)
    lib.based_probe_read_rows.restype = ctypes.c_int
    lib.based_probe_read_rows.argtypes = [ctypes.c_void_p] + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2
    assert lib.based_probe_read_rows(0x10000, 1, 64, 3, 0x20000, None) == 1
    assert lib.based_probe_read_rows(None, 1, 64, 8, 0x20000, None) == 1

"""bench.py's contract: the FLOP counts every TFLOP/s figure divides by, the
refusal of several GPUs, the traffic-summary reader, and (on a GPU) the shape
of the one JSON line it prints.

The FLOP counts are pinned to a brute-force count of the visible (query, key)
pairs of the masks the pages define (intra-stream: Figure 2(c); cross-stream:
Figure 2(a), windowed 2(b)), taken from the oracle's 1-based mask builder.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import brute  # noqa: E402

INTRA, CROSS = 0, 1


@pytest.mark.parametrize("n", [1, 2, 3, 5])
@pytest.mark.parametrize("L", [1, 7, 16])
@pytest.mark.parametrize("mode,window", [(INTRA, 0), (INTRA, 1), (INTRA, 4), (CROSS, 0), (CROSS, 1), (CROSS, 3),
                                         (INTRA, 100), (CROSS, 100)])
def test_useful_flops_counts_visible_pairs(n, L, mode, window):
    pairs = int(brute.mask(n, L, mode, window).sum())
    assert bench.useful_flops(1, L, n, 1, 1, mode, window) == 4 * pairs
    # linear in batch, heads and head dim
    assert bench.useful_flops(3, L, n, 5, 64, mode, window) == 4 * 3 * 5 * 64 * pairs


@pytest.mark.parametrize("n", [1, 2, 4])
@pytest.mark.parametrize("mode,window", [(INTRA, 0), (CROSS, 0), (INTRA, 3), (CROSS, 2)])
def test_useful_flops_final_counts_final_rows(n, mode, window):
    L = 9
    m = brute.mask(n, L, mode, window)
    final_rows = np.arange(n - 1, n * L, n)  # 0-based positions i*n + n-1
    pairs = int(m[final_rows].sum())
    assert bench.useful_flops_final(1, L, n, 1, 1, mode, window) == 4 * pairs


@pytest.mark.parametrize("mode,window", [(INTRA, 0), (CROSS, 0), (INTRA, 3), (CROSS, 2)])
def test_row_visible_keys_matches_mask(mode, window):
    n, L = 3, 11
    m = brute.mask(n, L, mode, window)
    t = np.arange(n * L)
    np.testing.assert_array_equal(bench.row_visible_keys(t, n, L, mode, window), m.sum(axis=1))


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_measured_traffic_reads_summary_and_digest(tmp_path, monkeypatch):
    import hashlib
    (tmp_path / "profiles").mkdir()
    (tmp_path / "src").mkdir()
    a, b = tmp_path / "src" / "a.hip", tmp_path / "src" / "a.inc"
    a.write_text("kernel source\n")
    b.write_text("included part\n")
    digest = hashlib.sha256(a.read_bytes() + b.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "k__hbm_bytes.md").write_text(
        "# summary\n\n- `source`: `src/a.hip, src/a.inc`\n"
        f"- `source_sha256`: `{digest}`\n- `traffic_bytes_per_launch`: `12345`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("k__hbm_bytes") == 12345
    assert bench.measured_traffic("missing") is None
    b.write_text("included part, changed\n")  # counters no longer describe the kernel
    assert bench.measured_traffic("k__hbm_bytes") is None


REQUIRED = {"metric": str, "value": (int, float), "unit": str, "n_gpus": int, "steps": int, "warmup": int,
            "ms_per_step": (int, float), "higher_is_better": bool, "scaling": str, "dtype": str, "data": str,
            "config": dict, "roofline": dict, "cpu_baseline": dict}


@pytest.mark.gpu
def test_bench_json_line():
    """A short default-shaped run prints one JSON line with the contract's
    fields; the roofline fraction is achieved / peak."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-extra", "--cpu-seconds", "2"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key, typ in REQUIRED.items():
        assert isinstance(d.get(key), typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    assert "workload" in d["config"]
    for name, comp in d["components"].items():  # mean, min and median of every timed row
        assert {"ms", "ms_min", "ms_median"} <= set(comp), name
        assert comp["ms_min"] <= comp["ms_median"] + 1e-9, name
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["cores"] >= 1

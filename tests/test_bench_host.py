"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard and the CPU
baseline leg (the float64 oracle timed on a bounded channel sample)."""
import numpy as np

import bench
from workloads import WORKLOADS, make_inputs


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.delenv("WORLD_SIZE", raising=False)
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main(["--gpus", "1"]) == 2


def test_cpu_baseline_reports_a_bounded_oracle_sample():
    w = WORKLOADS[1]
    v, g = make_inputs(w)
    rec = bench.cpu_baseline(w, v, g, budget_s=0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "outputs/s"
    assert rec["cores"] >= 1 and rec["value"] > 0
    n = int(rec["sample"].split()[0])
    assert 8 <= n <= w.B * w.C
    assert "of %d channels (L=%d)" % (w.B * w.C, w.L) in rec["sample"]
    assert np.isfinite(rec["value"])

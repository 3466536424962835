"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=120)
        assert p.returncode != 0
        assert "one GPU" in p.stderr
        assert p.stdout.strip() == ""          # no JSON line for a refused run


def test_defaults_are_one_gpu_and_a_bounded_run(monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.gpus == 1 and a.workload == "quartet"
    assert 1 <= a.steps <= 200 and 0 <= a.warmup <= 50
    assert not a.no_cpu_baseline and not a.no_extra

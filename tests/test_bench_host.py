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


def test_counter_records_match_the_sources_they_were_taken_on(monkeypatch, tmp_path):
    """The committed GEMM traffic and quantizer VALU records are used only
    while the kernel sources hash to the values they were taken on."""
    import json
    import types
    import bench
    st = types.SimpleNamespace(m=8192, n=4096, k=4096)
    avg = {"quant_x": 0.04, "quant_w": 0.02, "quant_dy": 0.045}
    r = bench.quant_alu_roofline(st, avg)
    assert r is not None and r["bound"] == "alu" and 0.0 < r["frac"] < 1.0
    assert bench.gemm_traffic(st) is not None
    # another workload, or a record whose source hash differs: no figure
    assert bench.quant_alu_roofline(types.SimpleNamespace(m=8192, n=14336, k=4096), avg) is None
    rec = json.load(open(bench.QUANT_VALU_RECORD))
    rec["source_sha256"] = {k: "0" * 64 for k in rec["source_sha256"]}
    fake = tmp_path / "rec.json"
    fake.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "QUANT_VALU_RECORD", str(fake))
    assert bench.quant_alu_roofline(st, avg) is None

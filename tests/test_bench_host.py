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


def test_counter_records_are_used_only_on_the_sources_they_were_taken_on(monkeypatch, tmp_path):
    """bench.py takes the GEMM traffic and the quantizer VALU counts from
    committed counter records only while the kernel sources hash to the
    values recorded with them and the workload matches."""
    import hashlib
    import json
    import types
    import bench

    def sha(rel):
        with open(os.path.join(ROOT, rel), "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()

    gsrc = "fp4_microscaled_quantized_amd/csrc/gemm_mx.hip"
    qsrc = ["fp4_microscaled_quantized_amd/csrc/quant_mx.hip", "fp4_microscaled_quantized_amd/csrc/mx_device.h"]
    st = types.SimpleNamespace(m=8192, n=4096, k=4096)
    avg = {"quant_x": 0.04, "quant_w": 0.02, "quant_dy": 0.045}
    traffic = {"workload": "8192x4096x4096", "source": gsrc, "source_sha256": sha(gsrc),
               "bytes_per_launch": {"gemm_y": 2.4e8, "gemm_dx": 2.4e8, "gemm_dw": 1.8e8}}
    valu = {"workload": "8192x4096x4096", "source_sha256": {p: sha(p) for p in qsrc},
            "valu_per_launch": {"quant_x": 1.6e7, "quant_w": 8e6, "quant_dy": 2.1e7},
            "trans_per_launch": {"quant_x": 0, "quant_w": 0, "quant_dy": 0}}
    tr, vr = tmp_path / "traffic.json", tmp_path / "valu.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tr))
    monkeypatch.setattr(bench, "QUANT_VALU_RECORD", str(vr))
    tr.write_text(json.dumps(traffic))
    vr.write_text(json.dumps(valu))
    assert bench.gemm_traffic(st) == round((2.4e8 + 2.4e8 + 1.8e8) / 3)
    r = bench.quant_alu_roofline(st, avg)
    assert r["bound"] == "alu" and 0.0 < r["frac"] < 1.0
    # another workload: no figure
    other = types.SimpleNamespace(m=8192, n=14336, k=4096)
    assert bench.gemm_traffic(other) is None and bench.quant_alu_roofline(other, avg) is None
    # a source changed since the counters were taken: no figure
    traffic["source_sha256"] = "0" * 64
    valu["source_sha256"][qsrc[1]] = "0" * 64
    tr.write_text(json.dumps(traffic))
    vr.write_text(json.dumps(valu))
    assert bench.gemm_traffic(st) is None and bench.quant_alu_roofline(st, avg) is None
    # a missing record: no figure
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "none.json"))
    assert bench.gemm_traffic(st) is None

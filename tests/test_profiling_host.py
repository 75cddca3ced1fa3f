"""Host logic of the measurement helpers (gpt_pretraining_step_amd.profiling):
attribution of counter rows to the dispatch after each marker, the traffic
record's scaling by the calibration copy, and the per-site, per-workload,
per-source-hash lookup that bench.py uses, bench.py's refusal of more than one
GPU and its FLOP accounting.  CPU only: synthetic CSV rows."""

import csv
import json
import os

import pytest

from gpt_pretraining_step_amd import profiling as P

MARK = P.MARKER


def _rows(counter, seq):
    """Counter rows for a sequence of (kernel name, value) dispatches; each
    dispatch reports two dimension instances that must be summed."""
    out = []
    for i, (name, v) in enumerate(seq, start=1):
        for part in (0.25, 0.75):
            out.append({"Dispatch_Id": str(i), "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": str(v * part)})
    return out


def _write(dirname, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def test_attribute_takes_the_dispatch_after_each_marker():
    seq = [("other", 5), (MARK, 0), ("site_kernel", 100), ("other", 7), (MARK, 0), ("site_kernel", 300),
           (MARK, 0), ("copy", 64)]
    name, vals, copy = P.attribute(_rows("FETCH_SIZE", seq), "FETCH_SIZE")
    assert name == "site_kernel" and vals == [100, 300] and copy == 64


def test_attribute_rejects_mixed_kernels():
    seq = [(MARK, 0), ("a", 1), (MARK, 0), ("b", 2), (MARK, 0), ("copy", 3)]
    with pytest.raises(ValueError):
        P.attribute(_rows("FETCH_SIZE", seq), "FETCH_SIZE")


def test_traffic_record_scales_and_is_found_only_for_its_site_workload_and_sources(tmp_path):
    site = "gemm.dw"
    # 256 MiB copy read as half its bytes by FETCH_SIZE (KiB), written in full
    copy = 1 << 28
    f_dir, w_dir = str(tmp_path / "f"), str(tmp_path / "w")
    _write(f_dir, _rows("FETCH_SIZE", [(MARK, 0), ("k", 1000.0), (MARK, 0), ("copy", copy / 1024 / 2)]))
    _write(w_dir, _rows("WRITE_SIZE", [(MARK, 0), ("k", 10.0), (MARK, 0), ("copy", copy / 1024)]))
    text = P.traffic_record(f_dir, w_dir, site, copy, "cmd f", "cmd w")
    rec = json.loads([l for l in text.splitlines() if l.startswith("traffic: ")][0][len("traffic: "):])
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == round(1000.0 * 1024 * 2 + 10.0 * 1024)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x_hbm_traffic.md").write_text(text)
    assert P.load_traffic(str(prof), site) == rec["bytes_per_launch"]
    assert P.load_traffic(str(prof), site, "rotary") is None       # another workload
    assert P.load_traffic(str(prof), "gemm.qkv") is None           # another site
    stale = text.replace(rec["sources_sha256_16"], "0" * 16)
    (prof / "x_hbm_traffic.md").write_text(stale)
    assert P.load_traffic(str(prof), site) is None                  # sources changed since


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and r.stdout == ""
    assert "one GPU" in r.stderr


def test_bench_flop_accounting():
    """The FLOPs per token of the MFU line and the grouped weight-gradient
    launch's FLOPs, against sums written out from the shapes."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    # 6N + 12 L H Q T with the padded-vocabulary parameter count
    assert bench.flops_per_token(124_475_904) == 6 * 124_475_904 + 12 * 12 * 12 * 64 * 1024 == 860_101_632
    M, C, V, F = 16 * 1024, 768, 50304, 3072
    fl = bench.gemm_site_flops(M, F)
    per_layer = 2 * M * C * (3 * C) + 2 * M * C * C + 2 * M * C * F + 2 * M * F * C
    assert fl["gemm.dw"] == 12 * per_layer == 2_783_138_807_808
    # the lm_head's products run per chunk of 8192 rows: two chunks at B=16
    assert fl["gemm.lm_head"] == 2 * 8192 * V * C
    assert fl["gemm.lm_head_bwd"] == 2 * fl["gemm.lm_head"]
    assert 2 * (fl["gemm.lm_head"] + fl["gemm.lm_head_bwd"]) == 3 * 2 * M * V * C
    assert fl["gemm.qkv"] == 2 * M * 3 * C * C

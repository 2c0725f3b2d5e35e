"""Host logic of bench.py that needs no GPU: the traffic record built from two
rocprofv3 counter CSVs, its validity check against the kernel sources, and the
single-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def counter_rows(ref_kib, mine_kib, launches, tail_copies):
    """A run as --copy-ref records it: input conversions (copies), this library's
    kernels (two per call), the three reference copies, then unrelated copies."""
    rows = [("void at::native::copy_kernel<float>", 999999.0)] * 2
    for _ in range(launches):
        rows.append(("void dw::(anonymous namespace)::pass1_kernel<float>", mine_kib * 0.75))
        rows.append(("void dw::(anonymous namespace)::reduce_kernel<float>", mine_kib * 0.25))
    rows += [("__amd_rocclr_copyBuffer", ref_kib)] * 3
    rows += [("void at::native::copy_kernel<float>", 4 * ref_kib)] * tail_copies
    return rows


@pytest.mark.parametrize("tail_copies", [0, 6])
def test_traffic_record_scales_by_the_reference_copy(tmp_path, monkeypatch, tail_copies):
    # the counters of this run read 2x low for fetches and exactly for writes
    ref = bench.COPY_REF_BYTES / 1024.0
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fetch, "FETCH_SIZE", counter_rows(ref / 2, 1000.0, 4, tail_copies))
    write_csv(write, "WRITE_SIZE", counter_rows(ref, 300.0, 4, tail_copies))
    out = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda tag: str(out))
    bench.traffic_from(str(fetch), str(write), "t.x", 0, "cmd")
    rec = json.loads(out.read_text())
    assert rec["launches"] == 4
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(2.0 * 1000.0 * 1024)
    assert rec["write_bytes_per_launch"] == pytest.approx(300.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(2.0 * 1000.0 * 1024 + 300.0 * 1024)
    assert rec["source_sha256"] == bench.kernel_sources_sha256()


def test_traffic_record_needs_the_reference_copy(tmp_path, monkeypatch):
    # copies before the library's kernels are input conversions, not the reference
    rows = [r for r in counter_rows(100.0, 10.0, 2, 0) if "rocclr" not in r[0]]
    f = tmp_path / "f.csv"
    write_csv(f, "FETCH_SIZE", rows)
    monkeypatch.setattr(bench, "traffic_path", lambda tag: str(tmp_path / "rec.json"))
    with pytest.raises(SystemExit):
        bench.traffic_from(str(f), str(f), "t.x", 0, "cmd")
    assert not (tmp_path / "rec.json").exists()


def test_committed_traffic_follows_the_sources(tmp_path, monkeypatch):
    path = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda tag: str(path))
    assert bench.committed_traffic("t.x") is None
    path.write_text(json.dumps({"source_sha256": bench.kernel_sources_sha256(), "bytes_per_launch": 123.0}))
    assert bench.committed_traffic("t.x") == 123.0
    path.write_text(json.dumps({"source_sha256": "0" * 64, "bytes_per_launch": 123.0}))
    assert bench.committed_traffic("t.x") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ceiling_model():
    import bench
    ceil = {"copy_gbs": 5000.0, "read_gbs": 6000.0, "write_gbs": 5500.0, "mfma_f32_tflops": 140.0,
            "mfma_f16_tflops": 2000.0, "valu_fma_f32_tflops": 100.0}
    assert bench.ceiling_of("fwd.x.k3", "bytes", 0.5, ceil)[0] == 5000.0
    assert bench.ceiling_of("fwd.x.k3", "bytes", 1.0, ceil)[0] == 6000.0
    assert bench.ceiling_of("fwd.x.k3", "bytes", 0.0, ceil)[0] == 5500.0
    assert abs(bench.ceiling_of("fwd.x.k3", "bytes", 0.75, ceil)[0] - 5500.0) < 1e-9
    assert bench.ceiling_of("bwd_weight.largek_mfma_f32.k31_s1_m1_f32", "flops", 1, ceil)[0] == 140.0
    assert bench.ceiling_of("fwd.largek_mfma.k31_s1_m1_f16", "flops", 1, ceil)[0] == 2000.0
    assert bench.ceiling_of("bwd_weight.largek_mfma_h16.k13_s1_m1_f16", "flops", 1, ceil)[0] == 2000.0
    assert bench.ceiling_of("fwd.largek_mfma_h16.k7_s1_m1_bf16", "flops", 1, ceil)[0] == 2000.0
    assert bench.ceiling_of("bwd_input.largek_roll16.k31_s1_m1_f16", "flops", 1, ceil)[0] == 2000.0
    assert bench.tag_peak("fwd.largek_roll16.k31_s1_m1_bf16", "flops")[0] == "mfma"
    assert bench.tag_peak("fwd.largek_roll_f32.k31_s1_m1_f32", "flops") == ("mfma", bench.FP32_PEAK_TFLOPS, "TFLOP/s")
    assert bench.tag_peak("bwd_weight.largek_regtile.k7_s1_m1_f32", "flops")[0] == "alu"
    assert bench.ceiling_of("bwd_input.largek_roll_f32.k31_s1_m1_f32", "flops", 1, ceil)[1:] == ("TFLOP/s", "fp32 matrix instructions")
    assert bench.ceiling_of("bwd_weight.stream_7x7.k7_s1_m1_f16", "flops", 1, ceil)[0] == 100.0
    assert bench.ceiling_of("fwd.largek_regtile.k13_s1_m1_f32", "flops", 1, ceil)[0] == 100.0
    assert bench.ceiling_of("bwd_weight.largek_mfma_t16.k13_s1_m1_f32", "flops", 1, ceil)[0] == 140.0
    assert bench.ceiling_of("fwd.x", "bytes", 0.5, None) is None

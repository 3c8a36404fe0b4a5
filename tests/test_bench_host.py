"""bench.py's host-side bookkeeping on the CPU: counter summaries scaled by the
copy calibration, the out-proj / fc2 split by fetch size, the source digest that
voids stale traffic figures, and the comment stripping behind it."""

import csv
import json

import pytest

import bench


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture
def traffic_json(tmp_path, monkeypatch):
    path = tmp_path / "hbm_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    return path


def test_summary_scales_by_the_copy_and_splits_residual_gemms(tmp_path, traffic_json):
    copy = "void at::native::vectorized_elementwise_kernel<bfloat16_copy_kernel_cuda>"
    fc1 = "gemm_bf16_kernel<128, 128, 64, 2, 2, 2, EpiGeluBf16, AMapLinear>"
    res = "gemm_bf16_kernel<128, 128, 64, 2, 2, 2, EpiResidual, AMapLinear>"
    # the 256 MiB calibration copy reads 262144 KiB; FETCH_SIZE reports half of it
    fetch = [(copy, 131072.0)] * 3 + [(copy, 10.0), (fc1, 1000.0), (fc1, 1200.0), (res, 100.0), (res, 120.0),
                                      (res, 400.0), (res, 440.0)]
    write = [(copy, 262144.0)] * 3 + [(fc1, 500.0), (res, 50.0), (res, 50.0)]
    _write_pmc(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_pmc(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "vitl16_1024_b1")
    doc = json.loads(traffic_json.read_text())
    w = doc["workloads"]["vitl16_1024_b1"]
    assert w["scale_fetch"] == pytest.approx(2.0) and w["scale_write"] == pytest.approx(1.0)
    assert w["source_digest"] == bench._source_digest()
    ops = w["ops"]
    assert ops["fc1"]["bytes_per_launch"] == pytest.approx((1100.0 * 2 + 500.0) * 1024)
    # residual dispatches split at the midpoint of their fetch range: small = out-proj, large = fc2
    assert ops["out_proj"]["dispatches"] == 2 and ops["fc2"]["dispatches"] == 2
    assert ops["out_proj"]["bytes_per_launch"] == pytest.approx((110.0 * 2 + 50.0) * 1024)
    assert ops["fc2"]["bytes_per_launch"] == pytest.approx((420.0 * 2 + 50.0) * 1024)
    assert bench.traffic_for("vitl16_1024_b1", "fc2") == pytest.approx((420.0 * 2 + 50.0) * 1024)
    assert bench.traffic_for("vitl16_1024_b1", "attention") is None   # no dispatches: no figure
    assert bench.traffic_for("vits16_336_b32", "fc2") is None          # workload never summarised


def test_head_workload_selects_the_bottleneck_convx(tmp_path, traffic_json):
    copy = "copyBuffer"
    conv = "gemm_bf16_kernel<32, 128, 64, 1, 4, 2, EpiChanLN<128>, AMapConv3, MmaBf16, 0>"
    other = "gemm_bf16_kernel<32, 256, 64, 1, 4, 2, EpiChanLN<256>, AMapLinear, MmaBf16, 0>"
    lin128 = "gemm_bf16_kernel<32, 128, 64, 1, 4, 2, EpiChanLN<128>, AMapLinear, MmaBf16, 0>"
    _write_pmc(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 131072.0)] * 3 + [(conv, 3000.0), (other, 9e6), (lin128, 9e6)])
    _write_pmc(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 262144.0)] * 3 + [(conv, 2800.0), (other, 9e6), (lin128, 9e6)])
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "semantic_head_b8")
    assert bench.traffic_for("semantic_head_b8", "convx") == pytest.approx((3000.0 * 2 + 2800.0) * 1024)


def test_summary_needs_the_calibration_copy(tmp_path, traffic_json):
    _write_pmc(tmp_path / "f.csv", "FETCH_SIZE", [("attention_kernel<4>", 5.0)])
    _write_pmc(tmp_path / "w.csv", "WRITE_SIZE", [("attention_kernel<4>", 5.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "vits16_336_b32")


def test_stale_digest_voids_the_traffic_figure(traffic_json):
    traffic_json.write_text(json.dumps({"workloads": {"vits16_336_b32": {
        "source_digest": "0" * 16, "ops": {"fc2": {"bytes_per_launch": 1.0}}}}}))
    assert bench.traffic_for("vits16_336_b32", "fc2") is None
    traffic_json.write_text(json.dumps({"workloads": {"vits16_336_b32": {
        "source_digest": bench._source_digest(), "ops": {"fc2": {"bytes_per_launch": 1.0}}}}}))
    assert bench.traffic_for("vits16_336_b32", "fc2") == 1.0


def test_comment_edits_do_not_change_the_digest_input():
    code = "int a = 1;  // one\n/* block\n comment */\nint b = 2;\n\n   \nint c = a / b;\n"
    assert bench._strip_comments(code) == "int a = 1;\nint b = 2;\nint c = a / b;"
    assert bench._strip_comments(code.replace("// one", "// uno")) == bench._strip_comments(code)
    assert bench._strip_comments(code.replace("a / b", "a * b")) != bench._strip_comments(code)


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err

"""Host logic of bench.py (no GPU): the HBM-traffic summary built from
rocprofv3 counter CSVs (copy calibration, the split-K reduction launch counted
with its GEMM), the staleness check of a stored summary, and the refusal of
more than one GPU."""
import csv
import json
import os

import pytest

import bench
from quantized_gemm_qoq_amd import workloads

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(d, counter, rows):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "1_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def _summary(tmp_path, monkeypatch, fetch_rows, write_rows):
    d1, d2 = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write_counters(d1, "FETCH_SIZE", fetch_rows)
    _write_counters(d2, "WRITE_SIZE", write_rows)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda wl, layer: str(out))
    wl = workloads.WORKLOADS["llama3_8b_qkv_decode"]
    args = bench.parse_args(["--workload", wl.name, "--pmc-summary", d1, d2])
    assert bench.pmc_summary(args, wl, wl.layers[0]) == 0
    return json.loads(out.read_text()), out


GEMM = "void qoq::(anonymous namespace)::k_gemm_lds<0, 128, 1>(signed char const*)"
REDUCE = "void qoq::(anonymous namespace)::k_splitk_reduce<0>(int const*)"
PC = "void qoq::(anonymous namespace)::k_gemm_stream<1, 2, 3, 1, 16>(signed char const*)"
QACT = "void qoq::(anonymous namespace)::k_quantize_act_reg<256, 1>(unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"


def test_traffic_summary_calibration_and_split_k(tmp_path, monkeypatch):
    cal = bench.CALIBRATION_MIB * 1024.0
    # the copy reads half of what it moves by FETCH_SIZE's count (scale 2) and
    # writes all of it (scale 1); medians over three dispatches per kernel
    fetch = [(COPY, cal / 2)] * 3 + [(GEMM, 1000.0), (GEMM, 1000.0), (GEMM, 9999.0)] + \
        [(REDUCE, 300.0)] * 3 + [(PC, 700.0)] * 3 + [(QACT, 10.0)] * 3 + [("other_kernel", 5.0)]
    write = [(COPY, cal)] * 3 + [(GEMM, 200.0)] * 3 + [(REDUCE, 50.0)] * 3 + [(PC, 40.0)] * 3 + \
        [(QACT, 20.0)] * 3
    d, _ = _summary(tmp_path, monkeypatch, fetch, write)
    assert d["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert d["calibration"]["write_scale"] == pytest.approx(1.0)
    assert d["source_hash"] == bench.kernel_source_hash()
    k = d["kernels"]
    assert set(k) == {"w4a8_gemm_g128", "w4a8_gemm_per_channel", "quantize_act"}
    g = k["w4a8_gemm_g128"]  # the median ignores the outlier; the reduction launch is added
    assert g["hbm_read_bytes"] == round((1000 + 300) * 1024 * 2.0)
    assert g["hbm_write_bytes"] == round((200 + 50) * 1024 * 1.0)
    assert g["hbm_bytes"] == g["hbm_read_bytes"] + g["hbm_write_bytes"]
    assert g["reduce_FETCH_SIZE_KiB"] == 300.0
    pc = k["w4a8_gemm_per_channel"]
    assert pc["hbm_bytes"] == round(700 * 1024 * 2.0) + round(40 * 1024 * 1.0)
    assert "reduce_FETCH_SIZE_KiB" not in pc


def test_stored_traffic_only_while_sources_match(tmp_path, monkeypatch):
    fetch = [(COPY, 1000.0)] + [(PC, 10.0)]
    write = [(COPY, 2000.0)] + [(PC, 1.0)]
    d, out = _summary(tmp_path, monkeypatch, fetch, write)
    want = d["kernels"]["w4a8_gemm_per_channel"]["hbm_bytes"]
    assert bench.stored_traffic("any", "any", "w4a8_gemm_per_channel") == want
    assert bench.stored_traffic("any", "any", "w4a8_gemm_g128") is None
    d["source_hash"] = "0" * 16  # taken on other kernel sources
    out.write_text(json.dumps(d))
    assert bench.stored_traffic("any", "any", "w4a8_gemm_per_channel") is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_counter_summary_table(tmp_path, monkeypatch):
    """Medians per kernel and counter over the dispatches, one pass per
    directory, in a markdown table under profiles/ (redirected here)."""
    d1, d2 = str(tmp_path / "a"), str(tmp_path / "b")
    _write_counters(d1, "SQ_WAVES", [(PC, 4096.0), (PC, 4096.0), (QACT, 256.0), (COPY, 1.0)])
    _write_counters(d2, "TCC_HIT_sum", [(PC, 10.0), (PC, 30.0), (PC, 20.0), (GEMM, 7.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    wl = workloads.WORKLOADS["llama3_8b_qkv_decode"]
    args = bench.parse_args(["--workload", wl.name, "--counter-summary", d1, d2])
    assert bench.counter_summary(args, wl, wl.layers[0]) == 0
    text = (tmp_path / "profiles" / f"counters_{wl.name}_{wl.layers[0].name}.md").read_text()
    rows = {l.split("|")[1].strip(): [c.strip() for c in l.split("|")[2:-1]]
            for l in text.splitlines() if l.startswith("| SQ_") or l.startswith("| TCC_")}
    head = [l for l in text.splitlines() if l.startswith("| counter")][0]
    cols = [c.strip().strip("`") for c in head.split("|")[2:-1]]
    assert "__amd_rocclr_copyBuffer" not in cols and len(cols) == 3
    pc = cols.index("k_gemm_stream<1, 2, 3, 1, 16>")
    assert rows["SQ_WAVES"][pc] == "4096" and rows["TCC_HIT_sum"][pc] == "20"
    assert rows["SQ_WAVES"][cols.index("k_gemm_lds<0, 128, 1>")] == ""
    assert "--pmc SQ_WAVES" in text and "--pmc TCC_HIT_sum" in text


def test_fit_line_recovers_fixed_cost_and_slope():
    """The K sweep's line fit: exact on points of a line, least squares
    (mean residual zero) on noisy ones, and an error without two distinct K."""
    ks = [128, 256, 512, 1024, 2048, 4096]
    a, b = bench.fit_line(ks, [4.0 + 0.001 * k for k in ks])
    assert abs(a - 4.0) < 1e-12 and abs(b - 0.001) < 1e-15
    ys = [4.0 + 0.001 * k + (0.05 if i % 2 else -0.05) for i, k in enumerate(ks)]
    a, b = bench.fit_line(ks, ys)
    assert abs(sum(y - (a + b * k) for k, y in zip(ks, ys))) < 1e-9
    for bad in ([1], [512, 512]):
        with pytest.raises(ValueError):
            bench.fit_line(bad, [1.0] * len(bad))

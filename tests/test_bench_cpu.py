"""Host-side logic of bench.py that needs no GPU: the algorithmic byte
counts behind the HBM roofline, the comment-blind source digest that keys
the traffic records, the counter-to-bytes calibration of a traffic record
and its invalidation, and the one-GPU guard."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_algorithmic_bytes():
    w = workloads.BY_NAME["skinny_64x28672x8192"]
    assert bench.algorithmic_bytes(w, "f16") == 2 * (64 * 8192 + 28672 * 8192 + 64 * 28672)
    assert bench.algorithmic_bytes(w, "bf16") == bench.algorithmic_bytes(w, "f16")
    # one byte per operand element, one scale byte per 32 K elements of each row
    assert bench.algorithmic_bytes(w, "mxf8") == (64 * 8192 + 28672 * 8192) + 2 * 64 * 28672 + \
        (64 + 28672) * 8192 // 32
    lin = workloads.BY_NAME["linear_8192x14336x4096"]
    assert bench.algorithmic_bytes(lin, "f16") == 419_430_400


def test_code_text_ignores_comments_and_layout_only():
    src = 'int a = 1; // note\n/* block\n comment */  const char *s = "x//y /* z */";\n\n  f(a);\n'
    assert bench._code_text(src) == 'int a = 1;\nconst char *s = "x//y /* z */";\nf(a);'
    assert bench._code_text(src.replace("// note", "// other note")) == bench._code_text(src)
    assert bench._code_text(src.replace("int a = 1;", "int a = 2;")) != bench._code_text(src)
    assert bench._code_text("char c = '/'; // x") == "char c = '/';"


def _counter_csv(path, kernel, counter, values):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, v in enumerate(values):
            # counters summed over blocks per dispatch: split each value in two rows
            for part in (0.25, 0.75):
                wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter,
                             "Counter_Value": v * part})


def test_traffic_record_calibration_and_invalidation(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "digest-a")
    files = [tmp_path / n for n in ("gf.csv", "gw.csv", "cf.csv", "cw.csv")]
    _counter_csv(files[0], "gemm_f16_x", "FETCH_SIZE", [1000.0, 1200.0])  # mean 1100 units
    _counter_csv(files[1], "gemm_f16_x", "WRITE_SIZE", [300.0, 300.0])
    _counter_csv(files[2], "copyBuffer", "FETCH_SIZE", [512.0])  # 1 MiB copy: 2048 B/unit
    _counter_csv(files[3], "copyBuffer", "WRITE_SIZE", [1024.0])  # 1024 B/unit
    args = type("A", (), {})()
    args.traffic_record = [str(p) for p in files]
    args.copy_bytes = 1 << 20
    args.traffic_kernel, args.workload = "gemm_f16_x", "w"
    assert bench.traffic_record(args) == 0
    rec = json.load(open(tmp_path / "gemm_f16_x__w__traffic.json"))
    assert rec["bytes_per_fetch_unit"] == 2048.0 and rec["bytes_per_write_unit"] == 1024.0
    assert rec["hbm_bytes_per_launch"] == 1100.0 * 2048 + 300.0 * 1024
    assert bench.measured_traffic("gemm_f16_x", "w") == rec["hbm_bytes_per_launch"]
    # the kernel sources changed since the counters were taken: no figure
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "digest-b")
    assert bench.measured_traffic("gemm_f16_x", "w") is None
    assert bench.measured_traffic("gemm_f16_y", "w") is None


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err



def test_trace_summary_orders_dispatches_and_averages_the_timed_window(tmp_path):
    """The per-call series comes out in start order (not file order) and the
    window mean covers exactly the timed calls [warmup, warmup + steps)."""
    p = tmp_path / "kernel_trace.csv"
    starts = [500, 100, 300, 700, 900]
    durs_ns = [5000, 1000, 3000, 7000, 9000]  # by start order: 1, 3, 5, 7, 9 us
    with open(p, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        for s0, d in zip(starts, durs_ns):
            wr.writerow({"Kernel_Name": "gemm_x", "Start_Timestamp": s0, "End_Timestamp": s0 + d})
        wr.writerow({"Kernel_Name": "copyBuffer", "Start_Timestamp": 50, "End_Timestamp": 99999})
    t = bench.trace_summary(str(p), "gemm_", (1, 4))
    assert t["per_call_us"] == [1.0, 3.0, 5.0, 7.0, 9.0]
    assert t["calls"] == 5 and t["window_mean_us"] == 5.0 and t["mean_us"] == 5.0


def test_processes_only_for_the_single_line(capsys, monkeypatch):
    """--processes runs the one benchmark line in independent processes; it is
    refused with --all and the measurement-only modes (before any process or
    device is started)."""
    for extra in (["--all"], ["--mfma-ceiling"], ["--hbm-ceiling"]):
        monkeypatch.setattr(sys, "argv", ["bench.py", "--processes", "3", *extra])
        assert bench.main() == 2
        assert "single benchmark line" in capsys.readouterr().err

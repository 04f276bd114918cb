"""Host checks of the HBM-traffic summary used for bench.py's roofline.traffic:
copy calibration, per-kernel averages, and the source-hash guard."""
import csv
import json

from muon_adamw_amd import counters

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": 256, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_summary_calibrates_on_the_copy(tmp_path):
    copy = "void at::native::elementwise_kernel<copy>(...)"
    apply = "void ma::(anonymous namespace)::ns_mfma_kernel<2>(ma::(anonymous namespace)::NsArgs)"
    # the copy of 1 GiB reads as half its bytes in FETCH_SIZE and exactly in WRITE_SIZE
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 524288.0), (copy, 12.0), (apply, 1000.0), (apply, 1200.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1048576.0), (apply, 300.0), (apply, 300.0)])
    s = counters.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl", "cmd")
    assert abs(s["fetch_factor"] - 2.0) < 1e-3 and abs(s["write_factor"] - 1.0) < 1e-3
    k = s["kernels"]["ns_apply_bf16"]
    assert k["dispatches"] == 2 and k["fetch_kib"] == 1100.0 and k["write_kib"] == 300.0
    assert k["hbm_bytes_per_launch"] == round((1100.0 * 2.0 + 300.0) * 1024)


def test_traffic_only_while_sources_match(tmp_path):
    p = tmp_path / "c.json"
    body = {"source_sha256": counters.source_hash(),
            "kernels": {"ns_apply_bf16": {"hbm_bytes_per_launch": 123}}}
    p.write_text(json.dumps(body))
    assert counters.traffic_for(str(p), "ns_apply_bf16") == 123
    assert counters.traffic_for(str(p), "momentum") is None
    body["source_sha256"] = "0" * 64
    p.write_text(json.dumps(body))
    assert counters.traffic_for(str(p), "ns_apply_bf16") is None
    assert counters.traffic_for(str(tmp_path / "missing.json"), "ns_apply_bf16") is None

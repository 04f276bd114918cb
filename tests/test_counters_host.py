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


def test_mfma_pass_calibrates_on_the_ceiling_loop(tmp_path):
    """The MFMA-op counter is scaled by the ceiling loop's known flops (the
    full-length launch; the short warm-up launch is left out), and each
    library kernel gets its executed flops per launch."""
    copy = "void at::native::elementwise_kernel<copy>(...)"
    ceil = "ma::(anonymous namespace)::mfma_ceiling_kernel(float*, int)"
    ns = "ma::(anonymous namespace)::ns_persistent_kernel(ma::MatDesc const*, ma::NsQueue)"
    mom = "void ma::(anonymous namespace)::momentum_kernel<unsigned short>(...)"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 524288.0), (ns, 2000.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1048576.0), (ns, 500.0)])
    # counted in units of 512 flops, say: the ceiling's 1000-round launch reads
    # CEILING_FLOPS / 512, its 100-round warm-up a tenth of that
    unit = 512.0
    full = counters.CEILING_FLOPS / unit
    _csv(tmp_path / "m.csv", counters.MFMA_COUNTER,
         [(ceil, full / 10), (ceil, full), (ns, 2.0e9 / unit), (ns, 2.2e9 / unit), (mom, 0.0)])
    s = counters.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl", "cmd", str(tmp_path / "m.csv"))
    assert abs(s["mfma_factor"] - unit) < 1e-6 and s["mfma_counter"] == counters.MFMA_COUNTER
    assert s["kernels"]["ns_persistent_bf16"]["mfma_flops_per_launch"] == round(2.1e9)
    assert s["kernels"]["momentum"] == {"dispatches": 1, "mfma_flops_per_launch": 0}
    assert counters.CEILING_FLOPS == 1024 * 4 * 1000 * 8 * 32768
    p = tmp_path / "c.json"
    p.write_text(json.dumps(s))
    assert counters.flops_for(str(p), "ns_persistent_bf16") == round(2.1e9)
    assert counters.traffic_for(str(p), "momentum") is None      # an entry without the byte passes
    s["source_sha256"] = "0" * 64
    p.write_text(json.dumps(s))
    assert counters.flops_for(str(p), "ns_persistent_bf16") is None

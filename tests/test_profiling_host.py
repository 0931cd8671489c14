"""Host checks of the rocprofv3 summary tools (ssm_layer_decode_amd.profiling):
the counter scaling against the copy probe, the kernel-stats table and one
table per bench suite, on small synthetic inputs with known answers."""
import csv
import json

from ssm_layer_decode_amd import profiling


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_scales_by_the_copy_probe(tmp_path):
    copy = 1 << 30
    # the probe copies 1 GiB: FETCH reads half of it (x2 factor), WRITE all of it (x1)
    _counters(tmp_path / "f.csv", "FETCH_SIZE", [("probe_copy_kernel(...)", copy / 2048),
                                                 ("rssm_decode_kernel<...>", 1000.0),
                                                 ("rssm_decode_kernel<...>", 3000.0)])
    _counters(tmp_path / "w.csv", "WRITE_SIZE", [("probe_copy_kernel(...)", copy / 1024),
                                                 ("rssm_decode_kernel<...>", 100.0),
                                                 ("rssm_decode_kernel<...>", 300.0)])
    d = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "rssm_decode_kernel", copy,
                          sha="abc", algorithmic=4200.0 * 1024)
    assert abs(d["fetch_scale"] - 2.0) < 1e-12 and abs(d["write_scale"] - 1.0) < 1e-12
    assert abs(d["hbm_bytes_per_launch"] - (2000.0 * 2 + 200.0) * 1024) < 1e-6
    assert abs(d["traffic_over_algorithmic"] - 1.0) < 1e-12
    assert d["kernel_src_sha"] == "abc"


def test_stats_table(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "rssm_decode_kernel", "Calls": 3, "AverageNs": 225000, "MinNs": 200000,
                    "MaxNs": 450000, "Percentage": 45.5})
    t = profiling.stats_table(str(p))
    assert "| rssm_decode_kernel | 3 | 225.0 | 200.0 | 450.0 | 45.5% |" in t


def test_every_suite_renders(tmp_path):
    rows = [
        {"suite": "decode", "case": "gdn", "workload": "w", "tokens_per_s": 1e6, "GBps": 6000.0, "us_per_step": 200.0,
         "conventional_tokens_per_s": 5e5, "conventional_GBps": 5000.0, "speedup": 2.0},
        {"suite": "window", "L": 16, "tokens_per_s": 1e6, "GBps": 6000.0, "us_per_step": 225.0},
        {"suite": "batch", "B": 1, "layers_rotated": 256, "tokens_per_s": 8e4, "GBps": 430.0, "us_per_layer_step": 12.7,
         "conventional_us_per_layer_step": 14.0, "speedup": 1.1},
        {"suite": "spec", "T": 4, "replay_us_per_round": 675.0, "snapshot_us_per_round": 2146.0, "speedup": 3.18,
         "replay_verify_over_conv_decode_step": 0.76, "snapshot_round_over_conv_decode_step": 2.77,
         "replay_verified_tokens_per_s": 3e6, "snapshot_verified_tokens_per_s": 9.5e5, "conv_decode_step_us": 775.0,
         "replay_decode_step_us": 475.0},
        {"suite": "read_copy", "case": "mamba2", "read_copy": "fp8", "ckpt": "f32", "layers_rotated": 1,
         "tokens_per_s": 2e6, "GBps": 5300.0, "us_per_layer_step": 126.0},
        {"suite": "spec_copies", "ckpt": "f32", "read_copy": "fp8", "T": 8, "heads_per_tile": 1, "us_per_round": 783.0,
         "verify_only_us": 553.0, "verified_tokens_per_s": 5.2e6},
        {"suite": "verify_h7", "T": 4, "verify_us": 527.5, "algorithmic_bytes_per_launch": 3.1e9, "GBps": 5890.0},
        {"suite": "graph", "B": 1, "layers": 64, "eager_us_per_layer_step": 9.8, "graph_us_per_layer_step": 5.9},
        {"suite": "prefill", "case": "mamba2", "T": 512, "kernel": "rssm_prefill_mfma_kernel", "prefill_ms": 7.8,
         "prefill_tokens_per_s": 1.7e7, "decode_tokens_per_s": 1.1e6, "speedup_vs_decode": 15.0,
         "algorithmic_GBps": 3600.0, "TFLOPs": 77.0, "TFLOPs_peak": 157.3, "peak_of": "fp32 MFMA"},
    ]
    p = tmp_path / "suite.jsonl"
    p.write_text("\n".join(json.dumps(r) for r in rows) + "\n")
    md = profiling.suite_markdown(str(p))
    for title in ("## Decode at other shapes", "## Window sweep", "## Batch sweep", "## Speculative verify + commit, Mamba-2",
                  "## Read copies", "reading a copy or an fp16 checkpoint", "## Verify alone", "## Small batches",
                  "## Prefill"):
        assert title in md, title
    assert "| 1 | 64 | 9.8 | 5.9 |" in md
    assert "| 4 | 527.5 | 3.100 | 5890 |" in md


def test_counter_summary_splits_flush_dispatches(tmp_path):
    """Dispatch i of a layer that starts empty is at window position i mod L;
    position L - 1 is the flush step."""
    p = tmp_path / "c.csv"
    L = 4
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "VGPR_Count", "LDS_Block_Size"])
        w.writeheader()
        for i in range(12):                       # ids out of order on purpose
            did = 100 + (11 - i)
            pos = (11 - i) % L
            w.writerow({"Dispatch_Id": did, "Kernel_Name": "rssm_decode_kernel<128>", "Counter_Name": "SQ_WAVES",
                        "Counter_Value": 10.0 if pos == L - 1 else 1.0 + pos, "VGPR_Count": 64, "LDS_Block_Size": 8192})
            w.writerow({"Dispatch_Id": 500 + i, "Kernel_Name": "other", "Counter_Name": "SQ_WAVES",
                        "Counter_Value": 999.0, "VGPR_Count": 8, "LDS_Block_Size": 0})
    c, res = profiling.counter_summary([str(p)], "rssm_decode_kernel", L)
    assert c["SQ_WAVES"] == (2.0, 10.0)
    assert res["VGPR_Count"] == "64" and res["LDS_Block_Size"] == "8192"
    assert "| SQ_WAVES | 2 | 10 |" in profiling.counter_table([str(p)], "rssm_decode_kernel", L)

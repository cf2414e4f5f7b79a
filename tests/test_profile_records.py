"""The committed counter summaries that bench.py attaches to its line: the
fields it reads are there and well formed (CPU only; no GPU, no oracle)."""
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load(name):
    with open(os.path.join(ROOT, "profiles", name)) as f:
        return json.load(f)


def test_quantize_counter_record():
    rec = load("quantize_counters_llama8b.json")
    assert len(rec["quantize_source_sha256"]) == 64
    calls = rec["calls"]
    assert calls
    for name, c in calls.items():
        assert c["bound"] in ("valu", "hbm"), name
        # the bound follows the stated rule on the recorded busy fraction
        assert (c["bound"] == "valu") == (c["valu_busy_frac"] >= 0.70), name
        assert c["duration_us_under_counters"] > 0, name
        assert c["hbm_read_bytes"] >= 0 and c["hbm_write_bytes"] >= 0, name
        assert c["kernels"], name


def test_gemm_traffic_record():
    rec = load("gemm_traffic_llama8b.json")
    assert len(rec["gemm_source_sha256"]) == 64
    assert rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] > 0
    assert rec["launch_order"] == ["fprop_gu", "fprop_down", "dgrad_down", "wgrad_down",
                                   "dgrad_gu", "wgrad_gu"]


def test_bench_reads_records():
    import sys
    sys.path.insert(0, ROOT)
    import bench
    c = bench.quantize_counters()
    if c is not None:  # None only when the record is for another quantize source
        for v in c.values():
            assert v.get("bound") in ("valu", "hbm")

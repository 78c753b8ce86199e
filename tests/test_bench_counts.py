"""The benchmark's useful-work and byte counts (closed forms in bench.py) agree with a count
taken directly from the mask."""
import numpy as np
import pytest

import bench
import oracle
import workloads as wl


@pytest.mark.parametrize("Lq,Lk,causal,W", [(64, 64, False, 0), (64, 64, True, 0), (50, 80, True, 0),
                                            (80, 50, True, 0), (100, 100, True, 10), (100, 100, True, 150),
                                            (70, 120, True, 33)])
def test_visible_pairs_match_the_mask(Lq, Lk, causal, W):
    assert bench.visible_pairs(Lq, Lk, causal, W) == int(oracle.visibility(Lq, Lk, causal, W).sum())


def test_named_workload_counts():
    c3 = wl.PREFILL["gqa_causal_bf16_L4096"]
    assert bench.prefill_flops(c3) == 4 * 128 * 2 * 32 * (4096 * 4097 // 2)
    c4 = wl.PREFILL["swa_gqa_bf16_L16384_W4096"]
    W, L = 4096, 16384
    assert bench.prefill_flops(c4) == 4 * 128 * 32 * (W * (W + 1) // 2 + (L - W) * W)
    c2 = wl.PREFILL["mha_bf16_L1024"]
    assert bench.prefill_flops(c2) == 4 * 64 * 4 * 16 * 1024 * 1024
    assert bench.prefill_bytes(c3) == (2 * 2 * 32 * 4096 * 128 + 2 * 2 * 8 * 4096 * 128) * 2 + 4 * 2 * 32 * 4096
    # decode: one read of each live K and V row per KV head
    assert bench.decode_bytes(1000, 4, 32, 8, 128) == 2 * 1000 * 8 * 128 * 2 + 2 * 4 * 32 * 128 * 2 + 4 * 4 * 32 + 48


def test_gpus_above_one_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_mfma_counter_summary(tmp_path):
    """GRBM_GUI_ACTIVE arrives summed over the 8 XCDs and SQ_VALU_MFMA_BUSY_CYCLES over the 1024
    SIMDs; the summary divides both back and averages over dispatches."""
    import csv
    path = tmp_path / "run_counter_collection.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    # two dispatches of 100 us: 180k and 200k cycles per XCD, matrix core busy 90k / 120k per SIMD
    for disp, cyc, busy, t0 in ((1, 180_000, 90_000, 0), (2, 200_000, 120_000, 1_000_000)):
        for name, val in (("GRBM_GUI_ACTIVE", cyc * 8), ("SQ_VALU_MFMA_BUSY_CYCLES", busy * 1024)):
            rows.append({"Dispatch_Id": disp, "Kernel_Name": "k", "Counter_Name": name, "Counter_Value": val,
                         "Start_Timestamp": t0, "End_Timestamp": t0 + 100_000})
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        w.writerows(rows)
    m = bench._mfma_counters(str(path))["k"]
    assert m["dispatches"] == 2
    assert m["mfma_busy_frac"] == round(105_000 / 190_000, 4)
    assert m["engine_clock_ghz"] == round(190_000 / 100_000, 3)
    assert m["mean_us"] == 100.0

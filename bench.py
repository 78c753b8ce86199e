#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, in this order:
  * prefill: attn_fwd on the causal GQA workload (B=2, Hq=32, Hkv=8, L=4096, d=128, bf16, LSE),
  * prefill: attn_fwd on the sliding-window workload (B=1, Hq=32, Hkv=8, L=16384, W=4096, d=128),
  * decode: attn_decode on the GQA decode batch (64 sequences, Hq=32, Hkv=8, d=128, KV lengths
    uniform in [1024, 32768], one pooled K/V buffer with poisoned gaps),
  * decode: attn_decode on the MQA batch (same lengths, Hkv=1), rotated over pool replicas so
    that the 256 MB last-level cache cannot serve the 0.6 GB pool from one step to the next.
Inputs are generated on the device before timing.  The reported value is the causal GQA
prefill's useful TFLOP/s (4*d per visible (query, key) pair per query head); every part gets its
own roofline object.  Kernel times come from HIP events recorded on the stream the kernels run on,
around each part of each timed step.  After the timed steps the causal prefill is also timed back
to back (no other kernel between its calls) and reported beside the in-step figure.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --only PART    # one part of the step only (profiling)
  python bench.py --suite        # one JSON line per workload (the five, the backward of the dense
                                 # bf16 ones, both decode batches in a
                                 # paged cache, and a ragged chunked-prefill batch), for the tables
  python bench.py --mfma-ceiling # the matrix-core + LDS ceiling probe (include/attn_probe.h)
  python bench.py --gemm-reference  # a plain bf16 GEMM through the platform library, for reference
  python bench.py --copy-calib   # a plain device copy of known size, to scale HBM counters
  python bench.py --summarize-counters FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [MFMA_DIR]
                                 # rocprofv3 --pmc outputs -> per-launch HBM bytes (profiles/hbm_traffic.md)

The roofline "traffic" fields come from profiles/hbm_traffic.md (FETCH_SIZE / WRITE_SIZE counter
runs of this same command, scaled by what the counters read for a plain copy of known size); they
are reported only while the kernel sources still hash to what was profiled, and are null otherwise.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk/CU)
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA: twice the bf16 rate
# The FP8-input prefill runs S = Q K^T on the FP8 matrix cores and P V on the bf16 ones, half the
# useful FLOPs each: its roofline peak is 1 / (0.5 / 5033.2 + 0.5 / 2516.6) TFLOP/s.
PEAK_FP8_BF16_MIX_TFLOPS = round(1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS), 1)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# ---- work and byte counts (closed forms) ------------------------------------------------------

def visible_pairs(Lq: int, Lk: int, causal: bool, window: int) -> int:
    """Visible (query, key) pairs of one head: Lq*Lk without a mask; with causal masking (query
    i at position i + Lk - Lq) each row sees min(p+1, Lk) keys, at most W of them with a window."""
    total = 0
    if not causal:
        return Lq * Lk
    delta = Lk - Lq
    # rows whose position p = i + delta is < 0 see nothing
    for_rows = range(max(0, -delta), Lq)
    if window <= 0:
        # sum over p of min(p + 1, Lk)
        for i in for_rows:
            total += min(i + delta + 1, Lk)
        return total
    for i in for_rows:
        p = i + delta
        total += min(p, Lk - 1) - max(0, p - window + 1) + 1
    return total


def prefill_flops(c) -> int:
    return 4 * c.d * c.B * c.Hq * visible_pairs(c.Lq, c.Lk, c.causal, c.window)


def backward_flops(c) -> int:
    """Five products per visible pair and query head (S, dP, dV, dK, dQ), 2*d flops each: 2.5
    times the forward's; the recomputation of S and dP in the second kernel is not counted."""
    return 10 * c.d * c.B * c.Hq * visible_pairs(c.Lq, c.Lk, c.causal, c.window)


# FP8-input prefill lines of the suite: the two long workloads with FP8 Q, K, V.
FP8_PREFILL_WORKLOADS = ["gqa_causal_bf16_L4096", "swa_gqa_bf16_L16384_W4096"]

# Backward (training) lines of the suite: the dense bf16 workloads.
BWD_WORKLOADS = ["mha_bf16_L1024", "gqa_causal_bf16_L4096", "swa_gqa_bf16_L16384_W4096"]


def prefill_bytes(c) -> int:
    esz = 4 if c.dtype == "f32" else 2
    return (2 * c.B * c.Hq * c.Lq * c.d + 2 * c.B * c.Hkv * c.Lk * c.d) * esz + 4 * c.B * c.Hq * c.Lq


def decode_bytes(n_tokens: int, n_seq: int, Hq: int, Hkv: int, d: int, kv_bytes: int = 2) -> int:
    """One read of every live K and V row (kv_bytes per element: 2 for bf16, 1 for an FP8 cache),
    one read of q, one write of O (bf16) and LSE (fp32), plus offsets and lens."""
    return 2 * n_tokens * Hkv * d * kv_bytes + 2 * n_seq * Hq * d * 2 + 4 * n_seq * Hq + 12 * n_seq


def decode_flops(n_tokens: int, Hq: int, Hkv: int, d: int) -> int:
    return 4 * d * n_tokens * Hq


# ---- HBM traffic from counter runs -------------------------------------------------------------

KERNEL_SOURCES = ["attn_device.hpp", "fp8_device.hpp", "kernels.hpp", "plan.hpp", "prefill.hip", "decode.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_attn_fwd_03_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _counter_means(path: str) -> dict:
    """rocprofv3 --pmc CSV -> {kernel name: mean counter value per dispatch}."""
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


N_XCD, N_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def _mfma_counters(path: str) -> dict:
    """rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES CSV -> per kernel: the fraction of
    SIMD cycles the matrix core was busy, and the engine clock over the dispatch.  GRBM_GUI_ACTIVE
    comes summed over the XCDs (each counts the kernel's cycles); SQ_VALU_MFMA_BUSY_CYCLES summed
    over every SIMD."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = per.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {}
    for name, ds in per.items():
        ds = [d for d in ds.values() if "GRBM_GUI_ACTIVE" in d and "SQ_VALU_MFMA_BUSY_CYCLES" in d]
        if not ds:
            continue
        cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / len(ds) / N_XCD
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / len(ds) / N_SIMD
        ns = sum(d["ns"] for d in ds) / len(ds)
        out[name] = {"dispatches": len(ds), "mfma_busy_frac": round(busy / cyc, 4),
                     "engine_clock_ghz": round(cyc / ns, 3), "mean_us": round(ns / 1e3, 1)}
    return out


def _per_counter_means(path: str) -> dict:
    """rocprofv3 --pmc CSV with several counters -> {kernel name: {counter: mean per dispatch}}."""
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, mfma_dir=None, mops_dir=None) -> dict:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the attention kernels, scaled to bytes with the
    factors a 1 GiB device copy (--copy-calib) gives for the same counters; with `mfma_dir`, also
    the matrix-core busy fraction and engine clock of each kernel; with `mops_dir`, the executed
    matrix-core work (SQ_INSTS_VALU_MFMA_MOPS_*, units of 512 FLOP) and LDS counters.  `parts`
    names each part of the step with its workload and kernels."""
    def load(d):
        return _counter_means(os.path.join(d, "run_counter_collection.csv"))
    fetch, write = load(fetch_dir), load(write_dir)
    cf, cw = load(copy_fetch_dir), load(copy_write_dir)
    copy_bytes = 1 << 30
    # true bytes per counted byte (the counters report KiB)
    f_scale = copy_bytes / (max(cf.values()) * 1024)
    w_scale = copy_bytes / (max(cw.values()) * 1024)
    out = {"kernel_source_sha": kernel_source_hash(), "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "kernels": {}}
    mfma = _mfma_counters(os.path.join(mfma_dir, "run_counter_collection.csv")) if mfma_dir else {}
    for name in sorted(set(fetch) | set(write)):
        if "attnfwd::" not in name:
            continue
        short = re.sub(r"^void attnfwd::|\(attnfwd::\w+\)$", "", name)
        fb, wb = fetch.get(name, 0.0) * 1024 * f_scale, write.get(name, 0.0) * 1024 * w_scale
        out["kernels"][short] = {"FETCH_SIZE_KiB": round(fetch.get(name, 0.0), 1),
                                 "WRITE_SIZE_KiB": round(write.get(name, 0.0), 1),
                                 "read_bytes": int(fb), "write_bytes": int(wb), "traffic_bytes": int(fb + wb)}
        if name in mfma:
            out["kernels"][short].update(mfma[name])
    if mops_dir:
        for name, cs in _per_counter_means(os.path.join(mops_dir, "run_counter_collection.csv")).items():
            short = re.sub(r"^void attnfwd::|\(attnfwd::\w+\)$", "", name)
            if short in out["kernels"]:
                out["kernels"][short].update({c: round(v, 1) for c, v in cs.items() if c != "GRBM_GUI_ACTIVE"})
    out["parts"] = {name: {"workload": w, "kernels": PART_KERNELS[name]} for name, _, w in STEP_PARTS}
    return out


def load_traffic() -> dict | None:
    """The committed counter summary, if it was taken on the kernel sources as they are now."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    return data if data.get("kernel_source_sha") == kernel_source_hash() else None


# ---- timing helpers ---------------------------------------------------------------------------

def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def cpu_baseline(c, q, k, v):
    """The oracle as it stands, on the host cores, over the whole prefill workload."""
    import numpy as np
    import oracle
    import workloads as wl
    qn, kn, vn = wl.to_f64(q), wl.to_f64(k), wl.to_f64(v)
    t0 = time.perf_counter()
    oracle.attention(qn, kn, vn, scale=c.scale, causal=c.causal, window=c.window)
    dt = time.perf_counter() - t0
    return {"value": prefill_flops(c) / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.host_cores(), "kind": "oracle",
            "sample": f"all of {c.name} (B={c.B}, Hq={c.Hq}, Hkv={c.Hkv}, L={c.Lq}, d={c.d}, causal), fp64 numpy, "
                      f"{dt:.1f} s wall", "seconds": dt}


# The parts of one step, in order: (name, kind, workload).
STEP_PARTS = [("prefill", "prefill", "gqa_causal_bf16_L4096"),
              ("prefill_window", "prefill", "swa_gqa_bf16_L16384_W4096"),
              ("decode", "decode", "gqa_decode_bf16"),
              ("decode_mqa", "decode", "mqa_decode_bf16")]
# Kernel names as rocprofv3 reports them, for the counter summary's traffic fields.  Template
# arguments: prefill (head size, key tile, ragged, mask mode); decode split (head size, paged, pool
# format, packed layout); decode merge (head size, packed layout, paged).
PART_KERNELS = {"prefill": ["fwd_bf16_kernel<128, 32, false, 1>"],
                "prefill_window": ["fwd_bf16_kernel<128, 32, false, 2>"],
                "decode": ["decode_split_kernel<128, false, 0, true>", "decode_merge_kernel<128, true, false>"],
                "decode_mqa": ["decode_split_kernel<128, false, 0, false>", "decode_merge_kernel<128, false, false>"]}
MQA_REPLICAS = 4  # 4 x 0.62 GB of MQA pools: well past the 256 MB last-level cache


PROBE_SOURCE_BYTES = 64 * (9216 + 10240)  # the probe's mode-4 source blocks (include/attn_probe.h)


def mfma_ceiling(args):
    """The ceiling probe in its five modes, each adding one part of the prefill kernel's work: the
    matrix instructions alone, with LDS operands, with the softmax's vector work, with the
    per-step wait and barrier, with the global->LDS loads of K and V; the last once more on
    operands drawn like the workloads' (the matrix cores' power depends on the operands' bits).
    768 workgroups (three per CU), timed over several launches of `steps` 32-key steps each, as
    TFLOP/s and as a fraction of the nominal bf16 peak."""
    import torch
    import attention_attn_fwd_03_amd as af
    wgs, steps = 768, 4096
    # Source blocks of the load mode first, as bf16 pairs of 0.01 (0x3C24), then the results.
    sink = torch.empty(PROBE_SOURCE_BYTES // 4 + wgs * 256, device="cuda", dtype=torch.float32)
    sink.view(torch.int32).fill_(0x3C243C24)
    what = {0: "MFMAs alone, operands in registers", 1: "MFMAs with K / V^T operands read from LDS",
            2: "MFMAs, LDS operands and the softmax's vector work (max, fma, exp2, add, bf16 pack)",
            3: "mode 2 plus the per-step wait and workgroup barrier",
            4: "mode 3 plus the per-step global->LDS loads of K and V (19 KB per workgroup, from L2); "
               "Q, K, V all 0.01",
            5: "mode 4 with Q, K, V drawn from N(0, 1) in bf16, as the prefill workloads"}
    for mode in (0, 1, 2, 3, 4, 5):
        if args.probe_mode is not None and mode != args.probe_mode:
            continue
        if mode == 5:  # the same kernel as mode 4, on random operands
            g = torch.Generator(device="cuda").manual_seed(7)
            n = PROBE_SOURCE_BYTES // 2
            sink[:PROBE_SOURCE_BYTES // 4].view(torch.bfloat16).copy_(
                torch.randn(n, device="cuda", generator=g).to(torch.bfloat16))
        mode, label = min(mode, 4), mode
        for _ in range(3):
            af.probe_mfma_ceiling(wgs, steps, sink, mode=mode)
        torch.cuda.synchronize()
        ev = _events(2)
        # --probe-seconds: launch for that long (to sample power or clocks meanwhile), about 4 ms each
        reps = max(10, int(args.probe_seconds * 250)) if args.probe_seconds else 10
        ev[0].record()
        for i in range(reps):
            af.probe_mfma_ceiling(wgs, steps, sink, mode=mode)
            if i % 250 == 249:
                torch.cuda.synchronize()  # keep the queue short so that the launches stay timed
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        flops = wgs * 4 * steps * 16 * 2 * 32 * 32 * 16
        tf = flops / (ms * 1e-3) / 1e12
        print(json.dumps({"probe": "mfma_ceiling", "mode": mode, "operands": "N(0,1)" if label == 5 else "constant",
                          "what": what[label], "workgroups": wgs,
                          "steps": steps, "ms_per_launch": round(ms, 4), "TFLOP/s": round(tf, 1),
                          "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "peak_TFLOP/s": PEAK_BF16_TFLOPS}),
              flush=True)


def gemm_reference(args):
    """A plain bf16 matrix product C = A B (8192 x 8192 x 8192, fp32 accumulation, bf16 result)
    through the platform's tuned GEMM library (torch.matmul), on operands drawn from N(0, 1) and on
    constant operands: what the matrix cores sustain on the dense product alone, the reference
    beside which the attention kernels' fraction of the nominal peak is read.  Not part of the
    attention path."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(11)
    cases = {"N(0,1)": (torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16),
                        torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)),
             "constant": (torch.full((n, n), 0.01, device="cuda", dtype=torch.bfloat16),
                          torch.full((n, n), 0.01, device="cuda", dtype=torch.bfloat16))}
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for label, (a, b) in cases.items():
        for _ in range(5):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        reps = max(50, int(args.probe_seconds / 1.2e-3)) if args.probe_seconds else 50  # about 1.1 ms per call
        ev = _events(2)
        ev[0].record()
        for i in range(reps):
            torch.matmul(a, b, out=c)
            if i % 500 == 499:
                torch.cuda.synchronize()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"reference": "bf16_gemm", "M": n, "N": n, "K": n, "operands": label,
                          "ms_per_call": round(ms, 4), "TFLOP/s": round(tf, 1),
                          "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "peak_TFLOP/s": PEAK_BF16_TFLOPS}),
              flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--mfma-ceiling", action="store_true")
    ap.add_argument("--gemm-reference", action="store_true")
    ap.add_argument("--probe-mode", type=int, default=None, help="with --mfma-ceiling: run only this mode (0-5)")
    ap.add_argument("--probe-seconds", type=float, default=0.0,
                    help="with --mfma-ceiling: keep each mode running about this long")
    ap.add_argument("--only", choices=[p[0] for p in STEP_PARTS], default=None,
                    help="profile helper: run only this part of the step")
    ap.add_argument("--workload", default=None, help="with --suite: run only this workload")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR", default=None,
                    help="rocprofv3 --pmc output dirs: FETCH_SIZE, WRITE_SIZE, both for --copy-calib, "
                         "optionally a GRBM_GUI_ACTIVE + SQ_VALU_MFMA_BUSY_CYCLES pass, then a "
                         "SQ_INSTS_VALU_MFMA_MOPS_* + LDS pass")
    args = ap.parse_args()

    if args.summarize_counters:
        if len(args.summarize_counters) not in (4, 5, 6):
            ap.error("--summarize-counters takes 4 to 6 directories")
        print(json.dumps(summarize_counters(*args.summarize_counters), indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the attention kernels here run on a single device and this "
              "build has no multi-GPU path (prefill shards by KV head with no communication; see the "
              "design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_attn_fwd_03_amd as af
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    af.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"

    if args.copy_calib:
        n = 1 << 30
        x = torch.empty(n, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n}), flush=True)
        return
    if args.mfma_ceiling:
        return mfma_ceiling(args)
    if args.gemm_reference:
        return gemm_reference(args)
    if args.suite:
        return run_suite(args)

    parts = [p for p in STEP_PARTS if args.only in (None, p[0])]
    run = {}    # part -> callable enqueuing it
    info = {}   # part -> config dict and work / bytes per call
    for name, kind, wname in parts:
        if kind == "prefill":
            c = wl.PREFILL[wname]
            q, k, v = wl.prefill_inputs_for(c, device=dev)
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], device=dev, dtype=torch.float32)
            run[name] = (lambda c=c, q=q, k=k, v=v, o=o, lse=lse:
                         af.attn_fwd(q, k, v, causal=c.causal, window=c.window, scale=c.scale, return_lse=True,
                                     out=o, lse_out=lse))
            fl = prefill_flops(c)
            info[name] = {"cfg": c, "work": fl, "inputs": (q, k, v),
                          "config": {"workload": wname, "B": c.B, "Hq": c.Hq, "Hkv": c.Hkv, "L": c.Lq, "d": c.d,
                                     "causal": c.causal, "window": c.window, "lse": True,
                                     "useful_gflop": round(fl / 1e9, 3)}}
        else:
            c = wl.DECODE[wname]
            lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
            max_len = int(lens.max())
            n_rep = MQA_REPLICAS if c.Hkv == 1 else 1
            reps = []
            for r in range(n_rep):
                qd, kp, vp, offs, lens_t, _ = wl.decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens,
                                                               seed=c.value_seed + 100 * r, device=dev,
                                                               max_gap=c.max_gap)
                reps.append((qd, kp, vp, offs, lens_t))
            od = torch.empty_like(reps[0][0])
            lsed = torch.empty((c.n_seq, c.Hq), device=dev, dtype=torch.float32)
            ws = torch.empty(af.decode_workspace_size(c.n_seq, c.Hq, c.Hkv, c.d, max_len), device=dev,
                             dtype=torch.uint8)
            it = [0]

            def call(c=c, reps=reps, it=it, od=od, lsed=lsed, ws=ws, max_len=max_len):
                qd, kp, vp, offs, lens_t = reps[it[0] % len(reps)]
                it[0] += 1
                af.attn_decode(qd, kp, vp, offs, lens_t, max_len=max_len, scale=c.scale, return_lse=True,
                               workspace=ws, out=od, lse_out=lsed)
            run[name] = call
            n_tok = int(lens.sum())
            by = decode_bytes(n_tok, c.n_seq, c.Hq, c.Hkv, c.d)
            info[name] = {"cfg": c, "work": by,
                          "config": {"workload": wname, "n_seq": c.n_seq, "Hq": c.Hq, "Hkv": c.Hkv, "d": c.d,
                                     "kv_tokens": n_tok, "max_len": max_len, "pool_replicas": n_rep,
                                     "algorithmic_gb": round(by / 1e9, 4)}}
    torch.cuda.synchronize()

    def step(ev=None):
        for i, (name, _, _) in enumerate(parts):
            if ev is not None:
                ev[i].record()
            run[name]()
        if ev is not None:
            ev[len(parts)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [_events(len(parts) + 1) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
        if (i + 1) % 10 == 0 or i + 1 == args.steps:
            print(f"# step {i + 1}/{args.steps} enqueued", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    for i, (name, _, _) in enumerate(parts):
        ms = [e[i].elapsed_time(e[i + 1]) for e in evs]
        info[name]["ms"] = sum(ms) / len(ms)
        info[name]["ms_min"] = min(ms)

    # The causal prefill back to back: `steps` calls with nothing in between, one event pair.
    if "prefill" in run:
        ev = _events(2)
        ev[0].record()
        for _ in range(args.steps):
            run["prefill"]()
        ev[1].record()
        torch.cuda.synchronize()
        info["prefill"]["back_to_back_ms"] = ev[0].elapsed_time(ev[1]) / args.steps

    def roofline(name):
        x = info[name]
        if x["cfg"].__class__.__name__ == "PrefillConfig":
            tf = x["work"] / (x["ms"] * 1e-3) / 1e12
            r = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": PART_KERNELS[name][0],
                 "workload": x["config"]["workload"], "kernel_ms": round(x["ms"], 4),
                 "kernel_ms_min": round(x["ms_min"], 4),
                 "per_launch": f"{x['work'] / 1e9:.1f} GFLOP useful (4*d per visible pair, all heads)"}
            if "back_to_back_ms" in x:
                b2b = x["work"] / (x["back_to_back_ms"] * 1e-3) / 1e12
                r["back_to_back"] = {"kernel_ms": round(x["back_to_back_ms"], 4), "achieved": round(b2b, 2),
                                     "frac": round(b2b / PEAK_BF16_TFLOPS, 4)}
            return r
        gbs = x["work"] / (x["ms"] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernels": " + ".join(PART_KERNELS[name]),
                "workload": x["config"]["workload"], "kernels_ms": round(x["ms"], 4),
                "kernels_ms_min": round(x["ms_min"], 4),
                "per_launch": f"{x['work'] / 1e9:.3f} GB (one read of live K/V rows + q, O, LSE)"}

    head = "prefill" if "prefill" in info else parts[0][0]
    main_roof = roofline(head)
    line = {
        "metric": "prefill attn TFLOP/s (% MFMA peak) + decode KV-read GB/s (% HBM peak), 1 GPU",
        "value": main_roof["achieved"],
        "unit": main_roof["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v (bf16), decode pools with seeded lengths and NaN gaps",
        "config": {"workload": " + ".join(info[n]["config"]["workload"] for n, _, _ in parts),
                   **{n: info[n]["config"] for n, _, _ in parts}, "parallelism": "single GPU"},
        "roofline": main_roof,
    }
    for n, _, _ in parts:
        if n != head:
            line["roofline_" + n] = roofline(n)
    traffic = load_traffic()
    if traffic is not None:
        for n, _, _ in parts:
            key = "roofline" if n == head else "roofline_" + n
            ks = [traffic["kernels"].get(k) for k in PART_KERNELS[n]]
            if all(ks):
                line[key]["traffic"] = sum(k["traffic_bytes"] for k in ks)
                for field in ("mfma_busy_frac", "engine_clock_ghz"):
                    if field in ks[0]:
                        line[key]["counters_" + field] = ks[0][field]
    if not args.no_cpu_baseline and "prefill" in info:
        print("# timing the oracle on the host", file=sys.stderr, flush=True)
        q, k, v = info["prefill"]["inputs"]
        cb = cpu_baseline(info["prefill"]["cfg"], q.cpu(), k.cpu(), v.cpu())
        line["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(line), flush=True)


PAGE_SIZE = 64  # tokens per page of the paged-cache suite lines
FP8_FORMATS = ("e4m3fn", "e5m2")  # FP8 suite lines (KV cache, prefill inputs)


def run_suite(args):
    """One JSON line per workload: median kernel time over timed calls, TFLOP/s or GB/s."""
    import torch
    import attention_attn_fwd_03_amd as af
    import workloads as wl
    dev = "cuda"
    reps, warm = max(args.steps, 10), max(args.warmup, 3)

    def timeit(fn):
        # Warm up for at least 0.2 s of wall time, not a fixed count: the engine clock takes some
        # milliseconds to settle after the host-side input generation, and a short kernel's first
        # few dozen calls would otherwise run at a clock the steady state does not have.
        t0, n = time.perf_counter(), 0
        while True:
            fn()
            n += 1
            if n >= warm and n % 4 == 0:
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= 0.2:
                    break
        ev = [_events(2) for _ in range(reps)]
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        ts = sorted(e[0].elapsed_time(e[1]) for e in ev)
        return ts[len(ts) // 2], ts[0]

    def wanted(name):
        return args.workload is None or args.workload == name

    for name, c in wl.PREFILL.items():
        if not wanted(name):
            continue
        q, k, v = wl.prefill_inputs_for(c, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], device=dev, dtype=torch.float32)
        med, mn = timeit(lambda: af.attn_fwd(q, k, v, causal=c.causal, window=c.window, scale=c.scale,
                                             return_lse=True, out=o, lse_out=lse))
        fl = prefill_flops(c)
        peak = PEAK_F32_MFMA_TFLOPS if c.dtype == "f32" else PEAK_BF16_TFLOPS
        tf = fl / (med * 1e-3) / 1e12
        print(json.dumps({"workload": name, "kind": "prefill", "dtype": c.dtype, "median_ms": round(med, 4),
                          "min_ms": round(mn, 4), "useful_gflop": round(fl / 1e9, 4), "TFLOP/s": round(tf, 2),
                          "frac_mfma_peak": round(tf / peak, 4), "peak_TFLOP/s": peak,
                          "GB/s_algorithmic": round(prefill_bytes(c) / (med * 1e-3) / 1e9, 1)}), flush=True)
        del q, k, v, o, lse
    for name in FP8_PREFILL_WORKLOADS:
        c = wl.PREFILL[name]
        for fmt in FP8_FORMATS:
            fname = name.replace("_bf16_", f"_fp8_{fmt}_")
            if not wanted(fname):
                continue
            qc, kc, vc, qs, ks, vs = wl.fp8_prefill_inputs(c.B, c.Hq, c.Hkv, c.Lq, c.Lk, c.d, fmt, seed=c.seed,
                                                           device=dev)
            o = torch.empty(qc.shape, device=dev, dtype=torch.bfloat16)
            lse = torch.empty(qc.shape[:3], device=dev, dtype=torch.float32)
            med, mn = timeit(lambda: af.attn_fwd_fp8(qc, kc, vc, qkv_format=fmt, q_scale=qs, k_scale=ks, v_scale=vs,
                                                     causal=c.causal, window=c.window, scale=c.scale,
                                                     return_lse=True, out=o, lse_out=lse))
            fl = prefill_flops(c)
            tf = fl / (med * 1e-3) / 1e12
            print(json.dumps({"workload": fname, "kind": "prefill", "dtype": f"fp8 {fmt} q/k/v, bf16 P",
                              "median_ms": round(med, 4), "min_ms": round(mn, 4), "useful_gflop": round(fl / 1e9, 4),
                              "TFLOP/s": round(tf, 2), "frac_mfma_peak": round(tf / PEAK_FP8_BF16_MIX_TFLOPS, 4),
                              "peak_TFLOP/s": PEAK_FP8_BF16_MIX_TFLOPS,
                              "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
            del qc, kc, vc, o, lse
    for name in BWD_WORKLOADS:
        c = wl.PREFILL[name]
        if not wanted(name + "_bwd"):
            continue
        q, k, v, do = wl.backward_inputs(c.B, c.Hq, c.Hkv, c.Lq, c.Lk, c.d, seed=c.seed, device=dev)
        o, lse = af.attn_fwd(q, k, v, causal=c.causal, window=c.window, scale=c.scale, return_lse=True)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(af.bwd_workspace_size(c.B, c.Hq, c.Lq), device=dev, dtype=torch.uint8)
        med, mn = timeit(lambda: af.attn_bwd(q, k, v, o, do, lse, causal=c.causal, window=c.window, scale=c.scale,
                                             workspace=ws, out=grads))
        fl = backward_flops(c)
        tf = fl / (med * 1e-3) / 1e12
        print(json.dumps({"workload": name + "_bwd", "kind": "backward", "dtype": "bf16", "median_ms": round(med, 4),
                          "min_ms": round(mn, 4), "useful_gflop": round(fl / 1e9, 4), "TFLOP/s": round(tf, 2),
                          "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "peak_TFLOP/s": PEAK_BF16_TFLOPS}),
              flush=True)
        del q, k, v, do, o, lse, grads, ws
    for name, c in wl.VARLEN.items():
        if not wanted(name):
            continue
        lq, lk = c.lengths()
        q, kp, vp, cu, offs, lens, layout = wl.varlen_inputs(lq, lk, c.Hq, c.Hkv, c.d, seed=c.seed, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], device=dev, dtype=torch.float32)
        med, mn = timeit(lambda: af.attn_fwd_varlen(q, kp, vp, cu, offs, lens, max_seqlen_q=int(lq.max()),
                                                    causal=c.causal, window=c.window, scale=c.scale,
                                                    return_lse=True, out=o, lse_out=lse))
        fl = sum(4 * c.d * c.Hq * visible_pairs(int(a), int(b), c.causal, c.window) for a, b in zip(lq, lk))
        tf = fl / (med * 1e-3) / 1e12
        print(json.dumps({"workload": name, "kind": "prefill_varlen", "dtype": "bf16", "median_ms": round(med, 4),
                          "min_ms": round(mn, 4), "sequences": c.n_seq, "new_tokens": int(lq.sum()),
                          "keys": int(lk.sum()), "useful_gflop": round(fl / 1e9, 4), "TFLOP/s": round(tf, 2),
                          "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "peak_TFLOP/s": PEAK_BF16_TFLOPS}),
              flush=True)
        del q, kp, vp, o, lse
    for name, c in wl.DECODE.items():
        paged_name = f"{name}_paged_P{PAGE_SIZE}"
        fp8_names = {fmt: name.replace("_bf16", "") + f"_fp8_{fmt}" for fmt in FP8_FORMATS}
        if not wanted(name) and not wanted(paged_name) and not any(wanted(n) for n in fp8_names.values()):
            continue
        lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
        max_len = int(lens.max())
        # Several replicas of the pool are rotated so that the 256 MB last-level cache cannot hold the
        # working set between calls.
        pool_bytes = 2 * (int(lens.sum()) + 256 * 65) * c.Hkv * c.d * 2
        n_rep = max(1, min(8, math.ceil(2.0e9 / pool_bytes)))
        reps_data = []
        for r in range(n_rep):
            qd, kp, vp, offs, lens_t, layout = wl.decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens,
                                                                seed=c.value_seed + 100 * r, device=dev,
                                                                max_gap=c.max_gap)
            reps_data.append((qd, kp, vp, offs, lens_t))
        od = torch.empty_like(reps_data[0][0])
        lsed = torch.empty((c.n_seq, c.Hq), device=dev, dtype=torch.float32)
        ws = torch.empty(af.decode_workspace_size(c.n_seq, c.Hq, c.Hkv, c.d, max_len), device=dev, dtype=torch.uint8)
        it = [0]

        def call():
            qd, kp, vp, offs, lens_t = reps_data[it[0] % n_rep]
            it[0] += 1
            af.attn_decode(qd, kp, vp, offs, lens_t, max_len=max_len, scale=c.scale, return_lse=True,
                           workspace=ws, out=od, lse_out=lsed)
        n_tok = int(lens.sum())
        by = decode_bytes(n_tok, c.n_seq, c.Hq, c.Hkv, c.d)

        def report(wname, med, mn, extra, by=by, dtype="bf16", reps=n_rep):
            gbs = by / (med * 1e-3) / 1e9
            print(json.dumps({"workload": wname, "kind": "decode", "dtype": dtype, "median_ms": round(med, 4),
                              "min_ms": round(mn, 4), "kv_tokens": n_tok, "pool_replicas": reps, **extra,
                              "algorithmic_gb": round(by / 1e9, 4), "GB/s": round(gbs, 1),
                              "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                              "useful_gflop": round(decode_flops(n_tok, c.Hq, c.Hkv, c.d) / 1e9, 3)}), flush=True)

        if wanted(name):
            med, mn = timeit(call)
            report(name, med, mn, {})
        del reps_data
        if wanted(paged_name):
            # The same batch in a paged cache: 64-token pages scattered over the pool in a seeded
            # order, 97 spare pages, unused rows NaN.
            paged = [wl.paged_decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens, PAGE_SIZE, seed=c.value_seed + 100 * r,
                                            device=dev, extra_pages=97)[:5] for r in range(n_rep)]

            def call_paged():
                qd, kp, vp, table, lens_t = paged[it[0] % n_rep]
                it[0] += 1
                af.attn_decode_paged(qd, kp, vp, table, lens_t, page_size=PAGE_SIZE, max_len=max_len, scale=c.scale,
                                     return_lse=True, workspace=ws, out=od, lse_out=lsed)
            med, mn = timeit(call_paged)
            report(paged_name, med, mn, {"page_size": PAGE_SIZE})
            del paged
        for fmt, fp8_name in fp8_names.items():
            if not wanted(fp8_name):
                continue
            # The same batch with an FP8 cache (per-pool scales); half the bytes, so more replicas.
            n_rep8 = max(1, min(16, math.ceil(2.0e9 / (pool_bytes / 2))))
            reps8 = [wl.fp8_decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens, fmt, seed=c.value_seed + 100 * r,
                                          device=dev, max_gap=c.max_gap) for r in range(n_rep8)]

            def call_fp8():
                qd, kc, vc, offs, lens_t, _, ks, vs = reps8[it[0] % n_rep8]
                it[0] += 1
                af.attn_decode(qd, kc, vc, offs, lens_t, max_len=max_len, scale=c.scale, return_lse=True,
                               workspace=ws, out=od, lse_out=lsed, kv_format=fmt, k_scale=ks, v_scale=vs)
            med, mn = timeit(call_fp8)
            by8 = decode_bytes(n_tok, c.n_seq, c.Hq, c.Hkv, c.d, kv_bytes=1)
            report(fp8_name, med, mn, {"kv_format": fmt}, by=by8, dtype=f"bf16 (kv {fmt})", reps=n_rep8)
            del reps8


if __name__ == "__main__":
    main()

"""Benchmark: absorbed MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv2] [--no-others]

A step is one pass of the path over one batch: absorb_q, rope_append,
decode_latent, then the split merge and W_UV as the one fused call
combine_up_v.  Inputs are seeded synthetic tensors already
resident in HBM; the timed loop rotates over several independent input sets
(each with its own cache and weights, like successive layers) so that the
256 MB Infinity Cache cannot hold the cache and weights; the per-step
temporaries share one workspace.  The timed steps replay a HIP graph that
holds one step of every set in turn (as the layers of one decode step);
back-to-back decode launches between HIP events give that kernel's
duration.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 * 2 ** 20
COUNTERS = os.path.join(ROOT, "profiles", "decode_latent_counters.json")
# the bf16 decode kernel's sources (counter-derived traffic is reported only
# while they are unchanged)
SOURCES = [os.path.join(ROOT, "head_latent_attention_12_amd", "csrc", f)
           for f in ("mla.hip", "mla_common.h", "decode_asm.inc")]


def workload_label(inp) -> str:
    lens = "ragged U[512,8192]" if inp.name == "dsv2_ragged" else f"T={int(inp.lens[0])}"
    return (f"MLA decode {inp.dtype} B={inp.B} H={inp.H} d_head={inp.d_head} d_v={inp.d_v} "
            f"r={inp.r} d_rope={inp.d_rope} {lens}")


def algorithmic(inp, fp8=False):
    """Algorithmic bytes and flops of the step and of the decode kernel alone.

    Bytes: every attended cache row read once, the appended row written once,
    W_UK and W_UV read once, q_nope/q_rope/new-token inputs read once, out
    written once.  Split partials, q_lat round trips and re-reads are
    implementation overhead and are not counted.
    """
    s = 2 if inp.dtype == "bf16" else 4
    rows = int(inp.seq_lens.sum())
    B, H, dh, dv, r, dr, W = inp.B, inp.H, inp.d_head, inp.d_v, inp.r, inp.d_rope, inp.W
    rb = r + 2 * dr + 4 if fp8 else W * s             # bytes per cache row (fp8: codes, bf16 RoPE, scale)
    step_bytes = (rows * rb + B * rb                  # cache read + new row written
                  + 2 * H * dh * r * s                # W_UK, W_UV (d_v = d_head here)
                  + B * H * (dh + dr) * s + B * (r + dr) * s  # q_nope, q_rope, c_kv_new, k_rope_new
                  + B * H * dv * 4)                   # out (fp32)
    step_flops = 2 * H * (W + r) * rows + 2 * B * H * dh * r + 2 * B * H * dv * r
    k3_bytes = rows * rb + B * H * W * s               # cache rows + q_lat
    k3_flops = 2 * H * (W + r) * rows
    return rows, step_bytes, step_flops, k3_bytes, k3_flops


def source_hash() -> str:
    h = hashlib.sha256()
    for f in SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    try:
        rec = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    e = rec.get(workload)
    if not e or e.get("source_sha") != source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


CALIB_BYTES = 512 * 2 ** 20     # calibration kernel: reads and writes this many bytes (above the 256 MB MALL)
CALIB_KERNEL = "neg_kernel"     # torch.neg on float32: one read and one write per element


def counters_run(workload: str, steps: int, warmup: int) -> None:
    """The workload's timed steps (also over an fp8 cache for the bf16
    DeepSeek-V2 shapes), then the calibration kernel 4 times: the program
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE profiles."""
    import torch
    run_workload(workload, steps, warmup, min_sets=5, verbose=True)
    if workload.startswith("dsv2"):  # the same steps over an fp8 cache (its decode kernel's counters)
        run_workload(workload, steps, warmup, min_sets=5, verbose=True, fp8=True)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"# counters run done: {workload}, {steps} steps; calibration {CALIB_KERNEL} x4 of {CALIB_BYTES} bytes",
          file=sys.stderr, flush=True)


def _per_dispatch(run_dir: str, counter: str):
    """{kernel name: [value per dispatch]} from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            key = (row["Kernel_Name"], row.get("Dispatch_Id") or row.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def ingest_counters(workload: str, fetch_dir: str, write_dir: str, command: str) -> dict:
    """Per-launch HBM bytes of the decode kernel from FETCH_SIZE and WRITE_SIZE
    runs (KiB per dispatch), each scaled by what the same counter reads for the
    calibration kernel of known size; written to profiles/decode_latent_counters.json."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _per_dispatch(d, counter)
        dec = [v for n, vs in per.items() if "decode_latent_kernel" in n for v in vs]
        cal = [v for n, vs in per.items() if CALIB_KERNEL in n for v in vs]
        if not dec or not cal:
            raise SystemExit(f"{d}: no {counter} rows for the decode or calibration kernel")
        kib = float(np.mean(dec))
        scale = (CALIB_BYTES / 1024.0) / float(np.median(cal))
        res[counter] = {"kib_per_launch": kib, "dispatches": len(dec), "calibration_kib": float(np.median(cal)),
                        "scale": scale, "bytes_per_launch": kib * 1024.0 * scale}
    entry = {
        "hbm_bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"],
        "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
        "calibration": f"torch.neg over {CALIB_BYTES} bytes of float32 (reads and writes that many bytes)",
        "source_sha": source_hash(), "command": command,
    }
    try:
        rec = json.load(open(COUNTERS))
    except (OSError, ValueError):
        rec = {}
    rec[workload] = entry
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
    return entry


def cpu_baseline(inp, budget_s: float):
    """Time the fp64 oracle (absorbed form) on this machine's host cores."""
    from threadpoolctl import threadpool_info

    from oracle import mla_oracle as orc
    seqs = []
    for b in range(inp.B):
        rows = inp.cached_rows_f64(b)
        seqs.append((rows[:, :inp.r], rows[:, inp.r:]))
    qn, qr, cn, kn = inp.f64("q_nope"), inp.f64("q_rope"), inp.f64("c_kv_new"), inp.f64("k_rope_new")
    wuk, wuv = inp.f64("w_uk"), inp.f64("w_uv")
    done_rows, n_seq = 0, 0
    t0 = time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < budget_s:
        orc.absorbed_decode_seq(qn[b], qr[b], seqs[b][0], seqs[b][1], cn[b], kn[b], wuk, wuv,
                                inp.softmax_scale, inp.rope_base)
        done_rows += int(inp.seq_lens[b])
        n_seq += 1
        b = (b + 1) % inp.B
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": done_rows / dt, "unit": "cached-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 absorbed oracle, {n_seq} sequence evaluations cycling over the step's {inp.B} "
                      f"sequences ({done_rows} attended rows) in {dt:.1f} s"}


def run_kv_down(B=16, d_model=5120, launches=50):
    """Latent KV production from the hidden state at the DeepSeek-V2 shape:
    back-to-back launches between one pair of HIP events, over 8 weight sets
    (5.9 MB each) so that they do not sit in the Infinity Cache together."""
    import torch

    from head_latent_attention_12_amd import mla, synthetic as syn
    from head_latent_attention_12_amd.step import _dev

    kin = syn.make_kv_down_inputs(B, d_model)
    dims = mla.make_dims(B, 128, 128, 128, kin.r, kin.d_rope, mla.MLA_BF16)
    n_sets = 8
    ws = [{k: _dev(getattr(kin, k), "cuda") for k in ("h", "w_dkv", "w_kr", "norm_w")} for _ in range(n_sets)]
    work = torch.empty(mla.mla_kv_down_workspace_size(dims, d_model) // 4, dtype=torch.float32, device="cuda")
    c = torch.empty((B, kin.r), dtype=torch.int16, device="cuda")
    k = torch.empty((B, kin.d_rope), dtype=torch.int16, device="cuda")
    call = lambda w: mla.mla_kv_down(dims, d_model, w["h"], w["w_dkv"], w["w_kr"], w["norm_w"], kin.eps, work, c, k)
    for i in range(10):
        call(ws[i % n_sets])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(launches):
        call(ws[i % n_sets])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    nbytes = (kin.r + kin.d_rope) * d_model * 2 + B * d_model * 2 + B * (kin.r + kin.d_rope) * 2
    print(f"# kv_down B={B} d_model={d_model}: {us:.2f} us per call (two launches), "
          f"{nbytes / (us * 1e-6) / 1e9:.0f} GB/s of weights and activations", file=sys.stderr, flush=True)
    return {"workload": f"latent KV production bf16 B={B} d_model={d_model} r={kin.r} d_rope={kin.d_rope}",
            "us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "timing": "HIP events around back-to-back calls over 8 weight sets"}


def capture_round(sets):
    """One HIP graph with one step of each input set, in order."""
    import torch

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for ds in sets:
            ds.run()  # one eager pass on the capture stream before recording
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        for ds in sets:
            ds.run()
    return graph


def run_workload(name, steps, warmup, min_sets, verbose=True, page_rows=None, fp8=False):
    import torch

    from head_latent_attention_12_amd import mla, synthetic as syn
    from head_latent_attention_12_amd.step import DeviceStep

    inp = syn.make_inputs(name)
    rows, step_bytes, step_flops, k3_bytes, k3_flops = algorithmic(inp, fp8)
    row_bytes = inp.r + 2 * inp.d_rope + 4 if fp8 else inp.W * (2 if inp.dtype == "bf16" else 4)
    set_bytes = inp.total_rows * row_bytes + 2 * inp.H * inp.d_head * inp.r * 2
    n_sets = max(min_sets, int(np.ceil(2 * MALL_BYTES / set_bytes)))
    # each set has its own cache and weights (like successive layers); the
    # per-step temporaries (q_lat, split partials, o_lat, out) are one shared
    # workspace, as a multi-layer decode would reuse them
    sets = [DeviceStep(inp, page_rows=page_rows, page_seed=0, fp8=fp8)]
    sets += [DeviceStep(inp, scratch=sets[0], page_rows=page_rows, page_seed=i, fp8=fp8, fp8_seed=3 + i)
             for i in range(1, n_sets)]
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        sets[i % n_sets].run()
    torch.cuda.synchronize()

    # the timed steps, recorded as HIP graphs (the kernels are the same as
    # eager launches; a graph removes the host-side launch cost between them):
    # one graph holds one step of every set in turn, as the layers of one
    # decode step would run, and per-set graphs cover a remainder of steps
    graphs = [ds.capture() for ds in sets]
    round_graph = capture_round(sets)
    n_rounds, n_rest = divmod(steps, n_sets)

    def timed_steps():
        for _ in range(n_rounds):
            round_graph.replay()
        for i in range(n_rest):
            graphs[i].replay()

    for _ in range(max(1, warmup // n_sets)):
        round_graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed_steps()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # device span of the replayed steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    timed_steps()
    e1.record(stream)
    torch.cuda.synchronize()
    dev_ms = e0.elapsed_time(e1) / steps

    # eager steps with HIP events around every decode launch (its duration for
    # the roofline), timed as a whole too
    k3_start = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    k3_end = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        ds = sets[i % n_sets]
        ds.absorb_rope()
        k3_start[i].record(stream)
        ds.decode_latent()
        k3_end[i].record(stream)
        ds.combine_up_v()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) * 1e3 / steps
    k3_event_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(k3_start, k3_end)]))
    # the decode kernel's duration for the roofline: back-to-back launches over
    # the rotated input sets between one event pair (a pair around a single
    # launch also counts its dispatch latency, ~3 us)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(steps):
        sets[i % n_sets].decode_latent()
    b1.record(stream)
    torch.cuda.synchronize()
    k3_ms = b0.elapsed_time(b1) / steps
    del graphs, round_graph

    ms = wall * 1e3 / steps
    res = {
        "name": (name if page_rows is None else f"{name}_paged{page_rows}") + ("_fp8" if fp8 else ""),
        "workload": workload_label(inp) + ("" if page_rows is None else
                                           f", paged cache ({page_rows}-row pages, shuffled block table)")
        + (", fp8 latent cache (E4M3 codes, one power-of-two scale per row, bf16 RoPE key)" if fp8 else ""),
        "cached_tokens_per_step": rows,
        "ms_per_step": ms,
        "device_ms_per_step": dev_ms,
        "eager_ms_per_step": eager_ms,
        "value": rows / (ms * 1e-3),
        "step_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "step_TFLOPs": step_flops / (ms * 1e-3) / 1e12,
        "decode_kernel_ms": k3_ms,
        "decode_kernel_event_ms": k3_event_ms,
        "decode_kernel_GBps": k3_bytes / (k3_ms * 1e-3) / 1e9,
        "decode_kernel_TFLOPs": k3_flops / (k3_ms * 1e-3) / 1e12,
        "k3_bytes": k3_bytes,
        "k3_flops": k3_flops,
        "step_bytes": step_bytes,
        "step_flops": step_flops,
        "num_splits": sets[0].num_splits,
        "input_sets": n_sets,
        "inp": inp,
    }
    if verbose:
        print(f"# {res['name']}: {ms * 1e3:.1f} us/step (device {dev_ms * 1e3:.1f}, eager {eager_ms * 1e3:.1f}), "
              f"decode kernel {k3_ms * 1e3:.1f} us "
              f"= {res['decode_kernel_GBps']:.0f} GB/s, {res['decode_kernel_TFLOPs']:.0f} TFLOP/s; "
              f"splits {res['num_splits']}, sets {n_sets}", file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv2", choices=["tiny", "small", "dsv2", "dsv2_ragged", "dsv2_long"])
    ap.add_argument("--no-others", action="store_true", help="skip the other DeepSeek-V2-shaped workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--counters-run", action="store_true",
                    help="run the workload's steps and the calibration kernel only (profiled with rocprofv3 --pmc)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE csv runs into profiles/decode_latent_counters.json")
    ap.add_argument("--counters-command", default="", help="command line recorded with ingested counters")
    args = ap.parse_args()
    if args.ingest_counters:
        print(json.dumps(ingest_counters(args.workload, *args.ingest_counters, args.counters_command), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Sequences are independent, so batch data-parallel scaling across GPUs needs no exchange.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from head_latent_attention_12_amd import mla
    mla.lib()
    if args.counters_run:
        counters_run(args.workload, args.steps, args.warmup)
        return

    main_res = run_workload(args.workload, args.steps, args.warmup, min_sets=5)
    others = {}
    if not args.no_others:
        for name, page_rows, fp8 in (("dsv2_ragged", None, False), ("dsv2_long", None, False),
                                     ("dsv2_ragged", 64, False), ("dsv2", None, True), ("dsv2_ragged", None, True)):
            if name == args.workload and page_rows is None and not fp8:
                continue
            r = run_workload(name, max(20, args.steps // 4), max(5, args.warmup // 4), min_sets=2,
                             page_rows=page_rows, fp8=fp8)
            others[r["name"]] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()
                                 if k not in ("inp", "k3_bytes", "k3_flops", "step_bytes", "step_flops")}
        others["kv_down_dsv2"] = run_kv_down()

    inp = main_res["inp"]
    bf16 = inp.dtype == "bf16"
    traffic = counter_traffic(main_res["name"])
    achieved = main_res["decode_kernel_GBps"]
    line = {
        "metric": "MLA decode cached-tokens/s + achieved HBM GB/s & MFMA util vs roofline (1 GPU)",
        "value": round(main_res["value"], 1),
        "unit": "cached-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded Gaussian inputs of the DeepSeek-V2 MLA shape; no dataset or weights)",
        "config": {
            "workload": main_res["workload"],
            "B": inp.B, "H": inp.H, "d_head": inp.d_head, "d_v": inp.d_v, "r": inp.r, "d_rope": inp.d_rope,
            "cached_tokens_per_step": main_res["cached_tokens_per_step"],
            "num_splits": main_res["num_splits"], "input_sets_rotated": main_res["input_sets"],
            "parallelism": "single GPU (split-KV across work-groups)",
        },
        "roofline": {
            "kernel": "decode_latent_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (round(traffic / (main_res["decode_kernel_ms"] * 1e-3) / 1e9, 1) if traffic else None),
            "traffic_bytes_per_launch": (round(traffic) if traffic else None),
            "algorithmic_bytes_per_launch": main_res["k3_bytes"],
            "avg_launch_us": round(main_res["decode_kernel_ms"] * 1e3, 2),
            "launch_timing": "HIP events around back-to-back launches of the kernel over the rotated input sets",
            "avg_launch_us_in_step": round(main_res["decode_kernel_event_ms"] * 1e3, 2),
            "mfma_tflops": round(main_res["decode_kernel_TFLOPs"], 1),
            "mfma_frac": round(main_res["decode_kernel_TFLOPs"] / (BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS), 4),
        },
        "step": {
            "timing": "HIP graph replay of the four calls per step (absorb_q, rope_append, decode_latent, combine_up_v); one graph holds one step of every rotated input set",
            "device_us_per_step": round(main_res["device_ms_per_step"] * 1e3, 2),
            "eager_us_per_step": round(main_res["eager_ms_per_step"] * 1e3, 2),
            "GBps": round(main_res["step_GBps"], 1),
            "hbm_frac": round(main_res["step_GBps"] / HBM_PEAK_GBS, 4),
            "TFLOPs": round(main_res["step_TFLOPs"], 1),
        },
        "other_workloads": others,
    }
    line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

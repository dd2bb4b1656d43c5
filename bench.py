#!/usr/bin/env python3
"""Benchmark of the E8RHTLinear forward on one MI355X.

Step = one decode pass (B = 1) through the Devstral-Small 24B-shaped MLP:
gate 5120->32768, up 5120->32768, down 32768->5120 at 4 bpw (16-bit primary +
16-bit residual index per 8-weight group), bf16 activations; each layer runs
input RHT, the decode matmul against the indices and output RHT.  The layers
run on seeded synthetic data (no activation between them); gate and up, whose
inputs are ready together in an MLP, run as one glq_e8rht_linear_group call (one
launch pair on half the CUs each), then down; the step as three single calls is
reported beside it (one_call_per_layer).
R copies of the three layers' index arrays (>= 1 GiB in total) are rotated so
every step reads its indices from HBM, not from the 256 MB Infinity Cache.
The 16-bit index arrays are relabelled once, before timing, as slot codes
(glq_slot_codes: the same codebook entries, decoded with one LDS read);
--index-format codebook times the codebook indices themselves, and the run
reports the other format beside the headline.

value   = sum over the step's layers of (index bytes + x bytes + y bytes + sign
          bytes) / step time, in GB/s (inputs resident in HBM before timing starts).
roofline: the dominant launch pair, the gate+up group (fused_group_kernel, then the
          small blocks_group_kernel): events around back-to-back group calls (same
          stream) give its average duration; achieved = the two layers' bytes / that
          time.  A single layer call is fused_decode_kernel + output_blocks_kernel,
          timed the same way for one_call_per_layer.
prefill: the 2048-token prefill of the SmolLM3-3B gate shape (2048->11008,
          3 bpw), its MFMA matmul timed the same way, in TFLOP/s.
block_b1: the seven linears of a SmolLM3-3B decoder block (3 bpw, fp16) at B = 1,
          issued eagerly from Python and replayed from one captured HIP graph; the
          small layers are launch-bound, and the graph removes the host launch cost.
configs: every layer of the other workloads at their batch sizes (tiny 256->256 at B=1;
          SmolLM2 up at B=1, 5; each SmolLM3 linear at B=1, 5; Devstral at B=4, 16, the
          staged decode path), each timed over rotating copies of its indices, in GB/s
          and as a fraction of the HBM peak.
cpu_baseline: the fp64 oracle on the step's layers in turn, for >= 10 s of host CPU work.

--only LEG runs one leg by itself (for profiler runs); --pmc-report summarizes
rocprofv3 --pmc folders of such a run into a counter file under profiles/.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LEGS = ["decode", "configs", "prefill", "block", "recipes", "blockdiag", "kv"]
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "fused E8-RHT linear: achieved HBM GB/s at B=1 decode; TFLOP/s at prefill"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def act_bytes(dtype):
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-padded-only", action="store_true",
                    help="time only the padded prefill workload (profiler runs of its kernels)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--block-steps", type=int, default=500)
    ap.add_argument("--no-recipes", action="store_true", help="skip the 5-8 bpw decode measurement")
    ap.add_argument("--recipe-steps", type=int, default=300)
    ap.add_argument("--no-blockdiag", action="store_true", help="skip the unpadded (block-diagonal) measurement")
    ap.add_argument("--no-kv", action="store_true", help="skip the E8 KV-cache decode attention measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-layer measurement of the other configs")
    ap.add_argument("--kv-steps", type=int, default=50)
    ap.add_argument("--index-format", choices=["slot", "codebook"], default="slot",
                    help="16-bit index arrays as slot codes (default) or as codebook indices")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run 10 plain device-to-device copies of BYTES (scale for HBM traffic counters)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only summarize four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of this "
                         "bench and of --calibrate-copy) into " + os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--copy-bytes", type=int, default=1 << 28, help="BYTES of the --calibrate-copy run summarized")
    ap.add_argument("--only", choices=LEGS, help="run one leg alone (profiler runs)")
    ap.add_argument("--config-calls", type=int, default=200, help="timed calls per layer in the configs leg")
    ap.add_argument("--config-workloads", nargs="+", metavar="KEY",
                    help="only these workloads in the configs leg (profiler runs)")
    ap.add_argument("--pmc-report", nargs="+", metavar="ARG",
                    help="OUT KERNEL DIR [DIR ...]: medians of every counter of the dispatches whose name "
                         "contains KERNEL in rocprofv3 --pmc folders DIR, written to OUT with --pmc-cmd")
    ap.add_argument("--pmc-cmd", action="append", default=[], help="a command line recorded in the report")
    ap.add_argument("--stats-report", nargs=2, metavar=("OUT", "DIR"),
                    help="only summarize the kernel_stats.csv of a rocprofv3 --kernel-trace --stats folder DIR into OUT "
                         "(commands from --pmc-cmd, notes from --note)")
    ap.add_argument("--note", action="append", default=[], help="a note line recorded in a --stats-report")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.copy_bytes)
        return
    if args.pmc_report:
        pmc_report(args.pmc_report, args.pmc_cmd)
        return
    if args.stats_report:
        stats_report(args.stats_report, args.pmc_cmd, args.note)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the E8RHTLinear path here has no multi-GPU "
              "implementation (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import e8_lattice_codebook_amd as glq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.calibrate_copy, "copies": 10}), flush=True)
        return
    log("bench: building codebooks")
    cb = glq.Codebooks(dev)
    if args.only and args.only != "decode":
        fn = {"configs": lambda: bench_configs(glq, synth, cb, dev, args, log),
              "prefill": lambda: bench_prefill(glq, synth, cb, dev, args, log),
              "block": lambda: {"b1": bench_block_graph(glq, synth, cb, dev, args, log), "b5": bench_block_b5(glq, synth, cb, dev, args, log)},
              "recipes": lambda: bench_recipes(glq, synth, cb, dev, args, log, None),
              "blockdiag": lambda: bench_blockdiag(glq, synth, cb, dev, args, log, None),
              "kv": lambda: bench_kv(glq, synth, cb, dev, args, log)}[args.only]
        print(json.dumps({"only": args.only, args.only: fn()}), flush=True)
        return

    wl = synth.WORKLOADS["devstral_mlp"]
    B = args.batch
    host_layers = [synth.make_layer(s, wl.resid_bits, wl.seed, k) for k, s in enumerate(wl.layers)]
    idx_bytes = sum(l.index_bytes() for l in host_layers)
    copies = max(2, math.ceil((1 << 30) / idx_bytes))
    log("bench: %d layers, %.1f MiB of indices per step, %d rotating copies" % (
        len(host_layers), idx_bytes / 2 ** 20, copies))
    qls_cb = [[glq.QuantizedLayer.from_synth(l, cb) for l in host_layers] for _ in range(copies)]
    qls_slot = [[q.to_slot_codes() for q in row] for row in qls_cb]
    slot = args.index_format == "slot"
    qls, qls_other = (qls_slot, qls_cb) if slot else (qls_cb, qls_slot)
    xs = []
    for k, l in enumerate(host_layers):
        _, raw = synth.make_x(l.n, B, wl.act_dtype, wl.seed, k)
        xs.append(torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16))
    ys = [torch.empty((B, l.m), dtype=torch.bfloat16, device=dev) for l in host_layers]
    ws = torch.zeros(max(glq.linear_workspace_bytes(q, B) for q in qls[0]), dtype=torch.uint8, device=dev)

    # algorithmic bytes of one layer call: indices + x + y + the two sign vectors
    launch_bytes = [l.index_bytes() + B * (l.n + l.m) * act_bytes(wl.act_dtype) + l.n_pad + l.m_pad
                    for l in host_layers]
    step_bytes = sum(launch_bytes)

    grouped = B == 1  # gate and up as one launch pair (glq_e8rht_linear_group)
    gws = torch.zeros(max(1, glq.linear_group_workspace_bytes(qls[0][:2], B)), dtype=torch.uint8, device=dev)

    def step_layers(i):  # one glq_e8rht_linear call per layer
        row = qls[i % copies]
        for k in range(len(row)):
            glq.e8rht_linear(row[k], xs[k], out=ys[k], workspace=ws)

    def group_call(i):  # gate and up: their inputs are ready together in an MLP
        row = qls[i % copies]
        glq.e8rht_linear_group(row[:2], xs[:2], outs=ys[:2], workspace=gws)

    def step_grouped(i):  # gate + up as one group, then down
        group_call(i)
        glq.e8rht_linear(qls[i % copies][2], xs[2], out=ys[2], workspace=ws)

    step = step_grouped if grouped else step_layers
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n, first=0):
        """ms per call of fn over n back-to-back calls, one event pair around them"""
        e0.record()
        for i in range(n):
            fn(first + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(i)
        if grouped:
            step_layers(i)
    torch.cuda.synchronize()
    log("bench: timing %d steps" % args.steps)
    t0 = time.perf_counter()
    ms_per_step = timed(step, args.steps, args.warmup)
    wall = time.perf_counter() - t0
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log("bench: %.4f ms/step (wall %.4f), %.1f GB/s%s" % (ms_per_step, wall * 1e3 / args.steps, value,
                                                          " (gate+up grouped)" if grouped else ""))

    # per launch pair: at B = 1 every call is fused_decode_kernel + output_blocks_kernel,
    # a group fused_group_kernel + blocks_group_kernel.  One pair of events (on the launch
    # stream) around `steps` back-to-back calls over the rotating copies, so the events
    # add nothing to the calls they time.
    per_layer_ms = []
    for k in range(len(host_layers)):
        per_layer_ms.append(timed(lambda i: glq.e8rht_linear(qls[i % copies][k], xs[k], out=ys[k], workspace=ws),
                                  args.steps))
    achieved_layers = sum(launch_bytes) / (sum(per_layer_ms) * 1e-3) / 1e9
    log("bench: per-call ms %s -> %.1f GB/s" % (["%.4f" % t for t in per_layer_ms], achieved_layers))
    if grouped:
        group_ms = timed(group_call, args.steps)
        group_bytes = launch_bytes[0] + launch_bytes[1]
        achieved = group_bytes / (group_ms * 1e-3) / 1e9
        log("bench: gate+up group %.4f ms per call -> %.1f GB/s" % (group_ms, achieved))
        layers_ms = timed(step_layers, args.steps)
        log("bench: one call per layer: %.4f ms/step, %.1f GB/s" % (layers_ms, step_bytes / (layers_ms * 1e-3) / 1e9))
    else:
        achieved = achieved_layers

    # the achievable HBM rate for context: a plain device copy of 1 GiB (reads and
    # writes 1 GiB each), the same event timing
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    copy_ms = timed(lambda i: dst.copy_(src), 10)
    copy_gbs = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del src, dst
    # codeword lookups per second over the timed step (one per group and index stage)
    stages = 1 + (1 if wl.resid_bits else 0)
    lookups = sum(q.m_pad * (q.n_pad // 8) for q in qls[0]) * stages
    log("bench: plain copy %.1f GB/s; %.3g codeword lookups/s" % (copy_gbs, lookups / (ms_per_step * 1e-3)))

    # the other index format, same loop and step count
    other_steps = min(args.steps, 300)
    qls, qls_other = qls_other, qls
    other_ms = timed(step, other_steps)
    qls, qls_other = qls_other, qls
    other_value = step_bytes / (other_ms * 1e-3) / 1e9
    log("bench: %s indices: %.1f GB/s" % ("codebook" if slot else "slot-code", other_value))

    layer_kernel = ("fused_decode_kernel + output_blocks_kernel (one E8RHTLinear call at B = 1: input RHT, "
                    "decode matmul, row-block output transform; then the fixed-order split sum and the "
                    "cross-block output transform)")
    layers_roofline = {
        "bound": "hbm",
        "kernel": layer_kernel if B == 1 else "staged decode launches (RHT, quant_u, gemv_lds, RHT)",
        "achieved": round(achieved_layers, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved_layers / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(TRAFFIC_FILE) if B == 1 else None,
        "per_call_ms": [round(t, 5) for t in per_layer_ms],
        "bytes_per_call": launch_bytes,
        "timing": "one event pair around %d back-to-back calls per layer (rotating copies)" % args.steps,
    }
    if grouped:
        roofline = {
            "bound": "hbm",
            "kernel": ("fused_group_kernel + blocks_group_kernel (the gate and up E8RHTLinear calls at B = 1 in "
                       "one launch pair, glq_e8rht_linear_group: each layer's workgroups run the fused input "
                       "RHT, decode matmul and row-block output transform on half the CUs; then the fixed-order "
                       "split sums and cross-block output transforms of both)"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(GROUP_TRAFFIC_FILE),
            "per_launch_ms": round(group_ms, 5),
            "bytes_per_launch": group_bytes,
            "timing": "one event pair around %d back-to-back group calls (rotating copies)" % args.steps,
        }
    else:
        roofline = dict(layers_roofline)
    roofline.update({"copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4),
                     "lookups_per_s": float("%.4g" % (lookups / (ms_per_step * 1e-3)))})

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i16 fixed point x i4 -> i32, f32 scale",
        "arith": "activations in 16-bit fixed point per 64 columns (a power-of-two-normalized scale per "
                 "block, 4 int4 digit planes), exact i32 dot products against the int4-packed codewords, "
                 "f32 scaling, reduction and transforms",
        "data": "synthetic",
        "config": {
            "workload": "Devstral-Small-24B MLP decode (gate 5120->32768, up 5120->32768, down 32768->5120), "
                        "4 bpw (16+16-bit E8 indices), B=%d, bf16 activations, uniform seeded indices" % B,
            "batch": B,
            "step": ("gate and up as one glq_e8rht_linear_group call (one launch pair), then down"
                     if grouped else "one glq_e8rht_linear call per layer"),
            "index_format": ("slot codes: the 16-bit indices relabelled once at load (glq_slot_codes), "
                             "same entries and bytes") if slot else "codebook indices",
            "index_bytes_per_step": idx_bytes,
            "algorithmic_bytes_per_step": step_bytes,
            "rotating_copies": copies,
        },
        "roofline": roofline,
    }
    if grouped:
        result["one_call_per_layer"] = {
            "ms_per_step": round(layers_ms, 5), "value": round(step_bytes / (layers_ms * 1e-3) / 1e9, 2),
            "unit": "GB/s", "roofline": layers_roofline}
    result["other_index_format"] = {"index_format": "codebook indices" if slot else "slot codes",
                                    "value": round(other_value, 2), "unit": "GB/s", "steps": other_steps}

    if args.only == "decode":
        # the decode leg alone (profiler runs): no other leg, no CPU baseline
        print(json.dumps(result), flush=True)
        return
    if not args.no_configs:
        result["configs"] = bench_configs(glq, synth, cb, dev, args, log, devstral=(host_layers, qls, copies))

    if not args.no_prefill:
        result["prefill"] = bench_prefill(glq, synth, cb, dev, args, log)

    if not args.no_block:
        result["block_b1"] = bench_block_graph(glq, synth, cb, dev, args, log)
        result["block_b5"] = bench_block_b5(glq, synth, cb, dev, args, log)

    if not args.no_recipes and B == 1:
        # the recipes run one call per layer: compared with the same form at 4 bpw
        result["recipes_b1"] = bench_recipes(glq, synth, cb, dev, args, log,
                                             step_bytes / (layers_ms * 1e-3) / 1e9 if grouped else value)

    if not args.no_blockdiag and B == 1:
        result["blockdiag_b1"] = bench_blockdiag(glq, synth, cb, dev, args, log, layers_ms if grouped else ms_per_step,
                                                 ms_per_step if grouped else None)

    if not args.no_kv:
        result["kv_attention"] = bench_kv(glq, synth, cb, dev, args, log)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host_layers, wl, B, log)

    print(json.dumps(result), flush=True)


# ---- HBM traffic of the B = 1 launches from rocprofv3 counters -------------------------
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_decode_kernel_devstral_mlp_b1_traffic.txt")
FUSED_KERNEL_NAMES = ("fused_decode_kernel", "output_blocks_kernel")  # the two launches of a B = 1 call
GROUP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_group_kernel_devstral_gate_up_b1_traffic.txt")
GROUP_KERNEL_NAMES = ("fused_group_kernel", "blocks_group_kernel")  # the two launches of the gate+up group
KERNEL_SOURCES = ["fused_decode.hip", "lds_codebook.h", "fwht_lds.h", "internal.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "e8_lattice_codebook_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _pmc_rows(folder, counter):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc csv output folder."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit("no %s rows under %s" % (counter, folder))
    return rows


def pmc_summary(dirs, copy_bytes):
    """Write TRAFFIC_FILE and GROUP_TRAFFIC_FILE: FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch) of the two kernels of a B = 1 call, and of the two kernels of the gate+up
    group, each scaled by bytes / counter of a plain copy of copy_bytes (reads and
    writes copy_bytes each)."""
    import numpy as np
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    rows = {"fetch": _pmc_rows(fetch_dir, "FETCH_SIZE"), "write": _pmc_rows(write_dir, "WRITE_SIZE")}
    copy = {}
    for name, folder, counter in (("copy_fetch", cfetch_dir, "FETCH_SIZE"), ("copy_write", cwrite_dir, "WRITE_SIZE")):
        crows = _pmc_rows(folder, counter)
        big = max(v for _, v in crows)
        copy[name + "_kib"] = float(np.median([v for _, v in crows if v > 0.5 * big]))  # the copy dispatches
    sf = copy_bytes / (copy["copy_fetch_kib"] * 1024.0)
    sw = copy_bytes / (copy["copy_write_kib"] * 1024.0)
    cmd = ("python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-prefill --no-block --no-recipes "
           "--no-blockdiag --no-kv --no-configs")
    for path, names, what in ((TRAFFIC_FILE, FUSED_KERNEL_NAMES, "one B = 1 call"),
                              (GROUP_TRAFFIC_FILE, GROUP_KERNEL_NAMES, "one B = 1 gate+up group call")):
        out = {}
        for name in ("fetch", "write"):
            out[name + "_kib"] = 0.0
            out[name + "_dispatches"] = 0
            for kname in names:  # per call: the sum of the two kernels' medians
                vals = [v for k, v in rows[name] if kname in k]
                out[name + "_kib"] += float(np.median(vals))
                out[name + "_dispatches"] += len(vals)
        traffic = out["fetch_kib"] * 1024.0 * sf + out["write_kib"] * 1024.0 * sw
        lines = [
            "# HBM traffic of %s (%s), Devstral-Small-24B MLP decode" % (what, " + ".join(names)),
            "# commands (from the repository root, after cd /tmp && export TMPDIR=/tmp for the profiler):",
            "#   rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR --output-format csv -- %s" % cmd,
            "#   rocprofv3 --pmc WRITE_SIZE -d WRITE_DIR --output-format csv -- (same)",
            "#   rocprofv3 --pmc FETCH_SIZE -d COPY_FETCH_DIR --output-format csv -- python3 bench.py --calibrate-copy %d"
            % copy_bytes,
            "#   rocprofv3 --pmc WRITE_SIZE -d COPY_WRITE_DIR --output-format csv -- (same)",
            "#   python3 bench.py --pmc-summary FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR --copy-bytes %d"
            % copy_bytes,
            "kernel_source_sha256: %s" % kernel_source_hash(),
            "fetch_kib_median: %.1f (%d dispatches)" % (out["fetch_kib"], out["fetch_dispatches"]),
            "write_kib_median: %.1f (%d dispatches)" % (out["write_kib"], out["write_dispatches"]),
            "copy_bytes: %d" % copy_bytes,
            "copy_fetch_kib: %.1f -> fetch scale %.4f" % (copy["copy_fetch_kib"], sf),
            "copy_write_kib: %.1f -> write scale %.4f" % (copy["copy_write_kib"], sw),
            "traffic_bytes_per_call: %d" % int(round(traffic)),
        ]
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print("\n".join(lines))


def measured_traffic(path):
    """HBM bytes per call from a traffic file written by pmc_summary, or None when it is
    missing or was taken on other kernel sources.  TRAFFIC_FILE holds medians over the
    three layers' dispatches (reported against their mean algorithmic bytes);
    GROUP_TRAFFIC_FILE those of the gate+up group calls."""
    try:
        with open(path) as fh:
            kv = dict(l.split(": ", 1) for l in fh.read().splitlines() if ": " in l and not l.startswith("#"))
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return int(kv["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def clone_layer(glq, q):
    """A device copy of a QuantizedLayer's index arrays (signs and codebooks shared)."""
    return glq.QuantizedLayer(q.n, q.m, q.n_pad, q.m_pad, q.resid_bits, q.sign_in, q.sign_out, q.idx0.clone(),
                              None if q.idx1 is None else q.idx1.clone(), q.codebooks, q.wscale, q.resid_scale,
                              q.device, q.index_format, extra=tuple((b, i.clone(), sc) for b, i, sc in q.extra))


def time_calls(torch, calls, reps):
    """ms per call of `calls` (a list of callables, run in turn `reps` times) between one
    pair of events on the current stream, after two warm-up passes."""
    for _ in range(2):
        for c in calls:
            c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for c in calls:
            c()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls))


CONFIG_LEGS = [("tiny", (1,)), ("smollm2_up", (1, 5)), ("smollm3_block", (1, 5)), ("devstral_mlp", (4, 16))]


def bench_configs(glq, synth, cb, dev, args, log, devstral=None):
    """Every layer of the other workloads at their batch sizes, one layer at a time:
    slot-code copies of its indices rotated so that the calls stream about 1 GiB of
    indices (cold past the 256 MB MALL where the layer is large enough: at most 2048
    copies), calls timed back to back with one pair of events.  GB/s counts index,
    activation, output and sign bytes per call; frac is against the 8 TB/s HBM peak.
    B = 1 runs the two-launch fused decode, 2 <= B <= 16 the staged decode (input RHT,
    quantization, GEMV, output RHT; the GEMV on the int8 matrix units for 2 <= B <= 16 on
    layers of at least 2^21 groups and for 4 <= B <= 16 from 2^17)."""
    import numpy as np
    import torch

    out = []
    for key, batches in CONFIG_LEGS:
        if args.config_workloads and key not in args.config_workloads:
            continue
        wl = synth.WORKLOADS[key]
        ab = act_bytes(wl.act_dtype)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.act_dtype]
        for k, shape in enumerate(wl.layers):
            if key == "devstral_mlp" and devstral is not None:
                host, rows, ncop = devstral
                l = host[k]
                cps = [row[k] for row in rows] if args.index_format == "slot" else None
            else:
                l = synth.make_layer(shape, wl.resid_bits, wl.seed, k)
                cps = None
            if cps is None:
                q0 = glq.QuantizedLayer.from_synth(l, cb)
                if args.index_format == "slot":
                    q0 = q0.to_slot_codes()
                ncop = max(2, min(2048, math.ceil((1 << 30) / l.index_bytes())))
                cps = [q0] + [clone_layer(glq, q0) for _ in range(ncop - 1)]
            ncop = len(cps)
            for B in batches:
                _, raw = synth.make_x(l.n, B, wl.act_dtype, wl.seed, k)
                x = torch.from_numpy(raw.view(np.int16) if wl.act_dtype == "bf16" else raw).to(dev)
                if wl.act_dtype == "bf16":
                    x = x.view(torch.bfloat16)
                y = torch.empty((B, l.m), dtype=tdt, device=dev)
                ws = glq.linear_workspace(cps[0], B, dev)
                calls = [lambda q=q: glq.e8rht_linear(q, x, out=y, workspace=ws) for q in cps]
                reps = max(1, math.ceil(args.config_calls / ncop))
                ms = time_calls(torch, calls, reps)
                nbytes = l.index_bytes() + B * (l.n + l.m) * ab + l.n_pad + l.m_pad
                gbs = nbytes / (ms * 1e-3) / 1e9
                path = ("fused B=1 (2 launches)" if B == 1 else
                        "staged (input RHT, quantization, GEMV, output RHT; the GEMV on the int8 matrix units "
                        "for 2 <= B <= 16 on layers of 2^21+ groups and 4 <= B <= 16 from 2^17, else the "
                        "LDS-codebook integer GEMV)")
                log("bench: %s %s B=%d: %.2f us per call, %.1f GB/s (%d copies)" % (key, shape.name, B, ms * 1e3,
                                                                                   gbs, ncop))
                out.append({"workload": key, "layer": "%s %d->%d (n_pad %d, m_pad %d)" % (
                    shape.name, l.n, l.m, l.n_pad, l.m_pad), "B": B, "bpw": l.bpw, "path": path,
                    "us_per_call": round(ms * 1e3, 3), "value": round(gbs, 2), "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_call": int(nbytes), "copies": ncop,
                    "cold": bool(ncop * l.index_bytes() >= (512 << 20)), "calls_timed": reps * ncop})
                del ws, x, y
            del cps
            torch.cuda.empty_cache()
        if key == "devstral_mlp" and args.index_format == "slot":
            # gate and up (one input) as one glq_e8rht_linear_group call: one int8 GEMV launch
            if devstral is not None:
                host, rows, _ = devstral
            else:  # the configs leg alone: three rotating copies of gate and up
                host = [synth.make_layer(wl.layers[k], wl.resid_bits, wl.seed, k) for k in (0, 1)]
                rows = [[glq.QuantizedLayer.from_synth(h, cb).to_slot_codes() for h in host] for _ in range(3)]
            for B in batches:
                _, raw = synth.make_x(host[0].n, B, wl.act_dtype, wl.seed, 0)
                x = torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
                ys = [torch.empty((B, l.m), dtype=tdt, device=dev) for l in host[:2]]
                gws = torch.empty(max(1, glq.linear_group_workspace_bytes(rows[0][:2], B)), dtype=torch.uint8,
                                  device=dev)
                calls = [lambda r=r: glq.e8rht_linear_group(r[:2], [x, x], outs=ys, workspace=gws) for r in rows]
                ms = time_calls(torch, calls, max(1, math.ceil(args.config_calls / len(rows))))
                nbytes = sum(l.index_bytes() + B * (l.n + l.m) * ab + l.n_pad + l.m_pad for l in host[:2])
                gbs = nbytes / (ms * 1e-3) / 1e9
                log("bench: %s gate+up grouped B=%d: %.2f us per call, %.1f GB/s" % (key, B, ms * 1e3, gbs))
                out.append({"workload": key, "layer": "gate+up as one glq_e8rht_linear_group call", "B": B,
                            "path": "grouped int8 GEMV (one launch for both layers)",
                            "us_per_call": round(ms * 1e3, 3), "value": round(gbs, 2), "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_call": int(nbytes),
                            "copies": len(rows)})
                del x, ys, gws
            torch.cuda.empty_cache()
    return out


def pmc_report(argv, cmds):
    """OUT KERNEL DIR [DIR ...]: per-counter medians over the dispatches whose kernel name
    contains KERNEL in rocprofv3 --pmc csv folders, with the derived MFMA, VALU and LDS
    figures where their counters are present."""
    import csv
    import glob
    import statistics
    out_file, kname, dirs = argv[0], argv[1], argv[2:]
    vals, names = {}, set()
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if kname in r.get("Kernel_Name", ""):
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                        names.add(r["Kernel_Name"])
    if not vals:
        raise SystemExit("no dispatches of %s under %s" % (kname, dirs))
    med = {k: statistics.median(v) for k, v in vals.items()}
    lines = ["# rocprofv3 --pmc counters (MI355X, one GPU): medians over the dispatches of %s" % kname,
             "# kernels: %s" % "; ".join(sorted(names)),
             "# commands (repository root; profiler runs after cd /tmp && export TMPDIR=/tmp):"]
    lines += ["#   %s" % c for c in cmds]
    lines += ["# values are sums over the device's XCDs / shader engines as rocprofv3 reports them"]
    for k in sorted(med):
        lines.append("%s: %.1f (%d dispatches)" % (k, med[k], len(vals[k])))
    g = med.get("GRBM_GUI_ACTIVE")
    if g:
        xcd_cycles = g / 8.0  # GRBM_GUI_ACTIVE is summed over the 8 XCDs
        lines.append("derived kernel_cycles_per_xcd: %.0f (%.2f us at 2.4 GHz)" % (xcd_cycles, xcd_cycles / 2400.0))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            # summed over the 1024 SIMDs (it reads 16 cycles per 16x16x32 f16 MFMA issued)
            lines.append("derived mfma_busy_per_simd: %.4f (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8) / "
                         "1024 SIMDs)" % (med["SQ_VALU_MFMA_BUSY_CYCLES"] / xcd_cycles / 1024.0))
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in med:
            fl = med["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512.0
            lines.append("derived mfma_f16_flops: %.4g (MOPS x 512) -> %.1f TFLOP/s over the kernel cycles"
                         % (fl, fl / (xcd_cycles / 2.4e9) / 1e12))
        if "SQ_INSTS_VALU" in med:
            lines.append("derived valu_busy_per_simd: %.4f (SQ_INSTS_VALU x 4 cycles / (kernel cycles x 1024 SIMDs))"
                         % (med["SQ_INSTS_VALU"] * 4.0 / (xcd_cycles * 1024.0)))
    if "SQ_LDS_BANK_CONFLICT" in med and "SQ_INSTS_LDS" in med:
        lines.append("derived lds_conflict_cycles_per_lds_inst: %.2f" % (med["SQ_LDS_BANK_CONFLICT"] / med["SQ_INSTS_LDS"]))
    os.makedirs(os.path.dirname(os.path.abspath(out_file)), exist_ok=True)
    with open(out_file, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_report(argv, cmds, notes):
    """OUT DIR: the kernels of a rocprofv3 --kernel-trace --stats csv folder, by total
    time (microseconds), with the recorded commands and notes."""
    import csv
    import glob
    out_file, folder = argv[0], argv[1]
    files = glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under %s" % folder)
    with open(files[0]) as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel statistics (MI355X, one GPU), durations in microseconds",
             "# commands (repository root; profiler runs after cd /tmp && export TMPDIR=/tmp):"]
    lines += ["#   %s" % c for c in cmds]
    lines += ["# %s" % n for n in notes]
    lines.append("%-100s %7s %9s %9s %9s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "total_ms"))
    for r in rows[:25]:
        name = r["Name"]
        if len(name) > 100:
            name = name[:97] + "..."
        lines.append("%-100s %7s %9.2f %9.2f %9.2f %10.3f" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e6))
    os.makedirs(os.path.dirname(os.path.abspath(out_file)), exist_ok=True)
    with open(out_file, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def bench_prefill(glq, synth, cb, dev, args, log):
    """The 2048-token prefill of the SmolLM3-3B gate shape, 3 bpw: the whole linear, and
    its MFMA matmul alone (events around it), on the padded layer (m_pad 16384, the
    workload as described) and on the unpadded one (m_pad = m = 11008, block-diagonal
    output transform).  TFLOP/s counts the matmul's algorithmic flops 2 M m_pad n_pad;
    the nominal figure divides the layer's own 2 M m n by the same time."""
    import numpy as np
    import torch

    wl = synth.WORKLOADS["prefill_gateup"]
    M = wl.batches[0]

    def measure(l):
        q_cb = glq.QuantizedLayer.from_synth(l, cb)
        q_slot = q_cb.to_slot_codes()
        q, q_other = (q_slot, q_cb) if args.index_format == "slot" else (q_cb, q_slot)
        _, raw = synth.make_x(l.n, M, wl.act_dtype, wl.seed, 0)
        x = torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
        u = torch.empty(glq.lib().glq_prefill_u_bytes(M, l.n_pad), dtype=torch.uint8, device=dev)
        u16 = torch.empty((M, l.n_pad), dtype=torch.float16, device=dev)
        z = torch.empty((1, M, l.m_pad), dtype=torch.float32, device=dev)
        y = torch.empty((M, l.m), dtype=torch.bfloat16, device=dev)
        ws = glq.linear_workspace(q, M, dev)
        lin_ms = time_calls(torch, [lambda: glq.e8rht_linear(q, x, out=y, workspace=ws)], args.prefill_steps)

        def matmul_ms(qq):
            # the linear's prefill steps one by one, events around the matmul: slot codes
            # on fragment-order u (gemm_shared_kernel), codebook indices on fragment-order
            # u (gemm_lds_kernel)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.prefill_steps)]
            frag = glq.e8_matmul_prefill_supported(qq)
            for a, b in evs:
                if frag:
                    glq.input_rht_prefill(x, l.n_pad, qq.sign_in, out=u)
                else:
                    glq.input_rht(x, l.n_pad, qq.sign_in, torch.float16, out=u16)
                a.record()
                if frag:
                    glq.e8_matmul_prefill(qq, u, M, out=z)
                else:
                    glq.e8_matmul(qq, u16, out=z)
                b.record()
                glq.output_rht(z, l.m, qq.sign_out, out=y)
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b) for a, b in evs[2:]])), frag

        gemm_ms, frag = matmul_ms(q)
        other_ms, _ = matmul_ms(q_other)
        return lin_ms, gemm_ms, other_ms, frag

    l = synth.make_layer(wl.layers[0], wl.resid_bits, wl.seed, 0)
    lin_ms, gemm_ms, other_ms, frag = measure(l)
    flops = 2.0 * M * l.m_pad * l.n_pad
    nominal = 2.0 * M * l.m * l.n
    tflops = flops / (gemm_ms * 1e-3) / 1e12
    log("bench: prefill linear %.4f ms, MFMA matmul %.4f ms = %.1f TFLOP/s (nominal %.1f)" % (
        lin_ms, gemm_ms, tflops, nominal / (gemm_ms * 1e-3) / 1e12))
    unpadded = None
    if not args.prefill_padded_only:
        lu = synth.make_layer(wl.layers[0], wl.resid_bits, wl.seed, 0, block_diag=True)
        ulin_ms, ugemm_ms, _, _ = measure(lu)
        uflops = 2.0 * M * lu.m_pad * lu.n_pad
        log("bench: unpadded prefill (m_pad %d) linear %.4f ms, matmul %.4f ms = %.1f TFLOP/s" % (
            lu.m_pad, ulin_ms, ugemm_ms, uflops / (ugemm_ms * 1e-3) / 1e12))
        unpadded = {"workload": "the same layer unpadded: m_pad = m = 11008 (block-diagonal output transform "
                                "over 8192 + 2048 + 512 + 256)",
                    "linear_ms": round(ulin_ms, 5), "matmul_ms": round(ugemm_ms, 5),
                    "value": round(uflops / (ugemm_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "flops": uflops,
                    "linear_speedup_vs_padded": round(lin_ms / ulin_ms, 3)}
    return {
        "workload": "SmolLM3-3B gate 2048->11008 (m_pad 16384), M=2048 tokens, 3 bpw, bf16 activations",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "linear_ms": round(lin_ms, 5),
        "matmul_ms": round(gemm_ms, 5),
        "nominal_tflops": round(nominal / (gemm_ms * 1e-3) / 1e12, 2),
        "nominal_flops": nominal,
        "other_index_format": {"index_format": "codebook indices" if args.index_format == "slot" else "slot codes",
                               "value": round(flops / (other_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s"},
        "unpadded": unpadded,
        "roofline": {"bound": "mfma", "kernel": ("gemm_shared_kernel (prefill matmul: a 64-row codeword tile per "
                                                 "k-step dequantized from the LDS codebook into LDS, shared by four "
                                                 "waves as fp16 MFMA operands, fp32 accumulation)") if frag else
                     ("gemm_lds_kernel (prefill matmul: codewords from the LDS codebook dequantized per wave into "
                      "fp16 MFMA operands, fp32 accumulation)"),
                     "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops},
    }


def bench_block_b5(glq, synth, cb, dev, args, log, B=5):
    """The seven linears of a SmolLM3-3B block at B = 5 (3 bpw, fp16, slot codes): as
    seven glq_e8rht_linear calls and as four glq_e8rht_linear_group calls (q+k+v, o,
    gate+up, down), the q+k+v and gate+up groups sharing one int8 GEMV launch each."""
    import numpy as np
    import torch

    wl = synth.WORKLOADS["smollm3_block"]
    host = [synth.make_layer(sh, wl.resid_bits, wl.seed, k) for k, sh in enumerate(wl.layers)]
    qs = [glq.QuantizedLayer.from_synth(l, cb) for l in host]
    if args.index_format == "slot":
        qs = [q.to_slot_codes() for q in qs]
    xs = []
    for k, l in enumerate(host):
        _, raw = synth.make_x(l.n, B, wl.act_dtype, wl.seed, k)
        xs.append(torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.float16))
    ys = [torch.empty((B, l.m), dtype=torch.float16, device=dev) for l in host]
    groups = [(0, 1, 2), (3,), (4, 5), (6,)]
    ws = torch.empty(max(max(glq.linear_workspace_bytes(q, B) for q in qs),
                         max(glq.linear_group_workspace_bytes([qs[k] for k in g], B) for g in groups)),
                     dtype=torch.uint8, device=dev)

    def calls():
        for k in range(len(qs)):
            glq.e8rht_linear(qs[k], xs[k], out=ys[k], workspace=ws)

    def grouped():
        for g in groups:
            glq.e8rht_linear_group([qs[k] for k in g], [xs[k] for k in g], outs=[ys[k] for k in g], workspace=ws)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {"workload": "SmolLM3-3B decoder block, 7 linears, 3 bpw, fp16 activations, B=%d, indices resident in "
                       "the 256 MB MALL across iterations" % B}
    n = args.block_steps
    for name, fn in (("calls", calls), ("grouped", grouped)):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms_per_block"] = round(e0.elapsed_time(e1) / n, 5)
    out["speedup_grouped"] = round(out["calls_ms_per_block"] / out["grouped_ms_per_block"], 3)
    log("bench: SmolLM3 block B=%d: %.4f ms as seven calls, %.4f ms as four groups" % (
        B, out["calls_ms_per_block"], out["grouped_ms_per_block"]))
    return out


def bench_block_graph(glq, synth, cb, dev, args, log):
    import numpy as np
    import torch

    wl = synth.WORKLOADS["smollm3_block"]
    host = [synth.make_layer(sh, wl.resid_bits, wl.seed, k) for k, sh in enumerate(wl.layers)]
    qs = [glq.QuantizedLayer.from_synth(l, cb) for l in host]
    if args.index_format == "slot":
        qs = [q.to_slot_codes() for q in qs]
    xs = []
    for k, l in enumerate(host):
        _, raw = synth.make_x(l.n, 1, wl.act_dtype, wl.seed, k)
        xs.append(torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.float16))
    ys = [torch.empty((1, l.m), dtype=torch.float16, device=dev) for l in host]
    ws = torch.empty(max(glq.linear_workspace_bytes(q, 1) for q in qs), dtype=torch.uint8, device=dev)
    nbytes = sum(l.index_bytes() + 2 * (l.n + l.m) + l.n_pad + l.m_pad for l in host)

    def block():
        for k in range(len(qs)):
            glq.e8rht_linear(qs[k], xs[k], out=ys[k], workspace=ws)

    n = args.block_steps
    for _ in range(50):
        block()
    torch.cuda.synchronize()
    eager_ref = [y.clone() for y in ys]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        block()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        block()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            block()
    torch.cuda.synchronize()
    for y in ys:
        y.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ys, eager_ref))
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / n
    log("bench: SmolLM3 block B=1: eager %.4f ms, graph %.4f ms per block (replay equals eager: %s)" % (
        eager_ms, graph_ms, same))

    # the same block with the linears that a decoder block can run together as groups
    # (glq_e8rht_linear_group): q, k, v; o; gate, up; down -- 8 launches instead of 14
    groups = [(0, 1, 2), (3,), (4, 5), (6,)]
    gws = torch.empty(max(glq.linear_group_workspace_bytes([qs[k] for k in gr], 1) for gr in groups),
                      dtype=torch.uint8, device=dev)

    def block_grouped():
        for gr in groups:
            glq.e8rht_linear_group([qs[k] for k in gr], [xs[k] for k in gr], outs=[ys[k] for k in gr],
                                   workspace=gws)

    for _ in range(50):
        block_grouped()
    torch.cuda.synchronize()
    grouped_diff = max(float((y.float() - r.float()).abs().max() / r.float().abs().max())
                       for y, r in zip(ys, eager_ref))
    e0.record()
    for _ in range(n):
        block_grouped()
    e1.record()
    torch.cuda.synchronize()
    grouped_ms = e0.elapsed_time(e1) / n
    per_group = []
    for gr in groups:
        e0.record()
        for _ in range(n):
            glq.e8rht_linear_group([qs[k] for k in gr], [xs[k] for k in gr], outs=[ys[k] for k in gr],
                                   workspace=gws)
        e1.record()
        torch.cuda.synchronize()
        per_group.append(round(e0.elapsed_time(e1) / n * 1e3, 2))
    log("bench: SmolLM3 block B=1 grouped: %.4f ms per block; per group (us) %s" % (grouped_ms, per_group))
    return {
        "workload": "SmolLM3-3B decoder block, 7 linears (q, k, v, o 2048-wide; gate, up 2048->11008; down "
                    "11008->2048), 3 bpw, fp16 activations, B=1; %.1f MB of indices, resident in the 256 MB "
                    "MALL across iterations" % (sum(l.index_bytes() for l in host) / 1e6),
        "eager_ms_per_block": round(eager_ms, 5),
        "graph_ms_per_block": round(graph_ms, 5),
        "layer_calls_per_s_eager": round(len(host) / (eager_ms * 1e-3), 1),
        "layer_calls_per_s_graph": round(len(host) / (graph_ms * 1e-3), 1),
        "graph_speedup": round(eager_ms / graph_ms, 3),
        "graph_gbs": round(nbytes / (graph_ms * 1e-3) / 1e9, 1),
        "replay_equals_eager": bool(same),
        "launches_per_block": 2 * len(host),
        "grouped": {
            "groups": "q+k+v, o, gate+up, down (glq_e8rht_linear_group: one pair of launches per group)",
            "ms_per_block": round(grouped_ms, 5),
            "us_per_group": per_group,
            "gbs": round(nbytes / (grouped_ms * 1e-3) / 1e9, 1),
            "speedup_vs_eager": round(eager_ms / grouped_ms, 3),
            "launches_per_block": 2 * len(groups),
            "max_rel_diff_vs_single_calls": grouped_diff,
        },
    }


def bench_recipes(glq, synth, cb, dev, args, log, value_4bpw):
    """The Devstral MLP decode step at B = 1 with the 5-8 bpw recipes (16-bit
    primary and residual stage plus one or two further 8/16-bit stages), same
    activations, rotating copies and loop as the 4 bpw measurement: one call per
    layer, and with gate and up as one group."""
    import numpy as np
    import torch

    wl = synth.WORKLOADS["devstral_mlp"]
    xs, ys = [], []
    for k, s in enumerate(wl.layers):
        sp = s.padded()
        _, raw = synth.make_x(sp.n, 1, wl.act_dtype, wl.seed, k)
        xs.append(torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16))
        ys.append(torch.empty((1, sp.m), dtype=torch.bfloat16, device=dev))
    out = {"workload": "Devstral-Small-24B MLP decode (gate, up, down), B=1, bf16 activations; recipes of the "
                       "bit-width table: 16+16+8, 16+16+16, 16+16+16+8, 16+16+16+16 bits per 8 weights",
           "index_format": args.index_format, "steps": args.recipe_steps, "unit": "GB/s",
           "value_4bpw": None if value_4bpw is None else round(value_4bpw, 2), "by_bpw": {}}
    for bpw in (5, 6, 7, 8):
        resid_bits, extra_bits = synth.RECIPES[bpw]
        host = [synth.make_layer(s, resid_bits, wl.seed, k, extra_bits=extra_bits) for k, s in enumerate(wl.layers)]
        idx_bytes = sum(l.index_bytes() for l in host)
        copies = max(2, math.ceil((1 << 30) / idx_bytes))
        qls = [[glq.QuantizedLayer.from_synth(l, cb) for l in host] for _ in range(copies)]
        if args.index_format == "slot":
            qls = [[q.to_slot_codes() for q in row] for row in qls]
        del host
        ws = torch.zeros(max(glq.linear_workspace_bytes(q, 1) for q in qls[0]), dtype=torch.uint8, device=dev)
        step_bytes = sum(q.index_bytes() + (q.n + q.m) * 2 + q.n_pad + q.m_pad for q in qls[0])

        def step(i):
            row = qls[i % copies]
            for k in range(len(row)):
                glq.e8rht_linear(row[k], xs[k], out=ys[k], workspace=ws)

        for i in range(50):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.recipe_steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.recipe_steps
        gbs = step_bytes / (ms * 1e-3) / 1e9
        log("bench: %d bpw Devstral MLP B=1: %.4f ms/step, %.1f GB/s (%d copies)" % (bpw, ms, gbs, copies))
        # gate and up as one group, then down (as the 4 bpw headline step)
        gws = torch.zeros(max(1, glq.linear_group_workspace_bytes(qls[0][:2], 1)), dtype=torch.uint8, device=dev)

        def gstep(i):
            row = qls[i % copies]
            glq.e8rht_linear_group(row[:2], xs[:2], outs=ys[:2], workspace=gws)
            glq.e8rht_linear(row[2], xs[2], out=ys[2], workspace=ws)

        for i in range(50):
            gstep(i)
        e0.record()
        for i in range(args.recipe_steps):
            gstep(i)
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / args.recipe_steps
        ggbs = step_bytes / (gms * 1e-3) / 1e9
        log("bench: %d bpw Devstral MLP B=1, gate+up grouped: %.4f ms/step, %.1f GB/s" % (bpw, gms, ggbs))
        out["by_bpw"][str(bpw)] = {"ms_per_step": round(ms, 5), "value": round(gbs, 2),
                                   "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": step_bytes,
                                   "launches_per_layer": 2,
                                   "grouped": {"ms_per_step": round(gms, 5), "value": round(ggbs, 2),
                                               "frac": round(ggbs / HBM_PEAK_GBS, 4)}}
        del qls, ws, gws
        torch.cuda.empty_cache()
    return out


def bench_blockdiag(glq, synth, cb, dev, args, log, padded_ms, padded_grouped_ms=None):
    """The Devstral MLP decode step at B = 1 with unpadded layers: 5120 is
    transformed block-diagonally (4096 + 1024) instead of being padded to 8192, so
    gate and up store 5120 / 8 groups per row and down 5120 rows."""
    import numpy as np
    import torch

    wl = synth.WORKLOADS["devstral_mlp"]
    host = [synth.make_layer(s, wl.resid_bits, wl.seed, k, block_diag=True) for k, s in enumerate(wl.layers)]
    idx_bytes = sum(l.index_bytes() for l in host)
    copies = max(2, math.ceil((1 << 30) / idx_bytes))
    qls = [[glq.QuantizedLayer.from_synth(l, cb) for l in host] for _ in range(copies)]
    if args.index_format == "slot":
        qls = [[q.to_slot_codes() for q in row] for row in qls]
    xs, ys = [], []
    for k, l in enumerate(host):
        _, raw = synth.make_x(l.n, 1, wl.act_dtype, wl.seed, k)
        xs.append(torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16))
        ys.append(torch.empty((1, l.m), dtype=torch.bfloat16, device=dev))
    del host
    ws = torch.zeros(max(glq.linear_workspace_bytes(q, 1) for q in qls[0]), dtype=torch.uint8, device=dev)
    step_bytes = sum(q.index_bytes() + (q.n + q.m) * 2 + q.n_pad + q.m_pad for q in qls[0])

    def step(i):
        row = qls[i % copies]
        for k in range(len(row)):
            glq.e8rht_linear(row[k], xs[k], out=ys[k], workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log("bench: unpadded Devstral MLP B=1: %.4f ms/step, %.1f GB/s" % (ms, gbs))
    # gate and up as one group (same n_pad = 5120, block-diagonal), then down
    gws = torch.zeros(max(1, glq.linear_group_workspace_bytes(qls[0][:2], 1)), dtype=torch.uint8, device=dev)

    def gstep(i):
        row = qls[i % copies]
        glq.e8rht_linear_group(row[:2], xs[:2], outs=ys[:2], workspace=gws)
        glq.e8rht_linear(row[2], xs[2], out=ys[2], workspace=ws)

    for i in range(args.warmup):
        gstep(i)
    e0.record()
    for i in range(args.steps):
        gstep(i)
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / args.steps
    ggbs = step_bytes / (gms * 1e-3) / 1e9
    log("bench: unpadded Devstral MLP B=1, gate+up grouped: %.4f ms/step, %.1f GB/s" % (gms, ggbs))
    out = {"workload": "Devstral-Small-24B MLP decode, B=1, bf16, 4 bpw, unpadded: gate, up 5120 -> 32768 and down "
                       "32768 -> 5120 with block-diagonal transforms over 5120 = 4096 + 1024",
           "index_format": args.index_format, "steps": args.steps, "ms_per_step": round(ms, 5),
           "value": round(gbs, 2), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "algorithmic_bytes_per_step": step_bytes, "index_bytes_per_step": idx_bytes,
           "padded_ms_per_step": None if padded_ms is None else round(padded_ms, 5),
           "step_speedup_vs_padded": None if padded_ms is None else round(padded_ms / ms, 3),
           "grouped": {"step": "gate and up as one glq_e8rht_linear_group call, then down",
                       "ms_per_step": round(gms, 5), "value": round(ggbs, 2), "unit": "GB/s",
                       "frac": round(ggbs / HBM_PEAK_GBS, 4),
                       "padded_grouped_ms_per_step": None if padded_grouped_ms is None else round(padded_grouped_ms, 5),
                       "step_speedup_vs_padded_grouped":
                           None if padded_grouped_ms is None else round(padded_grouped_ms / gms, 3)}}
    del qls, ws, gws
    torch.cuda.empty_cache()
    return out


def bench_kv(glq, synth, cb, dev, args, log, layers=36, B=4, ctx=16384):
    """Decode attention over E8-compressed K/V caches, SmolLM3-3B shapes: 16 query
    heads on 4 KV heads, head_dim 128, the 4 bpw recipe (two 16-bit stages), pages of
    16 tokens; B sequences of ctx tokens in every one of the model's layers (one
    call per layer, each with its own cache), so a step streams every cache once."""
    import numpy as np
    import torch

    Hq, Hkv, D = 16, 4, 128
    caches, tables = [], []
    for layer in range(layers):
        host = synth.make_kv([ctx] * B, Hkv, D, 2, 16, seed=2000 + layer, spare_pages=0)
        c = glq.KVCache.from_synth(host, cb)
        if args.index_format == "slot":
            c = c.to_slot_codes()
        caches.append(c)
        tables.append(torch.from_numpy(host.block_table).to(dev))
        kv_bytes = host.kv_bytes()
    lens = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    _, raw = synth.make_q(B, Hq, D, "bf16", seed=2999)
    q = torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(glq.e8kv_attention_workspace_bytes(caches[0], B, Hq, ctx), dtype=torch.uint8, device=dev)

    def step():
        for layer in range(layers):
            glq.e8kv_attention_decode(caches[layer], q, tables[layer], lens, ctx, out=out, workspace=ws)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.kv_steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.kv_steps
    gbs = layers * kv_bytes / (ms * 1e-3) / 1e9
    log("bench: E8 KV attention, SmolLM3-3B shapes, B=%d ctx=%d, %d layers: %.4f ms/step (%.2f us per layer call), "
        "%.1f GB/s of cache" % (B, ctx, layers, ms, ms * 1e3 / layers, gbs))
    out_d = {"workload": "decode attention over E8-compressed paged K/V caches, SmolLM3-3B shapes (16 query heads, 4 KV "
                         "heads, head_dim 128), 4 bpw cache (two 16-bit E8 stages per 8 values, fp32 scale per vector), "
                         "pages of 16 tokens, B=%d sequences of %d tokens, %d layers' caches per step, bf16 q and out"
                         % (B, ctx, layers),
             "index_format": args.index_format, "steps": args.kv_steps, "ms_per_step": round(ms, 5),
             "us_per_layer_call": round(ms * 1e3 / layers, 3), "value": round(gbs, 2), "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4), "cache_bytes_per_layer_call": kv_bytes,
             "tokens_attended_per_s": round(layers * B * ctx / (ms * 1e-3), 1)}
    del caches, tables, ws
    torch.cuda.empty_cache()
    return out_d


def cpu_baseline(layers, wl, B, log, min_seconds=10.0):
    """The oracle (fp64 NumPy, dequantize-then-matmul) on the step's layers, repeated
    until at least min_seconds of CPU work: a bounded sample of the same workload."""
    import numpy as np
    import synth
    from oracle import glq as og

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:  # noqa: BLE001
        pass
    xs = [synth.make_x(l.n, B, wl.act_dtype, wl.seed, k)[0] for k, l in enumerate(layers)]
    t0 = time.perf_counter()
    nbytes, calls = 0, 0
    while time.perf_counter() - t0 < min_seconds:
        k = calls % len(layers)
        l = layers[k]
        og.linear(xs[k], l.sign_in, l.sign_out, l.n_pad, l.m, l.idx0, l.idx1, l.resid_bits, l.wscale,
                  l.resid_scale)
        nbytes += l.index_bytes() + B * (l.n + l.m) * act_bytes(wl.act_dtype) + l.n_pad + l.m_pad
        calls += 1
    dt = time.perf_counter() - t0
    log("bench: cpu oracle %d layer calls in %.2f s -> %.3f GB/s" % (calls, dt, nbytes / dt / 1e9))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": "oracle.glq.linear (fp64 NumPy: row-block dequantization, BLAS matmul, FWHTs) on the "
                      "step's layers in turn at B=%d: %d layer calls (%.2f steps) in %.1f s; dequantization "
                      "runs single-threaded, BLAS on `cores` threads" % (B, calls, calls / len(layers), dt),
            "seconds": round(dt, 3)}


if __name__ == "__main__":
    main()

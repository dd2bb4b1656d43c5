#!/usr/bin/env python3
"""Benchmark of the E8RHTLinear forward on one MI355X.

Step = one decode pass (B = 1) through the Devstral-Small 24B-shaped MLP:
gate 5120->32768, up 5120->32768, down 32768->5120 at 4 bpw (16-bit primary +
16-bit residual index per 8-weight group), bf16 activations; each layer runs
input RHT, the decode matmul against the indices and output RHT.  The layers
are independent calls on seeded synthetic data (no activation between them).
R copies of the three layers' index arrays (>= 1 GiB in total) are rotated so
every step reads its indices from HBM, not from the 256 MB Infinity Cache.
The 16-bit index arrays are relabelled once, before timing, as slot codes
(glq_slot_codes: the same codebook entries, decoded with one LDS read);
--index-format codebook times the codebook indices themselves, and the run
reports the other format beside the headline.

value   = sum over the step's layers of (index bytes + x bytes + y bytes + sign
          bytes) / step time, in GB/s (inputs resident in HBM before timing starts).
roofline: at B = 1 each layer call is two kernel launches (fused_decode_kernel,
          then the small output_blocks_kernel); events around every call (same
          stream) in a second loop give their average duration; achieved = the
          calls' bytes / their time.
prefill: the 2048-token prefill of the SmolLM3-3B gate shape (2048->11008,
          3 bpw), its MFMA matmul timed the same way, in TFLOP/s.
block_b1: the seven linears of a SmolLM3-3B decoder block (3 bpw, fp16) at B = 1,
          issued eagerly from Python and replayed from one captured HIP graph; the
          small layers are launch-bound, and the graph removes the host launch cost.
cpu_baseline: the fp64 oracle on the step's layers in turn, for >= 10 s of host CPU work.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--block-steps", type=int, default=500)
    ap.add_argument("--no-recipes", action="store_true", help="skip the 5-8 bpw decode measurement")
    ap.add_argument("--recipe-steps", type=int, default=300)
    ap.add_argument("--no-blockdiag", action="store_true", help="skip the unpadded (block-diagonal) measurement")
    ap.add_argument("--no-kv", action="store_true", help="skip the E8 KV-cache decode attention measurement")
    ap.add_argument("--kv-steps", type=int, default=50)
    ap.add_argument("--index-format", choices=["slot", "codebook"], default="slot",
                    help="16-bit index arrays as slot codes (default) or as codebook indices")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run 10 plain device-to-device copies of BYTES (scale for HBM traffic counters)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only summarize four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of this "
                         "bench and of --calibrate-copy) into " + os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--copy-bytes", type=int, default=1 << 28, help="BYTES of the --calibrate-copy run summarized")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.copy_bytes)
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

    def step(i):
        row = qls[i % copies]
        for k in range(len(row)):
            glq.e8rht_linear(row[k], xs[k], out=ys[k], workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("bench: timing %d steps" % args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log("bench: %.4f ms/step (wall %.4f), %.1f GB/s" % (ms_per_step, wall * 1e3 / args.steps, value))

    # per-call timing: at B = 1 every layer call is fused_decode_kernel followed by
    # output_blocks_kernel; events on the launch stream around each call
    n_ev = args.steps * len(host_layers)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i in range(args.steps):
        row = qls[(args.warmup + i) % copies]
        for k in range(len(row)):
            a, b = evs[i * len(row) + k]
            a.record()
            glq.e8rht_linear(row[k], xs[k], out=ys[k], workspace=ws)
            b.record()
    torch.cuda.synchronize()
    per_layer_ms = [float(np.mean([evs[i * len(host_layers) + k][0].elapsed_time(evs[i * len(host_layers) + k][1])
                                   for i in range(args.steps)])) for k in range(len(host_layers))]
    achieved = sum(launch_bytes) / (sum(per_layer_ms) * 1e-3) / 1e9
    log("bench: per-launch ms %s -> %.1f GB/s" % (["%.4f" % t for t in per_layer_ms], achieved))

    # the other index format, same loop and step count
    other_steps = min(args.steps, 300)
    e0.record()
    for i in range(other_steps):
        row = qls_other[i % copies]
        for k in range(len(row)):
            glq.e8rht_linear(row[k], xs[k], out=ys[k], workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    other_value = step_bytes / (e0.elapsed_time(e1) / other_steps * 1e-3) / 1e9
    log("bench: %s indices: %.1f GB/s" % ("codebook" if slot else "slot-code", other_value))

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
        "dtype": "f32",
        "arith": "activations in 16-bit fixed point per 64 columns (4 int4 digit planes), exact i32 dot "
                 "products against the int4-packed codewords, f32 scaling, reduction and transforms",
        "data": "synthetic",
        "config": {
            "workload": "Devstral-Small-24B MLP decode (gate 5120->32768, up 5120->32768, down 32768->5120), "
                        "4 bpw (16+16-bit E8 indices), B=%d, bf16 activations, uniform seeded indices" % B,
            "batch": B,
            "index_format": ("slot codes: the 16-bit indices relabelled once at load (glq_slot_codes), "
                             "same entries and bytes") if slot else "codebook indices",
            "index_bytes_per_step": idx_bytes,
            "algorithmic_bytes_per_step": step_bytes,
            "rotating_copies": copies,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("fused_decode_kernel + output_blocks_kernel (one E8RHTLinear call at B = 1: input RHT, "
                       "decode matmul, row-block output transform; then the fixed-order split sum and the "
                       "cross-block output transform)") if B == 1 else
                      "staged decode launches (RHT, quant_u, gemv_lds, RHT)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(launch_bytes) if B == 1 else None,
            "per_launch_ms": [round(t, 5) for t in per_layer_ms],
            "bytes_per_launch": launch_bytes,
        },
    }

    result["other_index_format"] = {"index_format": "codebook indices" if slot else "slot codes",
                                    "value": round(other_value, 2), "unit": "GB/s", "steps": other_steps}

    if not args.no_prefill:
        result["prefill"] = bench_prefill(glq, synth, cb, dev, args, log)

    if not args.no_block:
        result["block_b1"] = bench_block_graph(glq, synth, cb, dev, args, log)

    if not args.no_recipes and B == 1:
        result["recipes_b1"] = bench_recipes(glq, synth, cb, dev, args, log, value)

    if not args.no_blockdiag and B == 1:
        result["blockdiag_b1"] = bench_blockdiag(glq, synth, cb, dev, args, log, ms_per_step)

    if not args.no_kv:
        result["kv_attention"] = bench_kv(glq, synth, cb, dev, args, log)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host_layers, wl, B, log)

    print(json.dumps(result), flush=True)


# ---- HBM traffic of the fused kernel from rocprofv3 counters -------------------------
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_decode_kernel_devstral_mlp_b1_traffic.txt")
FUSED_KERNEL_NAMES = ("fused_decode_kernel", "output_blocks_kernel")  # the two launches of a B = 1 call
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
    """Write TRAFFIC_FILE: FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the two kernels of
    a B = 1 call, each scaled by bytes / counter of a plain copy of copy_bytes (reads
    and writes copy_bytes each)."""
    import numpy as np
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    out = {}
    for name, folder, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(folder, counter)
        out[name + "_kib"] = 0.0
        out[name + "_dispatches"] = 0
        for kname in FUSED_KERNEL_NAMES:  # per call: the sum of the two kernels' medians
            vals = [v for k, v in rows if kname in k]
            out[name + "_kib"] += float(np.median(vals))
            out[name + "_dispatches"] += len(vals)
    for name, folder, counter in (("copy_fetch", cfetch_dir, "FETCH_SIZE"), ("copy_write", cwrite_dir, "WRITE_SIZE")):
        rows = _pmc_rows(folder, counter)
        big = max(v for _, v in rows)
        vals = [v for _, v in rows if v > 0.5 * big]  # the copy dispatches (not small setup kernels)
        out[name + "_kib"] = float(np.median(vals))
    sf = copy_bytes / (out["copy_fetch_kib"] * 1024.0)
    sw = copy_bytes / (out["copy_write_kib"] * 1024.0)
    traffic = out["fetch_kib"] * 1024.0 * sf + out["write_kib"] * 1024.0 * sw
    lines = [
        "# HBM traffic of one B = 1 call (%s), Devstral-Small-24B MLP decode" % " + ".join(FUSED_KERNEL_NAMES),
        "# commands (from the repository root, after cd /tmp && export TMPDIR=/tmp for the profiler):",
        "#   rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR --output-format csv -- python3 bench.py --steps 3 --warmup 1 "
        "--no-cpu-baseline --no-prefill --no-block --no-recipes --no-blockdiag --no-kv",
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
        "copy_fetch_kib: %.1f -> fetch scale %.4f" % (out["copy_fetch_kib"], sf),
        "copy_write_kib: %.1f -> write scale %.4f" % (out["copy_write_kib"], sw),
        "traffic_bytes_per_call: %d" % int(round(traffic)),
    ]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_traffic(launch_bytes):
    """HBM bytes per B = 1 call from TRAFFIC_FILE, or None when it is missing or was
    taken on other kernel sources.  The file holds medians over the three layers'
    dispatches, so it is reported against their mean algorithmic bytes."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(l.split(": ", 1) for l in fh.read().splitlines() if ": " in l and not l.startswith("#"))
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return int(kv["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def bench_prefill(glq, synth, cb, dev, args, log):
    import numpy as np
    import torch

    wl = synth.WORKLOADS["prefill_gateup"]
    l = synth.make_layer(wl.layers[0], wl.resid_bits, wl.seed, 0)
    M = wl.batches[0]
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
    flops = 2.0 * M * l.m_pad * l.n_pad
    for _ in range(3):
        glq.e8rht_linear(q, x, out=y, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.prefill_steps):
        glq.e8rht_linear(q, x, out=y, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    lin_ms = e0.elapsed_time(e1) / args.prefill_steps

    def matmul_ms(qq):
        # the linear's prefill steps one by one, events around the matmul: slot codes
        # on fragment-order u (gemm_shared_kernel), codebook indices on row-order u
        # (gemm_lds_kernel)
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
        return float(np.mean([a.elapsed_time(b) for a, b in evs])), frag

    gemm_ms, frag = matmul_ms(q)
    tflops = flops / (gemm_ms * 1e-3) / 1e12
    other_tflops = flops / (matmul_ms(q_other)[0] * 1e-3) / 1e12
    log("bench: prefill linear %.4f ms, MFMA matmul %.4f ms = %.1f TFLOP/s" % (lin_ms, gemm_ms, tflops))
    return {
        "workload": "SmolLM3-3B gate 2048->11008 (m_pad 16384), M=2048 tokens, 3 bpw, bf16 activations",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "linear_ms": round(lin_ms, 5),
        "other_index_format": {"index_format": "codebook indices" if args.index_format == "slot" else "slot codes",
                               "value": round(other_tflops, 2), "unit": "TFLOP/s"},
        "roofline": {"bound": "mfma", "kernel": ("gemm_shared_kernel (prefill matmul: a 64-row codeword tile per "
                                                 "k-step dequantized from the LDS codebook into LDS, shared by four "
                                                 "waves as fp16 MFMA operands, fp32 accumulation)") if frag else
                     ("gemm_lds_kernel (prefill matmul: codewords from the LDS codebook dequantized per wave into "
                      "fp16 MFMA operands, fp32 accumulation)"),
                     "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops},
    }


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
    }


def bench_recipes(glq, synth, cb, dev, args, log, value_4bpw):
    """The Devstral MLP decode step at B = 1 with the 5-8 bpw recipes (16-bit
    primary and residual stage plus one or two further 8/16-bit stages), same
    activations, rotating copies and loop as the 4 bpw measurement."""
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
           "value_4bpw": round(value_4bpw, 2), "by_bpw": {}}
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
        out["by_bpw"][str(bpw)] = {"ms_per_step": round(ms, 5), "value": round(gbs, 2),
                                   "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": step_bytes,
                                   "launches_per_layer": 2}
        del qls, ws
        torch.cuda.empty_cache()
    return out


def bench_blockdiag(glq, synth, cb, dev, args, log, padded_ms):
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
    log("bench: unpadded Devstral MLP B=1: %.4f ms/step, %.1f GB/s (padded %.4f ms/step)" % (ms, gbs, padded_ms))
    out = {"workload": "Devstral-Small-24B MLP decode, B=1, bf16, 4 bpw, unpadded: gate, up 5120 -> 32768 and down "
                       "32768 -> 5120 with block-diagonal transforms over 5120 = 4096 + 1024",
           "index_format": args.index_format, "steps": args.steps, "ms_per_step": round(ms, 5),
           "value": round(gbs, 2), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "algorithmic_bytes_per_step": step_bytes, "index_bytes_per_step": idx_bytes,
           "padded_ms_per_step": round(padded_ms, 5), "step_speedup_vs_padded": round(padded_ms / ms, 3)}
    del qls, ws
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

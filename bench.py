"""Benchmark of one packed DiT block forward on one MI355X.

A step is one dit_block_forward call (adaLN, pre-norms, QKV, qk-norm/RoPE,
attention, out projection, SwiGLU FFN) over the text-to-audio+video packing:
512 text + 512 audio + 24576 video tokens, D=2688, 21 heads x 128, SwiGLU
10752, two timestep slots.  Inputs are seeded synthetic tensors already resident
in HBM.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "packed DiT block tokens/s + attention TFLOP/s (% MFMA peak), 25.6k tokens"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(spec, wl, seq_starts=None):
    """The fp64 oracle on the same workload, on the host cores: two bounded
    samples of query rows (K/V for all tokens are always computed), timed and
    extrapolated linearly to the whole block."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    sig = O.resolve_sigmas(wl.slot_plan)
    m1, m2 = 64, 4096  # about 10-15 s of host work at the 25.6k-token block
    times = {}
    for m in (m1, m2):
        rows = np.linspace(0, spec.n - 1, m).astype(np.int64)
        t0 = time.perf_counter()
        O.block(spec, wl.x, wl.rows, wl.pos, sig, wl.weights, qrows=rows, seq_starts=seq_starts)
        times[m] = time.perf_counter() - t0
        log(f"cpu oracle: {m} query rows in {times[m]:.2f} s")
    per_row = max((times[m2] - times[m1]) / (m2 - m1), 1e-9)
    fixed = max(times[m1] - m1 * per_row, 0.0)
    full = fixed + per_row * spec.n
    return {"value": spec.n / full, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"fp64 numpy oracle of the full {spec.n}-token block evaluated at {m1} and "
                       f"{m2} query rows ({times[m1]:.1f} s, {times[m2]:.1f} s; xn, K and V of all "
                       f"tokens in both); block time extrapolated linearly in query rows to "
                       f"{full:.0f} s")}


def measured_traffic(kernel_sources):
    """HBM bytes per attention dispatch from the committed counter summary, if
    it was taken on the current kernel sources (sha256 match), else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attention_t2va_hbm_traffic.md")
    try:
        txt = open(path).read()
        block = txt.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    for rel in kernel_sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["sources_sha256"].get(rel):
                return None
    return rec["traffic_bytes"]


ATTN_SOURCES = ("packed_sequence_diffusion_amd/csrc/k_attn.hip",
                "packed_sequence_diffusion_amd/csrc/dev_common.h",
                "packed_sequence_diffusion_amd/csrc/dit_kernels.h")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t2va")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seqs", type=int, default=1,
                    help="pack the workload as this many independent samples of equal length "
                         "(block-diagonal attention); 1 = one sequence")
    ap.add_argument("--blocks", type=int, default=1,
                    help="a stack of this many blocks with their own weights per step "
                         "(dit_stack_forward); value stays tokens/s per block")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES three times (the "
                         "calibration kernel for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the block is "
              "measured at its single-GPU shape", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {args.copy_probe} bytes")
        return
    from packed_sequence_diffusion_amd import dit
    from synth import workloads as W
    from synth.device import to_device

    spec = W.spec_by_name(args.workload)
    seq_starts = None
    if args.seqs > 1:
        seq_starts = [spec.n * i // args.seqs for i in range(args.seqs + 1)]
    t0 = time.perf_counter()
    wl = W.make_workload(spec)
    dev = to_device(wl)
    cfg = dit.make_config(spec)
    blk = dit.Block(cfg, dev.weights)
    blocks = [blk]
    for i in range(1, args.blocks):  # further blocks: same shape, their own seeded weights
        blocks.append(dit.Block(cfg, to_device(W.make_custom_workload(
            spec, 0xD17200 + i)).weights))
    sig = dit.resolve_sigmas(wl.slot_plan)
    out = torch.empty_like(dev.x)
    ws = blk.workspace(spec.n)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t0:.1f} s; workspace {ws.numel() / 2**30:.2f} GiB; "
        f"{len(blocks)} block(s)")

    def step():
        if len(blocks) == 1:
            blk.forward(dev.x, dev.rows, dev.pos, sig, out=out, workspace=ws, seq_starts=seq_starts)
        else:
            dit.stack_forward(blocks, dev.x, dev.rows, dev.pos, sig, out=out, workspace=ws,
                              seq_starts=seq_starts)

    stream = torch.cuda.current_stream()
    run = step
    if args.graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        run = graph.replay

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log("warmup done")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # one event after every step as well: per-step median and min
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    if not args.graph:
        dit.profile_begin(args.steps * len(blocks))
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        run()
        evs[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    step_ms = sorted([ev0.elapsed_time(evs[0])] +
                     [evs[i - 1].elapsed_time(evs[i]) for i in range(1, args.steps)])
    step_ms = [v / len(blocks) for v in step_ms]
    if args.graph:  # phase split from an eager pass of the same steps
        dit.profile_begin(args.steps * len(blocks))
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    phases = dit.profile_end()
    total_ms = ev0.elapsed_time(ev1)
    ms = total_ms / args.steps / len(blocks)  # per block
    calls = phases.pop("calls")
    ph = {k: v / calls for k, v in phases.items()}
    log("phases (ms/step): " + ", ".join(f"{k}={v:.3f}" for k, v in ph.items()))

    # practical HBM ceiling on this machine: a device copy of the residual stream
    xc = torch.empty_like(dev.x)
    xc.copy_(dev.x)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(20):
        xc.copy_(dev.x)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * dev.x.numel() * 4 * 20 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del xc

    attn_flops = spec.attn_flops()
    if seq_starts is not None:  # block-diagonal: 4 * sum(len^2) * D
        attn_flops = 4.0 * spec.D * sum((b - a) ** 2 for a, b in zip(seq_starts, seq_starts[1:]))
    gemm_flops = spec.gemm_flops()
    attn_ms = ph["attention"]
    gemm_ms = ph["qkv_gemm"] + ph["out_gemm"] + ph["fc1_gemm"] + ph["fc2_gemm"]
    attn_tf = attn_flops / (attn_ms * 1e-3) / 1e12
    gemm_tf = gemm_flops / (gemm_ms * 1e-3) / 1e12
    # bandwidth-bound pre-norm: read x fp32, write xn bf16 per element
    norm_bytes = spec.n * spec.D * (4 + 2)
    norm_gbs = norm_bytes / (ph["norm1"] * 1e-3) / 1e9

    res = {
        "metric": METRIC if spec.name == "t2va" else METRIC.replace("25.6k tokens",
                                                                     f"{spec.n} tokens"),
        "value": spec.n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": step_ms[len(step_ms) // 2],
        "ms_per_step_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded normal inputs and weights; no checkpoint)",
        "config": {
            "workload": (f"{spec.name}: packed DiT block, {spec.n} tokens (512 text + 512 audio + "
                         f"24576 video 16x32x48), D={spec.D}, {spec.H}x{spec.hd} heads, SwiGLU "
                         f"{spec.F}, {spec.slots} timestep slots x 3 tags, rank-24 adaLN")
            if spec.name == "t2va" else f"{spec.name}: n={spec.n} D={spec.D}",
            "n": spec.n, "D": spec.D, "heads": spec.H, "head_dim": spec.hd, "ffn": spec.F,
            "parallelism": "single GPU",
            "samples": args.seqs,
            "blocks_per_step": args.blocks,
            "hip_graph": bool(args.graph),
        },
        "attention_tflops": attn_tf,
        "attention_frac_mfma_peak": attn_tf / PEAK_BF16_TFLOPS,
        "gemm_tflops": gemm_tf,
        "gemm_frac_mfma_peak": gemm_tf / PEAK_BF16_TFLOPS,
        "norm1_gbs": norm_gbs,
        "norm1_frac_hbm_peak": norm_gbs / PEAK_HBM_GBS,
        "hbm_copy_gbs": copy_gbs,
        "norm1_frac_of_copy": norm_gbs / copy_gbs,
        "phases_ms": ph,
        "roofline": {
            "kernel": "k_attn_bf16<128,true> (attention; + k_attn_merge)",
            "bound": "mfma",
            "achieved": attn_tf,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": attn_tf / PEAK_BF16_TFLOPS,
            "traffic": (measured_traffic(ATTN_SOURCES)
                        if spec.name == "t2va" and seq_starts is None else None),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, wl, seq_starts)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

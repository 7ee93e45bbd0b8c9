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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, wl, seq_starts=None):
    """The fp64 oracle run over the whole block (every query row) on the same
    workload, on the host cores, timed once.  At the 25.6k-token block it
    holds one head's [n, n] fp64 score plane at a time (about 16 GB at peak)
    and takes well under a minute on the GPU host."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    sig = O.resolve_sigmas(wl.slot_plan)
    t0 = time.perf_counter()
    O.block(spec, wl.x, wl.rows, wl.pos, sig, wl.weights, seq_starts=seq_starts)
    full = time.perf_counter() - t0
    log(f"cpu oracle: whole block ({spec.n} tokens) in {full:.1f} s")
    return {"value": spec.n / full, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"the whole {spec.n}-token block, every query row: fp64 numpy oracle "
                       f"(BLAS matmuls on {int(cores)} threads), {full:.1f} s"),
            "cpu": cpu_model()}


def profile_record(name, kernel_sources):
    """The JSON record of a committed profile summary, if it was taken on the
    current kernel sources (sha256 match), else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
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
    return rec


def measured_traffic(kernel_sources):
    """HBM bytes per attention dispatch from the committed counter summary."""
    rec = profile_record("attention_t2va_hbm_traffic.md", kernel_sources)
    return rec["traffic_bytes"] if rec else None


def measured_mfma(kernel_sources):
    """MFMA-busy fraction and sustained clock of the attention kernel from the
    committed counter summary."""
    rec = profile_record("t2va_block_mfma_counters.md", kernel_sources)
    return (rec["mfma_busy"], rec["clock_ghz"]) if rec else (None, None)


ATTN_SOURCES = ("packed_sequence_diffusion_amd/csrc/k_attn.hip",
                "packed_sequence_diffusion_amd/csrc/dev_common.h",
                "packed_sequence_diffusion_amd/csrc/dit_kernels.h")


def shard_bench(args, spec):
    """One GPU's share of a P-way token shard: the token-local steps of the block
    (adaLN, pre-norms, GEMMs with their epilogues) at n/P tokens, timed as the
    block at that size minus its attention phase, and the attention of the
    shard's n/P queries against all n keys (dit_attention_shard), timed alone.
    The all-gather of K and V that would precede it is not run (one GPU)."""
    import torch
    from packed_sequence_diffusion_amd import dit
    from synth import workloads as W
    from synth.device import to_device

    P = args.shard
    if spec.n % P or (spec.n // P) % 128:
        print(f"--shard {P}: n = {spec.n} must split into shards of a multiple of 128 tokens",
              file=sys.stderr)
        sys.exit(2)
    m = spec.n // P
    wl = W.make_workload(spec, n=m)  # the packing's first n/P tokens
    dev = to_device(wl)
    cfg = dit.make_config(spec)
    blk = dit.Block(cfg, dev.weights)
    sig = dit.resolve_sigmas(wl.slot_plan)
    out = torch.empty_like(dev.x)
    ws = blk.workspace(m)
    for _ in range(args.warmup):
        blk.forward(dev.x, dev.rows, dev.pos, sig, out=out, workspace=ws)
    torch.cuda.synchronize()
    dit.profile_begin(args.steps)
    for _ in range(args.steps):
        blk.forward(dev.x, dev.rows, dev.pos, sig, out=out, workspace=ws)
    torch.cuda.synchronize()
    ph = dit.profile_end()
    calls = ph.pop("calls")
    ph = {k: v / calls for k, v in ph.items()}
    local_ms = sum(v for k, v in ph.items() if k != "attention")

    # the shard's attention: synthetic q (its m rows), k and v^T of all n tokens
    n, H, hd = spec.n, spec.H, spec.hd
    gen = torch.Generator(device="cuda").manual_seed(0xD17500)
    q = (torch.randn((H, m, hd), generator=gen, device="cuda") * 0.1).to(torch.bfloat16)
    k = (torch.randn((H, n, hd), generator=gen, device="cuda") * 0.1).to(torch.bfloat16)
    vt = torch.randn((H, hd, n), generator=gen, device="cuda").to(torch.bfloat16)
    o = torch.empty((m, H * hd), dtype=torch.bfloat16, device="cuda")
    acfg = dit.make_config(spec)
    wsa = torch.empty(dit.lib.dit_attention_shard_workspace_size(acfg), dtype=torch.uint8,
                      device="cuda")
    qlo = (P // 2) * m  # a middle shard; every shard does the same work
    stream = torch.cuda.current_stream()

    def attn():
        dit.attention_shard(acfg, q, m, qlo, qlo + m, k, vt, n, n, hd ** -0.5, o, workspace=wsa)

    for _ in range(args.warmup):
        attn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        attn()
    ev1.record(stream)
    torch.cuda.synchronize()
    attn_ms = ev0.elapsed_time(ev1) / args.steps
    attn_tf = 4.0 * m * n * spec.D / (attn_ms * 1e-3) / 1e12
    gemm_ms = ph["qkv_gemm"] + ph["out_gemm"] + ph["fc1_gemm"] + ph["fc2_gemm"]
    per_gpu_ms = local_ms + attn_ms
    kv_bytes = 2 * n * spec.D * 2 * (P - 1) / P  # K and V of the other shards, bf16
    res = {
        "metric": f"one GPU's share of a {P}-way token shard of the {spec.name} block",
        "value": m / (per_gpu_ms * 1e-3),
        "unit": "tokens/s per GPU (the K/V all-gather not included)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "shard_tokens": m,
        "keys": n,
        "per_gpu_ms": per_gpu_ms,
        "token_local_ms": local_ms,
        "shard_attention_ms": attn_ms,
        "shard_attention_tflops": attn_tf,
        "shard_attention_frac_mfma_peak": attn_tf / PEAK_BF16_TFLOPS,
        "shard_gemm_tflops": spec.gemm_flops() / P / (gemm_ms * 1e-3) / 1e12,
        "kv_allgather_bytes_per_gpu": kv_bytes,
        "phases_ms": ph,
        "dtype": spec.dtype,
        "data": "synthetic",
    }
    print(json.dumps(res), flush=True)


def device_weights(dit, gen, cfg, seed):
    """Seeded synthetic weights of one prepared piece, made on the device:
    linear weights and biases N(0, 0.02), norm gains 1 + N(0, 0.02), adaLN
    tables N(0, 1)."""
    import torch
    gains = ("norm1", "norm2", "q_norm", "k_norm", "post_attn_norm", "post_ffn_norm")
    gen.manual_seed(seed)
    out = {}
    for f, (dt, shp) in dit.weight_shapes(cfg).items():
        t = torch.randn(shp, generator=gen, device="cuda")
        if f in gains:
            t = 1.0 + 0.02 * t
        elif f != "adaln_table":
            t = 0.02 * t
        out[f] = t.to(torch.bfloat16 if dt == "bf16" else torch.float32).contiguous()
    return out


def time_steps(run, steps, warmup):
    """Mean, median and min milliseconds of `steps` calls of run(i) after
    `warmup` untimed ones, by events on the current stream."""
    import statistics
    import torch
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        run(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, statistics.median(per), min(per)


def zimage_bench(args, spec):
    """Z-Image denoise steps (dit_zimage_forward) at the zimage block shape: a
    128 x 128 latent of 16 channels (4096 image tokens) and 512 caption tokens
    of width 2560, L main layers, 2 noise and 2 context refiners and the final
    layer, with their own seeded device-generated weights.  Each step timed
    without the step cache, then with it (the first L/2 main layers reused
    between refreshes every second step, the caption refined once)."""
    import torch
    from packed_sequence_diffusion_amd import dit
    from synth import workloads as W

    if spec.name != "zimage":
        print("--zimage runs the zimage shape only (--workload zimage)", file=sys.stderr)
        sys.exit(2)
    L, C, cap_len, cap_dim = args.zimage, 16, 512, 2560
    hw = 128
    gen = torch.Generator(device="cuda")
    t0 = time.perf_counter()
    common = dict(D=spec.D, H=spec.H, hd=spec.hd, rope=spec.rope, rope_axes=spec.rope_axes,
                  rope_theta=spec.rope_theta, temb_freq=spec.temb_freq, temb_hidden=spec.temb_hidden)
    cfg = dit.make_config(spec)
    ccfg = dit.make_config(W.BlockSpec("zctx", "zcontext", spec.dtype, n=cap_len, F=spec.F, **common))
    fcfg = dit.make_config(W.BlockSpec("zfin", "zfinal", spec.dtype, n=(hw // 2) ** 2, F=4 * C,
                                       eps=1e-6, **common))
    mk = lambda c, seed: dit.Block(c, device_weights(dit, gen, c, seed))  # noqa: E731
    layers = [mk(cfg, 0xD17900 + i) for i in range(L)]
    noise = [mk(cfg, 0xD17A00 + i) for i in range(2)]
    context = [mk(ccfg, 0xD17B00 + i) for i in range(2)]
    final = mk(fcfg, 0xD17C00)
    gen.manual_seed(0xD17D00)
    rn = lambda *shp: torch.randn(shp, generator=gen, device="cuda")  # noqa: E731
    model = dit.ZimageModel(layers, noise, context, final, C, (0.05 * rn(spec.D, 4 * C)).to(torch.bfloat16),
                            0.02 * rn(spec.D), 1.0 + 0.02 * rn(cap_dim),
                            (0.02 * rn(spec.D, cap_dim)).to(torch.bfloat16), 0.02 * rn(spec.D), 1e-6)
    lat = rn(C, hw, hw)
    cap = rn(cap_len, cap_dim)
    pos = torch.from_numpy(W.zimage_positions(hw // 2, hw // 2, cap_len).astype("float32")).cuda()
    torch.cuda.synchronize()
    log(f"zimage setup ({L} layers + refiners + final): {time.perf_counter() - t0:.1f} s")
    ts = [1.0 - (i + 0.5) / max(args.steps, 1) for i in range(max(args.steps, args.warmup))]
    plain = time_steps(lambda i: model.forward(lat, cap, pos, ts[i % len(ts)]), args.steps, args.warmup)
    cache = dit.ZimageCache(model, hw, hw, cap_len, layers=L // 2, interval=2)
    for i in range(args.warmup):
        model.forward(lat, cap, pos, ts[i % len(ts)], step=i, cache=cache)
    torch.cuda.synchronize()
    cache.reset()  # the timed steps start a new generation: step 0 refreshes
    cached = time_steps(lambda i: model.forward(lat, cap, pos, ts[i % len(ts)], step=i, cache=cache),
                        args.steps, 0)
    res = {
        "metric": f"Z-Image denoise step ({L} layers + 2 noise + 2 context refiners + final), "
                  f"{(hw // 2) ** 2} image + {cap_len} caption tokens",
        "value": 1e3 / cached[0],
        "unit": "steps/s with the step cache",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step_uncached": plain[0],
        "ms_per_step_uncached_median": plain[1],
        "ms_per_step_cached": cached[0],
        "ms_per_step_cached_median": cached[1],
        "cache": {"layers": L // 2, "interval": 2, "caption_refined_once": True},
        "speedup": plain[0] / cached[0],
        "dtype": spec.dtype,
        "data": "synthetic (seeded device-generated weights, latent and caption; no checkpoint)",
    }
    print(json.dumps(res), flush=True)


def evaluation_bench(args, spec):
    """One whole MMH3 denoise evaluation per step (dit_mmh3_forward): patch and
    audio embeddings, the slot plan and token rows, a stack of B blocks of the
    t2va shape with their own weights, the video and audio heads and the
    unpacking of their rows, over the t2va layout (512 text + 512 audio +
    24576 video tokens).  Weights and inputs are seeded synthetic tensors made
    on the device (linear weights N(0, 0.02), gains 1 + N(0, 0.02), adaLN basis
    and bias N(0, 0.02), its table N(0, 1); text, latents N(0, 1)); latent
    channels 16 (video) and 64 (audio) are a synthetic choice."""
    import torch
    from packed_sequence_diffusion_amd import dit
    from synth import workloads as W

    if spec.name != "t2va":
        print("--evaluation runs the t2va layout only", file=sys.stderr)
        sys.exit(2)
    B, C, Ca = args.evaluation, 16, 64
    lay = W.build_layout(512, 16, 64, 96, 256)
    n = lay.seq_len
    gen = torch.Generator(device="cuda")
    weights = lambda cfg, seed: device_weights(dit, gen, cfg, seed)  # noqa: E731

    t0 = time.perf_counter()
    cfg = dit.make_config(spec)
    blocks = [dit.Block(cfg, weights(cfg, 0xD17600 + i)) for i in range(B)]
    heads = []
    for name, F, seed in (("head-video", 4 * C, 0xD17700), ("head-audio", Ca, 0xD17701)):
        hs = W.BlockSpec(name, "final", spec.dtype, n=n, D=spec.D, H=spec.H, hd=spec.hd, F=F,
                         slots=spec.slots, tags=1)
        hc = dit.make_config(hs)
        heads.append(dit.Block(hc, weights(hc, seed)))
    gen.manual_seed(0xD17800)
    lin = lambda *shp: (0.02 * torch.randn(shp, generator=gen, device="cuda"))  # noqa: E731
    model = dit.Mmh3Model(blocks, heads[0], heads[1], C, Ca, lin(spec.D, 4 * C).to(torch.bfloat16),
                          lin(spec.D), lin(spec.D, Ca).to(torch.bfloat16), lin(spec.D))
    text = torch.randn((512, spec.D), generator=gen, device="cuda")
    video = torch.randn((C, 16, 64, 96), generator=gen, device="cuda")
    audio = torch.randn((Ca, 2, 256), generator=gen, device="cuda")
    pos = torch.from_numpy(lay.pos.astype("float32")).cuda()
    sigma_v = 0.42
    torch.cuda.synchronize()
    log(f"evaluation setup ({B} blocks + heads): {time.perf_counter() - t0:.1f} s")

    def step():
        return model.forward(lay.segments, pos, text, video, audio, (), sigma_v)

    run = step
    if args.graph:
        step()  # sizes the workspace before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        run = g.replay
    ms, med, mn = time_steps(lambda i: run(), args.steps, args.warmup)
    res = {
        "metric": f"one MMH3 denoise evaluation ({B} blocks + embeddings + heads), t2va layout",
        "value": 1e3 / ms,
        "unit": "evaluations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_evaluation": ms,
        "ms_per_evaluation_median": med,
        "ms_per_evaluation_min": mn,
        "ms_per_block": ms / B,
        "tokens": n,
        "block_tokens_per_s": n * B / (ms * 1e-3),
        "hip_graph": bool(args.graph),
        "dtype": spec.dtype,
        "data": "synthetic (seeded device-generated weights and latents; no checkpoint)",
    }
    print(json.dumps(res), flush=True)


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
    ap.add_argument("--shard", type=int, default=1, metavar="P",
                    help="time one GPU's share of a P-way token shard of the workload instead "
                         "(the block's token-local phases at n/P tokens and the attention of "
                         "n/P queries against all n keys) and print that line")
    ap.add_argument("--evaluation", type=int, default=0, metavar="B",
                    help="time one whole MMH3 denoise evaluation per step instead (embeddings, "
                         "B blocks of the t2va shape with their own weights, both heads) and "
                         "print that line")
    ap.add_argument("--zimage", type=int, default=0, metavar="L",
                    help="with --workload zimage: time Z-Image denoise steps instead (L main "
                         "layers + refiners + final layer), without and with the step cache, "
                         "and print that line")
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
    if args.shard > 1:
        shard_bench(args, spec)
        return
    if args.evaluation > 0:
        evaluation_bench(args, spec)
        return
    if args.zimage > 0:
        zimage_bench(args, spec)
        return
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

    mfma_busy, clock_ghz = (measured_mfma(ATTN_SOURCES)
                            if spec.name == "t2va" and seq_starts is None else (None, None))
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
            # rocprofv3 counters of the same kernel: the matrix pipe's busy fraction and
            # the clock the chip sustained (the peak above assumes 2.4 GHz)
            "mfma_busy": mfma_busy,
            "clock_ghz": clock_ghz,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, wl, seq_starts)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

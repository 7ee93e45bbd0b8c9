"""Seeded random small block configurations on the GPU against the fp64
oracle, every stage and every token: variant (MMH3, SigLIP, Z-Image, the two
refiners), dtype, head size, head count, FFN width (up to the depths whose
GEMMs run as split-K tails), ragged token counts around the 64/128/256 tile
edges, timestep slots, the checkpoint RoPE and shared adaLN forms, and packed
samples.  The fixed cases of test_gpu_parity.py pin each feature; this sweep
covers their combinations."""

import numpy as np
import pytest

from synth import workloads as W
from tests.gpu_common import compare, log, run_gpu

pytestmark = pytest.mark.gpu
CASES_PER_CHUNK = 40


@pytest.fixture(scope="module")
def dit():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from packed_sequence_diffusion_amd import dit as d
    return d


def random_case(rng, i):
    variant = str(rng.choice(["mmh3", "siglip", "zimage", "refiner", "zcontext"]))
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    hd = int(rng.choice([64, 128]))
    H = int(rng.choice([1, 2, 3, 4]))
    if (H * hd) % 128:
        H += 1
    D = H * hd
    F = int(rng.choice([128, 256, 384, 512] + ([2048, 4096] if dtype == "bf16" else [])))
    n = int(rng.choice([1, 2, 31, 64, 65, 127, 128, 129, 255, 256, 257, 300, 511, 513]))
    rope = {"mmh3": "split_half", "zimage": "interleaved", "siglip": "none", "refiner": "none",
            "zcontext": "interleaved"}[variant]
    if variant == "mmh3" and rng.random() < 0.3:
        rope = "partial"
    if rope == "partial":
        axes = (hd // 4,) * 3
    elif rope == "none":
        axes = (0, 0, 0)
    else:
        axes = (hd // 4, hd // 8 * 3, hd // 8 * 3) if hd == 128 else (16, 24, 24)
    kw = dict(n=n, D=D, H=H, hd=hd, F=F, slots=int(rng.choice([1, 2, 3])) if variant == "mmh3" else 1,
              rope=rope, rope_axes=axes, rope_theta=float(rng.choice([256.0, 1e4])),
              eps=1e-6 if variant == "siglip" else 1e-5, temb_hidden=64, temb_freq=32)
    if variant == "mmh3" and rng.random() < 0.3:
        kw["adaln_shared"] = 1
    starts = None
    if n >= 4 and rng.random() < 0.3:
        cuts = np.sort(rng.choice(np.arange(1, n), size=int(rng.integers(1, 4)), replace=False))
        starts = [0] + [int(c) for c in cuts] + [n]
    return W.BlockSpec(f"random{i}-{variant}-{dtype}", variant, dtype, **kw), starts


@pytest.mark.parametrize("chunk", range(4))
def test_random_small_blocks(dit, chunk):
    rng = np.random.default_rng(9000 + chunk)
    for i in range(CASES_PER_CHUNK):
        spec, starts = random_case(rng, i)
        wl = W.make_custom_workload(spec, 9100 + 100 * chunk + i)
        log(f"[case] chunk {chunk} #{i}: {spec.variant} {spec.dtype} n={spec.n} D={spec.D} "
            f"H={spec.H}x{spec.hd} F={spec.F} slots={spec.slots} rope={spec.rope} "
            f"shared={spec.adaln_shared} starts={starts}")
        _, st = run_gpu(spec, wl, dit, seq_starts=starts)
        errs, bad, t = compare(spec, wl, st, seq_starts=starts)
        assert not bad, f"chunk {chunk} #{i} {spec}: stages over {t}: {bad}"

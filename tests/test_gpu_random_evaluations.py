"""Seeded random whole MMH3 evaluations on the GPU against the oracle's
evaluation: prompt length, frames, latent size, audio length, first / last
keyframes (condition frames at their own timestep slot), the noise level, the
checkpoint forms with a vision block inside the prompt, and the dtype."""

import numpy as np
import pytest

import oracle as O
from synth import workloads as W
from tests.gpu_common import log

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def dit():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from packed_sequence_diffusion_amd import dit as d
    return d


def _case(dit, rng, i):
    import torch
    from synth.device import to_device
    dtype = str(rng.choice(["bf16", "f32"]))
    compat = bool(rng.random() < 0.4)
    text_len = int(rng.choice([1, 7, 16, 33]))
    T = int(rng.choice([1, 2, 3, 5]))
    lh, lw = int(rng.choice([4, 6, 8])), int(rng.choice([4, 8, 10]))
    at = int(rng.choice([2, 5, 12]))
    kf = [[], [(0, T)], [(T - 1, T)], [(0, T), (T - 1, T)]][int(rng.integers(4))] if T > 1 else []
    lay = W.build_layout(text_len, T, lh, lw, at, keyframes=kf)
    hd = 128 if dtype == "bf16" else 64
    C, Ca, D = 16, 64, 256
    rope = dict(rope="partial", rope_axes=(hd // 4,) * 3) if compat else dict(
        rope="split_half", rope_axes=(hd // 4, hd // 8 * 3, hd // 8 * 3))
    sh = int(compat)
    n = lay.seq_len
    bspec = W.BlockSpec(f"reval{i}-{dtype}", "mmh3", dtype, n=n, D=D, H=D // hd, hd=hd,
                        F=384 if dtype == "bf16" else 256, slots=3, adaln_shared=sh, **rope)
    hv = W.BlockSpec("head-v", "final", dtype, n=n, D=D, H=D // hd, hd=hd, F=4 * C, slots=3, tags=1,
                     adaln_shared=sh)
    ha = W.BlockSpec("head-a", "final", dtype, n=n, D=D, H=D // hd, hd=hd, F=Ca, slots=3, tags=1,
                     adaln_shared=sh)
    nb = int(rng.choice([1, 2]))
    wblocks = [W.make_custom_workload(bspec, 12000 + 10 * i + b).weights for b in range(nb)]
    whv = W.make_custom_workload(hv, 12500 + i).weights
    wha = W.make_custom_workload(ha, 12600 + i).weights

    def lin(shape):
        w = (0.02 * rng.standard_normal(shape)).astype(np.float32)
        return W.bf16_round(w) if dtype == "bf16" else w
    wv, bv = lin((D, 4 * C)), (0.02 * rng.standard_normal(D)).astype(np.float32)
    wa, ba = lin((D, Ca)), (0.02 * rng.standard_normal(D)).astype(np.float32)
    text = rng.standard_normal((text_len, D)).astype(np.float32)
    video = rng.standard_normal((C, T, lh, lw)).astype(np.float32)
    audio = rng.standard_normal((Ca, 2, at)).astype(np.float32)
    conds = [rng.standard_normal((C, 1, lh, lw)).astype(np.float32) for _ in kf]
    tags = None
    if compat and text_len > 2:
        tags = np.ones(text_len, np.int32)
        tags[1:text_len // 2] = 0
    sigma_v = float(rng.choice([0.03, 0.42, 0.97]))
    td = torch.bfloat16 if dtype == "bf16" else torch.float32

    def dev_w(spec, w):
        return to_device(W.Workload(spec, np.zeros((1, D), np.float32), None, None, [], w, 0)).weights
    cu = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()  # noqa: E731
    model = dit.Mmh3Model([dit.Block(dit.make_config(bspec), dev_w(bspec, w)) for w in wblocks],
                          dit.Block(dit.make_config(hv), dev_w(hv, whv)),
                          dit.Block(dit.make_config(ha), dev_w(ha, wha)), C, Ca, cu(wv, td), cu(bv),
                          cu(wa, td), cu(ba), audio_slope_rescale=compat)
    pos = lay.pos.astype(np.float32)
    vout, aout = model.forward(lay.segments, cu(pos), cu(text), cu(video), cu(audio),
                               [cu(c) for c in conds], sigma_v,
                               text_tags=None if tags is None else cu(tags, torch.int32))
    torch.cuda.synchronize()
    rv, ra = O.mmh3_forward(bspec, hv, ha, lay.segments, pos.astype(np.float64), text, video, audio,
                            conds, sigma_v, wblocks, whv, wha, wv, bv, wa, ba,
                            audio_slope_rescale=compat, text_tags=tags)
    ev, ea = O.rel_rms(vout.cpu().numpy(), rv), O.rel_rms(aout.cpu().numpy(), ra)
    log(f"[case] random evaluation {i}: {dtype} compat={compat} text={text_len} T={T} {lh}x{lw} "
        f"audio={at} keyframes={kf} blocks={nb} sigma_v={sigma_v} n={n}: video={ev:.2e} audio={ea:.2e}")
    return ev, ea, TOL[dtype]


@pytest.mark.parametrize("i", range(12))
def test_random_mmh3_evaluation(dit, i):
    rng = np.random.default_rng(1200 + i)
    ev, ea, tol = _case(dit, rng, i)
    assert ev <= tol and ea <= tol

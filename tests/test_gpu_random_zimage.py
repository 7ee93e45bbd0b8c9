"""Seeded random Z-Image forwards on the GPU against the oracle: image size,
caption length, main layers, noise and context refiners, and the step-level
cache (shallow layers, refresh interval) over a few denoise steps, both dtypes."""

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


@pytest.mark.parametrize("i", range(6))
def test_random_zimage_forward(dit, i):
    import torch
    from synth.device import to_device
    rng = np.random.default_rng(1500 + i)
    dtype = "bf16" if i % 2 == 0 else "f32"
    hd = 128 if dtype == "bf16" else 64
    D, C, cap_dim = 256, 16, 128
    F = 384 if dtype == "bf16" else 256
    Hl, Wl = int(rng.choice([4, 8, 12, 16])), int(rng.choice([4, 8, 10, 16]))
    cap = int(rng.choice([1, 9, 40]))
    nl, nn, nc = int(rng.integers(1, 4)), int(rng.integers(0, 3)), int(rng.integers(0, 3))
    shallow = int(rng.integers(0, nl + 1))
    interval = int(rng.choice([1, 2, 3]))
    common = dict(D=D, H=D // hd, hd=hd, F=F, rope="interleaved",
                  rope_axes=(hd // 4, hd // 8 * 3, hd // 8 * 3), rope_theta=256.0,
                  temb_freq=256, temb_hidden=1024)
    ntok = (Hl // 2) * (Wl // 2)
    bspec = W.BlockSpec(f"rz{i}-{dtype}", "zimage", dtype, n=ntok + cap, **common)
    cspec = W.BlockSpec(f"rzc{i}-{dtype}", "zcontext", dtype, n=cap, **common)
    fspec = W.BlockSpec(f"rzf{i}-{dtype}", "zfinal", dtype, n=ntok, eps=1e-6, **dict(common, F=4 * C))
    wl = [W.make_custom_workload(bspec, 15000 + 10 * i + j).weights for j in range(nl)]
    wn = [W.make_custom_workload(bspec, 15100 + 10 * i + j).weights for j in range(nn)]
    wc = [W.make_custom_workload(cspec, 15200 + 10 * i + j).weights for j in range(nc)]
    wf = W.make_custom_workload(fspec, 15300 + i).weights

    def lin(shape, s):
        w = (s * rng.standard_normal(shape)).astype(np.float32)
        return W.bf16_round(w) if dtype == "bf16" else w
    emb = dict(x_embed_w=lin((D, 4 * C), 0.2), x_embed_b=(0.02 * rng.standard_normal(D)).astype(np.float32),
               cap_norm=(1 + 0.02 * rng.standard_normal(cap_dim)).astype(np.float32), cap_eps=1e-6,
               cap_embed_w=lin((D, cap_dim), 0.1),
               cap_embed_b=(0.02 * rng.standard_normal(D)).astype(np.float32))

    def dev_w(spec, w):
        return to_device(W.Workload(spec, np.zeros((1, D), np.float32), None, None, [], w, 0)).weights
    blocks = lambda spec, ws: [dit.Block(dit.make_config(spec), dev_w(spec, w)) for w in ws]  # noqa: E731
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    cu = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()  # noqa: E731
    model = dit.ZimageModel(blocks(bspec, wl), blocks(bspec, wn), blocks(cspec, wc),
                            dit.Block(dit.make_config(fspec), dev_w(fspec, wf)), C,
                            cu(emb["x_embed_w"], td), cu(emb["x_embed_b"]), cu(emb["cap_norm"]),
                            cu(emb["cap_embed_w"], td), cu(emb["cap_embed_b"]), emb["cap_eps"])
    pos = W.zimage_positions(Hl // 2, Wl // 2, cap)
    capf = rng.standard_normal((cap, cap_dim)).astype(np.float32)
    cache = dit.ZimageCache(model, Hl, Wl, cap, layers=shallow, interval=interval)
    ocache = {"layers": shallow, "interval": interval}
    ts = [0.9, 0.6, 0.35, 0.1]
    for s, t in enumerate(ts):
        lat = rng.standard_normal((C, Hl, Wl)).astype(np.float32)
        got = model.forward(cu(lat), cu(capf), cu(pos.astype(np.float32)), t, step=s, cache=cache)
        torch.cuda.synchronize()
        ref = O.zimage_forward(bspec, cspec, fspec, lat, capf, pos, t, wl, wn, wc, wf, emb["x_embed_w"],
                               emb["x_embed_b"], emb["cap_norm"], emb["cap_eps"], emb["cap_embed_w"],
                               emb["cap_embed_b"], step=s, cache=ocache)
        e = O.rel_rms(got.cpu().numpy(), ref)
        log(f"[case] random zimage {i} {dtype} {Hl}x{Wl} cap={cap} layers={nl} refiners={nn}/{nc} "
            f"cache={shallow}/{interval} step {s}: rel_rms={e:.2e}")
        assert e <= TOL[dtype]

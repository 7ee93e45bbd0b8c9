"""The Z-Image model around its blocks, on the GPU against the fp64 oracle: the
final layer (LayerNorm without affine, scale from silu(temb), projection), the
channel-last patch layout, and the transformer forward (x and caption
embedders, noise and context refiners, main layers, final layer) over several
denoise steps with and without the step-level cache."""

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


@pytest.mark.parametrize("dtype,n,F", [("bf16", 300, 64), ("f32", 77, 128)])
def test_zimage_final_layer(dit, dtype, n, F):
    import torch
    from synth.device import to_device
    spec = W.BlockSpec(f"zfinal-{dtype}", "zfinal", dtype, n=n, D=256, H=2, hd=128, F=F, eps=1e-6,
                       temb_freq=256, temb_hidden=1024)
    wl = W.make_custom_workload(spec, 6100 + n)
    dev = to_device(wl)
    blk = dit.Block(dit.make_config(spec), dev.weights)
    t = dit.resolve_sigmas(wl.slot_plan)
    out = dit.final_forward(blk, dev.x, None, t)
    torch.cuda.synchronize()
    ref = O.zimage_final_layer(spec, wl.x, O.resolve_sigmas(wl.slot_plan)[0], wl.weights)["out"]
    err = O.rel_rms(out.cpu().numpy(), ref)
    log(f"[case] zimage final layer {dtype} n={n} F={F}: rel_rms={err:.2e}")
    assert err <= TOL[dtype]


def test_patchify_image_bitwise(dit):
    import torch
    rng = np.random.default_rng(91)
    x = rng.standard_normal((16, 10, 14)).astype(np.float32)
    ref = O.patchify_image(x)
    xd = torch.from_numpy(x).cuda()
    for dt in ("f32", "bf16"):
        want = ref if dt == "f32" else W.bf16_round(ref)
        assert np.array_equal(dit.patchify_image(xd, dt).float().cpu().numpy(), want)
    back = dit.unpatchify_image(torch.from_numpy(ref).cuda(), 16, 10, 14).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(back, x)


def _model(dit, dtype):
    """A small Z-Image transformer: 3 main layers, 1 noise refiner, 1 context
    refiner; a 16 x 16 latent of 16 channels (64 image tokens), 40 caption
    tokens of width 128."""
    import torch
    from synth.device import to_device
    hd = 128 if dtype == "bf16" else 64
    D, F, C, cap_dim = 256, 384 if dtype == "bf16" else 256, 16, 128
    common = dict(D=D, H=D // hd, hd=hd, F=F, rope="interleaved",
                  rope_axes=(hd // 4, hd // 8 * 3, hd // 8 * 3), rope_theta=256.0,
                  temb_freq=256, temb_hidden=1024)
    bspec = W.BlockSpec(f"zmain-{dtype}", "zimage", dtype, n=104, **common)
    cspec = W.BlockSpec(f"zctx-{dtype}", "zcontext", dtype, n=40, **common)
    fspec = W.BlockSpec(f"zfin-{dtype}", "zfinal", dtype, n=64, eps=1e-6, **dict(common, F=4 * C))
    wl = [W.make_custom_workload(bspec, 9000 + i).weights for i in range(3)]
    wn = [W.make_custom_workload(bspec, 9100).weights]
    wc = [W.make_custom_workload(cspec, 9200).weights]
    wf = W.make_custom_workload(fspec, 9300).weights
    rng = np.random.default_rng(93)

    def lin(shape, s=0.05):
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
    pos = W.zimage_positions(8, 8, 40)
    oracle_args = (bspec, cspec, fspec, wl, wn, wc, wf, emb)
    return model, oracle_args, pos, C, cap_dim, rng, cu


def _oracle(args, lat, cap, pos, t, step=0, cache=None):
    bspec, cspec, fspec, wl, wn, wc, wf, emb = args
    return O.zimage_forward(bspec, cspec, fspec, lat, cap, pos, t, wl, wn, wc, wf, emb["x_embed_w"],
                            emb["x_embed_b"], emb["cap_norm"], emb["cap_eps"], emb["cap_embed_w"],
                            emb["cap_embed_b"], step=step, cache=cache)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zimage_forward_steps_with_cache(dit, dtype):
    """Four denoise steps, cache interval 2 over the first 2 of 3 main layers:
    steps 0 and 2 refresh, 1 and 3 reuse the stored stream; the caption is
    refined on step 0 only.  Each step against the oracle's evaluation of the
    same cache rules, and the uncached forward on step 0."""
    import torch
    model, args, pos, C, cap_dim, rng, cu = _model(dit, dtype)
    lats = [rng.standard_normal((C, 16, 16)).astype(np.float32) for _ in range(4)]
    cap = rng.standard_normal((40, cap_dim)).astype(np.float32)
    ts = [0.95, 0.7, 0.45, 0.2]
    posd, capd = cu(pos.astype(np.float32)), cu(cap)
    cache = dit.ZimageCache(model, 16, 16, 40, layers=2, interval=2)
    ocache = {"layers": 2, "interval": 2}
    plain = model.forward(cu(lats[0]), capd, posd, ts[0])
    torch.cuda.synchronize()
    ref0 = _oracle(args, lats[0], cap, pos, ts[0])
    e = O.rel_rms(plain.cpu().numpy(), ref0)
    log(f"[case] zimage forward {dtype} uncached: rel_rms={e:.2e}")
    assert e <= TOL[dtype]
    for s in range(4):
        got = model.forward(cu(lats[s]), capd, posd, ts[s], step=s, cache=cache)
        torch.cuda.synchronize()
        ref = _oracle(args, lats[s], cap, pos, ts[s], s, ocache)
        e = O.rel_rms(got.cpu().numpy(), ref)
        log(f"[case] zimage forward {dtype} step {s} (cache interval 2, 2 layers): rel_rms={e:.2e}")
        assert e <= TOL[dtype]
    assert cache.c.caption_valid == 1 and cache.c.shallow_valid == 1
    # a reused step depends on t only: other latents give the same result bit for bit
    a = model.forward(cu(lats[0]), capd, posd, ts[1], step=3, cache=cache)
    b = model.forward(cu(lats[2]), capd, posd, ts[1], step=3, cache=cache)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

"""Pieces around the blocks of the MMH3 model, on the GPU against the fp64
oracle: the output head (final RMSNorm, single-modality shift/scale of the
token's timestep slot, head projection, sign flip), the linear projections on
the block GEMM kernels, and a stack of blocks with their own weights."""

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


@pytest.mark.parametrize("dtype,n,F", [("bf16", 333, 192), ("bf16", 64, 32), ("f32", 130, 128)])
def test_final_layer(dit, dtype, n, F):
    import torch
    from synth.device import to_device
    spec = W.BlockSpec(f"head-{dtype}", "final", dtype, n=n, D=256, H=2, hd=128, F=F, slots=2,
                       tags=1)
    wl = W.make_custom_workload(spec, 6000 + n)
    dev = to_device(wl)
    blk = dit.Block(dit.make_config(spec), dev.weights)
    sig = dit.resolve_sigmas(wl.slot_plan)
    out = dit.final_forward(blk, dev.x, dev.rows, sig)
    torch.cuda.synchronize()
    ref = O.final_layer(spec, wl.x, wl.rows, O.resolve_sigmas(wl.slot_plan), wl.weights)["out"]
    err = O.rel_rms(out.cpu().numpy(), ref)
    log(f"[case] final layer {dtype} n={n} F={F}: rel_rms={err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,m,k,nout,alpha", [("bf16", 300, 192, 96, -0.5),
                                                  ("bf16", 77, 64, 512, 1.0),
                                                  ("bf16", 300, 128, 576, 1.0),  # 192-wide tiles
                                                  ("f32", 130, 48, 128, 2.0)])
def test_linear(dit, dtype, m, k, nout, alpha):
    import torch
    rng = np.random.default_rng(m + k)
    a = rng.standard_normal((m, k)).astype(np.float32)
    w = (0.1 * rng.standard_normal((nout, k))).astype(np.float32)
    b = rng.standard_normal(nout).astype(np.float32)
    if dtype == "bf16":
        a, w = W.bf16_round(a), W.bf16_round(w)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = dit.linear(torch.from_numpy(a).to(td).cuda(), torch.from_numpy(w).to(td).cuda(),
                     torch.from_numpy(b).cuda(), alpha)
    torch.cuda.synchronize()
    ref = O.linear(a.astype(np.float64), w.astype(np.float64), b.astype(np.float64), alpha)
    err = O.rel_rms(out.cpu().numpy(), ref)
    log(f"[case] linear {dtype} {m}x{k} -> {nout} alpha={alpha}: rel_rms={err:.2e}")
    # fp32 accumulation of exact bf16 products: far inside either bar
    assert err <= 1e-5


@pytest.mark.parametrize("dtype,starts", [("bf16", None), ("bf16", [0, 111, 333]), ("f32", None)])
def test_stack_of_blocks(dit, dtype, starts):
    """Three blocks with their own weights: against the oracle's sequence of
    blocks, and bit for bit against three single-block calls."""
    import torch
    from synth.device import to_device
    hd = 128 if dtype == "bf16" else 64
    spec = W.BlockSpec(f"stack-{dtype}", "mmh3", dtype, n=333 if dtype == "bf16" else 130,
                       D=256, H=256 // hd, hd=hd, F=384 if dtype == "bf16" else 256, slots=2,
                       rope="split_half", rope_axes=(hd // 4, hd // 8 * 3, hd // 8 * 3))
    wls = [W.make_custom_workload(spec, 7000 + i) for i in range(3)]
    base = wls[0]  # x, rows, positions and sigmas of the first; weights of each
    devs = [to_device(wl) for wl in wls]
    cfg = dit.make_config(spec)
    blocks = [dit.Block(cfg, d.weights) for d in devs]
    sig = dit.resolve_sigmas(base.slot_plan)
    x, rows, pos = devs[0].x, devs[0].rows, devs[0].pos
    out = dit.stack_forward(blocks, x, rows, pos, sig, seq_starts=starts)
    h = x
    for b in blocks:
        h = b.forward(h, rows, pos, sig, seq_starts=starts)
    torch.cuda.synchronize()
    assert torch.equal(out, h)
    ref = O.stack(spec, base.x, base.rows, base.pos, O.resolve_sigmas(base.slot_plan),
                  [wl.weights for wl in wls], seq_starts=starts)
    got = out.cpu().numpy().astype(np.float64)
    x64 = base.x.astype(np.float64)
    e_out = O.rel_rms(got, ref)
    e_delta = O.rel_rms(got - x64, ref - x64)
    log(f"[case] stack {dtype} starts={starts}: out={e_out:.2e} out-x={e_delta:.2e}")
    tol = TOL[dtype]
    # out - x is a difference of fp32-stored vectors: add their storage rounding
    rms = lambda a: float(np.sqrt(np.mean(a * a)))  # noqa: E731
    floor = 2 * 2.0 ** -24 * (rms(ref) + rms(x64)) / rms(ref - x64)
    assert e_out <= tol and e_delta <= tol + floor


def test_stream_packing_kernels(dit):
    """patchify / unpatchify / pack / unpack against the oracle's layouts,
    bit for bit (bf16 rows are the RNE rounding of the same values)."""
    import torch
    rng = np.random.default_rng(71)
    v = rng.standard_normal((16, 3, 8, 12)).astype(np.float32)
    a = rng.standard_normal((64, 2, 10)).astype(np.float32)
    vd, ad = torch.from_numpy(v).cuda(), torch.from_numpy(a).cuda()
    rv, ra = O.patchify_video(v), O.pack_audio(a)
    for dt in ("f32", "bf16"):
        want_v = rv if dt == "f32" else W.bf16_round(rv)
        want_a = ra if dt == "f32" else W.bf16_round(ra)
        got_v = dit.patchify_video(vd, dt).float().cpu().numpy()
        got_a = dit.pack_audio(ad, dt).float().cpu().numpy()
        assert np.array_equal(got_v, want_v) and np.array_equal(got_a, want_a)
    back_v = dit.unpatchify_video(torch.from_numpy(rv).cuda(), 16, 3, 8, 12).cpu().numpy()
    back_a = dit.unpack_audio(torch.from_numpy(ra).cuda(), 64, 10).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(back_v, v) and np.array_equal(back_a, a)


def test_rms_norm(dit):
    import torch
    rng = np.random.default_rng(72)
    x = rng.standard_normal((77, 384)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(384)).astype(np.float32)
    got = dit.rms_norm(torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda(), 1e-5).cpu().numpy()
    ref = O.rms_norm(x.astype(np.float64), g.astype(np.float64), 1e-5)
    assert O.rel_rms(got, ref) <= 1e-6


def _mmh3_setup(dit, dtype, compat):
    """A small MMH3 model and one evaluation's inputs: text, a first-frame
    keyframe, stereo audio and two video frames; two blocks with their own
    weights; video and audio heads.  ``compat``: the checkpoint forms (shared
    RoPE frequencies over 3k pairs, one adaLN basis for every slot in blocks and
    heads), the audio velocity pre-multiplied by d(sigma_a)/d(sigma_v) and a
    vision block inside the prompt (per-token text tags)."""
    import torch
    from synth.device import to_device
    hd = 128 if dtype == "bf16" else 64
    lay = W.build_layout(16, 2, 8, 8, 12, keyframes=[(0, 2)])
    n = lay.seq_len
    C, Ca, D = 16, 64, 256
    rope = dict(rope="partial", rope_axes=(hd // 4,) * 3) if compat else dict(
        rope="split_half", rope_axes=(hd // 4, hd // 8 * 3, hd // 8 * 3))
    sh = int(compat)
    bspec = W.BlockSpec(f"model-{dtype}", "mmh3", dtype, n=n, D=D, H=D // hd, hd=hd,
                        F=384 if dtype == "bf16" else 256, slots=3, adaln_shared=sh, **rope)
    hv = W.BlockSpec("head-v", "final", dtype, n=n, D=D, H=D // hd, hd=hd, F=4 * C, slots=3, tags=1,
                     adaln_shared=sh)
    ha = W.BlockSpec("head-a", "final", dtype, n=n, D=D, H=D // hd, hd=hd, F=Ca, slots=3, tags=1,
                     adaln_shared=sh)
    wblocks = [W.make_custom_workload(bspec, 8000 + i).weights for i in range(2)]
    whv = W.make_custom_workload(hv, 8100).weights
    wha = W.make_custom_workload(ha, 8101).weights
    rng = np.random.default_rng(81)

    def lin(shape):
        w = (0.02 * rng.standard_normal(shape)).astype(np.float32)
        return W.bf16_round(w) if dtype == "bf16" else w
    wv, bv = lin((D, 4 * C)), (0.02 * rng.standard_normal(D)).astype(np.float32)
    wa, ba = lin((D, Ca)), (0.02 * rng.standard_normal(D)).astype(np.float32)
    host = dict(text=rng.standard_normal((16, D)).astype(np.float32),
                video=rng.standard_normal((C, 2, 8, 8)).astype(np.float32),
                audio=rng.standard_normal((Ca, 2, 12)).astype(np.float32),
                cond=rng.standard_normal((C, 1, 8, 8)).astype(np.float32),
                pos=lay.pos.astype(np.float32), sigma_v=0.42, tags=None)
    if compat:
        host["tags"] = np.full(16, 1, np.int32)
        host["tags"][4:10] = 0
    td = torch.bfloat16 if dtype == "bf16" else torch.float32

    def dev_weights(spec, w):
        wl = W.Workload(spec, np.zeros((1, D), np.float32), None, None, [], w, 0)
        return to_device(wl).weights
    blocks = [dit.Block(dit.make_config(bspec), dev_weights(bspec, w)) for w in wblocks]
    head_v = dit.Block(dit.make_config(hv), dev_weights(hv, whv))
    head_a = dit.Block(dit.make_config(ha), dev_weights(ha, wha))
    cu = lambda a, t=torch.float32: torch.from_numpy(a).to(t).cuda()  # noqa: E731
    model = dit.Mmh3Model(blocks, head_v, head_a, C, Ca, cu(wv, td), cu(bv), cu(wa, td), cu(ba),
                          audio_slope_rescale=compat)
    dev = dict(pos=cu(host["pos"]), text=cu(host["text"]), video=cu(host["video"]),
               audio=cu(host["audio"]), conds=[cu(host["cond"])],
               tags=None if host["tags"] is None else cu(host["tags"], torch.int32))
    oracle_args = (bspec, hv, ha, wblocks, whv, wha, wv, bv, wa, ba)
    return lay, model, dev, host, oracle_args


def _run(model, lay, dev, sigma_v):
    return model.forward(lay.segments, dev["pos"], dev["text"], dev["video"], dev["audio"], dev["conds"],
                         sigma_v, text_tags=dev["tags"])


@pytest.mark.parametrize("dtype,compat", [("bf16", False), ("f32", False), ("bf16", True),
                                          ("f32", True)])
def test_mmh3_denoise_evaluation(dit, dtype, compat):
    """One whole evaluation at a small size against the oracle's evaluation
    from the same seeded pieces."""
    import torch
    lay, model, dev, host, oa = _mmh3_setup(dit, dtype, compat)
    vout, aout = _run(model, lay, dev, host["sigma_v"])
    torch.cuda.synchronize()
    bspec, hv, ha, wblocks, whv, wha, wv, bv, wa, ba = oa
    rv, ra = O.mmh3_forward(bspec, hv, ha, lay.segments, host["pos"].astype(np.float64), host["text"],
                            host["video"], host["audio"], [host["cond"]], host["sigma_v"], wblocks, whv,
                            wha, wv, bv, wa, ba, audio_slope_rescale=compat, text_tags=host["tags"])
    ev = O.rel_rms(vout.cpu().numpy(), rv)
    ea = O.rel_rms(aout.cpu().numpy(), ra)
    log(f"[case] mmh3 evaluation {dtype} compat={compat} n={lay.seq_len}: video={ev:.2e} audio={ea:.2e}")
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


def test_mmh3_evaluation_graph_replay(dit):
    """The whole evaluation (patch and audio embeddings, token rows, two blocks,
    both heads, unpacking) captured in one HIP graph replays to the eager result
    bit for bit, with eager evaluations at another sigma between the replays."""
    import torch
    lay, model, dev, host, _ = _mmh3_setup(dit, "bf16", True)
    sv = host["sigma_v"]
    v_ref, a_ref = _run(model, lay, dev, sv)  # also sizes the workspace before capture
    torch.cuda.synchronize()
    v_ref, a_ref = v_ref.clone(), a_ref.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            v_g, a_g = _run(model, lay, dev, sv)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        v_g.fill_(float("nan"))
        a_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(v_g, v_ref) and torch.equal(a_g, a_ref)
        log(f"[case] mmh3 evaluation graph replay {rep}: equal={same}")
        assert same
        _run(model, lay, dev, 0.9)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
    assert torch.isfinite(v_ref).all() and torch.isfinite(a_ref).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reference_layout_stack(dit, dtype):
    """A reference layout ([MMH3] Layout::ref2va: a reference image, a
    reference clip with its soundtrack and a reference audio block before the
    target's audio and video) through two blocks: four timestep slots (video,
    audio, the condition slot at max(t_v, 0.999) and the reference-audio slot
    at t = 1 exactly), token rows slot * 3 + tag as [MMH3] MiniMaxH3::forward
    assigns them.  The library's slot planner and the oracle's are run
    independently and must agree; the stack's output is checked per token
    row, and the modulation rows of the t = 1 slot are checked directly
    (they read the adaLN table's last row with weight 1)."""
    import torch
    from synth.device import to_device
    from tests.gpu_common import row_rel
    lay = W.build_layout(16, 3, 8, 8, 4, refs=[("image", 8, 8), ("video", 2, 8, 8, 3), ("audio", 4)])
    n = lay.seq_len
    sv = 0.6
    lib_sig, lib_slot = dit.mmh3_slots(sv, has_cond=True, has_ref_audio=True)
    ts, o_slot = O.mmh3_slots(sv, 12.0, 3.0, 0.999, 1.0, True, True)
    assert len(lib_sig) == 4 and lib_slot == o_slot
    assert ts[o_slot["ref_audio"]] == 1.0 and lib_sig[lib_slot["ref_audio"]] == 0.0
    np.testing.assert_allclose(lib_sig, [1.0 - t for t in ts], rtol=0, atol=1e-15)
    kind_slot_tag = {"text": (lib_slot["video"], W.TAG_TEXT), "video": (lib_slot["video"], W.TAG_VIDEO),
                     "audio": (lib_slot["audio"], W.TAG_AUDIO), "ref_image": (lib_slot["cond"], W.TAG_VIDEO),
                     "ref_audio": (lib_slot["ref_audio"], W.TAG_AUDIO)}
    rows = W._rows_for(lay, kind_slot_tag, 3)
    np.testing.assert_array_equal(rows, O.mmh3_token_rows(lay.segments, o_slot))
    hd = 128 if dtype == "bf16" else 64
    spec = W.BlockSpec(f"ref-{dtype}", "mmh3", dtype, n=n, D=256, H=256 // hd, hd=hd,
                       F=384 if dtype == "bf16" else 256, slots=4, rope="split_half",
                       rope_axes=(hd // 4, hd // 8 * 3, hd // 8 * 3))
    pos = lay.pos.astype(np.float32)
    wls = [W.make_custom_workload(spec, 7100 + i, pos=pos, rows=rows, sigmas=lib_sig) for i in range(2)]
    devs = [to_device(wl) for wl in wls]
    cfg = dit.make_config(spec)
    blocks = [dit.Block(cfg, d.weights) for d in devs]
    x, drows, dpos = devs[0].x, devs[0].rows, devs[0].pos
    out = dit.stack_forward(blocks, x, drows, dpos, lib_sig)
    mods = torch.empty(dit.mod_shape(cfg), dtype=torch.float32, device="cuda")
    blocks[0].adaln_eval(lib_sig, mods)
    torch.cuda.synchronize()
    o_sig = [1.0 - t for t in ts]
    ref = O.stack(spec, wls[0].x, rows, pos, o_sig, [wl.weights for wl in wls])
    got = out.cpu().numpy().astype(np.float64)
    x64 = wls[0].x.astype(np.float64)
    u = 2.0 ** -24
    nrm = lambda a: np.sqrt(np.sum(a * a, axis=-1))  # noqa: E731
    e_out = row_rel(got, ref)
    e_delta = row_rel(got - x64, ref - x64) - 2 * u * (nrm(ref) + nrm(x64)) / nrm(ref - x64)
    w0 = {k: v.astype(np.float64) for k, v in wls[0].weights.items()}
    tsv = [O.mmh3_timestep(s) for s in o_sig]
    ref_mods = O.adaln_mods(w0["adaln_basis"], w0["adaln_bias"], w0["adaln_table"], tsv, 3, 6, spec.D)
    e_mods = row_rel(mods.cpu().numpy(), ref_mods)
    ra = lib_slot["ref_audio"]
    log(f"[case] reference layout {dtype} n={n} slots={len(lib_sig)}: out max={e_out.max():.2e} "
        f"out-x max={e_delta.max():.2e} mods max={e_mods.max():.2e} "
        f"(t=1 slot rows {e_mods[3 * ra:3 * ra + 3].max():.2e})")
    tol = TOL[dtype]
    assert e_out.max() <= tol and e_delta.max() <= tol
    assert e_mods.max() <= 1e-5  # modulation rows are fp32 in both configurations

"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and refuses bad arguments on the host before any launch (no
GPU call is made: every case fails validation)."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit.h")
LIB = os.path.join(ROOT, "packed_sequence_diffusion_amd", "libdit.so")


@pytest.fixture(scope="module")
def dit():
    if not os.path.exists(LIB):
        from packed_sequence_diffusion_amd import build
        build.build()
    from packed_sequence_diffusion_amd import dit as d
    return d


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z_0-9]+)\s*\(", txt)))


def test_header_functions_exported(dit):
    names = declared_functions()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dit_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(dit.lib, n)


def test_binding_refuses_to_import_without_the_library(tmp_path):
    """The binding has no CPU fallback: a copy of it next to no built library
    raises ImportError on import instead of running anything."""
    pkg = tmp_path / "pkg_without_lib"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    src = os.path.join(ROOT, "packed_sequence_diffusion_amd", "dit.py")
    (pkg / "dit.py").write_text(open(src).read())
    code = ("import sys\n"
            "try:\n"
            "    import pkg_without_lib.dit\n"
            "except ImportError as e:\n"
            "    print('refused:', e); sys.exit(0)\n"
            "sys.exit(3)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout and "no CPU fallback" in r.stdout


def test_abi_version(dit):
    assert dit.lib.dit_abi_version() == 7


def test_sigma_remap_printed_points(dit):
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "sigma_remap.json")))
    for s in g["involution_points"]:
        a = dit.sigma_remap(s, 12.0, 3.0)
        assert abs(dit.sigma_remap(a, 3.0, 12.0) - s) < g["involution_tol"]
        assert abs(a - s / (4.0 - 3.0 * s)) < 1e-14
    h = g["slope_step"]
    for s in g["slope_points"]:
        num = (dit.sigma_remap(s + h, 12.0, 3.0) - dit.sigma_remap(s - h, 12.0, 3.0)) / (2 * h)
        assert abs(num - dit.sigma_remap_slope(s, 12.0, 3.0)) < g["slope_tol"]


def test_configs_validate(dit):
    for spec in W.SPECS:
        dit.validate(dit.make_config(spec))
        assert dit.lib.dit_prepared_size(ctypes.byref(dit.make_config(spec))) > 0


def _cfg(dit, **kw):
    spec = W.spec_by_name("t2va")
    c = dit.make_config(spec)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("hd", 96, -6), ("D", 2560, -2), ("dtype", 7, -3), ("variant", 9, -1), ("slots", 0, -6),
    ("slots", 9, -6), ("F", 100, -6), ("rank", 0, -6), ("grid", 1, -1), ("rope", 5, -1),
    ("adaln_shared", -1, -1),
])
def test_config_refusals(dit, field, value, status):
    c = _cfg(dit, **{field: value})
    assert dit.lib.dit_validate_config(ctypes.byref(c)) == status
    assert dit.last_error()
    assert dit.lib.dit_prepared_size(ctypes.byref(c)) == 0


def test_rope_axes_must_sum_to_head_dim(dit):
    c = _cfg(dit)
    c.rope_axes[0] = 30
    assert dit.lib.dit_validate_config(ctypes.byref(c)) == -2


def test_partial_rope_and_shared_adaln_configs(dit):
    ok = _cfg(dit, rope=dit.ROPE_PARTIAL)
    for a in range(3):
        ok.rope_axes[a] = 32  # k = 16 shared frequencies, 96 of 128 dims rotated
    assert dit.lib.dit_validate_config(ctypes.byref(ok)) == 0
    # the shared frequency vector is part of the prepared weights
    assert dit.lib.dit_prepared_size(ctypes.byref(ok)) > dit.lib.dit_prepared_size(ctypes.byref(_cfg(dit)))
    bad = _cfg(dit, rope=dit.ROPE_PARTIAL)  # (32, 48, 48): axes differ
    assert dit.lib.dit_validate_config(ctypes.byref(bad)) == -1
    big = _cfg(dit, rope=dit.ROPE_PARTIAL)
    for a in range(3):
        big.rope_axes[a] = 44  # 3 * 44 > 128
    assert dit.lib.dit_validate_config(ctypes.byref(big)) == -2
    z = dit.make_config(W.spec_by_name("zimage"))
    z.rope = dit.ROPE_PARTIAL
    for a in range(3):
        z.rope_axes[a] = 32
    assert dit.lib.dit_validate_config(ctypes.byref(z)) == -6
    sh = _cfg(dit, adaln_shared=1)
    assert dit.lib.dit_validate_config(ctypes.byref(sh)) == 0
    assert dit.lib.dit_prepared_size(ctypes.byref(sh)) == dit.lib.dit_prepared_size(ctypes.byref(_cfg(dit)))
    assert dit.lib.dit_validate_config(ctypes.byref(_cfg(dit, adaln_shared=2))) == -1
    sg = dit.make_config(W.spec_by_name("siglip"))
    sg.adaln_shared = 1
    assert dit.lib.dit_validate_config(ctypes.byref(sg)) == -1
    # a partial-RoPE block needs its frequency vector
    w = dit.DitWeights()
    for f in ("w_qkv", "w_out", "w_fc1", "w_fc2", "norm1", "norm2", "q_norm", "k_norm",
              "adaln_basis", "adaln_table"):
        setattr(w, f, 256)
    need = dit.lib.dit_prepared_size(ctypes.byref(ok))
    assert dit.lib.dit_prepare_weights(ctypes.byref(ok), ctypes.byref(w), 256, need, None) == -1
    assert "rope_freq" in dit.last_error()


def test_zimage_model_configs_and_workspace(dit):
    z = W.spec_by_name("zimage")
    cfgs = {v: dit.make_config(W.small_spec(z, variant=v, F=64 if v == "zfinal" else z.F))
            for v in ("zimage", "zcontext", "zfinal")}
    for c in cfgs.values():
        assert dit.lib.dit_validate_config(ctypes.byref(c)) == 0
    # the context refiner has no timestep tensors; the final layer no block weights
    assert dit.lib.dit_prepared_size(ctypes.byref(cfgs["zcontext"])) < \
        dit.lib.dit_prepared_size(ctypes.byref(cfgs["zimage"]))
    Lc = dit.workspace_layout(cfgs["zcontext"], 512)
    assert Lc.mods == dit.NONE_OFFSET and Lc.temb == dit.NONE_OFFSET and Lc.y != dit.NONE_OFFSET
    Lf = dit.workspace_layout(cfgs["zfinal"], 4096)
    assert Lf.q == dit.NONE_OFFSET and Lf.temb != dit.NONE_OFFSET and Lf.mods != dit.NONE_OFFSET
    # a block entry point refuses the head, the head entry point refuses a block
    assert _fwd(dit, cfgs["zfinal"]) == -6
    m = dit.DitZimageModel()
    m.block, m.context, m.final_layer = (ctypes.pointer(cfgs[v]) for v in ("zimage", "zcontext", "zfinal"))
    arr = (ctypes.c_void_p * 2)(256, 512)
    m.layers, m.n_layers = arr, 2
    m.noise_refiners, m.n_noise_refiners = arr, 1
    m.context_refiners, m.n_context_refiners = arr, 1
    m.final_w, m.in_channels, m.cap_dim = 256, 16, 2560
    m.x_embed_w, m.cap_norm, m.cap_embed_w, m.cap_eps = 256, 256, 256, 1e-6
    size = dit.lib.dit_zimage_workspace_size(ctypes.byref(m), 128, 128, 512)
    assert size > 4608 * 3072 * 4
    assert dit.lib.dit_zimage_workspace_size(ctypes.byref(m), 127, 128, 512) == 0
    m.in_channels = 15  # 4C = 60: not a multiple of the bf16 GEMM depth
    assert dit.lib.dit_zimage_workspace_size(ctypes.byref(m), 128, 128, 512) == 0
    m.in_channels = 16
    m.context = ctypes.pointer(cfgs["zimage"])
    assert dit.lib.dit_zimage_workspace_size(ctypes.byref(m), 128, 128, 512) == 0


def test_workspace_layout_monotone(dit):
    c = _cfg(dit)
    L = dit.workspace_layout(c, 25600)
    assert L.ldn == 25600
    offs = [L.mods, L.rope, L.xn, L.q, L.k, L.vt, L.o, L.x1, L.a, L.part]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.y == dit.NONE_OFFSET
    # the bf16 QKV GEMM writes q, k and v^T directly: no staged qkv panel
    assert L.qkv == dit.NONE_OFFSET
    toy = dit.make_config(W.spec_by_name("toy"))
    Lt = dit.workspace_layout(toy, 256)
    assert Lt.qkv != dit.NONE_OFFSET and Lt.qkv % 256 == 0
    assert dit.lib.dit_workspace_size(ctypes.byref(c), 25600) == L.total
    assert dit.workspace_layout(c, 333).ldn == 384


def _fwd(dit, c, x=16, n=10, rows=16, pos=16, sig=(0.5, 0.2), out=16, ws=256, wsb=1 << 40,
         prep=256):
    arr = (ctypes.c_double * 2)(*sig)
    return dit.lib.dit_block_forward(ctypes.byref(c), prep, x, n, rows, pos, arr, len(sig), out,
                                     ws, wsb, None)


def test_block_forward_refusals(dit):
    c = _cfg(dit)
    assert _fwd(dit, c, n=-1) == -2
    assert _fwd(dit, c, prep=None) == -1
    assert _fwd(dit, c, sig=(0.5,)) == -2
    assert _fwd(dit, c, sig=(float("nan"), 0.2)) == -1
    assert _fwd(dit, c, x=None) == -1
    assert _fwd(dit, c, x=8) == -4
    assert _fwd(dit, c, pos=None) == -1
    assert _fwd(dit, c, ws=None) == -1
    assert _fwd(dit, c, ws=128) == -4
    assert _fwd(dit, c, wsb=1024) == -5
    assert "workspace" in dit.last_error()
    # n == 0 is a valid no-op: returns before touching anything
    assert _fwd(dit, c, n=0, x=None, out=None, ws=None) == 0


def test_prepare_refusals(dit):
    c = _cfg(dit)
    w = dit.DitWeights()
    assert dit.lib.dit_prepare_weights(ctypes.byref(c), ctypes.byref(w), 256, 1 << 40, None) == -1
    need = dit.lib.dit_prepared_size(ctypes.byref(c))
    assert dit.lib.dit_prepare_weights(ctypes.byref(c), ctypes.byref(w), 256, need - 1, None) == -5
    assert dit.lib.dit_prepare_weights(ctypes.byref(c), ctypes.byref(w), 16, need, None) == -4


def test_attention_refusals(dit):
    c = _cfg(dit)
    L = dit.lib.dit_attention
    assert L(ctypes.byref(c), 16, 16, 16, 100, 100, 1.0, 16, None) == -2  # ldn % 128
    assert L(ctypes.byref(c), 16, 16, 16, 300, 256, 1.0, 16, None) == -2  # ldn < n
    assert L(ctypes.byref(c), None, 16, 16, 10, 128, 1.0, 16, None) == -1
    assert L(ctypes.byref(c), 16, 16, 16, 0, 128, 1.0, 16, None) == 0


def test_attention_shard_refusals(dit):
    """dit_attention_shard checks its query range, q stride and workspace on the
    host (n = 25600, ldn = 25600, an 8-way shard of 3200 queries)."""
    c = _cfg(dit)
    L = dit.lib.dit_attention_shard
    need = dit.lib.dit_attention_shard_workspace_size(ctypes.byref(c))
    assert need == 256 * 256 * (128 + 2) * 4  # 256 slots x 256 rows x (O row, max, sum)
    f32 = dit.make_config(W.spec_by_name("toy"))
    assert dit.lib.dit_attention_shard_workspace_size(ctypes.byref(f32)) == 0

    def call(q=256, ldq=3200, qlo=3200, qhi=6400, n=25600, ldn=25600, ws=256, wsb=1 << 30, cfg=c):
        return L(ctypes.byref(cfg), q, ldq, qlo, qhi, 256, 256, n, ldn, 1.0, 256, ws, wsb, None)

    assert call(qlo=-1) == -2
    assert call(qlo=6400, qhi=6399) == -2
    assert call(qhi=25601) == -2
    assert call(ldq=3199) == -2   # < qhi - qlo
    assert call(ldq=3300) == -2   # % 128
    assert call(ldn=25500) == -2  # ldn < n
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5
    assert call(ws=16) == -4      # workspace not 256-byte aligned
    assert call(q=8) == -4        # q not 16-byte aligned
    assert call(q=None) == -1
    assert call(qlo=100, qhi=100) == 0  # empty range: nothing to do


def test_profile_arming(dit):
    ms = (ctypes.c_double * dit.NPHASES)()
    calls = ctypes.c_int32(0)
    assert dit.lib.dit_profile_end(ms, ctypes.byref(calls)) == -1
    assert dit.lib.dit_profile_begin(0) == -1
    assert [dit.lib.dit_phase_name(i).decode() for i in range(dit.NPHASES)][4] == "attention"


def test_packed_refusals(dit):
    """Bad sample tables are refused on the host before any launch."""
    c = _cfg(dit)
    arr = (ctypes.c_double * 2)(0.5, 0.2)

    def fwd(starts, nseq, n=10):
        st = (ctypes.c_int32 * max(len(starts), 1))(*starts)
        return dit.lib.dit_block_forward_packed(ctypes.byref(c), 256, 16, n, 16, 16, arr, 2, st,
                                                nseq, 16, 256, 1 << 40, None)

    assert fwd([0, 10], 0) == -2          # nseq < 1
    assert fwd([0] * 66, 65) == -2        # nseq > DIT_MAX_SEQS
    assert fwd([1, 10], 1) == -2          # must start at 0
    assert fwd([0, 6, 4, 10], 3) == -2    # decreasing
    assert fwd([0, 9], 1) == -2           # must end at n
    assert "seq_starts" in dit.last_error()
    assert dit.lib.dit_block_forward_packed(ctypes.byref(c), 256, 16, 10, 16, 16, arr, 2, None, 1,
                                            16, 256, 1 << 40, None) == -1
    A = dit.lib.dit_attention_packed
    st = (ctypes.c_int32 * 3)(0, 5, 9)
    assert A(ctypes.byref(c), 16, 16, 16, 10, 128, st, 2, 1.0, 16, None) == -2
    assert A(ctypes.byref(c), 16, 16, 16, 10, 128, None, 1, 1.0, 16, None) == -1


def test_given_mods_refusals(dit):
    c = _cfg(dit)
    F = dit.lib.dit_block_forward_mods
    assert F(ctypes.byref(c), 256, 16, 10, 16, 16, None, None, 0, 16, 256, 1 << 40, None) == -1
    assert F(ctypes.byref(c), 256, 16, 10, 16, 16, 8, None, 0, 16, 256, 1 << 40, None) == -4
    sig = dit.make_config(W.spec_by_name("siglip"))
    assert F(ctypes.byref(sig), 256, 16, 10, 16, 16, 256, None, 0, 16, 256, 1 << 40, None) == -6
    st = (ctypes.c_int32 * 2)(0, 9)
    assert F(ctypes.byref(c), 256, 16, 10, 16, 16, 256, st, 1, 16, 256, 1 << 40, None) == -2


def test_mmh3_layout_printed_facts(dit):
    """The library's layout builder against the page's printed layout tests."""
    import json
    import numpy as np
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layouts.json")))
    tl, lt, lh, lw, at = g["t2va_args"]
    segs, pos = dit.mmh3_layout(tl, lt, lh, lw, at)
    frame_rows = (lh // 2) * (lw // 2)
    assert frame_rows == g["t2va_frame_rows"] and len(pos) == g["t2va_seq_len"]
    assert [s[0] for s in segs] == g["t2va_order"]
    v = [s for s in segs if s[0] == "video"][0]
    assert abs(pos[v[1] + frame_rows, 0] - pos[v[1], 0] - g["video_t_first_step"]) < 1e-12
    ksegs, kpos = dit.mmh3_layout(tl, lt, lh, lw, at, keyframes=g["keyframes"])
    assert [s[0] for s in ksegs] == g["keyframe_order"]
    assert len(kpos) == len(pos) + 2 * frame_rows
    conds = [s for s in ksegs if s[0] == "cond"]
    spans = sum(5.0 / 3.0 * (1.0, 4.0, 4.0, 4.0, 4.0)[k % 5] for k in range(lt))
    assert kpos[conds[0][1], 0] == tl
    assert abs(kpos[conds[1][1], 0] - (tl + spans - 5.0 / 3.0)) < 1e-12
    kv = [s for s in ksegs if s[0] == "video"][0]
    # keyframes share the target grid and do not move the audio or video
    np.testing.assert_array_equal(kpos[conds[0][1]:conds[0][2], 1:], kpos[kv[1]:kv[1] + frame_rows, 1:])
    np.testing.assert_array_equal(kpos[kv[1]:kv[2]], pos[v[1]:v[2]])


def test_mmh3_layout_matches_the_input_recipe(dit):
    """dit_mmh3_layout equals the layouts the workloads are built from, bit for
    bit, for t2va, keyframes and every kind of reference."""
    import numpy as np
    cases = [((512, 16, 64, 96, 256), {}), ((64, 3, 16, 16, 0), {}),
             ((8, 3, 8, 12, 5), dict(keyframes=[(0, 39), (38, 39)])),
             ((512, 1, 128, 128, 0), dict(ref_images=[(128, 128)])),
             ((8, 3, 8, 12, 5), dict(refs=[("image", 8, 8), ("audio", 4), ("video", 2, 8, 8, 3),
                                           ("audio", 0), ("video", 3, 6, 10, 0)]))]
    for args, kw in cases:
        lay = W.build_layout(*args, **kw)
        refs = [("image", h, w) for h, w in kw.get("ref_images", [])] + list(kw.get("refs", []))
        segs, pos = dit.mmh3_layout(*args, keyframes=kw.get("keyframes", ()), refs=refs)
        assert segs == lay.segments
        np.testing.assert_array_equal(pos, lay.pos)


def test_mmh3_layout_refusals(dit):
    import pytest as pt
    with pt.raises(dit.DitError):
        dit.mmh3_layout(8, 3, 8, 12, 5, keyframes=[(5, 39)])  # neither first nor last frame
    with pt.raises(dit.DitError):
        dit.mmh3_layout(8, 3, 1, 12, 5)
    with pt.raises(dit.DitError):
        dit.mmh3_layout(8, 3, 8, 12, 5, refs=[("image", 8, 1)])
    n = ctypes.c_int32()
    pos = (ctypes.c_double * 30)()
    segs = (dit.DitSegment * 3)()
    # outputs too small for the 90 rows
    assert dit.lib.dit_mmh3_layout(8, 3, 8, 12, 5, None, 0, None, 0, pos, 10, segs, 3, ctypes.byref(n)) == -2


def test_mmh3_slots_match_the_oracle(dit):
    """The host slot planner against the oracle's, over random and edge sigmas
    and every combination of condition streams."""
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(5)
    for sv in [0.0, 1e-9, 1e-6, 0.001, 0.5, 0.999, 1.0] + list(rng.uniform(0, 1, 20)):
        for hc in (False, True):
            for hr in (False, True):
                sig, slot = dit.mmh3_slots(float(sv), has_cond=hc, has_ref_audio=hr)
                ts, oslot = O.mmh3_slots(float(sv), 12.0, 3.0, 0.999, 1.0, hc, hr)
                assert slot == oslot
                np.testing.assert_allclose([1.0 - s for s in sig], ts, rtol=0, atol=1e-15)
    assert dit.lib.dit_mmh3_slots(float("nan"), 12.0, 3.0, 0.999, 1.0, 0, 0,
                                  (ctypes.c_double * 4)(), (ctypes.c_int32 * 4)()) == -1


def _mmh3_model_struct(dit):
    """A DitMmh3Model over valid configs and placeholder (aligned, never
    dereferenced) pointers: the host-side checks run before any launch."""
    spec = W.small_spec(W.spec_by_name("t2va"), D=256, H=2, F=384, slots=3)
    blk = dit.make_config(spec)
    hv = dit.make_config(W.BlockSpec("hv", "final", "bf16", n=1, D=256, H=2, hd=128, F=64, slots=3, tags=1))
    ha = dit.make_config(W.BlockSpec("ha", "final", "bf16", n=1, D=256, H=2, hd=128, F=64, slots=3, tags=1))
    keep = (blk, hv, ha, (ctypes.c_void_p * 2)(256, 512))
    m = dit.DitMmh3Model()
    m.block, m.blocks, m.n_blocks = ctypes.pointer(blk), keep[3], 2
    m.head_video, m.head_video_w = ctypes.pointer(hv), 256
    m.head_audio, m.head_audio_w = ctypes.pointer(ha), 256
    m.latent_c, m.audio_c = 16, 64
    m.video_patch_w, m.audio_patch_w = 256, 256
    m.shift_video, m.shift_audio, m.cond_aug, m.cond_aug_audio = 12.0, 3.0, 0.999, 1.0
    return m, keep


def _segs(dit, spec):
    return (dit.DitSegment * len(spec))(*[dit.DitSegment(dit.SEG_KINDS[k], a, b) for k, a, b in spec])


def test_mmh3_evaluation_refusals(dit):
    m, keep = _mmh3_model_struct(dit)
    good = [("text", 0, 16), ("audio", 16, 40), ("video", 40, 72)]
    assert dit.lib.dit_mmh3_workspace_size(ctypes.byref(m), _segs(dit, good), 3) > 0
    bad = {
        "gap": [("text", 0, 16), ("video", 20, 52)],
        "two videos": [("video", 0, 32), ("video", 32, 64)],
        "no video": [("text", 0, 16), ("audio", 16, 40)],
        "reference in an evaluation": [("text", 0, 16), ("ref_image", 16, 32), ("video", 32, 64)],
    }
    for why, sg in bad.items():
        assert dit.lib.dit_mmh3_workspace_size(ctypes.byref(m), _segs(dit, sg), len(sg)) == 0, why
        assert dit.last_error(), why
    m.audio_slope_rescale = 2
    assert dit.lib.dit_mmh3_workspace_size(ctypes.byref(m), _segs(dit, good), 3) == 0
    m.audio_slope_rescale = 0
    # token rows are slot * 3 + tag: a block with another tag count is refused
    # (its modulation rows would be indexed with the wrong stride)
    blk = keep[0]
    for tags in (1, 2, 4):
        blk.tags = tags
        assert dit.lib.dit_mmh3_workspace_size(ctypes.byref(m), _segs(dit, good), 3) == 0, tags
        assert "tags = 3" in dit.last_error()
    blk.tags = 3
    assert dit.lib.dit_mmh3_workspace_size(ctypes.byref(m), _segs(dit, good), 3) > 0
    m.latent_c = 15  # 4 * latent_c not a multiple of the bf16 GEMM depth
    assert dit.lib.dit_mmh3_workspace_size(ctypes.byref(m), _segs(dit, good), 3) == 0
    assert dit.lib.dit_mmh3_workspace_size(None, _segs(dit, good), 3) == 0


def _zimage_model_struct(dit):
    """A DitZimageModel over valid configs and placeholder (aligned, never
    dereferenced) pointers: 3 main layers, 1 noise and 1 context refiner."""
    z = W.spec_by_name("zimage")
    cfgs = [dit.make_config(W.small_spec(z, variant=v, D=256, H=2, F=384 if v != "zfinal" else 64))
            for v in ("zimage", "zcontext", "zfinal")]
    arr = (ctypes.c_void_p * 3)(256, 512, 768)
    m = dit.DitZimageModel()
    m.block, m.context, m.final_layer = (ctypes.pointer(c) for c in cfgs)
    m.layers, m.n_layers, m.noise_refiners, m.n_noise_refiners = arr, 3, arr, 1
    m.context_refiners, m.n_context_refiners = arr, 1
    m.final_w, m.in_channels, m.cap_dim, m.cap_eps = 256, 16, 128, 1e-6
    m.x_embed_w, m.cap_norm, m.cap_embed_w = 256, 256, 256
    return m, (cfgs, arr)


def test_zimage_forward_cache_refusals(dit):
    m, keep = _zimage_model_struct(dit)
    need = dit.lib.dit_zimage_workspace_size(ctypes.byref(m), 16, 16, 40)
    assert need > 0

    def fwd(cache, step=0):
        return dit.lib.dit_zimage_forward(ctypes.byref(m), 256, 16, 16, 512, 40, 768, 0.5, step,
                                          ctypes.byref(cache), 1024, 256, need, None)
    c = dit.DitZimageCache()
    c.caption, c.shallow, c.layers, c.interval = 256, 512, 2, 0
    assert fwd(c) == -1 and "interval" in dit.last_error()
    c.interval, c.layers = 2, 4  # more shallow layers than main layers
    assert fwd(c) == -1
    c.layers, c.shallow = 2, None
    assert fwd(c) == -1
    c.shallow = 512
    assert fwd(c, step=-1) == -1
    # workspace too small
    c.layers = 1
    assert dit.lib.dit_zimage_forward(ctypes.byref(m), 256, 16, 16, 512, 40, 768, 0.5, 0,
                                      ctypes.byref(c), 1024, 256, need - 1, None) == -5


def test_model_piece_refusals(dit):
    L = dit.lib
    # output head entry point takes head configs only; blocks refuse head configs
    blk = _cfg(dit)
    arr = (ctypes.c_double * 2)(0.5, 0.2)
    assert L.dit_final_forward(ctypes.byref(blk), 256, 256, 10, None, arr, 2, 256, 256, 1 << 30, None) == -1
    # linear: depth / width multiples, finite alpha
    assert L.dit_linear(dit.BF16, 256, 100, 10, 100, 256, 64, None, 1.0, 256, None) == -6
    assert L.dit_linear(dit.BF16, 256, 64, 10, 64, 256, 48, None, 1.0, 256, None) == -6
    assert L.dit_linear(dit.BF16, 256, 64, 10, 64, 256, 64, None, float("nan"), 256, None) == -1
    assert L.dit_linear(7, 256, 64, 10, 64, 256, 64, None, 1.0, 256, None) == -3
    assert L.dit_linear(dit.BF16, 256, 64, 0, 64, 256, 64, None, 1.0, None, None) == 0  # m = 0: no-op
    # stack: at least one block
    assert L.dit_stack_forward(ctypes.byref(blk), (ctypes.c_void_p * 1)(256), 0, 256, 10, 256, 256,
                               arr, 2, None, 0, 256, 256, 1 << 30, None) == -2
    # rms_norm: row width
    assert L.dit_rms_norm(256, 10, 6, 256, 1e-5, 256, None) == -2
    assert L.dit_rms_norm(256, 10, 8192, 256, 1e-5, 256, None) == -2
    # stream layouts: even spatial sizes, known dtype
    assert L.dit_patchify_video(dit.BF16, 256, 4, 2, 7, 8, 256, None) == -2
    assert L.dit_patchify_video(9, 256, 4, 2, 8, 8, 256, None) == -3
    assert L.dit_patchify_image(dit.F32, 256, 4, 8, 5, 256, None) == -2
    assert L.dit_pack_audio(dit.F32, 256, -1, 3, 256, None) == -2


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    """bench.py measures one GPU: asked for several, it exits with status 2 and
    says so before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("p", [3, 256])
def test_bench_shard_refuses_uneven_shards(p):
    """bench.py --shard P needs shards of a multiple of 128 tokens (25600 / 3 is
    not whole, 25600 / 256 = 100): it exits with status 2 before any device work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--shard", str(p)],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "multiple of 128 tokens" in r.stderr and r.stdout == ""


def test_bench_evaluation_refuses_other_layouts():
    """bench.py --evaluation B runs the t2va layout only: another workload exits
    with status 2 before any device work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--evaluation", "2",
                        "--workload", "edit"], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "t2va layout only" in r.stderr and r.stdout == ""


def test_bench_zimage_refuses_other_shapes():
    """bench.py --zimage L runs the zimage shape only: the default workload
    exits with status 2 before any device work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--zimage", "4"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "zimage shape only" in r.stderr and r.stdout == ""


def test_adaln_eval_noalloc_refusals(dit):
    """The no-allocation adaLN entry point refuses a timestep MLP larger than
    its scratch array, and the usual bad arguments, before any launch."""
    z = W.spec_by_name("zimage")
    ok = dit.make_config(W.small_spec(z, D=256, H=2, F=384, temb_hidden=64, temb_freq=32))
    huge = dit.make_config(W.small_spec(z, D=256, H=2, F=384, temb_hidden=16384, temb_freq=32))
    sig = (ctypes.c_double * 1)(0.5)
    L = dit.lib
    assert L.dit_adaln_eval_noalloc(ctypes.byref(huge), 256, sig, 1, 256, None) == -6
    assert "scratch" in dit.last_error()
    assert L.dit_adaln_eval_noalloc(ctypes.byref(ok), None, sig, 1, 256, None) == -1
    assert L.dit_adaln_eval_noalloc(ctypes.byref(ok), 256, sig, 2, 256, None) == -2
    sl = dit.make_config(W.spec_by_name("siglip"))
    assert L.dit_adaln_eval_noalloc(ctypes.byref(sl), 256, sig, 1, 256, None) == -6

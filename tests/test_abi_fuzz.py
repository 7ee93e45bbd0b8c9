"""Host-side robustness of the C ABI (CPU, no device work): seeded random and
malformed arguments to the entry points that validate or plan on the host --
configuration checks, size and layout queries, the MMH3 layout builder, the
slot planner, the sigma remap -- must come back with a status or a size, never
crash, and agree with one another (a configuration the checker refuses has no
prepared or workspace size)."""

import ctypes
import math
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if not os.path.exists(os.path.join(ROOT, "packed_sequence_diffusion_amd", "libdit.so")):
    from packed_sequence_diffusion_amd import build
    build.build()
from packed_sequence_diffusion_amd import dit  # noqa: E402
from synth import workloads as W  # noqa: E402

L = dit.lib


def _pick(rng, vals):
    return vals[int(rng.integers(len(vals)))]


_FIELDS = {
    "variant": [-1, 0, 1, 2, 3, 4, 5, 6, 7],
    "dtype": [-1, 0, 1, 2],
    "D": [-64, 0, 64, 100, 128, 256, 768, 2688, 3072, 4096, 4160],
    "H": [0, 1, 2, 7, 21, 24],
    "hd": [0, 32, 64, 128, 256],
    "F": [0, 64, 100, 256, 384, 3072, 10752, 1 << 20],
    "slots": [-1, 0, 1, 2, 8, 9],
    "tags": [0, 1, 3, 4],
    "rank": [0, 1, 24, 64, 65],
    "grid": [0, 1, 2, 1025],
    "rope": [-1, 0, 1, 2, 3, 4],
    "rope_theta": [-1.0, 0.0, 256.0, 1e4, math.nan, math.inf],
    "eps": [-1e-5, 0.0, 1e-6, 1e-5, math.nan],
    "qk_eps": [0.0, 1e-5, -1.0],
    "temb_freq": [0, 32, 256, 257],
    "temb_hidden": [0, 64, 1024],
    "t_scale": [0.0, 1.0, 1000.0],
    "adaln_shared": [0, 1, 2],
}


def _random_config(rng):
    """A workload's configuration with zero to three fields replaced by values
    drawn from lists that mix valid and invalid ones."""
    spec = W.spec_by_name(_pick(rng, ["toy", "siglip", "zimage", "edit", "t2va"]))
    c = dit.make_config(spec)
    for _ in range(int(rng.integers(4))):
        f = _pick(rng, list(_FIELDS) + ["rope_axes"])
        if f == "rope_axes":
            c.rope_axes[int(rng.integers(3))] = _pick(rng, [-2, 0, 8, 16, 24, 32, 48, 64])
        else:
            setattr(c, f, _pick(rng, _FIELDS[f]))
    return c


def test_config_checks_and_sizes_agree():
    rng = np.random.default_rng(2024)
    seen_ok = 0
    for _ in range(3000):
        c = _random_config(rng)
        st = L.dit_validate_config(ctypes.byref(c))
        assert st <= 0
        ps = L.dit_prepared_size(ctypes.byref(c))
        n = _pick(rng, [-5, 0, 1, 77, 25600, 1 << 30])
        ws = L.dit_workspace_size(ctypes.byref(c), n)
        lay = dit.DitWsLayout()
        ls = L.dit_workspace_layout(ctypes.byref(c), n, ctypes.byref(lay))
        if st != 0:
            assert ps == 0 and ws == 0
            assert ls < 0
            continue
        seen_ok += 1
        assert ps > 0
        if ls == 0:
            assert ws == lay.total
            offs = [getattr(lay, f) for f in ("mods", "rope", "xn", "qkv", "q", "k", "vt", "o",
                                               "x1", "a", "y", "temb", "part")]
            assert all(o == dit.NONE_OFFSET or (o % 256 == 0 and o <= lay.total) for o in offs)
        else:
            assert ws == 0
    assert 300 < seen_ok < 2900  # both sides of the check are exercised


def test_null_arguments_are_refused():
    c = dit.DitConfig()
    assert L.dit_validate_config(None) < 0
    assert L.dit_prepared_size(None) == 0
    assert L.dit_workspace_size(None, 10) == 0
    assert L.dit_workspace_layout(None, 10, None) < 0
    assert L.dit_workspace_layout(ctypes.byref(c), 10, None) < 0
    assert L.dit_last_error()  # a message is left behind


def test_layout_builder_never_crashes():
    rng = np.random.default_rng(7)
    ns = ctypes.c_int32()
    for _ in range(2000):
        args = [_pick(rng, [-3, 0, 1, 2, 5, 16, 48, 512, 1 << 20]) for _ in range(5)]
        nk = _pick(rng, [0, 0, 1, 2, 3])
        kf = (ctypes.c_int32 * max(2 * nk, 1))(*[_pick(rng, [-1, 0, 1, 3, 7, 1000])
                                               for _ in range(2 * nk)])
        nr = _pick(rng, [0, 0, 1, 2])
        refs = (dit.DitLayoutRef * max(nr, 1))()
        for i in range(nr):
            refs[i].kind = _pick(rng, [-1, 0, 1, 2, 3])
            refs[i].latent_t, refs[i].lat_h, refs[i].lat_w, refs[i].audio_t = (
                _pick(rng, [-1, 0, 1, 4, 16]) for _ in range(4))
        # count only
        n = L.dit_mmh3_layout(*args, kf, nk, refs, nr, None, 0, None, 0, ctypes.byref(ns))
        if n < 0:
            continue
        assert ns.value >= 0
        if n > 200000:
            continue
        # too-small buffers are refused, exact ones are filled
        pos = np.zeros((n + 1, 3), dtype=np.float64)
        segs = (dit.DitSegment * (ns.value + 1))()
        pptr = pos.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        if n > 0:
            assert L.dit_mmh3_layout(*args, kf, nk, refs, nr, pptr, n - 1, segs, ns.value,
                                     ctypes.byref(ns)) < 0
        got = L.dit_mmh3_layout(*args, kf, nk, refs, nr, pptr, n, segs, ns.value + 1,
                                ctypes.byref(ns))
        assert got == n
        assert np.all(pos[n] == 0.0)  # nothing written past max_rows
        stops = [segs[i].stop for i in range(ns.value)]
        assert all(segs[i].start <= segs[i].stop for i in range(ns.value))
        assert (max(stops) if stops else 0) == n


def test_slot_planner_and_remap_never_crash():
    rng = np.random.default_rng(11)
    vals = [-1.0, 0.0, 1e-9, 0.25, 0.5, 0.999, 1.0, 1.5, math.nan, math.inf, -math.inf]
    sig = (ctypes.c_double * 8)()
    slots = (ctypes.c_int32 * 8)()
    for _ in range(2000):
        a = [_pick(rng, vals) for _ in range(5)]
        flags = [_pick(rng, [-1, 0, 1, 2]) for _ in range(2)]
        r = L.dit_mmh3_slots(*a, *flags, sig, slots)
        assert r <= 4
        if r > 0:
            assert all(-1 <= slots[i] < r for i in range(4))
            assert all(sig[i] <= sig[i - 1] for i in range(1, r))  # t ascending
        s = L.dit_sigma_remap(_pick(rng, vals), _pick(rng, [0.0, 3.0, 12.0, -1.0]),
                              _pick(rng, [0.0, 3.0, 12.0]))
        assert isinstance(s, float)


def test_model_workspace_queries_never_crash():
    """The MMH3 and Z-Image evaluation planners on random segment lists, image
    sizes and model fields: a size or 0, never a crash."""
    from tests.test_abi import _mmh3_model_struct, _zimage_model_struct
    rng = np.random.default_rng(19)
    m, keep = _mmh3_model_struct(dit)
    kinds = [-1, 0, 1, 2, 3, 4, 5, 6]
    for _ in range(1500):
        nseg = int(rng.integers(0, 7))
        segs = (dit.DitSegment * max(nseg, 1))()
        pos = 0
        for i in range(nseg):
            ln = _pick(rng, [-4, 0, 1, 16, 32, 77, 1 << 20, (1 << 31) - 1])
            start = pos if rng.random() < 0.8 else _pick(rng, [-1, 0, pos + 3])
            segs[i] = dit.DitSegment(_pick(rng, kinds), start, max(-(1 << 31), min(start + ln, (1 << 31) - 1)))
            pos = segs[i].stop
        m.n_blocks = _pick(rng, [-1, 0, 1, 2])
        m.latent_c = _pick(rng, [-16, 0, 15, 16, 1 << 20])
        m.audio_c = _pick(rng, [0, 64, 100])
        m.audio_slope_rescale = _pick(rng, [0, 1, 2])
        got = L.dit_mmh3_workspace_size(ctypes.byref(m), segs, nseg)
        assert got >= 0
    z, zkeep = _zimage_model_struct(dit)
    for _ in range(1500):
        hw = [_pick(rng, [-2, 0, 1, 2, 15, 16, 128, 1 << 15, 1 << 20, (1 << 31) - 2]) for _ in range(2)]
        cap = _pick(rng, [-1, 0, 1, 40, 512, 1 << 20, (1 << 31) - 1])
        z.n_layers = _pick(rng, [-1, 0, 1, 2])
        z.n_noise_refiners = _pick(rng, [-1, 0, 1])
        z.n_context_refiners = _pick(rng, [-1, 0, 1])
        z.in_channels = _pick(rng, [-16, 0, 15, 16, 1 << 20])
        z.cap_dim = _pick(rng, [-1, 0, 64, 128, 100])
        got = L.dit_zimage_workspace_size(ctypes.byref(z), hw[0], hw[1], cap)
        assert got >= 0


def test_token_counts_past_the_cap_are_refused():
    """Token counts past 2^24 (where int row products in the planners used to
    wrap) give no size rather than a wrong one."""
    from tests.test_abi import _mmh3_model_struct, _zimage_model_struct
    z, zkeep = _zimage_model_struct(dit)
    assert L.dit_zimage_workspace_size(ctypes.byref(z), 16, 16, 40) > 0
    for h, w, cap in [(1 << 20, 1 << 20, 40), ((1 << 31) - 2, (1 << 31) - 2, 40),
                      (128, 128, (1 << 31) - 1), (8192, 8192, 1)]:
        assert L.dit_zimage_workspace_size(ctypes.byref(z), h, w, cap) == 0
    m, keep = _mmh3_model_struct(dit)
    big = (1 << 24) + 64
    segs = (dit.DitSegment * 3)(dit.DitSegment(0, 0, big - 56), dit.DitSegment(2, big - 56, big - 32),
                                dit.DitSegment(1, big - 32, big))
    assert L.dit_mmh3_workspace_size(ctypes.byref(m), segs, 3) == 0
    assert "tokens" in dit.last_error()
    cfg = dit.make_config(W.spec_by_name("t2va"))
    assert L.dit_workspace_size(ctypes.byref(cfg), 1 << 24) > 0
    assert L.dit_workspace_size(ctypes.byref(cfg), (1 << 24) + 1) == 0
    assert L.dit_mmh3_layout(1 << 24, 1, 2, 2, 0, None, 0, None, 0, None, 0, None, 0,
                             ctypes.byref(ctypes.c_int32())) < 0

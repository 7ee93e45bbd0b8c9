"""The GPU parity criterion itself (CPU): stages taken from the oracle pass,
and an error confined to one head or one token row fails the per-unit bar
even where the whole-stage relative RMS stays under the tolerance."""

import numpy as np

import oracle as O
from synth import workloads as W
from tests.gpu_common import compare, row_rel


def _stages():
    spec = W.BlockSpec("crit", "mmh3", "bf16", n=96, D=2048, H=32, hd=64, F=256, slots=2,
                       rope="split_half", rope_axes=(16, 24, 24))
    wl = W.make_custom_workload(spec, 5)
    ref = O.block(spec, wl.x, wl.rows, wl.pos, O.resolve_sigmas(wl.slot_plan), wl.weights)
    st = {k: np.array(ref[k]) for k in ("mods", "xn", "q", "k", "v", "o", "x1", "xn2", "a", "out")}
    return spec, wl, st


def test_row_rel_floor():
    ref = np.array([[3.0, 4.0], [0.0, 0.0], [6.0, 8.0]])
    got = ref + np.array([[0.05, 0.0], [1e-4, 0.0], [0.0, 0.0]])
    e = row_rel(got, ref)
    assert abs(e[0] - 0.01) < 1e-12 and e[2] == 0.0
    # the zero row is measured against a thousandth of the median row norm (5)
    assert abs(e[1] - 1e-4 / 5e-3) < 1e-12


def test_oracle_stages_pass():
    spec, wl, st = _stages()
    errs, bad, _ = compare(spec, wl, st)
    assert not bad and max(errs.values()) < 1e-12


def test_one_head_wrong_fails_though_the_aggregate_passes():
    spec, wl, st = _stages()
    o = st["o"].reshape(spec.n, spec.H, spec.hd)
    o[:, 7] *= 1.05  # one head of thirty-two 5% off on every row
    st["o"] = o.reshape(spec.n, spec.D)
    ref = O.block(spec, wl.x, wl.rows, wl.pos, O.resolve_sigmas(wl.slot_plan), wl.weights)
    assert O.rel_rms(st["o"], ref["o"]) < 1e-2  # the whole-stage figure would pass
    _, bad, _ = compare(spec, wl, st)
    assert "o" in bad


def test_one_row_wrong_fails_though_the_aggregate_passes():
    spec, wl, st = _stages()
    st["a"][40] *= 1.05
    ref = O.block(spec, wl.x, wl.rows, wl.pos, O.resolve_sigmas(wl.slot_plan), wl.weights)
    assert O.rel_rms(st["a"], ref["a"]) < 1e-2
    _, bad, _ = compare(spec, wl, st)
    assert "a" in bad
    spec, wl, st = _stages()
    st["k"][3, 17] *= 0.97  # one (head, key token)
    _, bad, _ = compare(spec, wl, st)
    assert "k" in bad


def test_logit_bound_covers_bf16_q_k_rounding():
    """The o bound: the oracle with only q and k rounded to bf16 (RNE, as the
    block's panels are) stays within it on every (token, head), with room."""
    import math
    import torch
    from tests.gpu_common import LOGIT_UNIT, logit_max
    spec, wl, st = _stages()
    ref = O.block(spec, wl.x, wl.rows, wl.pos, O.resolve_sigmas(wl.slot_plan), wl.weights)
    bf = lambda a: torch.from_numpy(np.asarray(a)).to(torch.bfloat16).double().numpy()  # noqa: E731
    sc = 1.0 / math.sqrt(spec.hd)
    o16 = O.attention(bf(ref["q"]), bf(ref["k"]), ref["v"], sc)
    o64 = O.attention(ref["q"], ref["k"], ref["v"], sc)
    e = row_rel(o16, o64)  # [H, m]
    smax = logit_max(ref["q"], ref["k"], spec.hd, np.arange(spec.n))
    assert np.all(e <= 0.5 * LOGIT_UNIT * smax)

"""Pins of the fp64 oracle against things other than itself.

Each test ties one oracle function to a printed test point, a closed form, an
independent library routine, an invariant of the definition or a pure-Python
brute force on tiny inputs.  No GPU is used.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O
from synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- remap ----

def test_remap_involution_printed_points():
    g = gold("sigma_remap.json")
    for s in g["involution_points"]:
        a = O.sigma_remap(s, g["from_shift"], g["to_shift"])
        back = O.sigma_remap(a, g["to_shift"], g["from_shift"])
        assert abs(back - s) < g["involution_tol"]


def test_remap_closed_form_12_to_3():
    # Derived by hand: u = s/(12 - 11 s), 3u/(1 + 2u) = s / (4 - 3 s).
    for s in np.linspace(0.0, 1.0, 101):
        assert abs(O.sigma_remap(s, 12.0, 3.0) - s / (4.0 - 3.0 * s)) < 1e-14
    assert abs(O.sigma_remap(0.972973, 12.0, 3.0) - 0.9000001) < 1e-7
    assert O.sigma_remap(1.0, 12.0, 3.0) == 1.0
    assert O.sigma_remap(0.0, 12.0, 3.0) == 0.0


def test_remap_slope_finite_difference_printed_points():
    g = gold("sigma_remap.json")
    h = g["slope_step"]
    for s in g["slope_points"]:
        num = (O.sigma_remap(s + h, 12.0, 3.0) - O.sigma_remap(s - h, 12.0, 3.0)) / (2 * h)
        assert abs(num - O.sigma_remap_slope(s, 12.0, 3.0)) < g["slope_tol"]
        # closed form d/ds [s/(4-3s)] = 4/(4-3s)^2
        assert abs(O.sigma_remap_slope(s, 12.0, 3.0) - 4.0 / (4.0 - 3.0 * s) ** 2) < 1e-12


def test_mmh3_slots_rules():
    """The evaluation's timestep list, from the page's rules written out as
    cases: ascending, deduplicated, conditions pinned near 1."""
    # no conditions: audio is always later than video (sigma_a <= sigma_v)
    ts, slot = O.mmh3_slots(0.5, 12.0, 3.0, 0.999, 1.0, False, False)
    np.testing.assert_allclose(ts, [0.5, 1.0 - 0.2], rtol=0, atol=1e-15)
    assert slot == {"video": 0, "audio": 1, "cond": -1, "ref_audio": -1}
    # sigma_v = 1: both streams at t = 0 -> one slot
    ts, slot = O.mmh3_slots(1.0, 12.0, 3.0, 0.999, 1.0, False, False)
    assert ts == [0.0] and slot["video"] == slot["audio"] == 0
    # keyframes at max(t_v, 0.999); reference audio at max(t_a, 1.0) = 1
    ts, slot = O.mmh3_slots(0.6, 12.0, 3.0, 0.999, 1.0, True, True)
    sa = 0.6 / (4.0 - 3.0 * 0.6)
    np.testing.assert_allclose(ts, [0.4, 1.0 - sa, 0.999, 1.0], rtol=0, atol=1e-15)
    assert slot == {"video": 0, "audio": 1, "cond": 2, "ref_audio": 3}
    # sigma floor: t_v = 1 - 1e-6 is later than 0.999, so the condition rows
    # share the video slot
    ts, slot = O.mmh3_slots(0.0, 12.0, 3.0, 0.999, 1.0, True, False)
    assert slot["cond"] == slot["video"] and len(ts) == 2
    rows = O.mmh3_token_rows([("text", 0, 2), ("cond", 2, 3), ("audio", 3, 5), ("video", 5, 6)],
                             {"video": 0, "audio": 1, "cond": 2, "ref_audio": -1})
    assert rows.tolist() == [1, 1, 6, 5, 5, 0]


def test_token_rows_with_text_tags():
    # rows = slot * 3 + tag; a vision block in the prompt takes the video tag at the text's slot
    segs = [("text", 0, 5), ("cond", 5, 9), ("audio", 9, 11), ("video", 11, 15)]
    slot = {"video": 0, "audio": 1, "cond": 2, "ref_audio": -1}
    plain = O.mmh3_token_rows(segs, slot)
    assert plain.tolist() == [1] * 5 + [6] * 4 + [5] * 2 + [0] * 4
    tagged = O.mmh3_token_rows(segs, slot, text_tags=[1, 0, 0, 1, 2])
    assert tagged.tolist() == [1, 0, 0, 1, 2] + plain[5:].tolist()


def test_timestep_of_sigma():
    # the page floors the video sigma inside its forward only; a slot sigma of
    # 0 is the condition timestep t = 1 exactly
    assert O.mmh3_timestep(0.3) == pytest.approx(0.7, abs=1e-15)
    assert O.mmh3_timestep(0.0) == 1.0
    # the evaluation's floor: sigma_v = 0 puts video at 1 - 1e-6 and audio at
    # 1 - 1e-6 / (4 - 3e-6), later, so ascending order is [video, audio]
    ts, _ = O.mmh3_slots(0.0, 12.0, 3.0, 0.999, 1.0, False, False)
    assert ts == [1.0 - 1e-6, 1.0 - 1e-6 / (4.0 - 3e-6)]


def test_slot_at_t_one_reads_the_last_table_row():
    """A reference-audio slot (t = max(t_a, 1) = 1) evaluates the curve at the
    table's last row with weight 1 ([MMH3] Adaln::eval keeps the last
    interval whole): mods = basis @ table[G-1] + bias, exactly."""
    rng = np.random.default_rng(7)
    T, E, D, r, G = 3, 6, 4, 5, 9
    basis = rng.normal(size=(2 * T * E * D, r))
    bias = rng.normal(size=2 * T * E * D)
    table = rng.normal(size=(G, r))
    ts, slot = O.mmh3_slots(0.4, 12.0, 3.0, 0.999, 1.0, False, True)
    assert ts[slot["ref_audio"]] == 1.0
    sig = [0.4, 0.0]  # a video slot and a slot at t = 1 exactly
    mods = O.adaln_mods(basis, bias, table, [O.mmh3_timestep(s) for s in sig], T, E, D)
    half = T * E * D
    want = basis[half:] @ table[G - 1] + bias[half:]
    np.testing.assert_allclose(mods[T:].reshape(-1), want, rtol=1e-13, atol=1e-13)
    # and not the coordinates one millionth of t earlier (the floor applied to
    # every slot would move them by 1e-6 * (G - 1) of a table step)
    p = (1.0 - 1e-6) * (G - 1)
    c = table[G - 2] + (p - (G - 2)) * (table[G - 1] - table[G - 2])
    assert np.max(np.abs(mods[T:].reshape(-1) - (basis[half:] @ c + bias[half:]))) > 1e-7


def test_resolve_sigmas_plan():
    s = O.resolve_sigmas([("value", 0.5), ("remap", 0, 12.0, 3.0)])
    assert s == [0.5, pytest.approx(0.2, abs=1e-15)]


# ---------------------------------------------------------------- adaLN ----

def test_adaln_lerp_special_points():
    rng = np.random.default_rng(1)
    tab = rng.standard_normal((1025, 24))
    for k in (0, 1, 17, 512, 1023):
        np.testing.assert_array_equal(O.adaln_coords(tab, k / 1024.0), tab[k])
    # t >= 1 lands on the last row with weight 1 (f = 1 on the last interval)
    np.testing.assert_allclose(O.adaln_coords(tab, 1.0), tab[1024], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.adaln_coords(tab, 1.7), tab[1024], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(O.adaln_coords(tab, -0.3), tab[0])
    k = 300
    np.testing.assert_allclose(O.adaln_coords(tab, (k + 0.25) / 1024.0),
                               0.75 * tab[k] + 0.25 * tab[k + 1], rtol=0, atol=1e-13)


def test_adaln_coords_match_numpy_interp():
    rng = np.random.default_rng(2)
    tab = rng.standard_normal((1025, 24))
    grid = np.arange(1025) / 1024.0
    for t in rng.uniform(0, 1, 50):
        want = np.array([np.interp(t, grid, tab[:, j]) for j in range(24)])
        np.testing.assert_allclose(O.adaln_coords(tab, t), want, rtol=0, atol=1e-12)


def test_adaln_rank_basis_equals_full_matrix_map():
    """A full adaLN map W_full applied to an embedding that lies on the curve
    spanned by A equals the rank-r basis map with basis W_full A."""
    rng = np.random.default_rng(3)
    D, r, S, T, E = 16, 24, 2, 3, 6
    tab = rng.standard_normal((1025, r))
    A = rng.standard_normal((D, r))
    Wf = rng.standard_normal((S * T * E * D, D))
    bias = rng.standard_normal(S * T * E * D)
    ts = [0.123, 0.877]
    got = O.adaln_mods(Wf @ A, bias, tab, ts, T, E, D)
    grid = np.arange(1025) / 1024.0
    per = T * E * D
    for s, t in enumerate(ts):
        c = np.array([np.interp(t, grid, tab[:, j]) for j in range(r)])
        emb = A @ c  # the full map's input
        want = Wf[s * per:(s + 1) * per] @ emb + bias[s * per:(s + 1) * per]
        np.testing.assert_allclose(got[s * T:(s + 1) * T].ravel(), want, rtol=1e-12, atol=1e-10)


def test_adaln_one_hot_basis_returns_coords_and_layout():
    rng = np.random.default_rng(4)
    D, r, T, E = 8, 24, 3, 6
    tab = rng.standard_normal((1025, r))
    basis = np.zeros((2 * T * E * D, r))
    # row j picks coordinate j % r
    basis[np.arange(basis.shape[0]), np.arange(basis.shape[0]) % r] = 1.0
    ts = [0.25, 0.5]
    m = O.adaln_mods(basis, None, tab, ts, T, E, D)
    assert m.shape == (2 * T, E * D)
    for s, t in enumerate(ts):
        c = tab[int(t * 1024)]
        for tag in range(T):
            for e in range(E):
                for d in range(D):
                    j = ((s * T + tag) * E + e) * D + d
                    assert m[s * T + tag, e * D + d] == c[j % r]


# ---------------------------------------------------------- norms/acts ----

def test_rms_norm_unit_gain_closed_form_and_torch():
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 64)) * 3.0
    eps = 1e-5
    y = O.rms_norm(x, None, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)),
                               rtol=1e-13)
    g = 1.0 + 0.02 * rng.standard_normal(64)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps)
    np.testing.assert_allclose(O.rms_norm(x, g, eps), want.numpy(), rtol=1e-13, atol=1e-13)
    # scale invariance as eps -> 0
    np.testing.assert_allclose(O.rms_norm(5.0 * x, g, 0.0), O.rms_norm(x, g, 0.0), rtol=1e-13)


def test_layer_norm_matches_torch():
    import torch
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 96)) * 2.0 + 1.5
    g = 1.0 + 0.02 * rng.standard_normal(96)
    b = 0.02 * rng.standard_normal(96)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g),
                                          torch.from_numpy(b), 1e-6)
    np.testing.assert_allclose(O.layer_norm(x, g, b, 1e-6), want.numpy(), rtol=1e-12, atol=1e-12)
    y = O.layer_norm(x, np.ones(96), np.zeros(96), 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-12)


def test_silu_against_expit():
    from scipy.special import expit
    v = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(O.silu(v), v * expit(v), rtol=1e-13, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([50.0]))[0] - 50.0) < 1e-15 * 50 + 1e-18


def test_gelu_landmarks_printed():
    g = gold("gelu_landmarks.json")
    y = O.gelu_tanh(np.array(g["xs"]))
    assert abs(y[0]) < g["abs_at_minus_10_below"]
    assert abs(y[3]) < g["abs_at_zero_below"]
    assert abs(y[6] - 10.0) < g["abs_err_at_10_below"]
    lo, hi = g["dip_range_at_minus_0_75"]
    assert lo < y[2] < hi
    assert y[1] < 0.0
    tail = y[g["monotone_from_index"]:]
    assert np.all(np.diff(tail) >= -g["monotone_slack"])


def test_gelu_tanh_close_to_erf_gelu():
    # The tanh form approximates x * Phi(x) to within a few 1e-4 everywhere.
    v = np.linspace(-8, 8, 4001)
    exact = np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in v])
    assert np.max(np.abs(O.gelu_tanh(v) - exact)) < 1e-3


def test_gelu_tanh_matches_torch():
    import torch
    v = np.linspace(-12, 12, 3001)
    want = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(v), want, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ RoPE ----

def test_rope_angles_axis_structure():
    pos = np.array([[3.0, 5.0, 7.0]])
    ang = O.rope_angles(pos, (32, 48, 48), 1e4)
    assert ang.shape == (1, 64)
    # the first frequency of every axis is 1: the angle is the coordinate
    assert ang[0, 0] == 3.0 and ang[0, 16] == 5.0 and ang[0, 40] == 7.0
    # the last frequency of axis a is theta^(-(d_a - 2)/d_a)
    assert ang[0, 15] == pytest.approx(3.0 * 1e4 ** (-30.0 / 32.0), rel=1e-14)
    assert ang[0, 39] == pytest.approx(5.0 * 1e4 ** (-46.0 / 48.0), rel=1e-14)
    assert ang[0, 63] == pytest.approx(7.0 * 1e4 ** (-46.0 / 48.0), rel=1e-14)
    # [ZIMG] frequencies exp(-ln(theta) i / half) are the same numbers
    half = 24
    f = np.exp(-math.log(256.0) * np.arange(half) / half)
    np.testing.assert_allclose(O.rope_angles(np.array([[0.0, 1.0, 0.0]]), (32, 48, 48), 256.0)[0, 16:40],
                               f, rtol=1e-14)


def test_rope_split_half_is_complex_rotation():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 5, 128))
    ang = rng.uniform(-600, 600, (5, 64))
    y = O.rope_rotate(x, ang[None], "split_half")
    z = (x[..., :64] + 1j * x[..., 64:]) * np.exp(1j * ang)[None]
    np.testing.assert_allclose(y[..., :64], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., 64:], z.imag, atol=1e-12)
    # norms preserved, zero angle is the identity
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(O.rope_rotate(x, np.zeros((1, 5, 64)), "split_half"), x)


def test_rope_interleaved_is_permuted_split_half():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 4, 128))
    ang = rng.uniform(-50, 50, (4, 64))
    perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])  # interleaved -> split
    inv = np.argsort(perm)
    got = O.rope_rotate(x, ang[None], "interleaved")
    via = O.rope_rotate(x[..., perm], ang[None], "split_half")[..., inv]
    np.testing.assert_allclose(got, via, atol=1e-13)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)[None]
    np.testing.assert_allclose(got[..., 0::2], z.real, atol=1e-12)


def test_rope_partial_angles_structure_and_full_special_case():
    # [MMH3] rope_angles: k shared frequencies, axis-major, angle = pos[axis] * freq
    rng = np.random.default_rng(9)
    pos = rng.uniform(0, 600, (4, 3))
    freq = np.exp(-rng.uniform(0, 9, 16))
    ang = O.rope_angles_shared(pos, freq)
    assert ang.shape == (4, 48)
    unit = O.rope_angles_shared(np.array([[1.0, 2.0, 3.0]]), np.ones(16))
    np.testing.assert_array_equal(unit[0], np.repeat([1.0, 2.0, 3.0], 16))
    # frequencies theta^(-m/k) and 6k = hd: the per-axis table with three equal axes
    k, theta = 16, 1e4
    f = theta ** (-np.arange(k) / k)
    np.testing.assert_allclose(O.rope_angles_shared(pos, f), O.rope_angles(pos, (32, 32, 32), theta),
                               rtol=1e-14)


def test_rope_partial_rotates_3k_pairs_and_keeps_the_tail():
    # pairs (j, j + 48) turn as complex numbers; head dims 96..127 are untouched
    rng = np.random.default_rng(10)
    x = rng.standard_normal((2, 5, 128))
    ang = O.rope_angles_shared(rng.uniform(0, 600, (5, 3)), np.exp(-rng.uniform(0, 9, 16)))
    y = O.rope_rotate(x, ang[None], "split_half")
    z = (x[..., :48] + 1j * x[..., 48:96]) * np.exp(1j * ang)[None]
    np.testing.assert_allclose(y[..., :48], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., 48:96], z.imag, atol=1e-12)
    np.testing.assert_array_equal(y[..., 96:], x[..., 96:])


def test_rope_for_selects_the_layout():
    spec = W.small_spec(W.spec_by_name("t2va"), rope="partial", rope_axes=(32, 32, 32))
    pos = np.array([[1.0, 2.0, 3.0]])
    ang, mode = O.rope_for(spec, pos, {"rope_freq": np.ones(16)})
    assert mode == "split_half" and ang.shape == (1, 48)
    ang, mode = O.rope_for(W.spec_by_name("t2va"), pos, {})
    assert mode == "split_half" and ang.shape == (1, 64)


# ------------------------------------------------------------- attention ----

def _brute_attention(q, k, v, scale):
    H, m, hd = q.shape
    n = k.shape[1]
    out = np.zeros((H, m, v.shape[2]))
    for h in range(H):
        for i in range(m):
            s = [scale * sum(q[h, i, d] * k[h, j, d] for d in range(hd)) for j in range(n)]
            mx = max(s)
            e = [math.exp(si - mx) for si in s]
            tot = sum(e)
            for d in range(v.shape[2]):
                out[h, i, d] = sum(e[j] * v[h, j, d] for j in range(n)) / tot
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 5, 8)) * 2
    k = rng.standard_normal((2, 11, 8)) * 2
    v = rng.standard_normal((2, 11, 8))
    np.testing.assert_allclose(O.attention(q, k, v, 0.35), _brute_attention(q, k, v, 0.35),
                               rtol=1e-12, atol=1e-13)


def test_attention_matches_torch_sdpa():
    import torch
    rng = np.random.default_rng(10)
    q = rng.standard_normal((3, 40, 64))
    k = rng.standard_normal((3, 70, 64))
    v = rng.standard_normal((3, 70, 64))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.125).numpy()
    np.testing.assert_allclose(O.attention(q, k, v, 0.125), want, rtol=1e-11, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((2, 33, 16))
    q = rng.standard_normal((2, 9, 16))
    vconst = np.broadcast_to(rng.standard_normal((2, 1, 16)), (2, 33, 16)).copy()
    np.testing.assert_allclose(O.attention(q, k, vconst, 1.0), np.broadcast_to(vconst[:, :1], (2, 9, 16)),
                               rtol=1e-13)
    v = rng.standard_normal((2, 33, 16))
    np.testing.assert_allclose(O.attention(np.zeros_like(q), k, v, 1.0),
                               np.broadcast_to(v.mean(axis=1, keepdims=True), (2, 9, 16)), rtol=1e-12)


def test_attention_extreme_scores_finite():
    g = gold("softmax_extremes.json")
    lo, hi = g["extreme_score_range"]
    rng = np.random.default_rng(12)
    # one-dimensional heads so the score is q*k: choose q=1, k in [lo, hi]
    k = rng.uniform(lo, hi, (1, 8, 1))
    q = np.ones((1, 8, 1))
    v = rng.standard_normal((1, 8, 4))
    o = O.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, _brute_attention(q, k, v, 1.0), rtol=1e-12)


# ---------------------------------------------------------------- layouts ----

# -------------------------------------------------- packed samples (ragged) ----

def _brute_masked_attention(q, k, v, scale, qtok, seq_starts):
    """Scalar loops over every key with an explicit block-diagonal mask: key j
    counts for query token i only when both lie in the same sample."""
    H, m, hd = q.shape
    n = k.shape[1]
    sample = [None] * n
    for s_, (a, e) in enumerate(zip(seq_starts[:-1], seq_starts[1:])):
        for t in range(a, e):
            sample[t] = s_
    out = np.zeros((H, m, v.shape[2]))
    for h in range(H):
        for i in range(m):
            keep = [j for j in range(n) if sample[j] == sample[qtok[i]]]
            s = [scale * sum(q[h, i, d] * k[h, j, d] for d in range(hd)) for j in keep]
            mx = max(s)
            e = [math.exp(si - mx) for si in s]
            tot = sum(e)
            for d in range(v.shape[2]):
                out[h, i, d] = sum(e[c] * v[h, j, d] for c, j in enumerate(keep)) / tot
    return out


def test_packed_attention_brute_force_tiny():
    rng = np.random.default_rng(21)
    starts = [0, 4, 5, 5, 13]  # lengths 4, 1, 0 (empty), 8
    q = rng.standard_normal((2, 13, 6)) * 2
    k = rng.standard_normal((2, 13, 6)) * 2
    v = rng.standard_normal((2, 13, 6))
    qtok = np.arange(13)
    np.testing.assert_allclose(O.attention_packed(q, k, v, 0.4, qtok, starts),
                               _brute_masked_attention(q, k, v, 0.4, qtok, starts),
                               rtol=1e-12, atol=1e-13)
    # a subset of query rows, out of order
    sel = np.array([12, 4, 0, 7])
    np.testing.assert_allclose(O.attention_packed(q[:, sel], k, v, 0.4, sel, starts),
                               _brute_masked_attention(q[:, sel], k, v, 0.4, sel, starts),
                               rtol=1e-12, atol=1e-13)


def test_packed_attention_single_sample_is_full_attention():
    rng = np.random.default_rng(22)
    q, k, v = (rng.standard_normal((3, 17, 8)) for _ in range(3))
    np.testing.assert_array_equal(O.attention_packed(q, k, v, 0.3, np.arange(17), [0, 17]),
                                  O.attention(q, k, v, 0.3))


def test_packed_attention_rejects_bad_starts():
    q = np.zeros((1, 4, 2))
    for bad in ([0, 5], [1, 4], [0, 3, 2, 4], [0]):
        with pytest.raises(ValueError):
            O.attention_packed(q, q, q, 1.0, np.arange(4), bad)


def test_refiner_is_the_mmh3_block_with_neutral_modulation():
    """The unmodulated block equals the (brute-force pinned) MMH3 block whose
    adaLN rows are shift 0, scale 0, gate 1 in both halves: zero basis, bias
    holding those values."""
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(17, n=11)
    D = spec.D
    neutral = np.zeros(6 * D)
    neutral[2 * D:3 * D] = 1.0
    neutral[5 * D:6 * D] = 1.0
    wn = dict(w)
    wn["adaln_basis"] = np.zeros_like(w["adaln_basis"])
    wn["adaln_bias"] = np.tile(neutral, spec.slots * spec.tags)
    for rope, p in (("none", None), ("split_half", pos)):
        mspec = W.small_spec(spec, rope=rope)
        rspec = W.small_spec(mspec, variant="refiner")
        want = O.mmh3_block(mspec, x, rows, p, sig, wn)
        got = O.refiner_block(rspec, x, p, w)
        for name in ("xn", "o", "x1", "a", "out"):
            np.testing.assert_allclose(got[name], want[name], rtol=1e-13, atol=1e-13)


def test_final_layer_matches_torch_composition():
    """The head against torch fp64: table lerp at the slot timesteps,
    basis map, rms_norm, shift/scale of the token's slot, linear, negation."""
    import torch
    import torch.nn.functional as Fn
    spec = W.BlockSpec("head", "final", "f32", n=9, D=16, H=2, hd=8, F=12, slots=2, tags=1,
                       rank=3, grid=9)
    wl = W.make_custom_workload(spec, 51, sigmas=[0.3, 0.85])
    w = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    got = O.final_layer(spec, wl.x, wl.rows, [0.3, 0.85], w)["out"]
    tw = {k: torch.from_numpy(v) for k, v in w.items()}
    rows_per_slot = 2 * spec.D
    mods = []
    for s_, sig in enumerate([0.3, 0.85]):
        t = 1.0 - sig
        p = min(max(t, 0.0), 1.0) * (spec.grid - 1)
        i0 = min(int(math.floor(p)), spec.grid - 2)
        c = tw["adaln_table"][i0] + (p - i0) * (tw["adaln_table"][i0 + 1] - tw["adaln_table"][i0])
        blk = slice(s_ * rows_per_slot, (s_ + 1) * rows_per_slot)
        mods.append(tw["adaln_basis"][blk] @ c + tw["adaln_bias"][blk])
    mods = torch.stack(mods)
    r = torch.from_numpy(wl.rows.astype(np.int64))
    hn = Fn.rms_norm(torch.from_numpy(wl.x.astype(np.float64)), (spec.D,), tw["norm1"], spec.eps)
    hn = hn * (1 + mods[r, spec.D:]) + mods[r, :spec.D]
    want = -Fn.linear(hn, tw["w_fc1"], tw["b_fc1"])
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


def test_stack_is_sequential_blocks():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(18, n=8)
    w2 = {k: v * (1.1 if k.startswith("w_") else 1.0) for k, v in w.items()}
    a = O.mmh3_block(spec, O.mmh3_block(spec, x, rows, pos, sig, w)["out"], rows, pos, sig, w2)["out"]
    np.testing.assert_array_equal(O.stack(spec, x, rows, pos, sig, [w, w2]), a)


def test_patchify_is_the_einsum_layout_and_inverts():
    """The page's patch layout is einsum("nctrhpwq->nthwcrpq") of [C, T, H/2,
    2, W/2, 2]: rows (t, h, w), columns (c, r, p, q) -> (c, p, q)."""
    rng = np.random.default_rng(61)
    x = rng.standard_normal((3, 2, 6, 4))
    C, T, H, W = x.shape
    want = np.einsum("ctrhpw->trpchw", x.reshape(C, T, H // 2, 2, W // 2, 2)).reshape(-1, 4 * C)
    rows = O.patchify_video(x)
    np.testing.assert_array_equal(rows, want)
    np.testing.assert_array_equal(O.unpatchify_video(rows, C, T, H, W), x)


def test_pack_audio_layout_and_inverse():
    rng = np.random.default_rng(62)
    x = rng.standard_normal((5, 2, 7))
    rows = O.pack_audio(x)
    assert rows.shape == (14, 5)
    for ch in range(2):
        for t in range(7):
            np.testing.assert_array_equal(rows[ch * 7 + t], x[:, ch, t])
    np.testing.assert_array_equal(O.unpack_audio(rows, 5, 7), x)


def test_packed_block_equals_samples_run_alone():
    """[ENC]: a ragged batch behaves exactly like its sequences run solo."""
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(16, n=12)
    starts = [0, 5, 6, 12]
    packed = O.mmh3_block(spec, x, rows, pos, sig, w, seq_starts=starts)
    for a, e in zip(starts[:-1], starts[1:]):
        alone = O.mmh3_block(spec, x[a:e], rows[a:e], pos[a:e], sig, w)
        for name in ("o", "x1", "out"):
            np.testing.assert_allclose(packed[name][a:e], alone[name], rtol=1e-12, atol=1e-12)
    # and differs from attending across samples
    full = O.mmh3_block(spec, x, rows, pos, sig, w)
    assert np.abs(full["o"] - packed["o"]).max() > 1e-3


def test_layout_t2va_printed():
    g = gold("layouts.json")
    lay = W.build_layout(*g["t2va_args"])
    assert lay.frame_rows == g["t2va_frame_rows"]
    assert lay.seq_len == g["t2va_seq_len"]
    assert [s[0] for s in lay.segments] == g["t2va_order"]
    v = lay.segment("video")
    t0 = lay.pos[v[1], 0]
    t1 = lay.pos[v[1] + lay.frame_rows, 0]
    assert abs(t1 - t0 - g["video_t_first_step"]) < 1e-12


def test_layout_keyframes_printed():
    g = gold("layouts.json")
    tl, lt, lh, lw, at = g["t2va_args"]
    base = W.build_layout(tl, lt, lh, lw, at)
    lay = W.build_layout(tl, lt, lh, lw, at, keyframes=[tuple(k) for k in g["keyframes"]])
    assert lay.cond_rows() == 2 * lay.frame_rows
    assert lay.seq_len == base.seq_len + 2 * lay.frame_rows
    assert [s[0] for s in lay.segments] == g["keyframe_order"]
    a0, v0 = lay.segment("audio"), lay.segment("video")
    assert lay.pos[a0[1], 0] == base.pos[base.segment("audio")[1], 0]
    assert lay.pos[v0[1], 0] == base.pos[base.segment("video")[1], 0]
    conds = [s for s in lay.segments if s[0] == "cond"]
    assert lay.pos[conds[0][1], 0] == tl
    spans = sum(5.0 / 3.0 * (1.0, 4.0, 4.0, 4.0, 4.0)[k % 5] for k in range(lt))
    assert abs(lay.pos[conds[1][1], 0] - (tl + spans - 5.0 / 3.0)) < 1e-12
    assert lay.pos[conds[0][1], 1] == lay.pos[v0[1], 1]


def test_workload_shapes():
    for spec in W.SPECS:
        pos, rows = W.layout_for(spec)
        if pos is not None:
            assert pos.shape == (spec.n, 3)
        if rows is not None:
            assert rows.shape == (spec.n,)
            assert rows.min() >= 0 and rows.max() < spec.mod_rows
    pos, rows = W.layout_for(W.spec_by_name("t2va"))
    assert sorted(set(rows.tolist())) == [0, 1, 5]
    # video t spans [512, 512 + 5/3 * 51]; audio frames sit at 512 + i
    vid = rows == 0
    assert pos[vid, 0].min() == 512.0 and pos[vid, 0].max() == pytest.approx(597.0)
    assert pos[rows == 5, 0].max() == 767.0
    pos, rows = W.layout_for(W.spec_by_name("edit"))
    assert sorted(set(rows.tolist())) == [0, 1]


# ---------------------------------------------------------- whole block ----

def _tiny_mmh3_spec(n=7):
    return W.BlockSpec("tiny", "mmh3", "f32", n=n, D=16, H=2, hd=8, F=12, slots=2, rank=3,
                       grid=9, rope="split_half", rope_axes=(2, 2, 4), rope_theta=100.0)


def _brute_mmh3(spec, x, rows, pos, sigmas, w):
    """Scalar loops, written independently of the oracle's array code.
    ``spec.rope == "partial"``: the k frequencies of w["rope_freq"] serve every
    axis, pair (j, j + 3k), dims from 6k on unrotated.  ``spec.adaln_shared``:
    one slot's basis rows at every slot."""
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    n = len(x)
    T, E = spec.tags, 6
    G = spec.grid
    mods = {}
    for s, sg in enumerate(sigmas):
        t = 1.0 - sg
        p = min(max(t, 0.0), 1.0) * (G - 1)
        i0 = min(int(math.floor(p)), G - 2)
        f = p - i0
        c = [w["adaln_table"][i0][k] * (1 - f) + w["adaln_table"][i0 + 1][k] * f
             for k in range(spec.rank)]
        for tag in range(T):
            for e in range(E):
                for d in range(D):
                    j = ((s * T + tag) * E + e) * D + d
                    if spec.adaln_shared:
                        j = (tag * E + e) * D + d
                    mods[(s * T + tag, e, d)] = w["adaln_bias"][j] + sum(
                        w["adaln_basis"][j][k] * c[k] for k in range(spec.rank))

    def rms(vec, g, eps):
        ms = sum(v * v for v in vec) / len(vec)
        inv = 1.0 / math.sqrt(ms + eps)
        return [vec[i] * inv * g[i] for i in range(len(vec))]

    def mv(W_, vec, r0, r1):
        return [sum(W_[r][c] * vec[c] for c in range(len(vec))) for r in range(r0, r1)]

    freqs = []
    if spec.rope == "partial":
        for a in range(3):
            for f in w["rope_freq"]:
                freqs.append((a, float(f)))
    else:
        for a, d in enumerate(spec.rope_axes):
            for m in range(d // 2):
                freqs.append((a, spec.rope_theta ** (-2.0 * m / d)))
    P = len(freqs)

    def rope(vec, i):
        out = list(vec)
        for j, (a, om) in enumerate(freqs):
            ang = pos[i][a] * om
            c, s_ = math.cos(ang), math.sin(ang)
            out[j] = vec[j] * c - vec[j + P] * s_
            out[j + P] = vec[j] * s_ + vec[j + P] * c
        return out

    xn = []
    for i in range(n):
        r = rows[i]
        z = rms(list(x[i]), w["norm1"], spec.eps)
        xn.append([z[d] * (1 + mods[(r, 1, d)]) + mods[(r, 0, d)] for d in range(D)])
    Q, K, V = [], [], []
    for i in range(n):
        qkv = mv(w["w_qkv"], xn[i], 0, 3 * D)
        Q.append([rope(rms(qkv[h * hd:(h + 1) * hd], w["q_norm"], spec.qk_eps), i) for h in range(H)])
        K.append([rope(rms(qkv[D + h * hd:D + (h + 1) * hd], w["k_norm"], spec.qk_eps), i) for h in range(H)])
        V.append([qkv[2 * D + h * hd:2 * D + (h + 1) * hd] for h in range(H)])
    out = np.zeros((n, D))
    for i in range(n):
        r = rows[i]
        o = []
        for h in range(H):
            s = [sum(Q[i][h][d] * K[j][h][d] for d in range(hd)) / math.sqrt(hd) for j in range(n)]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            tot = sum(e)
            o += [sum(e[j] * V[j][h][d] for j in range(n)) / tot for d in range(hd)]
        proj = mv(w["w_out"], o, 0, D)
        x1 = [x[i][d] + mods[(r, 2, d)] * proj[d] for d in range(D)]
        z = rms(x1, w["norm2"], spec.eps)
        h2 = [z[d] * (1 + mods[(r, 4, d)]) + mods[(r, 3, d)] for d in range(D)]
        gu = mv(w["w_fc1"], h2, 0, 2 * F)
        act = [gu[f] / (1 + math.exp(-gu[f])) * gu[F + f] for f in range(F)]
        y = mv(w["w_fc2"], act, 0, D)
        out[i] = [x1[d] + mods[(r, 5, d)] * y[d] for d in range(D)]
    return out


def _tiny_mmh3_inputs(seed=13, n=7):
    spec = _tiny_mmh3_spec(n)
    wl = W.make_custom_workload(spec, seed, sigmas=[0.37, 0.81])
    w = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    # make the modulation visible: larger basis, table of unit scale
    w["adaln_basis"] = w["adaln_basis"] * 10.0
    for k in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
        w[k] = w[k] * 10.0
    return spec, wl.x.astype(np.float64), wl.rows, wl.pos.astype(np.float64), [0.37, 0.81], w


def test_mmh3_block_brute_force_tiny():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs()
    got = O.mmh3_block(spec, x, rows, pos, sig, w)["out"]
    want = _brute_mmh3(spec, x, rows, pos, sig, w)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)
    # the sampled-row form returns the same rows
    sel = np.array([5, 0, 3])
    np.testing.assert_allclose(O.mmh3_block(spec, x, rows, pos, sig, w, qrows=sel)["out"],
                               got[sel], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(10))
def test_mmh3_block_brute_force_random_tiny(seed):
    """Seeded random tiny shapes (tokens, width, heads, FFN, slots, adaLN rank
    and grid, RoPE axes and base, random segment rows) against the scalar
    brute force."""
    rng = np.random.default_rng(300 + seed)
    hd = int(rng.choice([8, 12, 16]))
    H = int(rng.choice([1, 2]))
    axes = {8: (2, 2, 4), 12: (4, 4, 4), 16: (4, 6, 6)}[hd]
    slots = int(rng.integers(1, 4))
    spec = W.BlockSpec("rtiny", "mmh3", "f32", n=int(rng.integers(1, 10)), D=H * hd, H=H, hd=hd,
                       F=int(rng.choice([4, 12])), slots=slots, rank=int(rng.integers(1, 5)),
                       grid=int(rng.choice([3, 9])), rope="split_half", rope_axes=axes,
                       rope_theta=float(rng.choice([10.0, 100.0, 1e4])))
    sig = [float(v) for v in rng.uniform(0.0, 1.0, size=slots)]
    wl = W.make_custom_workload(spec, 400 + seed, sigmas=sig)
    w = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    w["adaln_basis"] = w["adaln_basis"] * 10.0
    for k in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
        w[k] = w[k] * 10.0
    x, pos = wl.x.astype(np.float64), wl.pos.astype(np.float64)
    rows = rng.integers(0, slots * spec.tags, size=spec.n).astype(np.int32)
    got = O.mmh3_block(spec, x, rows, pos, sig, w)["out"]
    want = _brute_mmh3(spec, x, rows, pos, sig, w)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_mmh3_block_brute_force_tiny_compat_modes():
    # partial RoPE (k = 1: 3 of 4 pairs turn, dims 6, 7 stay) and a shared adaLN basis
    spec = W.small_spec(_tiny_mmh3_spec(7), rope="partial", rope_axes=(2, 2, 2), adaln_shared=1)
    wl = W.make_custom_workload(spec, 21, sigmas=[0.37, 0.81])
    w = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    assert w["adaln_basis"].shape[0] == spec.tags * 6 * spec.D and w["rope_freq"].shape == (1,)
    w["adaln_basis"] = w["adaln_basis"] * 10.0
    w["rope_freq"] = np.array([0.37])
    for k in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
        w[k] = w[k] * 10.0
    x, pos = wl.x.astype(np.float64), wl.pos.astype(np.float64)
    got = O.mmh3_block(spec, x, wl.rows, pos, [0.37, 0.81], w)
    want = _brute_mmh3(spec, x, wl.rows, pos, [0.37, 0.81], w)
    np.testing.assert_allclose(got["out"], want, rtol=1e-11, atol=1e-11)
    # unrotated dims: q's last two dims are the qk-normed projection as is
    proj = (got["xn"] @ w["w_qkv"][:spec.D].T).reshape(-1, spec.H, spec.hd).transpose(1, 0, 2)
    q_plain = O.rms_norm(proj, w["q_norm"], spec.qk_eps)
    np.testing.assert_array_equal(got["q"][..., 6:], q_plain[..., 6:])
    # relative positions only
    b = O.mmh3_block(spec, x, wl.rows, pos + np.array([5.0, -2.5, 9.0]), [0.37, 0.81], w)
    np.testing.assert_allclose(b["out"], got["out"], rtol=1e-11, atol=1e-12)


def test_shared_adaln_is_the_slot_major_basis_repeated():
    rng = np.random.default_rng(11)
    T, E, D, r = 3, 6, 8, 5
    B = rng.standard_normal((T * E * D, r))
    b = rng.standard_normal(T * E * D)
    tab = rng.standard_normal((9, r))
    ts = [0.3, 0.999]
    shared = O.adaln_mods(B, b, tab, ts, T, E, D, shared=True)
    tiled = O.adaln_mods(np.tile(B, (2, 1)), np.tile(b, 2), tab, ts, T, E, D)
    np.testing.assert_array_equal(shared, tiled)
    # equal timesteps give equal slot blocks
    same = O.adaln_mods(B, b, tab, [0.6, 0.6], T, E, D, shared=True)
    np.testing.assert_array_equal(same[:T], same[T:])


def test_mmh3_forward_audio_slope_rescale_closed_form():
    # the pre-multiplied audio velocity is the unscaled one times d(sigma_a)/d(sigma_v),
    # which for the 12 -> 3 remap sigma / (4 - 3 sigma) is 4 / (4 - 3 sigma)^2
    lay = W.build_layout(3, 1, 4, 4, 2)
    n, D, C, Ca = lay.seq_len, 16, 4, 4
    bs = W.BlockSpec("fwd-tiny", "mmh3", "f32", n=n, D=D, H=2, hd=8, F=12, slots=2, rank=3,
                     grid=9, rope="split_half", rope_axes=(2, 2, 4), rope_theta=100.0)
    hv = W.BlockSpec("hv", "final", "f32", n=n, D=D, H=2, hd=8, F=4 * C, slots=2, tags=1, rank=3, grid=9)
    ha = W.BlockSpec("ha", "final", "f32", n=n, D=D, H=2, hd=8, F=Ca, slots=2, tags=1, rank=3, grid=9)
    rng = np.random.default_rng(12)
    wb = [W.make_custom_workload(bs, 40).weights]
    whv, wha = W.make_custom_workload(hv, 41).weights, W.make_custom_workload(ha, 42).weights
    wv, wa = 0.1 * rng.standard_normal((D, 4 * C)), 0.1 * rng.standard_normal((D, Ca))
    text = rng.standard_normal((3, D))
    video, audio = rng.standard_normal((C, 1, 4, 4)), rng.standard_normal((Ca, 2, 2))
    sv = 0.63
    args = (bs, hv, ha, lay.segments, lay.pos, text, video, audio, [], sv, wb, whv, wha, wv, None,
            wa, None)
    v0, a0 = O.mmh3_forward(*args)
    v1, a1 = O.mmh3_forward(*args, audio_slope_rescale=True)
    np.testing.assert_array_equal(v1, v0)
    np.testing.assert_allclose(a1, a0 * 4.0 / (4.0 - 3.0 * sv) ** 2, rtol=1e-14)


def test_mmh3_block_permutation_equivariant():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(14, n=9)
    perm = np.random.default_rng(0).permutation(9)
    a = O.mmh3_block(spec, x, rows, pos, sig, w)["out"]
    b = O.mmh3_block(spec, x[perm], rows[perm], pos[perm], sig, w)["out"]
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_mmh3_block_rope_translation_invariant():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(15, n=9)
    a = O.mmh3_block(spec, x, rows, pos, sig, w)
    b = O.mmh3_block(spec, x, rows, pos + np.array([3.0, -7.5, 11.25]), sig, w)
    np.testing.assert_allclose(b["o"], a["o"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-11, atol=1e-12)


def test_mmh3_block_zero_gates_identity():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(16)
    D, T, E = spec.D, spec.tags, 6
    basis, bias = w["adaln_basis"].copy(), w["adaln_bias"].copy()
    for r in range(spec.slots * T):
        for e in (2, 5):
            sl = slice((r * E + e) * D, (r * E + e + 1) * D)
            basis[sl] = 0.0
            bias[sl] = 0.0
    w2 = dict(w, adaln_basis=basis, adaln_bias=bias)
    out = O.mmh3_block(spec, x, rows, pos, sig, w2)["out"]
    np.testing.assert_array_equal(out, x)


def test_mmh3_block_scale_minus_one_kills_attention_branch():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(17)
    D, T, E = spec.D, spec.tags, 6
    basis, bias = w["adaln_basis"].copy(), w["adaln_bias"].copy()
    for r in range(spec.slots * T):
        for e, val in ((0, 0.0), (1, -1.0)):
            sl = slice((r * E + e) * D, (r * E + e + 1) * D)
            basis[sl] = 0.0
            bias[sl] = val
    st = O.mmh3_block(spec, x, rows, pos, sig, dict(w, adaln_basis=basis, adaln_bias=bias))
    np.testing.assert_array_equal(st["xn"], 0.0)
    np.testing.assert_array_equal(st["x1"], x)


def test_mmh3_equal_rows_modulated_identically():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(18, n=6)
    x = np.repeat(x[:1], 6, axis=0)
    rows = np.array([1, 1, 4, 4, 1, 4], dtype=np.int32)
    st = O.mmh3_block(spec, x, rows, pos, sig, w)
    np.testing.assert_array_equal(st["xn"][0], st["xn"][1])
    np.testing.assert_array_equal(st["xn"][2], st["xn"][3])
    assert not np.array_equal(st["xn"][0], st["xn"][2])


def test_mmh3_rejects_out_of_range_rows():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(19)
    rows = rows.copy()
    rows[2] = 6
    with pytest.raises(ValueError):
        O.mmh3_block(spec, x, rows, pos, sig, w)


def test_qk_norm_unit_rms_in_block():
    spec, x, rows, pos, sig, w = _tiny_mmh3_inputs(20)
    w = dict(w, q_norm=np.ones(spec.hd), k_norm=np.ones(spec.hd))
    st = O.mmh3_block(spec, x, rows, pos, sig, w)
    # RoPE preserves norms, so q and k keep the RMS sqrt(ms / (ms + eps)) ~ 1
    rq = np.sqrt(np.mean(st["q"] ** 2, axis=-1))
    assert np.all(np.abs(rq - 1.0) < 1e-3)


@pytest.mark.parametrize("shape", [(20, 32, 4, 8, 48, 21), (1, 16, 1, 16, 8, 22), (9, 48, 3, 16, 20, 23),
                                   (33, 24, 2, 12, 64, 24)])
def test_siglip_layer_matches_torch_composition(shape):
    import torch
    import torch.nn.functional as Fn
    n, D, H, hd, F, seed = shape
    spec = W.BlockSpec("tiny_siglip", "siglip", "f32", n=n, D=D, H=H, hd=hd, F=F, eps=1e-6)
    wl = W.make_custom_workload(spec, seed)
    w = {k: torch.from_numpy(v.astype(np.float64)) for k, v in wl.weights.items()}
    x = torch.from_numpy(wl.x.astype(np.float64))
    D, H, hd = spec.D, spec.H, spec.hd
    xn = Fn.layer_norm(x, (D,), w["ln1_w"], w["ln1_b"], 1e-6)
    qkv = Fn.linear(xn, w["w_qkv"], w["b_qkv"])
    q, k, v = (qkv[:, i * D:(i + 1) * D].reshape(-1, H, hd).transpose(0, 1) for i in range(3))
    o = Fn.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(-1, D)
    x1 = x + Fn.linear(o, w["w_out"], w["b_out"])
    h = Fn.gelu(Fn.linear(Fn.layer_norm(x1, (D,), w["ln2_w"], w["ln2_b"], 1e-6), w["w_fc1"], w["b_fc1"]),
                approximate="tanh")
    want = x1 + Fn.linear(h, w["w_fc2"], w["b_fc2"])
    got = O.siglip_layer(spec, wl.x, {k: v.numpy() for k, v in w.items()})["out"]
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)


def test_timestep_embedding_closed_forms():
    e = O.timestep_embedding(0.0, 256)
    np.testing.assert_array_equal(e[:128], 1.0)
    np.testing.assert_array_equal(e[128:], 0.0)
    e = O.timestep_embedding(0.7, 256)
    assert e[0] == pytest.approx(math.cos(0.7)) and e[128] == pytest.approx(math.sin(0.7))
    # the last frequency is 10000^(-127/128)
    assert e[255] == pytest.approx(math.sin(0.7 * 10000.0 ** (-127.0 / 128.0)), rel=1e-13)


def _tiny_zimage(n=10, H=2, hd=8, F=12, axes=(2, 2, 4), seed=22):
    spec = W.BlockSpec("tiny_z", "zimage", "f32", n=n, D=H * hd, H=H, hd=hd, F=F,
                       rope="interleaved", rope_axes=axes, rope_theta=256.0,
                       temb_freq=16, temb_hidden=24)
    wl = W.make_custom_workload(spec, seed)
    w = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    return spec, wl.x.astype(np.float64), wl.pos.astype(np.float64), w


def test_zimage_zero_gates_identity():
    spec, x, pos, w = _tiny_zimage()
    D = spec.D
    aw, ab = w["ada_w"].copy(), w["ada_b"].copy()
    for c in (1, 3):  # gate_msa, gate_mlp -> tanh(0) = 0
        aw[c * D:(c + 1) * D] = 0.0
        ab[c * D:(c + 1) * D] = 0.0
    out = O.zimage_block(spec, x, pos, 0.4, dict(w, ada_w=aw, ada_b=ab))["out"]
    np.testing.assert_array_equal(out, x)


@pytest.mark.parametrize("shape", [(10, 2, 8, 12, (2, 2, 4), 22, 0.3), (1, 1, 16, 8, (4, 6, 6), 23, 0.9),
                                   (17, 3, 8, 20, (2, 2, 4), 24, 0.05), (6, 2, 12, 16, (4, 4, 4), 25, 0.6)])
def test_zimage_block_matches_torch_composition(shape):
    import torch
    import torch.nn.functional as Fn
    spec, x, pos, w = _tiny_zimage(*shape[:6])
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    tw = {k: torch.from_numpy(v) for k, v in w.items()}
    t = shape[6]
    half = spec.temb_freq // 2
    f = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
    arg = t * spec.t_scale * f
    emb = torch.cat([torch.cos(arg), torch.sin(arg)])
    temb = Fn.linear(Fn.silu(Fn.linear(emb, tw["temb_w1"], tw["temb_b1"])), tw["temb_w2"], tw["temb_b2"])
    m = Fn.linear(temb, tw["ada_w"], tw["ada_b"])
    sc1, g1, sc2, g2 = (m[i * D:(i + 1) * D] for i in range(4))
    xt = torch.from_numpy(x)
    xn = Fn.rms_norm(xt, (D,), tw["norm1"], 1e-5) * (1 + sc1)
    qkv = Fn.linear(xn, tw["w_qkv"])
    q, k, v = (qkv[:, i * D:(i + 1) * D].reshape(-1, H, hd) for i in range(3))
    q = Fn.rms_norm(q, (hd,), tw["q_norm"], 1e-5)
    k = Fn.rms_norm(k, (hd,), tw["k_norm"], 1e-5)
    # interleaved rotation through complex multiplication
    ang = []
    for a, d in enumerate(spec.rope_axes):
        om = spec.rope_theta ** (-torch.arange(d // 2, dtype=torch.float64) * 2.0 / d)
        ang.append(torch.from_numpy(pos[:, a:a + 1]) * om[None])
    ang = torch.cat(ang, dim=1)[:, None, :]
    rot = torch.polar(torch.ones_like(ang), ang)

    def rope(z):
        c = torch.view_as_complex(z.reshape(*z.shape[:-1], hd // 2, 2).contiguous()) * rot
        return torch.view_as_real(c).reshape(z.shape)

    q, k = rope(q), rope(k)
    o = Fn.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
    o = o.transpose(0, 1).reshape(-1, D)
    x1 = xt + torch.tanh(g1) * Fn.rms_norm(Fn.linear(o, tw["w_out"]), (D,), tw["post_attn_norm"], 1e-5)
    xf = Fn.rms_norm(x1, (D,), tw["norm2"], 1e-5) * (1 + sc2)
    gu = Fn.linear(xf, tw["w_fc1"])
    y2 = Fn.linear(Fn.silu(gu[:, :F]) * gu[:, F:], tw["w_fc2"])
    want = x1 + torch.tanh(g2) * Fn.rms_norm(y2, (D,), tw["post_ffn_norm"], 1e-5)
    got = O.zimage_block(spec, x, pos, t, w)["out"]
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)


def test_zimage_context_block_is_the_block_with_unit_gates():
    # no modulation: scale 0 and tanh(gate) = 1 (tanh(+inf) is exactly 1)
    spec, x, pos, w = _tiny_zimage()
    cspec = W.small_spec(spec, variant="zcontext")
    D = spec.D
    mods = np.zeros((1, 4 * D))
    mods[0, D:2 * D] = np.inf
    mods[0, 3 * D:] = np.inf
    got = O.zimage_context_block(cspec, x, pos, w)
    want = O.zimage_block(spec, x, pos, None, w, mods=mods)
    for k in ("xn", "q", "o", "x1", "a", "out"):
        np.testing.assert_allclose(got[k], want[k], rtol=1e-13, atol=1e-14)
    assert O.block(cspec, x, None, pos, [], w)["out"] is not None


def test_zimage_final_layer_matches_torch_composition():
    import torch
    import torch.nn.functional as Fn
    fspec = W.BlockSpec("tiny_zf", "zfinal", "f32", n=5, D=16, H=2, hd=8, F=32, eps=1e-6,
                        temb_freq=16, temb_hidden=24)
    w = {k: v.astype(np.float64) for k, v in W.make_custom_workload(fspec, 31).weights.items()}
    h = np.random.default_rng(5).standard_normal((5, 16)) * 3.0 + 1.0
    tw = {k: torch.from_numpy(v) for k, v in w.items()}
    t = 0.7
    half = 8
    f = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
    arg = t * fspec.t_scale * f
    emb = torch.cat([torch.cos(arg), torch.sin(arg)])
    temb = Fn.linear(Fn.silu(Fn.linear(emb, tw["temb_w1"], tw["temb_b1"])), tw["temb_w2"], tw["temb_b2"])
    scale = Fn.linear(Fn.silu(temb), tw["ada_w"], tw["ada_b"])
    xn = Fn.layer_norm(torch.from_numpy(h), (16,), eps=1e-6) * (1 + scale)
    want = Fn.linear(xn, tw["w_fc1"], tw["b_fc1"])
    got = O.zimage_final_layer(fspec, h, t, w)["out"]
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


def test_patchify_image_is_the_page_layout_and_inverts():
    rng = np.random.default_rng(6)
    C, H, W_ = 3, 6, 8
    x = rng.standard_normal((C, H, W_))
    # [C, H, W] -> [C, 1, 1, H/2, 2, W/2, 2] -> axes (1, 2, 3, 5, 4, 6, 0) -> [L, 4C]
    via = x.reshape(C, 1, 1, H // 2, 2, W_ // 2, 2).transpose(1, 2, 3, 5, 4, 6, 0).reshape(-1, 4 * C)
    rows = O.patchify_image(x)
    np.testing.assert_array_equal(rows, via)
    np.testing.assert_array_equal(O.unpatchify_image(rows, C, H, W_), x)


def _tiny_zimage_model():
    D, H_, hd, F, C, cap_dim = 16, 2, 8, 12, 4, 8
    common = dict(D=D, H=H_, hd=hd, F=F, rope="interleaved", rope_axes=(2, 2, 4), rope_theta=256.0,
                  temb_freq=16, temb_hidden=24, t_scale=1000.0)
    bspec = W.BlockSpec("zm", "zimage", "f32", n=7, **common)
    cspec = W.BlockSpec("zc", "zcontext", "f32", n=3, **common)
    fspec = W.BlockSpec("zf", "zfinal", "f32", n=4, eps=1e-6, **dict(common, F=4 * C))
    f64 = lambda d: {k: v.astype(np.float64) for k, v in d.items()}  # noqa: E731
    wl = [f64(W.make_custom_workload(bspec, 50 + i).weights) for i in range(3)]
    wn = [f64(W.make_custom_workload(bspec, 60).weights)]
    wc = [f64(W.make_custom_workload(cspec, 70).weights)]
    wf = f64(W.make_custom_workload(fspec, 80).weights)
    rng = np.random.default_rng(81)
    emb = dict(x_embed_w=0.3 * rng.standard_normal((D, 4 * C)), x_embed_b=0.1 * rng.standard_normal(D),
               cap_norm=1 + 0.1 * rng.standard_normal(cap_dim), cap_eps=1e-6,
               cap_embed_w=0.3 * rng.standard_normal((D, cap_dim)), cap_embed_b=0.1 * rng.standard_normal(D))
    pos = W.zimage_positions(2, 2, 3)
    return (bspec, cspec, fspec, wl, wn, wc, wf, emb, pos, C, cap_dim, rng)


def _zf(m, lat, cap, t, step=0, cache=None):
    bspec, cspec, fspec, wl, wn, wc, wf, emb, pos = m[:9]
    return O.zimage_forward(bspec, cspec, fspec, lat, cap, pos, t, wl, wn, wc, wf, emb["x_embed_w"],
                            emb["x_embed_b"], emb["cap_norm"], emb["cap_eps"], emb["cap_embed_w"],
                            emb["cap_embed_b"], step=step, cache=cache)


def test_zimage_forward_composes_the_pinned_pieces():
    m = _tiny_zimage_model()
    bspec, cspec, fspec, wl, wn, wc, wf, emb, pos, C, cap_dim, rng = m
    lat = rng.standard_normal((C, 4, 4))
    cap = rng.standard_normal((3, cap_dim))
    t = 0.45
    x = O.patchify_image(lat) @ emb["x_embed_w"].T + emb["x_embed_b"]
    x = O.zimage_block(bspec, x, pos[:4], t, wn[0])["out"]
    c = O.rms_norm(cap, emb["cap_norm"], 1e-6) @ emb["cap_embed_w"].T + emb["cap_embed_b"]
    c = O.zimage_context_block(cspec, c, pos[4:], wc[0])["out"]
    u = np.concatenate([x, c])
    for w in wl:
        u = O.zimage_block(bspec, u, pos, t, w)["out"]
    want = O.unpatchify_image(O.zimage_final_layer(fspec, u[:4], t, wf)["out"], C, 4, 4)
    np.testing.assert_allclose(_zf(m, lat, cap, t), want, rtol=1e-12, atol=1e-12)


def test_zimage_forward_step_cache_semantics():
    m = _tiny_zimage_model()
    bspec, cspec, fspec, wl, wn, wc, wf, emb, pos, C, cap_dim, rng = m
    lats = [rng.standard_normal((C, 4, 4)) for _ in range(4)]
    cap = rng.standard_normal((3, cap_dim))
    ts = [0.9, 0.7, 0.5, 0.3]
    # interval 1: every step refreshes, so every step is the plain forward
    c1 = {"layers": 2, "interval": 1}
    for s in range(3):
        np.testing.assert_allclose(_zf(m, lats[s], cap, ts[s], s, c1), _zf(m, lats[s], cap, ts[s]),
                                   rtol=1e-12, atol=1e-12)
    # interval 2, two shallow layers of three: step 0 stores, step 1 reads them
    c2 = {"layers": 2, "interval": 2}
    _zf(m, lats[0], cap, ts[0], 0, c2)
    u_stored = c2["outs"][1]
    got = _zf(m, lats[1], cap, ts[1], 1, c2)
    u = O.zimage_block(bspec, u_stored, pos, ts[1], wl[2])["out"]
    want = O.unpatchify_image(O.zimage_final_layer(fspec, u[:4], ts[1], wf)["out"], C, 4, 4)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # a reused step does not see its latents or the caption features (computed once)
    again = _zf(m, lats[3], rng.standard_normal((3, cap_dim)), ts[1], 1, c2)
    np.testing.assert_array_equal(again, got)
    # step 2 refreshes: the plain forward again (the caption is the stored one, equal)
    np.testing.assert_allclose(_zf(m, lats[2], cap, ts[2], 2, c2), _zf(m, lats[2], cap, ts[2]),
                               rtol=1e-12, atol=1e-12)


def test_rel_rms():
    assert O.rel_rms(np.array([1.0, 2.0]), np.array([1.0, 2.0])) == 0.0
    assert O.rel_rms(np.array([2.0, 0.0]), np.array([1.0, 0.0])) == 1.0


def _tiny_mmh3_model(seed=60):
    """A two-block, three-slot MMH3 model on a keyframe layout small enough
    to compose by hand: text 3, one condition frame, audio 2 x 2, video 2
    frames of a 4 x 4 latent (2 x 2 patch grid)."""
    lay = W.build_layout(3, 2, 4, 4, 2, keyframes=[(0, 9)])
    n, D, C, Ca = lay.seq_len, 16, 4, 8
    bs = W.BlockSpec("fwd-tiny", "mmh3", "f32", n=n, D=D, H=2, hd=8, F=12, slots=3, rank=3,
                     grid=9, rope="split_half", rope_axes=(2, 2, 4), rope_theta=100.0)
    hv = W.BlockSpec("hv", "final", "f32", n=n, D=D, H=2, hd=8, F=4 * C, slots=3, tags=1, rank=3, grid=9)
    ha = W.BlockSpec("ha", "final", "f32", n=n, D=D, H=2, hd=8, F=Ca, slots=3, tags=1, rank=3, grid=9)
    rng = np.random.default_rng(seed)
    wb = []
    for i in range(2):
        w = {k: v.astype(np.float64) for k, v in W.make_custom_workload(bs, seed + 10 + i).weights.items()}
        for k in ("w_qkv", "w_out", "w_fc1", "w_fc2", "adaln_basis"):
            w[k] = w[k] * 10.0  # strong branches, so every piece shows in the output
        wb.append(w)
    whv = {k: v.astype(np.float64) for k, v in W.make_custom_workload(hv, seed + 20).weights.items()}
    wha = {k: v.astype(np.float64) for k, v in W.make_custom_workload(ha, seed + 21).weights.items()}
    for w in (whv, wha):
        w["adaln_basis"] = w["adaln_basis"] * 10.0
    wv, bv = rng.standard_normal((D, 4 * C)), rng.standard_normal(D)
    wa, ba = rng.standard_normal((D, Ca)), rng.standard_normal(D)
    text = rng.standard_normal((3, D))
    video = rng.standard_normal((C, 2, 4, 4))
    audio = rng.standard_normal((Ca, 2, 2))
    cond = [rng.standard_normal((C, 1, 4, 4))]
    return lay, bs, hv, ha, wb, whv, wha, wv, bv, wa, ba, text, video, audio, cond


def test_mmh3_forward_composes_the_pinned_pieces():
    """[MMH3] MiniMaxH3::forward written out step by step from pinned pieces:
    slot timesteps by hand (t_v = 1 - sigma_v, the 12 -> 3 audio remap
    sigma / (4 - 3 sigma), condition frames at 0.999), token rows slot * 3 +
    tag, video and condition frames through the video patch projection, audio
    through the audio one, text as given, the blocks in order, each head at its
    stream's slot, unpacked.  Wrong pairings (condition frames through the
    audio projection, the two heads' slots exchanged, the condition frame at
    the video slot) each change the result."""
    (lay, bs, hv, ha, wb, whv, wha, wv, bv, wa, ba, text, video, audio, cond) = _tiny_mmh3_model()
    sv = 0.63
    got_v, got_a = O.mmh3_forward(bs, hv, ha, lay.segments, lay.pos, text, video, audio, cond, sv,
                                  wb, whv, wha, wv, bv, wa, ba)
    seg = {k: (a, b) for k, a, b in lay.segments}
    assert set(seg) == {"text", "cond", "audio", "video"}

    def compose(cond_proj=(wv, bv), head_slots=(0, 1), cond_slot=2):
        ts = [1.0 - sv, 1.0 - sv / (4.0 - 3.0 * sv), 0.999]  # ascending: video, audio, cond
        assert ts == sorted(ts)
        sig = [1.0 - t for t in ts]
        rows = np.empty(lay.seq_len, np.int64)
        rows[slice(*seg["text"])] = 0 * 3 + 1
        rows[slice(*seg["cond"])] = cond_slot * 3 + 0
        rows[slice(*seg["audio"])] = 1 * 3 + 2
        rows[slice(*seg["video"])] = 0 * 3 + 0
        h = np.zeros((lay.seq_len, bs.D))
        h[slice(*seg["text"])] = text
        h[slice(*seg["video"])] = O.patchify_video(video) @ wv.T + bv
        cw, cb = cond_proj  # the audio projection is narrower: its first columns only
        h[slice(*seg["cond"])] = O.patchify_video(cond[0])[:, :cw.shape[1]] @ cw.T + cb
        h[slice(*seg["audio"])] = O.pack_audio(audio) @ wa.T + ba
        for w in wb:
            h = O.mmh3_block(bs, h, rows, lay.pos, sig, w)["out"]
        a, b = seg["video"]
        rv = O.final_layer(hv, h[a:b], np.full(b - a, head_slots[0]), sig, whv)["out"]
        a, b = seg["audio"]
        ra = O.final_layer(ha, h[a:b], np.full(b - a, head_slots[1]), sig, wha)["out"]
        return (O.unpatchify_video(rv, *video.shape), O.unpack_audio(ra, audio.shape[0], audio.shape[2]))

    want_v, want_a = compose()
    np.testing.assert_allclose(got_v, want_v, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(got_a, want_a, rtol=1e-11, atol=1e-11)
    scale = float(np.sqrt(np.mean(want_v ** 2)))
    for why, kw in {"condition frames through the audio projection": dict(cond_proj=(wa, ba)),
                    "heads' slots exchanged": dict(head_slots=(1, 0)),
                    "condition frame at the video slot": dict(cond_slot=0)}.items():
        bad_v, bad_a = compose(**kw)
        d = max(np.max(np.abs(bad_v - got_v)), np.max(np.abs(bad_a - got_a)))
        assert d > 1e-3 * scale, why

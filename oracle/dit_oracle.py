"""fp64 CPU oracle of one packed diffusion-transformer block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code,
constant table or helper with the HIP library.

Every function is the plain definition, in float64, of one step of the block as
the pages define it.  Matrix products use numpy's ``@`` as a library primitive;
nothing is blocked, fused or reordered beyond what the definition states.

Citation tags (web pages, cited by title and the item on the page):

* [MMH3]   docs.rs source page of cortiq-engine 0.5.72, ``src/mmh3.rs``
* [SIGLIP] docs.rs source page of ffai-argus 0.7.0, ``src/siglip.rs``
* [ENC]    docs.rs source page of inferencelayer 0.2.1, ``src/encoder_cpu.rs``
* [ZIMG]   ollama fork, ``x/imagegen/models/zimage/transformer.go``

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: printed test points, closed forms, library routines (numpy.interp,
torch's scaled-dot-product attention, layer_norm and rms_norm in float64),
invariants and pure-Python brute force on tiny inputs.  No function is left
without a pin.  The pages print no golden forward of a whole block or
evaluation at any size, so those are pinned through code that is the same at
every size: the block by brute force at tiny sizes (random seeds, the
checkpoint modes), by torch compositions (SigLIP layer, Z-Image block) and by
invariants (permutation equivariance, zero-gate identity, RoPE translation
invariance); the MMH3 and Z-Image evaluations as compositions of their pinned
pieces and by their own identities (the Z-Image cache rules, the audio
slope's closed form).
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64

# ---------------------------------------------------------------------------
# Flow-schedule remap ([MMH3] ``time_shift_sigma`` / ``time_shift_slope``)
# ---------------------------------------------------------------------------


def _to_base(sigma: float, shift: float) -> float:
    """Point u of the shared base grid whose shifted sigma is ``sigma``.

    A schedule with shift k maps u to k*u / (1 + (k-1)*u); this is its inverse,
    u = sigma / (k - (k-1)*sigma)."""
    return sigma / (shift - (shift - 1.0) * sigma)


def _from_base(u: float, shift: float) -> float:
    return shift * u / (1.0 + (shift - 1.0) * u)


def sigma_remap(sigma: float, from_shift: float, to_shift: float) -> float:
    """sigma on the ``to_shift`` schedule at the same base-grid point as
    ``sigma`` on the ``from_shift`` schedule ([MMH3] ``time_shift_sigma``)."""
    return _from_base(_to_base(sigma, from_shift), to_shift)


def sigma_remap_slope(sigma: float, from_shift: float, to_shift: float) -> float:
    """d sigma_to / d sigma_from by the chain rule through the base grid
    ([MMH3] ``time_shift_slope``): d(from_base)/du at u times du/dsigma."""
    u = _to_base(sigma, from_shift)
    d_out_du = to_shift / (1.0 + (to_shift - 1.0) * u) ** 2
    du_dsigma = from_shift / (from_shift - (from_shift - 1.0) * sigma) ** 2
    return d_out_du * du_dsigma


def resolve_sigmas(plan: Sequence[tuple]) -> List[float]:
    """Slot sigmas from a workload's slot plan: ("value", v) or
    ("remap", src_slot, from_shift, to_shift)."""
    out: List[float] = []
    for item in plan:
        if item[0] == "value":
            out.append(float(item[1]))
        else:
            _, src, a, b = item
            out.append(sigma_remap(out[src], a, b))
    return out


def mmh3_slots(sigma_v: float, shift_video: float, shift_audio: float, cond_aug: float,
               cond_aug_audio: float, has_cond: bool, has_ref_audio: bool):
    """Timestep slots of one evaluation ([MMH3] ``MiniMaxH3::forward``): video
    at 1 - max(sigma_v, 1e-6), audio at 1 - remap of that sigma, condition
    frames / reference images at max(t_v, cond_aug), reference audio at
    max(t_a, cond_aug_audio); distinct values ascending.  Returns (slot
    timesteps, {stream: slot index or -1})."""
    sv = max(sigma_v, 1e-6)
    tv = 1.0 - sv
    ta = 1.0 - sigma_remap(sv, shift_video, shift_audio)
    ts = [tv, ta]
    tc = max(tv, cond_aug)
    tca = max(ta, cond_aug_audio)
    if has_cond:
        ts.append(tc)
    if has_ref_audio:
        ts.append(tca)
    ts = sorted(set(ts))
    slot = {"video": ts.index(tv), "audio": ts.index(ta),
            "cond": ts.index(tc) if has_cond else -1,
            "ref_audio": ts.index(tca) if has_ref_audio else -1}
    return ts, slot


def mmh3_token_rows(segments, slot, tags: int = 3, text_tags=None) -> np.ndarray:
    """Per-token modulation row slot * tags + tag from (kind, start, stop)
    segments ([MMH3] ``MiniMaxH3::forward``): text at the video slot with the
    text tag, or with its own entry of ``text_tags`` (the layout's per-token
    modality of the prompt span); video, condition frames and reference images
    with the video tag (the latter two at the condition slot); audio and
    reference audio with the audio tag."""
    video, text, audio = 0, 1, 2
    of = {"text": (slot["video"], text), "video": (slot["video"], video),
          "audio": (slot["audio"], audio), "cond": (slot["cond"], video),
          "ref_image": (slot["cond"], video), "ref_audio": (slot["ref_audio"], audio)}
    n = max(b for _, _, b in segments)
    rows = np.empty(n, dtype=np.int64)
    for kind, a, b in segments:
        s, t = of[kind]
        rows[a:b] = s * tags + t
        if kind == "text" and text_tags is not None:
            rows[a:b] = s * tags + np.asarray(text_tags, dtype=np.int64)
    return rows


def mmh3_timestep(sigma: float) -> float:
    """Slot timestep t = 1 - sigma of a block's slot sigma.  [MMH3]
    ``MiniMaxH3::forward`` floors only the video sigma at 1e-6, before the
    audio remap (``mmh3_slots`` does that); every slot timestep it hands to
    ``Adaln::eval`` is used as it is, so a condition slot at t = 1 reads the
    table's last row with weight 1."""
    return 1.0 - sigma


# ---------------------------------------------------------------------------
# Rank-r adaLN ([MMH3] module docs and ``Adaln::eval``)
# ---------------------------------------------------------------------------


def adaln_coords(table: np.ndarray, t: float) -> np.ndarray:
    """Curve coordinates at timestep t: linear interpolation of the [G, r]
    table at p = clamp(t, 0, 1) * (G - 1), the last interval kept whole so
    that t = 1 reads row G - 1 with weight 1 ([MMH3] ``Adaln::eval``).
    The grid coordinate is kept in fp64."""
    tab = np.asarray(table, dtype=F64)
    G = tab.shape[0]
    p = min(max(t, 0.0), 1.0) * (G - 1)
    i0 = min(int(math.floor(p)), G - 2)
    f = p - i0
    return tab[i0] + f * (tab[i0 + 1] - tab[i0])


def adaln_mods(basis: np.ndarray, bias: Optional[np.ndarray], table: np.ndarray,
               ts: Sequence[float], tags: int, chunks: int, D: int,
               shared: bool = False) -> np.ndarray:
    """Modulation rows [S*tags, chunks*D].

    Element (r, e, d) of row r = s*tags + tag is flat index (r*chunks + e)*D + d
    of the modulation buffer ([MMH3] ``Adaln::eval`` layout).  Flat element j
    is bias[j] + sum_k basis[j, k] * c_s[k], evaluated at its own slot's
    coordinates c_s = adaln_coords(table, ts[s]) (slot-major basis: rows
    [s*tags*chunks*D, (s+1)*tags*chunks*D) belong to slot s).  ``shared``:
    the basis and bias hold one slot's tags*chunks*D rows and the same map is
    applied at every slot's timestep (``Adaln::eval`` evaluating one W at
    each distinct timestep)."""
    B = np.asarray(basis, dtype=F64)
    bvec = None if bias is None else np.asarray(bias, dtype=F64)
    per_slot = tags * chunks * D
    S = len(ts)
    if shared:
        assert B.shape[0] == per_slot, "a shared basis holds one slot's rows"
    else:
        assert B.shape[0] == S * per_slot, "basis rows must cover every slot"
    out = np.empty(S * per_slot, dtype=F64)
    for s, t in enumerate(ts):
        c = adaln_coords(table, t)
        blk = slice(s * per_slot, (s + 1) * per_slot)
        src = slice(0, per_slot) if shared else blk
        out[blk] = B[src] @ c
        if bvec is not None:
            out[blk] += bvec[src]
    return out.reshape(S * tags, chunks * D)


# ---------------------------------------------------------------------------
# Norms and activations
# ---------------------------------------------------------------------------


def rms_norm(x: np.ndarray, g: Optional[np.ndarray], eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis ([MMH3]
    ``rms_norm_into``; per head for qk-norm, [ENC] ``rms_norm_heads``)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    return y if g is None else y * np.asarray(g, dtype=F64)


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b, variance biased and taken in a
    second pass over (x - mean) ([ENC] ``layer_norm_rows``)."""
    x = np.asarray(x, dtype=F64)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, F64) + np.asarray(b, F64)


def modulate(xn: np.ndarray, shift: Optional[np.ndarray], scale: np.ndarray) -> np.ndarray:
    """x * (1 + scale) + shift ([MMH3] ``modulate``; no shift in [ZIMG])."""
    y = xn * (1.0 + scale)
    return y if shift is None else y + shift


def silu(v: np.ndarray) -> np.ndarray:
    """v / (1 + e^-v) ([MMH3] ``silu``)."""
    v = np.asarray(v, dtype=F64)
    return v / (1.0 + np.exp(-v))


def gelu_tanh(v: np.ndarray) -> np.ndarray:
    """Tanh-form GELU, 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
    ([SIGLIP] ``GeluBiasOp``, the ``gelu_pytorch_tanh`` activation)."""
    v = np.asarray(v, dtype=F64)
    return 0.5 * v * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))


# ---------------------------------------------------------------------------
# 3-axis RoPE
# ---------------------------------------------------------------------------


def rope_angles(pos: np.ndarray, axes: Sequence[int], theta: float) -> np.ndarray:
    """Rotation angles [n, P], P = sum(axes)/2.

    Axis a (t, h, w in order) with d_a dims contributes d_a/2 angles
    pos[a] * theta^(-2m/d_a), m < d_a/2, concatenated in axis order
    ([MMH3] ``rope_angles``; per-axis frequencies as in [ZIMG]
    ``prepareRoPE3D``)."""
    pos = np.asarray(pos, dtype=F64)
    parts = []
    for a, d in enumerate(axes):
        m = np.arange(d // 2, dtype=F64)
        omega = float(theta) ** (-2.0 * m / d)
        parts.append(pos[:, a:a + 1] * omega[None, :])
    return np.concatenate(parts, axis=1)


def rope_angles_shared(pos: np.ndarray, freq: np.ndarray) -> np.ndarray:
    """Rotation angles [n, 3k] of the checkpoint form: the k frequencies of
    ``freq`` serve all three axes, angle a*k + j = pos[a] * freq[j], axes in
    order t, h, w ([MMH3] ``rope_angles`` over ``inv_freq``).  With
    split-half pairs (j, j + 3k), head dims from 6k on stay unrotated
    ([MMH3] ``norm_rope_w``)."""
    pos = np.asarray(pos, dtype=F64)
    f = np.asarray(freq, dtype=F64)
    return np.concatenate([pos[:, a:a + 1] * f[None, :] for a in range(3)], axis=1)


def rope_for(spec, pos: np.ndarray, w: Dict[str, np.ndarray]):
    """(angles [n, P], pair layout) of a block's RoPE."""
    if spec.rope == "partial":
        return rope_angles_shared(pos, w["rope_freq"]), "split_half"
    return rope_angles(pos, spec.rope_axes, spec.rope_theta), spec.rope


def rope_rotate(x: np.ndarray, ang: np.ndarray, mode: str) -> np.ndarray:
    """Rotate pairs of the last axis by ``ang`` (broadcast over leading axes).

    split_half: pair (j, j + P) ([MMH3] ``norm_rope_w``);
    interleaved: pair (2j, 2j + 1) ([ZIMG] ``applyRoPE3D``).
    Each pair (a, b) becomes (a cos - b sin, a sin + b cos)."""
    x = np.array(x, dtype=F64, copy=True)
    P = ang.shape[-1]
    c, s = np.cos(ang), np.sin(ang)
    if mode == "split_half":
        a, b = x[..., :P].copy(), x[..., P:2 * P].copy()
        x[..., :P] = a * c - b * s
        x[..., P:2 * P] = a * s + b * c
    elif mode == "interleaved":
        a, b = x[..., 0:2 * P:2].copy(), x[..., 1:2 * P:2].copy()
        x[..., 0:2 * P:2] = a * c - b * s
        x[..., 1:2 * P:2] = a * s + b * c
    else:
        raise ValueError(mode)
    return x


# ---------------------------------------------------------------------------
# Attention ([MMH3] ``attention`` host loop and ``softmax_inplace``)
# ---------------------------------------------------------------------------


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full bidirectional softmax attention per head, no mask.

    q [H, m, hd], k and v [H, n, hd] -> [H, m, hd].  Scores are
    scale * q.k; each row has its maximum subtracted before exp and is divided
    by its sum."""
    H = q.shape[0]
    out = np.empty((H, q.shape[1], v.shape[2]), dtype=F64)
    for h in range(H):
        s = scale * (np.asarray(q[h], F64) @ np.asarray(k[h], F64).T)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        out[h] = p @ np.asarray(v[h], F64)
    return out


def sample_ranges(seq_starts: Sequence[int], n: int) -> List[tuple]:
    """[(a, e)] token ranges of the packed samples; checks 0 = s_0 <= ... <= s_N = n."""
    st = [int(v) for v in seq_starts]
    if len(st) < 2 or st[0] != 0 or st[-1] != n or any(b < a for a, b in zip(st, st[1:])):
        raise ValueError("seq_starts must rise from 0 to n")
    return list(zip(st[:-1], st[1:]))


def attention_packed(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     qtok: np.ndarray, seq_starts: Sequence[int]) -> np.ndarray:
    """Attention over independent samples packed in one sequence ([ENC]
    ``attention_ragged``): query row r (token qtok[r]) of sample s attends only
    to the keys of that sample, tokens [seq_starts[s], seq_starts[s+1]).

    q [H, m, hd]; k, v [H, n, hd] over all tokens -> [H, m, hd]."""
    qtok = np.asarray(qtok, dtype=np.int64)
    out = np.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=F64)
    for a, e in sample_ranges(seq_starts, k.shape[1]):
        r = np.nonzero((qtok >= a) & (qtok < e))[0]
        if r.size:
            out[:, r] = attention(q[:, r], k[:, a:e], v[:, a:e], scale)
    return out


def _attend(q, k, v, scale, sel, seq_starts):
    if seq_starts is None:
        return attention(q, k, v, scale)
    return attention_packed(q, k, v, scale, sel, seq_starts)


def _heads(y: np.ndarray, H: int, hd: int) -> np.ndarray:
    """[m, H*hd] -> [H, m, hd] (head h is columns [h*hd, (h+1)*hd))."""
    return np.ascontiguousarray(y.reshape(y.shape[0], H, hd).transpose(1, 0, 2))


def _merge(o: np.ndarray) -> np.ndarray:
    """[H, m, hd] -> [m, H*hd]."""
    H, m, hd = o.shape
    return np.ascontiguousarray(o.transpose(1, 0, 2).reshape(m, H * hd))


def _lin(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """x @ W^T (+ b), W stored [out, in]."""
    y = np.asarray(x, F64) @ np.asarray(w, F64).T
    return y if b is None else y + np.asarray(b, F64)


def _sel(qrows: Optional[np.ndarray], n: int) -> np.ndarray:
    return np.arange(n) if qrows is None else np.asarray(qrows, dtype=np.int64)


# ---------------------------------------------------------------------------
# MiniMax-H3 block ([MMH3] ``block_forward``, ``ffn_tail``, ``residual``)
# ---------------------------------------------------------------------------


def mmh3_block(spec, x: np.ndarray, rows: np.ndarray, pos: Optional[np.ndarray],
               sigmas: Sequence[float], w: Dict[str, np.ndarray],
               qrows: Optional[np.ndarray] = None,
               seq_starts: Optional[Sequence[int]] = None,
               mods: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One MiniMax-H3 block over the packed sequence.  ``mods`` [R, 6D], if
    given, replaces the rows evaluated from the basis (``sigmas`` unused).

    Stages (fp64): mods [R, 6D]; xn [n, D]; q, k, v [H, *, hd] (q and k after
    qk-norm and RoPE, q unscaled); o [m, D]; x1, xn2 [m, D]; a [m, F];
    out [m, D], where m indexes ``qrows`` (all tokens if None).  K and V always
    cover every token, because every query attends to all of them (to all of
    its own sample's, when ``seq_starts`` packs several samples)."""
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    n = x.shape[0]
    x = np.asarray(x, F64)
    rows = np.asarray(rows, dtype=np.int64)
    R = spec.slots * spec.tags
    if rows.size and (rows.min() < 0 or rows.max() >= R):
        raise ValueError("modulation row out of range")
    if mods is None:
        ts = [mmh3_timestep(s) for s in sigmas]
        mods = adaln_mods(w["adaln_basis"], w.get("adaln_bias"), w["adaln_table"], ts,
                          spec.tags, 6, D, bool(getattr(spec, "adaln_shared", 0)))
    mods = np.asarray(mods, F64)
    chunk = lambda r, e: mods[r, e * D:(e + 1) * D]  # noqa: E731

    # pre-norm + modulate (chunks 0 shift, 1 scale)
    xn = modulate(rms_norm(x, w["norm1"], spec.eps), chunk(rows, 0), chunk(rows, 1))
    sel = _sel(qrows, n)

    # QKV (no bias), head split; qk-norm then RoPE on q and k
    wq, wk, wv = (w["w_qkv"][i * D:(i + 1) * D] for i in range(3))
    k = rms_norm(_heads(_lin(xn, wk), H, hd), w["k_norm"], spec.qk_eps)
    v = _heads(_lin(xn, wv), H, hd)
    q = rms_norm(_heads(_lin(xn[sel], wq), H, hd), w["q_norm"], spec.qk_eps)
    if spec.rope != "none":
        ang, mode = rope_for(spec, pos, w)
        k = rope_rotate(k, ang[None], mode)
        q = rope_rotate(q, ang[sel][None], mode)

    o = _merge(_attend(q, k, v, 1.0 / math.sqrt(hd), sel, seq_starts))
    rs = rows[sel]
    x1 = x[sel] + chunk(rs, 2) * _lin(o, w["w_out"])

    # FFN half: chunks 3 shift, 4 scale, 5 gate; fc1 rows are [gate | up]
    xn2 = modulate(rms_norm(x1, w["norm2"], spec.eps), chunk(rs, 3), chunk(rs, 4))
    gu = _lin(xn2, w["w_fc1"])
    a = silu(gu[:, :F]) * gu[:, F:]
    out = x1 + chunk(rs, 5) * _lin(a, w["w_fc2"])
    return dict(mods=mods, xn=xn, q=q, k=k, v=v, o=o, x1=x1, xn2=xn2, a=a, out=out)


# ---------------------------------------------------------------------------
# Token refiner: the MiniMax-H3 block without modulation ([MMH3] ``refine_text``
# runs ``block_forward`` with no modulation buffer: ``norm_rows`` without
# ``modulate``, ``residual`` without a gate)
# ---------------------------------------------------------------------------


def refiner_block(spec, x: np.ndarray, pos: Optional[np.ndarray], w: Dict[str, np.ndarray],
                  qrows: Optional[np.ndarray] = None,
                  seq_starts: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """xn = RMSNorm(x; norm1); q, k with qk-norm (RoPE only if the spec has
    one; the refiner itself is unrotated); x1 = x + W_out o; xn2 =
    RMSNorm(x1; norm2); out = x1 + W2 (silu(g) * u).  Stages as mmh3_block."""
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    n = x.shape[0]
    x = np.asarray(x, F64)
    sel = _sel(qrows, n)
    xn = rms_norm(x, w["norm1"], spec.eps)
    wq, wk, wv = (w["w_qkv"][i * D:(i + 1) * D] for i in range(3))
    k = rms_norm(_heads(_lin(xn, wk), H, hd), w["k_norm"], spec.qk_eps)
    v = _heads(_lin(xn, wv), H, hd)
    q = rms_norm(_heads(_lin(xn[sel], wq), H, hd), w["q_norm"], spec.qk_eps)
    if spec.rope != "none":
        ang, mode = rope_for(spec, pos, w)
        k = rope_rotate(k, ang[None], mode)
        q = rope_rotate(q, ang[sel][None], mode)
    o = _merge(_attend(q, k, v, 1.0 / math.sqrt(hd), sel, seq_starts))
    x1 = x[sel] + _lin(o, w["w_out"])
    xn2 = rms_norm(x1, w["norm2"], spec.eps)
    gu = _lin(xn2, w["w_fc1"])
    a = silu(gu[:, :F]) * gu[:, F:]
    out = x1 + _lin(a, w["w_fc2"])
    return dict(xn=xn, q=q, k=k, v=v, o=o, x1=x1, xn2=xn2, a=a, out=out)


# ---------------------------------------------------------------------------
# Output head ([MMH3] ``MiniMaxH3::forward``, "heads": ``final_adaln.eval``, the
# final ``rms_norm_into``, the shift/scale of the token's timestep row, the
# head projection and the sign flip)
# ---------------------------------------------------------------------------


def linear(a: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None,
           alpha: float = 1.0) -> np.ndarray:
    """alpha * (a @ W^T + b), W stored [out, in] (the embedding and head
    projections)."""
    return alpha * _lin(a, w, b)


def final_layer(spec, h: np.ndarray, rows: Optional[np.ndarray], sigmas: Sequence[float],
                w: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """mods [S, 2D] = rank-r adaLN of the head (one modality: chunk 0 shift,
    chunk 1 scale per timestep slot); hn = RMSNorm(h; g) * (1 + scale_r) +
    shift_r with r the token's slot; out = -(W hn + b)."""
    D = spec.D
    h = np.asarray(h, F64)
    rows = np.zeros(h.shape[0], np.int64) if rows is None else np.asarray(rows, np.int64)
    ts = [mmh3_timestep(s) for s in sigmas]
    mods = adaln_mods(w["adaln_basis"], w.get("adaln_bias"), w["adaln_table"], ts, spec.tags, 2, D,
                      bool(getattr(spec, "adaln_shared", 0)))
    hn = modulate(rms_norm(h, w["norm1"], spec.eps), mods[rows, 0:D], mods[rows, D:2 * D])
    out = -_lin(hn, w["w_fc1"], w.get("b_fc1"))
    return dict(mods=mods, xn=hn, out=out)


def stack(spec, x, rows, pos, sigmas, ws: Sequence[Dict[str, np.ndarray]], qrows=None,
          seq_starts=None) -> np.ndarray:
    """Blocks in order, each with its own weights; returns out of the last
    (all rows: every block needs all tokens of the previous one)."""
    h = np.asarray(x, F64)
    for w in ws:
        h = block(spec, h, rows, pos, sigmas, w, None, seq_starts)["out"]
    return h if qrows is None else h[np.asarray(qrows)]


# ---------------------------------------------------------------------------
# Latent streams and one denoise evaluation ([MMH3] ``patchify_video``,
# ``unpatchify_video``, ``pack_audio``, ``unpack_audio``, ``MiniMaxH3::forward``)
# ---------------------------------------------------------------------------


def patchify_video(x: np.ndarray) -> np.ndarray:
    """[C, T, H, W] -> [T*(H/2)*(W/2), 4C]: row (t, h2, w2), column c*4 + p*2 + q
    = x[c, t, 2*h2 + p, 2*w2 + q]."""
    C, T, H, W = x.shape
    out = np.empty((T * (H // 2) * (W // 2), 4 * C), dtype=x.dtype)
    r = 0
    for t in range(T):
        for h2 in range(H // 2):
            for w2 in range(W // 2):
                out[r] = x[:, t, 2 * h2:2 * h2 + 2, 2 * w2:2 * w2 + 2].reshape(-1)
                r += 1
    return out


def unpatchify_video(rows: np.ndarray, C: int, T: int, H: int, W: int) -> np.ndarray:
    """Inverse of ``patchify_video``."""
    x = np.empty((C, T, H, W), dtype=rows.dtype)
    r = 0
    for t in range(T):
        for h2 in range(H // 2):
            for w2 in range(W // 2):
                x[:, t, 2 * h2:2 * h2 + 2, 2 * w2:2 * w2 + 2] = rows[r].reshape(C, 2, 2)
                r += 1
    return x


def pack_audio(x: np.ndarray) -> np.ndarray:
    """[C, 2, T] -> [2T, C]: row ch*T + t, column c = x[c, ch, t]."""
    return np.ascontiguousarray(np.concatenate([x[:, 0, :].T, x[:, 1, :].T], axis=0))


def unpack_audio(rows: np.ndarray, C: int, T: int) -> np.ndarray:
    """Inverse of ``pack_audio``."""
    x = np.empty((C, 2, T), dtype=rows.dtype)
    x[:, 0, :] = rows[:T].T
    x[:, 1, :] = rows[T:].T
    return x


def mmh3_forward(block_spec, head_v_spec, head_a_spec, segments, pos, text, video, audio, conds,
                 sigma_v: float, w_blocks, w_head_v, w_head_a, w_vpatch, b_vpatch, w_apatch,
                 b_apatch, shift_video=12.0, shift_audio=3.0, cond_aug=0.999,
                 cond_aug_audio=1.0, audio_slope_rescale=False, text_tags=None):
    """One denoise evaluation: embed (video and condition frames through the
    video patch projection, audio through the audio one, refined text as
    given), the blocks with the evaluation's slots and token rows, the two
    heads (negated) and the unpacking.  ``segments``: (kind, start, stop) with
    kinds "text", "video", "audio", "cond".  Returns (video velocity [C, T, H,
    W], audio velocity [Ca, 2, Ta] or None).  ``audio_slope_rescale``
    multiplies the audio velocity by d(sigma_a)/d(sigma_v) (the pre-multiplied
    single-schedule form the [MMH3] module docs describe of the reference
    model; unscaled otherwise)."""
    ts, slot = mmh3_slots(sigma_v, shift_video, shift_audio, cond_aug, cond_aug_audio,
                          any(k == "cond" for k, _, _ in segments), False)
    sig = [1.0 - t for t in ts] + [1.0 - ts[-1]] * (block_spec.slots - len(ts))
    rows = mmh3_token_rows(segments, slot, text_tags=text_tags)
    n, D = rows.shape[0], block_spec.D
    C, T, H, W = video.shape
    h = np.zeros((n, D))
    ci = 0
    for kind, a, b in segments:
        if kind == "text":
            h[a:b] = np.asarray(text, F64)
        elif kind == "video":
            h[a:b] = linear(patchify_video(np.asarray(video, F64)), w_vpatch, b_vpatch)
        elif kind == "cond":
            h[a:b] = linear(patchify_video(np.asarray(conds[ci], F64)), w_vpatch, b_vpatch)
            ci += 1
        elif kind == "audio":
            h[a:b] = linear(pack_audio(np.asarray(audio, F64)), w_apatch, b_apatch)
    for w in w_blocks:
        h = mmh3_block(block_spec, h, rows, pos, sig, w)["out"]
    out_v = out_a = None
    for kind, a, b in segments:
        if kind == "video":
            r = final_layer(head_v_spec, h[a:b], np.full(b - a, slot["video"]), sig, w_head_v)["out"]
            out_v = unpatchify_video(r, C, T, H, W)
        elif kind == "audio":
            r = final_layer(head_a_spec, h[a:b], np.full(b - a, slot["audio"]), sig, w_head_a)["out"]
            out_a = unpack_audio(r, audio.shape[0], audio.shape[2])
            if audio_slope_rescale:
                out_a = out_a * sigma_remap_slope(sigma_v, shift_video, shift_audio)
    return out_v, out_a


# ---------------------------------------------------------------------------
# SigLIP encoder layer ([SIGLIP] ``Layer::forward``, ``finish_attention``)
# ---------------------------------------------------------------------------


def siglip_layer(spec, x: np.ndarray, w: Dict[str, np.ndarray],
                 qrows: Optional[np.ndarray] = None,
                 seq_starts: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Pre-LN encoder layer: LN1 -> qkv (+bias) -> attention (scores scaled by
    hd^-1/2) -> out (+bias) + residual -> LN2 -> fc1 (+bias) -> GELU-tanh ->
    fc2 (+bias) + residual.  Stages as in ``mmh3_block`` (no mods)."""
    D, H, hd = spec.D, spec.H, spec.hd
    n = x.shape[0]
    x = np.asarray(x, F64)
    sel = _sel(qrows, n)
    xn = layer_norm(x, w["ln1_w"], w["ln1_b"], spec.eps)
    wq, wk, wv = (w["w_qkv"][i * D:(i + 1) * D] for i in range(3))
    bq, bk, bv = (w["b_qkv"][i * D:(i + 1) * D] for i in range(3))
    k = _heads(_lin(xn, wk, bk), H, hd)
    v = _heads(_lin(xn, wv, bv), H, hd)
    q = _heads(_lin(xn[sel], wq, bq), H, hd)
    o = _merge(_attend(q, k, v, 1.0 / math.sqrt(hd), sel, seq_starts))
    x1 = x[sel] + _lin(o, w["w_out"], w["b_out"])
    xn2 = layer_norm(x1, w["ln2_w"], w["ln2_b"], spec.eps)
    a = gelu_tanh(_lin(xn2, w["w_fc1"], w["b_fc1"]))
    out = x1 + _lin(a, w["w_fc2"], w["b_fc2"])
    return dict(xn=xn, q=q, k=k, v=v, o=o, x1=x1, xn2=xn2, a=a, out=out)


# ---------------------------------------------------------------------------
# Z-Image block ([ZIMG] ``TimestepEmbedder``, ``TransformerBlock.Forward``)
# ---------------------------------------------------------------------------


def timestep_embedding(t: float, dim: int) -> np.ndarray:
    """[cos(t f_i) | sin(t f_i)], f_i = exp(-ln(10000) i / (dim/2)), i < dim/2
    ([ZIMG] ``TimestepEmbedder.Forward``)."""
    half = dim // 2
    f = np.exp(-math.log(10000.0) * np.arange(half, dtype=F64) / half)
    return np.concatenate([np.cos(t * f), np.sin(t * f)])


def zimage_mods(spec, t: float, w: Dict[str, np.ndarray]) -> np.ndarray:
    """[1, 4D] = adaLN(temb), temb = L2(silu(L1(sinusoid(t * t_scale)))); the
    block's adaLN linear takes temb directly ([ZIMG] ``Forward`` and
    ``TransformerBlock.Forward``).  Chunks: scale_msa, gate_msa, scale_mlp,
    gate_mlp."""
    e = timestep_embedding(t * spec.t_scale, spec.temb_freq)
    h = silu(_lin(e[None], w["temb_w1"], w["temb_b1"]))
    temb = _lin(h, w["temb_w2"], w["temb_b2"])
    return _lin(temb, w["ada_w"], w["ada_b"])


def zimage_block(spec, x: np.ndarray, pos: np.ndarray, t: float, w: Dict[str, np.ndarray],
                 qrows: Optional[np.ndarray] = None,
                 seq_starts: Optional[Sequence[int]] = None,
                 mods: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Modulated Z-Image block: x1 = x + tanh(gate_msa) * RMSNorm(Attn(RMSNorm(x)
    * (1 + scale_msa))); out = x1 + tanh(gate_mlp) * RMSNorm(W2(silu(W1 xf) *
    W3 xf)) with xf = RMSNorm(x1) * (1 + scale_mlp).  Interleaved RoPE.
    fc1 rows are [W1 (gate) | W3 (up)].  Extra stages: mods [1, 4D], y (out
    projection before its norm), y2 (fc2 output before its norm)."""
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    n = x.shape[0]
    x = np.asarray(x, F64)
    sel = _sel(qrows, n)
    mods = zimage_mods(spec, t, w) if mods is None else np.asarray(mods, F64)
    sc_msa, g_msa, sc_mlp, g_mlp = (mods[0, i * D:(i + 1) * D] for i in range(4))
    xn = modulate(rms_norm(x, w["norm1"], spec.eps), None, sc_msa)
    wq, wk, wv = (w["w_qkv"][i * D:(i + 1) * D] for i in range(3))
    ang = rope_angles(pos, spec.rope_axes, spec.rope_theta)
    k = rope_rotate(rms_norm(_heads(_lin(xn, wk), H, hd), w["k_norm"], spec.qk_eps),
                    ang[None], spec.rope)
    v = _heads(_lin(xn, wv), H, hd)
    q = rope_rotate(rms_norm(_heads(_lin(xn[sel], wq), H, hd), w["q_norm"], spec.qk_eps),
                    ang[sel][None], spec.rope)
    o = _merge(_attend(q, k, v, 1.0 / math.sqrt(hd), sel, seq_starts))
    y = _lin(o, w["w_out"])
    x1 = x[sel] + np.tanh(g_msa) * rms_norm(y, w["post_attn_norm"], spec.eps)
    xn2 = modulate(rms_norm(x1, w["norm2"], spec.eps), None, sc_mlp)
    gu = _lin(xn2, w["w_fc1"])
    a = silu(gu[:, :F]) * gu[:, F:]
    y2 = _lin(a, w["w_fc2"])
    out = x1 + np.tanh(g_mlp) * rms_norm(y2, w["post_ffn_norm"], spec.eps)
    return dict(mods=mods, xn=xn, q=q, k=k, v=v, o=o, y=y, x1=x1, xn2=xn2, a=a, y2=y2,
                out=out)


def zimage_context_block(spec, x: np.ndarray, pos: np.ndarray, w: Dict[str, np.ndarray],
                         qrows: Optional[np.ndarray] = None,
                         seq_starts: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """The Z-Image block without modulation, as the context (caption) refiner
    runs it ([ZIMG] ``TransformerBlock.Forward`` with no adaLN): x1 = x +
    RMSNorm(Attn(RMSNorm(x; norm1)); post_attn_norm); out = x1 +
    RMSNorm(FFN(RMSNorm(x1; norm2)); post_ffn_norm).  Stages as zimage_block
    without mods."""
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    n = x.shape[0]
    x = np.asarray(x, F64)
    sel = _sel(qrows, n)
    xn = rms_norm(x, w["norm1"], spec.eps)
    wq, wk, wv = (w["w_qkv"][i * D:(i + 1) * D] for i in range(3))
    ang = rope_angles(pos, spec.rope_axes, spec.rope_theta)
    k = rope_rotate(rms_norm(_heads(_lin(xn, wk), H, hd), w["k_norm"], spec.qk_eps),
                    ang[None], spec.rope)
    v = _heads(_lin(xn, wv), H, hd)
    q = rope_rotate(rms_norm(_heads(_lin(xn[sel], wq), H, hd), w["q_norm"], spec.qk_eps),
                    ang[sel][None], spec.rope)
    o = _merge(_attend(q, k, v, 1.0 / math.sqrt(hd), sel, seq_starts))
    y = _lin(o, w["w_out"])
    x1 = x[sel] + rms_norm(y, w["post_attn_norm"], spec.eps)
    xn2 = rms_norm(x1, w["norm2"], spec.eps)
    gu = _lin(xn2, w["w_fc1"])
    a = silu(gu[:, :F]) * gu[:, F:]
    y2 = _lin(a, w["w_fc2"])
    out = x1 + rms_norm(y2, w["post_ffn_norm"], spec.eps)
    return dict(xn=xn, q=q, k=k, v=v, o=o, y=y, x1=x1, xn2=xn2, a=a, y2=y2, out=out)


def zimage_final_layer(spec, h: np.ndarray, t: float, w: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """[ZIMG] ``FinalLayer.Forward``: scale = W_a silu(temb) + b_a with temb
    the timestep MLP's output at t * t_scale; out = W (LayerNorm without
    affine(h; eps) * (1 + scale)) + b."""
    D = spec.D
    e = timestep_embedding(t * spec.t_scale, spec.temb_freq)
    temb = _lin(silu(_lin(e[None], w["temb_w1"], w["temb_b1"])), w["temb_w2"], w["temb_b2"])
    scale = _lin(silu(temb), w["ada_w"], w["ada_b"])
    hn = layer_norm(np.asarray(h, F64), np.ones(D), np.zeros(D), spec.eps) * (1.0 + scale)
    return dict(mods=scale, xn=hn, out=_lin(hn, w["w_fc1"], w.get("b_fc1")))


def patchify_image(x: np.ndarray) -> np.ndarray:
    """[C, H, W] -> [(H/2)*(W/2), 4C]: row (h2, w2), column (p*2 + q)*C + c =
    x[c, 2*h2 + p, 2*w2 + q] ([ZIMG] ``PatchifyLatents``, channel fastest)."""
    C, H, W = x.shape
    out = np.empty(((H // 2) * (W // 2), 4 * C), dtype=x.dtype)
    for h2 in range(H // 2):
        for w2 in range(W // 2):
            r = h2 * (W // 2) + w2
            for p in range(2):
                for q in range(2):
                    out[r, (p * 2 + q) * C:(p * 2 + q + 1) * C] = x[:, 2 * h2 + p, 2 * w2 + q]
    return out


def unpatchify_image(rows: np.ndarray, C: int, H: int, W: int) -> np.ndarray:
    """The inverse of patchify_image ([ZIMG] ``UnpatchifyLatents``)."""
    x = np.empty((C, H, W), dtype=rows.dtype)
    for h2 in range(H // 2):
        for w2 in range(W // 2):
            r = h2 * (W // 2) + w2
            for p in range(2):
                for q in range(2):
                    x[:, 2 * h2 + p, 2 * w2 + q] = rows[r, (p * 2 + q) * C:(p * 2 + q + 1) * C]
    return x


def zimage_forward(bspec, cspec, fspec, latents, cap_feats, pos, t: float, w_layers, w_noise,
                   w_context, w_final, x_embed_w, x_embed_b, cap_norm, cap_eps, cap_embed_w,
                   cap_embed_b, step: int = 0, cache: Optional[dict] = None) -> np.ndarray:
    """The Z-Image transformer ([ZIMG] ``Transformer.Forward``, and with
    ``cache`` ``ForwardWithCache``): image patches through the x embedder and
    the noise refiners (image positions), the caption through RMSNorm, the cap
    embedder and the context refiners (caption positions), the main layers over
    [image | caption], the final layer on the image tokens, unpatchified.

    ``cache``: {"layers": k, "interval": m} plus the state this function keeps
    in it across steps: the refined caption (computed once) and the output of
    each of the first k main layers, stored on refresh steps (step % m == 0)
    and read in place of computing the layer on the other steps."""
    C, H, W = latents.shape
    ni = (H // 2) * (W // 2)
    pos = np.asarray(pos, F64)
    x = linear(patchify_image(np.asarray(latents, F64)), x_embed_w, x_embed_b)
    if cache is not None and cache.get("caption") is not None:
        cap = cache["caption"]
    else:
        cap = linear(rms_norm(np.asarray(cap_feats, F64), cap_norm, cap_eps), cap_embed_w, cap_embed_b)
        for w in w_context:
            cap = zimage_context_block(cspec, cap, pos[ni:], w)["out"]
        if cache is not None:
            cache["caption"] = cap
    for w in w_noise:
        x = zimage_block(bspec, x, pos[:ni], t, w)["out"]
    u = np.concatenate([x, cap], axis=0)
    refresh = cache is None or step % cache["interval"] == 0
    stored = cache.setdefault("outs", {}) if cache is not None else {}
    k = cache["layers"] if cache is not None else 0
    for i, w in enumerate(w_layers):
        if i < k and not refresh and i in stored:
            u = stored[i]
        else:
            u = zimage_block(bspec, u, pos, t, w)["out"]
            if i < k and refresh:
                stored[i] = u
    out = zimage_final_layer(fspec, u[:ni], t, w_final)["out"]
    return unpatchify_image(out, C, H, W)


def block(spec, x, rows, pos, sigmas, w, qrows=None, seq_starts=None,
          mods=None) -> Dict[str, np.ndarray]:
    """Dispatch on the block variant.  ``sigmas``: slot sigmas (mmh3) or
    [t] (zimage); ignored for siglip and refiner.  ``seq_starts``: packed samples (None =
    one sequence).  ``mods``: modulation rows replacing the evaluated ones."""
    if spec.variant == "mmh3":
        return mmh3_block(spec, x, rows, pos, sigmas, w, qrows, seq_starts, mods)
    if spec.variant == "siglip":
        return siglip_layer(spec, x, w, qrows, seq_starts)
    if spec.variant == "zimage":
        return zimage_block(spec, x, pos, sigmas[0] if sigmas else None, w, qrows, seq_starts, mods)
    if spec.variant == "refiner":
        return refiner_block(spec, x, pos, w, qrows, seq_starts)
    if spec.variant == "zcontext":
        return zimage_context_block(spec, x, pos, w, qrows, seq_starts)
    raise ValueError(spec.variant)


def rel_rms(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 (the parity metric)."""
    a = np.asarray(a, F64)
    ref = np.asarray(ref, F64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((a - ref) ** 2)))
    return num / den if den > 0 else num


__all__ = [
    "sigma_remap", "sigma_remap_slope", "resolve_sigmas", "mmh3_timestep", "mmh3_slots",
    "mmh3_token_rows",
    "adaln_coords", "adaln_mods", "rms_norm", "layer_norm", "modulate", "silu",
    "gelu_tanh", "rope_angles", "rope_angles_shared", "rope_for", "rope_rotate", "attention",
    "sample_ranges",
    "attention_packed", "mmh3_block", "refiner_block", "linear", "final_layer", "stack",
    "patchify_video", "unpatchify_video", "pack_audio", "unpack_audio", "mmh3_forward",
    "siglip_layer", "timestep_embedding", "zimage_mods", "zimage_block", "zimage_context_block",
    "zimage_final_layer", "patchify_image", "unpatchify_image", "zimage_forward", "block",
    "rel_rms",
]

"""Shared helpers of the GPU parity tests: run the HIP block through the C ABI,
read its intermediates from the workspace and compare them stage by stage with
the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle as O
from synth.device import to_device

TOL = {"f32": 1e-5, "bf16": 1e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def ws_view(ws, off: int, dtype, shape):
    import torch
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).reshape(shape)


def partial_rope_dims(hd: int, k: int) -> np.ndarray:
    """The library's documented head-dim order of q and k under the partial
    RoPE: stored dim d holds the page's dim pi[d] (P = 3k rotated pairs, the
    rotated halves moved to (j, j + hd/2), the unrotated dims to the pairs
    between)."""
    P, h = 3 * k, hd // 2
    d = np.arange(hd)
    return np.where(d < P, d, np.where(d < h, d + P, np.where(d < h + P, d - (h - P), d)))


def act_dtype(spec):
    import torch
    return torch.bfloat16 if spec.dtype == "bf16" else torch.float32


def run_gpu(spec, wl, dit, out_alias=False, seq_starts=None, mods_in=None):
    """Prepare + forward on the GPU; returns (out, stage dict of numpy fp64
    arrays over ALL tokens, xn of the attention half, mods).  ``seq_starts``
    packs independent samples (dit_block_forward_packed); ``mods_in`` (numpy
    [R, E*D]) runs dit_block_forward_mods with those modulation rows."""
    import torch
    dev = to_device(wl)
    cfg = dit.make_config(spec)
    blk = dit.Block(cfg, dev.weights)
    sig = dit.resolve_sigmas(wl.slot_plan)
    n = wl.x.shape[0]
    ad = act_dtype(spec)
    # attention-half pre-norm through the standalone entry point
    xn_a = torch.empty((n, spec.D), dtype=ad, device="cuda")
    mods = None
    temb = None
    if spec.variant in ("mmh3", "zimage"):
        mods = torch.empty((spec.mod_rows, spec.chunks * spec.D), dtype=torch.float32, device="cuda")
        if spec.variant == "zimage":
            temb = torch.empty(spec.temb_hidden + spec.temb_freq, dtype=torch.float32, device="cuda")
    blk.adaln_modulate(dev.x, dev.rows, sig, 0, xn_a, mods, temb)
    if mods_in is not None:
        md = torch.from_numpy(np.ascontiguousarray(mods_in, dtype=np.float32)).cuda()
        out = blk.forward_mods(dev.x, dev.rows, dev.pos, md, seq_starts=seq_starts)
    elif out_alias:
        out = dev.x.clone()
        blk.forward(out, dev.rows, dev.pos, sig, out=out, seq_starts=seq_starts)
    else:
        out = blk.forward(dev.x, dev.rows, dev.pos, sig, seq_starts=seq_starts)
    torch.cuda.synchronize()
    L = dit.workspace_layout(cfg, n)
    ws = blk._ws
    H, hd, D, F, ldn = spec.H, spec.hd, spec.D, spec.F, L.ldn

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    st = {}
    st["xn"] = f64(xn_a)
    if mods is not None:
        st["mods"] = f64(mods)
    # q carries log2(e) * hd^-1/2 (the attention kernel works in base 2)
    st["q"] = f64(ws_view(ws, L.q, ad, (H, ldn, hd))[:, :n]) * (math.sqrt(hd) / math.log2(math.e))
    st["k"] = f64(ws_view(ws, L.k, ad, (H, ldn, hd))[:, :n])
    if spec.rope == "partial":  # back to the page's head-dim order
        pi = partial_rope_dims(hd, spec.rope_axes[0] // 2)
        for name in ("q", "k"):
            page = np.empty_like(st[name])
            page[..., pi] = st[name]
            st[name] = page
    st["v"] = f64(ws_view(ws, L.vt, ad, (H, hd, ldn))[:, :, :n].transpose(1, 2))
    st["o"] = f64(ws_view(ws, L.o, ad, (n, D)))
    st["x1"] = f64(ws_view(ws, L.x1, torch.float32, (n, D)))
    st["xn2"] = f64(ws_view(ws, L.xn, ad, (n, D)))
    st["a"] = f64(ws_view(ws, L.a, ad, (n, F)))
    if spec.variant in ("zimage", "zcontext"):
        st["y2"] = f64(ws_view(ws, L.y, torch.float32, (n, D)))
    st["out"] = f64(out)
    # padding of the head-major panels must be zero (finite keys/values)
    if ldn > n:
        pad_k = ws_view(ws, L.k, ad, (H, ldn, hd))[:, n:]
        pad_v = ws_view(ws, L.vt, ad, (H, hd, ldn))[:, :, n:]
        st["_pad_max"] = float(max(pad_k.abs().max().item(), pad_v.abs().max().item()))
    return out, st


# A row whose reference norm is below this fraction of the stage's median row
# norm is measured against that floor instead of its own norm (a relative
# error is meaningless for a row that is all but zero).
ROW_FLOOR = 1e-3


def row_rel(got, ref, floor_frac=ROW_FLOOR):
    """Relative RMS error of every row (last axis) of got against ref:
    ||g_i - r_i|| / max(||r_i||, floor_frac * median_i ||r_i||)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    num = np.sqrt(np.sum((g - r) ** 2, axis=-1))
    den = np.sqrt(np.sum(r * r, axis=-1))
    floor = floor_frac * float(np.median(den)) if den.size else 0.0
    return num / np.maximum(den, max(floor, 1e-300))


def per_unit(name, g, r, H, hd):
    """Per-unit views of a stage: q/k/v [H, m, hd] are compared per (head,
    token) and o [m, H*hd] per (token, head); the rest per token row."""
    if name in ("q", "k", "v"):
        return g, r
    if name == "o":
        return g.reshape(g.shape[0], H, hd), r.reshape(r.shape[0], H, hd)
    return g, r


# Units downstream of the softmax: the bf16 q and k panels (the block's stated
# rounding points) move a logit s_ij by about 2^-9 |s_ij| (RNE on each factor),
# and a softmax row passes such a shift into its output's relative error.  On
# the oracle with only q and k rounded (everything else exact), the error of
# every (token, head) of o stays within 1.21 * 2^-9 * max_j |s_ij| on the test
# shapes; the kernel also rounds xn upstream.  Their per-unit bound is
# max(tol, 4 * 2^-9 * max_j |s_ij|), from the oracle's own logits.
LOGIT_UNIT = 4.0 * 2.0 ** -9


def logit_max(q, k, hd, sel, seq_starts=None):
    """max_j |q_ih . k_jh| / sqrt(hd) per (head, checked token) over the keys
    the token attends to: q [H, m, hd] at the tokens ``sel``, k [H, n, hd]."""
    H, m = q.shape[0], q.shape[1]
    out = np.zeros((H, m))
    ranges = O.sample_ranges(seq_starts, k.shape[1]) if seq_starts is not None else [(0, k.shape[1])]
    sel = np.asarray(sel)
    for a, e in ranges:
        r = np.nonzero((sel >= a) & (sel < e))[0]
        if r.size == 0 or e == a:
            continue
        for h in range(H):
            out[h, r] = np.abs(q[h, r] @ k[h, a:e].T).max(axis=1) / math.sqrt(hd)
    return out


def compare(spec, wl, st, qrows=None, tol=None, skip=(), seq_starts=None, mods=None):
    """Stage-by-stage check against the oracle.  The bar holds for every unit:
    each token row of every stage, and each (token, head) of q, k, v and o,
    has a relative RMS error <= tol (rows of x1 - x and out - x1 with their
    fp32 storage floor added; o and x1 - x against the logit-scaled bound
    above), and every stage as a whole meets tol.  Returns ({stage: error of
    the unit nearest its bound}, {stage: (error, bound)} over a bar, tol);
    the whole-stage figures are logged."""
    tol = TOL[spec.dtype] if tol is None else tol
    sig = O.resolve_sigmas(wl.slot_plan)
    ref = O.block(spec, wl.x, wl.rows, wl.pos, sig, wl.weights, qrows, seq_starts, mods)
    n = wl.x.shape[0]
    sel = np.arange(n) if qrows is None else np.asarray(qrows)
    ub = None  # [m, H] bound of each (token, head) of o
    if "o" in ref and tol > TOL["f32"]:
        ub = np.maximum(tol, LOGIT_UNIT * logit_max(ref["q"], ref["k"], spec.hd, sel, seq_starts)).T
    errs, agg, lim, bad = {}, {}, {}, {}

    def judge(name, e, b):
        """e: per-unit errors, b: their bounds (broadcast)."""
        if e.size == 0:
            errs[name], lim[name] = 0.0, float(np.max(b))
            return
        b = np.broadcast_to(b, e.shape)
        i = np.unravel_index(int(np.argmax(e / b)), e.shape)
        errs[name], lim[name] = float(e[i]), float(b[i])
        if not (e[i] <= b[i]):
            bad[name] = (errs[name], lim[name])

    for name in ("mods", "xn", "q", "k", "v", "o", "x1", "xn2", "a", "y2", "out"):
        if name not in ref or name not in st or name in skip:
            continue
        g = st[name]
        if name in ("q",):
            g = g[:, sel]
        elif name in ("o", "x1", "xn2", "a", "y2", "out"):
            g = g[sel]
        agg[name] = O.rel_rms(g, ref[name])
        gu, ru = per_unit(name, g, ref[name], spec.H, spec.hd)
        judge(name, row_rel(gu, ru), ub if (name == "o" and ub is not None) else tol)
    # The attention branch is small next to x: check x1 - x and out - x1
    # directly, per token row.  x1 and out are stored in fp32, so a difference
    # of two of them carries their storage rounding (unit roundoff 2^-24 of
    # |x|); each row's bar adds that floor for the row.  x1 - x mixes every
    # head of the row: its bound is the row's largest o bound.
    x64 = wl.x.astype(np.float64)[sel]
    d1 = ref["x1"] - x64
    d2 = ref["out"] - ref["x1"]
    u = 2.0 ** -24
    nrm = lambda a: np.sqrt(np.sum(a * a, axis=-1))  # noqa: E731
    rms = lambda a: float(np.sqrt(np.mean(a * a)))  # noqa: E731
    for name, g, d, base in (("x1-x", st["x1"][sel] - x64, d1, nrm(ref["x1"])),
                             ("out-x1", st["out"][sel] - st["x1"][sel], d2,
                              nrm(ref["x1"]) + nrm(ref["out"]))):
        agg[name] = O.rel_rms(g, d) - 2 * u * rms(base) / max(rms(nrm(d)), 1e-300)
        e = row_rel(g, d) - 2 * u * base / np.maximum(nrm(d), 1e-300)  # above the storage floor
        b = ub.max(axis=1) if (name == "x1-x" and ub is not None) else tol
        judge(name, e, b)
    log("[aggregate] " + " ".join(f"{k}={v:.2e}" for k, v in agg.items()))
    bad.update({f"{k} (whole stage)": (v, tol) for k, v in agg.items() if not (v <= tol)})
    return errs, bad, tol

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


def compare(spec, wl, st, qrows=None, tol=None, skip=(), seq_starts=None, mods=None):
    """Stage-by-stage rel-RMS vs the oracle; returns {stage: err}."""
    tol = TOL[spec.dtype] if tol is None else tol
    sig = O.resolve_sigmas(wl.slot_plan)
    ref = O.block(spec, wl.x, wl.rows, wl.pos, sig, wl.weights, qrows, seq_starts, mods)
    n = wl.x.shape[0]
    sel = np.arange(n) if qrows is None else np.asarray(qrows)
    errs = {}
    for name in ("mods", "xn", "q", "k", "v", "o", "x1", "xn2", "a", "y2", "out"):
        if name not in ref or name not in st or name in skip:
            continue
        g = st[name]
        if name in ("q",):
            g = g[:, sel]
        elif name in ("o", "x1", "xn2", "a", "y2", "out"):
            g = g[sel]
        errs[name] = O.rel_rms(g, ref[name])
    # The attention branch is small next to x: check x1 - x and out - x1
    # directly.  x1 and out are stored in fp32, so a difference of two of them
    # carries their storage rounding (unit roundoff 2^-24 of |x|); the bar for
    # these two adds that floor.
    x64 = wl.x.astype(np.float64)[sel]
    d1 = ref["x1"] - x64
    d2 = ref["out"] - ref["x1"]
    errs["x1-x"] = O.rel_rms(st["x1"][sel] - x64, d1)
    errs["out-x1"] = O.rel_rms(st["out"][sel] - st["x1"][sel], d2)
    u = 2.0 ** -24
    rms = lambda a: float(np.sqrt(np.mean(a * a)))  # noqa: E731
    lim = {k: tol for k in errs}
    lim["x1-x"] = tol + 2 * u * rms(ref["x1"]) / max(rms(d1), 1e-300)
    lim["out-x1"] = tol + 2 * u * (rms(ref["x1"]) + rms(ref["out"])) / max(rms(d2), 1e-300)
    bad = {k: (v, lim[k]) for k, v in errs.items() if not (v <= lim[k])}
    return errs, bad, tol

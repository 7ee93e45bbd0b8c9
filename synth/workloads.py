"""Block shapes, packed layouts and seeded tensors for the five workloads.

Citation tags used below (the pages are web pages; each is cited by its title
and the item on it):

* [MMH3]  docs.rs source page of cortiq-engine 0.5.72, ``src/mmh3.rs``
* [SIGLIP] docs.rs source page of ffai-argus 0.7.0, ``src/siglip.rs``
* [ZIMG]  ollama fork, ``x/imagegen/models/zimage/transformer.go``

Nothing here computes any part of the block: the layout builder only places
tokens (3-D positions and modulation-row indices), and the tensor generator only
draws seeded normals and rounds GEMM weights to bf16 so that both sides of a
parity test read the same values.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Block shapes
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class BlockSpec:
    """Shape and variant of one block workload.

    variant: "mmh3" (six-chunk adaLN from a rank-r timestep-curve basis,
    [MMH3] ``block_forward``), "siglip" (pre-LayerNorm encoder layer,
    [SIGLIP] ``Layer::forward``), "zimage" (four-chunk tanh-gated
    sandwich-norm block, [ZIMG] ``TransformerBlock.Forward``), "refiner"
    (the mmh3 block without modulation, [MMH3] ``refine_text``), "zcontext"
    (the zimage block without modulation, its context refiner), and the output
    heads "final" ([MMH3] heads) and "zfinal" ([ZIMG] ``FinalLayer``).
    """

    name: str
    variant: str
    dtype: str  # "f32" or "bf16": GEMM operands and attention inputs
    n: int
    D: int
    H: int
    hd: int
    F: int
    slots: int = 1  # timestep slots S (mmh3)
    tags: int = 3  # modality tags T (mmh3)
    rank: int = 24
    grid: int = 1025
    rope: str = "none"  # "none" | "split_half" | "interleaved" | "partial"
    # partial: the checkpoint form, k = rope_axes[0] / 2 frequencies (weight
    # "rope_freq") shared by the three axes, head dims from 3 * rope_axes[0] on
    # unrotated
    rope_axes: Tuple[int, int, int] = (0, 0, 0)
    rope_theta: float = 10000.0
    eps: float = 1e-5
    qk_eps: float = 1e-5
    temb_freq: int = 256  # zimage sinusoid width
    temb_hidden: int = 1024  # zimage timestep MLP width
    t_scale: float = 1000.0
    adaln_shared: int = 0  # mmh3 / final: one slot's basis rows used at every slot

    @property
    def chunks(self) -> int:
        return {"mmh3": 6, "zimage": 4, "siglip": 0, "refiner": 0, "final": 2, "zcontext": 0,
                "zfinal": 1}[self.variant]

    @property
    def mod_rows(self) -> int:
        if self.variant in ("mmh3", "final"):
            return self.slots * self.tags
        if self.variant in ("zimage", "zfinal"):
            return 1
        return 0

    def gemm_flops(self) -> float:
        n, D, F = self.n, self.D, self.F
        if self.variant == "siglip":
            return 2.0 * n * D * (4 * D + 2 * F)
        return 2.0 * n * D * (4 * D + 3 * F)

    def attn_flops(self) -> float:
        return 4.0 * self.n * self.n * self.D


SPECS: List[BlockSpec] = [
    # Toy packed block, fp32: 64 text + 3 frames of an 8x8 grid.
    BlockSpec("toy", "mmh3", "f32", n=256, D=256, H=4, hd=64, F=768, slots=1,
              rope="split_half", rope_axes=(16, 24, 24), rope_theta=10000.0),
    # SigLIP-shaped encoder layer (one 1024-patch image).
    BlockSpec("siglip", "siglip", "bf16", n=1024, D=768, H=12, hd=64, F=3072,
              rope="none", eps=1e-6),
    # Z-Image single-stream block: 64x64 image patches + 512 caption tokens.
    BlockSpec("zimage", "zimage", "bf16", n=4608, D=3072, H=24, hd=128, F=8192,
              rope="interleaved", rope_axes=(32, 48, 48), rope_theta=256.0),
    # Image-edit block: 512 text + 4096 reference + 4096 target tokens.
    BlockSpec("edit", "mmh3", "bf16", n=8704, D=2688, H=21, hd=128, F=10752, slots=2,
              rope="split_half", rope_axes=(32, 48, 48), rope_theta=10000.0),
    # Text-to-audio+video block: 512 text + 512 audio rows + 16x32x48 video.
    BlockSpec("t2va", "mmh3", "bf16", n=25600, D=2688, H=21, hd=128, F=10752, slots=2,
              rope="split_half", rope_axes=(32, 48, 48), rope_theta=10000.0),
]


def spec_by_name(name: str) -> BlockSpec:
    for s in SPECS:
        if s.name == name:
            return s
    raise KeyError(name)


# ---------------------------------------------------------------------------
# Packed layouts ([MMH3] ``Layout``)
# ---------------------------------------------------------------------------

# Latent frames a video token spans, cycling with period 5, and the rescale of
# that span onto the time axis ([MMH3] ``FRAME_PER_TOKEN``, ``FRAME_RESCALE``).
FRAME_SPAN = (1.0, 4.0, 4.0, 4.0, 4.0)
FRAME_RESCALE = 5.0 / 3.0

# Modality tags in the adaLN row order ([MMH3] module constants).
TAG_VIDEO, TAG_TEXT, TAG_AUDIO = 0, 1, 2


def _frac_axis(dim: int, patch: int, sqrt_area: float) -> List[float]:
    """Fractional h or w coordinates of a patch grid: ``dim/patch`` points,
    evenly spaced without the end point over [(1-r)/2, (1+r)/2) scaled by 32,
    where r = dim / sqrt(area) ([MMH3] ``axis_from_sqrt_area``)."""
    r = dim / sqrt_area
    m = dim // patch
    lo = (1.0 - r) / 2.0
    return [(lo + i * (r / m)) * 32.0 for i in range(m)]


def _frame_t(k: int) -> float:
    return FRAME_RESCALE * FRAME_SPAN[k % 5]


@dataclasses.dataclass
class Layout:
    pos: np.ndarray  # float64 [n, 3]: (t, h, w)
    segments: List[Tuple[str, int, int]]  # (kind, start, stop)
    frame_rows: int

    @property
    def seq_len(self) -> int:
        return int(self.pos.shape[0])

    def segment(self, kind: str) -> Tuple[str, int, int]:
        for s in self.segments:
            if s[0] == kind:
                return s
        raise KeyError(kind)

    def cond_rows(self) -> int:
        return sum(b - a for k, a, b in self.segments if k == "cond")


def build_layout(text_len: int, latent_t: int, lat_h: int, lat_w: int, audio_t: int,
                 keyframes: Sequence[Tuple[int, int]] = (),
                 ref_images: Sequence[Tuple[int, int]] = (),
                 refs: Sequence[tuple] = ()) -> Layout:
    """Place ``[text | references | keyframes | audio | video]`` on the
    3-D position grid ([MMH3] ``Layout::t2va``/``fl2va``/``ref2va``).

    ``refs``: ("image", lat_h, lat_w), ("audio", t) or ("video", latent_t,
    lat_h, lat_w, audio_t), in order; ``ref_images`` (lat_h, lat_w) pairs are
    image references placed before them.

    * text token i sits at (i, 0, 0);
    * a reference image occupies one time step at the cursor and advances it;
    * a reference audio is a stereo block at the cursor (the target grid's w
      extremes) and advances it by its frames;
    * a reference clip packs its soundtrack (its own grid's w extremes) and then
      its frames from the cursor, and advances it by the longer of the two;
    * a keyframe shares the target grid, sits at the first frame's time (the
      cursor) or the last frame's (cursor + all spans - one rescale) and does
      not advance the cursor;
    * audio is stereo, channel-major, one row per latent frame per channel at
      (cursor + i, 0, w_lo) then (cursor + i, 0, w_hi), the extremes of the
      target's w axis;
    * video frames start at the cursor and advance t by the cycling spans.
    """
    sq = math.sqrt(lat_h * lat_w)
    h_axis = _frac_axis(lat_h, 2, sq)
    w_axis = _frac_axis(lat_w, 2, sq)
    pos: List[Tuple[float, float, float]] = []
    segs: List[Tuple[str, int, int]] = []

    segs.append(("text", 0, text_len))
    pos.extend((float(i), 0.0, 0.0) for i in range(text_len))
    cursor = float(text_len)

    def stereo(c0, t, w_lo, w_hi):
        for w in (w_lo, w_hi):
            pos.extend((c0 + i, 0.0, w) for i in range(t))

    for ref in [("image", rh, rw) for rh, rw in ref_images] + list(refs):
        if ref[0] == "image":
            rh, rw = ref[1], ref[2]
            rsq = math.sqrt(rh * rw)
            ha, wa = _frac_axis(rh, 2, rsq), _frac_axis(rw, 2, rsq)
            start = len(pos)
            pos.extend((cursor, h, w) for h in ha for w in wa)
            segs.append(("ref_image", start, len(pos)))
            cursor += 1.0
        elif ref[0] == "audio":
            t = ref[1]
            if t > 0:
                start = len(pos)
                stereo(cursor, t, w_axis[0], w_axis[-1])
                segs.append(("ref_audio", start, len(pos)))
            cursor += float(t)
        elif ref[0] == "video":
            vt, rh, rw, rat = ref[1:5]
            rsq = math.sqrt(rh * rw)
            ha, wa = _frac_axis(rh, 2, rsq), _frac_axis(rw, 2, rsq)
            if rat > 0:
                start = len(pos)
                stereo(cursor, rat, wa[0], wa[-1])
                segs.append(("ref_audio", start, len(pos)))
            start = len(pos)
            tc = cursor
            for k in range(vt):
                pos.extend((tc, h, w) for h in ha for w in wa)
                tc += _frame_t(k)
            segs.append(("ref_image", start, len(pos)))
            cursor += max(float(rat), sum(_frame_t(k) for k in range(vt)))
        else:
            raise ValueError(ref[0])

    spans = sum(_frame_t(k) for k in range(latent_t))
    for pix, count in keyframes:
        if pix == 0:
            t = cursor
        elif count > 0 and pix == count - 1:
            t = cursor + spans - FRAME_RESCALE
        else:
            raise ValueError("a keyframe must be the first or the last frame")
        start = len(pos)
        pos.extend((t, h, w) for h in h_axis for w in w_axis)
        segs.append(("cond", start, len(pos)))

    start = len(pos)
    for w in (w_axis[0], w_axis[-1]):
        pos.extend((cursor + i, 0.0, w) for i in range(audio_t))
    segs.append(("audio", start, len(pos)))

    start = len(pos)
    t = cursor
    for k in range(latent_t):
        pos.extend((t, h, w) for h in h_axis for w in w_axis)
        t += _frame_t(k)
    segs.append(("video", start, len(pos)))

    return Layout(np.asarray(pos, dtype=np.float64).reshape(-1, 3), segs,
                  len(h_axis) * len(w_axis))


def zimage_positions(h_tok: int, w_tok: int, cap_len: int) -> np.ndarray:
    """Unified Z-Image sequence ``[image | caption]``: image token (j, k) at
    (cap_len + 1, j, k) in row-major order, caption token i at (1 + i, 0, 0)
    ([ZIMG] ``PrepareRoPECache``, ``createCoordinateGrid``)."""
    img = [(float(cap_len + 1), float(j), float(k)) for j in range(h_tok) for k in range(w_tok)]
    cap = [(float(1 + i), 0.0, 0.0) for i in range(cap_len)]
    return np.asarray(img + cap, dtype=np.float64)


def _rows_for(layout: Layout, kind_slot_tag: Dict[str, Tuple[int, int]], tags: int) -> np.ndarray:
    rows = np.zeros(layout.seq_len, dtype=np.int32)
    for kind, a, b in layout.segments:
        slot, tag = kind_slot_tag[kind]
        rows[a:b] = slot * tags + tag
    return rows


# ---------------------------------------------------------------------------
# Seeded tensors
# ---------------------------------------------------------------------------


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs here are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 array holding the bfloat16-rounded values of ``a``."""
    return (bf16_bits(a).astype(np.uint32) << 16).view(np.float32)


def weight_shapes(spec: BlockSpec) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, init) for every weight tensor, in a fixed order.

    init: "lin" = N(0, 0.02) GEMM weight (bf16-rounded in bf16 blocks),
    "vec" = N(0, 0.02) fp32, "gain" = 1 + N(0, 0.02) fp32, "table" = N(0, 1),
    "freq" = the k frequencies theta^(-m/k), m < k (fp32; a checkpoint's shared
    RoPE frequency vector).
    """
    D, H, hd, F = spec.D, spec.H, spec.hd, spec.F
    extra = []
    if spec.rope == "partial":
        extra = [("rope_freq", (spec.rope_axes[0] // 2,), "freq")]
    if spec.variant == "mmh3":
        R = (1 if spec.adaln_shared else spec.slots) * spec.tags * 6 * D
        return [
            ("norm1", (D,), "gain"), ("norm2", (D,), "gain"),
            ("w_qkv", (3 * D, D), "lin"), ("w_out", (D, D), "lin"),
            ("q_norm", (hd,), "gain"), ("k_norm", (hd,), "gain"),
            ("w_fc1", (2 * F, D), "lin"), ("w_fc2", (D, F), "lin"),
            ("adaln_basis", (R, spec.rank), "vec"), ("adaln_bias", (R,), "vec"),
            ("adaln_table", (spec.grid, spec.rank), "table"),
        ] + extra
    if spec.variant == "final":  # output head: F = output width, tags = 1
        R = (1 if spec.adaln_shared else spec.slots) * spec.tags * 2 * D
        return [
            ("norm1", (D,), "gain"), ("w_fc1", (F, D), "lin"), ("b_fc1", (F,), "vec"),
            ("adaln_basis", (R, spec.rank), "vec"), ("adaln_bias", (R,), "vec"),
            ("adaln_table", (spec.grid, spec.rank), "table"),
        ]
    if spec.variant == "refiner":
        return [
            ("norm1", (D,), "gain"), ("norm2", (D,), "gain"),
            ("w_qkv", (3 * D, D), "lin"), ("w_out", (D, D), "lin"),
            ("q_norm", (hd,), "gain"), ("k_norm", (hd,), "gain"),
            ("w_fc1", (2 * F, D), "lin"), ("w_fc2", (D, F), "lin"),
        ] + extra
    if spec.variant == "siglip":
        return [
            ("ln1_w", (D,), "gain"), ("ln1_b", (D,), "vec"),
            ("ln2_w", (D,), "gain"), ("ln2_b", (D,), "vec"),
            ("w_qkv", (3 * D, D), "lin"), ("b_qkv", (3 * D,), "vec"),
            ("w_out", (D, D), "lin"), ("b_out", (D,), "vec"),
            ("w_fc1", (F, D), "lin"), ("b_fc1", (F,), "vec"),
            ("w_fc2", (D, F), "lin"), ("b_fc2", (D,), "vec"),
        ]
    if spec.variant == "zcontext":  # the Z-Image block without its timestep / adaLN tensors
        return [
            ("norm1", (D,), "gain"), ("post_attn_norm", (D,), "gain"),
            ("norm2", (D,), "gain"), ("post_ffn_norm", (D,), "gain"),
            ("w_qkv", (3 * D, D), "lin"), ("w_out", (D, D), "lin"),
            ("q_norm", (hd,), "gain"), ("k_norm", (hd,), "gain"),
            ("w_fc1", (2 * F, D), "lin"), ("w_fc2", (D, F), "lin"),
        ]
    if spec.variant == "zfinal":  # Z-Image final layer: F = output width
        return [
            ("w_fc1", (F, D), "lin"), ("b_fc1", (F,), "vec"),
            ("temb_w1", (spec.temb_hidden, spec.temb_freq), "vec"),
            ("temb_b1", (spec.temb_hidden,), "vec"),
            ("temb_w2", (spec.temb_freq, spec.temb_hidden), "vec"),
            ("temb_b2", (spec.temb_freq,), "vec"),
            ("ada_w", (D, spec.temb_freq), "vec"), ("ada_b", (D,), "vec"),
        ]
    if spec.variant == "zimage":
        return [
            ("norm1", (D,), "gain"), ("post_attn_norm", (D,), "gain"),
            ("norm2", (D,), "gain"), ("post_ffn_norm", (D,), "gain"),
            ("w_qkv", (3 * D, D), "lin"), ("w_out", (D, D), "lin"),
            ("q_norm", (hd,), "gain"), ("k_norm", (hd,), "gain"),
            ("w_fc1", (2 * F, D), "lin"), ("w_fc2", (D, F), "lin"),
            ("temb_w1", (spec.temb_hidden, spec.temb_freq), "vec"),
            ("temb_b1", (spec.temb_hidden,), "vec"),
            ("temb_w2", (spec.temb_freq, spec.temb_hidden), "vec"),
            ("temb_b2", (spec.temb_freq,), "vec"),
            ("ada_w", (4 * D, spec.temb_freq), "vec"), ("ada_b", (4 * D,), "vec"),
        ]
    raise ValueError(spec.variant)


@dataclasses.dataclass
class Workload:
    spec: BlockSpec
    x: np.ndarray  # float32 [n, D]
    rows: Optional[np.ndarray]  # int32 [n] modulation row per token, or None
    pos: Optional[np.ndarray]  # float32 [n, 3], or None
    # One entry per timestep slot: ("value", v) uses v directly; ("remap", s,
    # a, b) asks each side to remap slot s's sigma from shift a to shift b with
    # its own implementation of the remap.
    slot_plan: List[tuple]
    weights: Dict[str, np.ndarray]  # float32, GEMM weights bf16-representable in bf16 blocks
    seed: int


def _draw(seed: int, idx: int, shape: Tuple[int, ...]) -> np.ndarray:
    rng = np.random.default_rng([seed, idx])
    return rng.standard_normal(shape, dtype=np.float32)


def make_weights(spec: BlockSpec, seed: int) -> Dict[str, np.ndarray]:
    out: Dict[str, np.ndarray] = {}
    for idx, (name, shape, init) in enumerate(weight_shapes(spec)):
        z = _draw(seed, idx, shape)
        if init == "lin":
            a = z * np.float32(0.02)
            if spec.dtype == "bf16":
                a = bf16_round(a)
        elif init == "vec":
            a = z * np.float32(0.02)
        elif init == "gain":
            a = np.float32(1.0) + z * np.float32(0.02)
        elif init == "table":
            a = z
        elif init == "freq":
            k = shape[0]
            a = np.float64(spec.rope_theta) ** (-np.arange(k, dtype=np.float64) / k)
        else:  # pragma: no cover
            raise ValueError(init)
        out[name] = np.ascontiguousarray(a, dtype=np.float32)
    return out


def layout_for(spec: BlockSpec):
    """(positions float64 [n,3] or None, rows int32 [n] or None) of the
    workload's packing."""
    if spec.name == "toy":
        lay = build_layout(64, 3, 16, 16, 0)
        rows = _rows_for(lay, {"text": (0, TAG_TEXT), "audio": (0, TAG_AUDIO),
                               "video": (0, TAG_VIDEO)}, spec.tags)
        return lay.pos, rows
    if spec.name == "edit":
        lay = build_layout(512, 1, 128, 128, 0, ref_images=[(128, 128)])
        rows = _rows_for(lay, {"text": (0, TAG_TEXT), "ref_image": (0, TAG_VIDEO),
                               "audio": (0, TAG_AUDIO), "video": (0, TAG_VIDEO)}, spec.tags)
        return lay.pos, rows
    if spec.name == "t2va":
        lay = build_layout(512, 16, 64, 96, 256)
        rows = _rows_for(lay, {"text": (0, TAG_TEXT), "audio": (1, TAG_AUDIO),
                               "video": (0, TAG_VIDEO)}, spec.tags)
        return lay.pos, rows
    if spec.name == "zimage":
        return zimage_positions(64, 64, 512), np.zeros(4608, dtype=np.int32)
    if spec.name == "siglip":
        return None, None
    raise KeyError(spec.name)


def make_workload(spec: BlockSpec, seed: Optional[int] = None, rows_mode: str = "layout",
                  n: Optional[int] = None, weight_seed: Optional[int] = None) -> Workload:
    """Seeded workload for ``spec``.

    Seeds: activations 0xD17000 + config index, weights 0xD17100 + config
    index, unless given.  ``rows_mode="random"`` draws every token's row
    uniformly from all modulation rows instead of the layout's.  ``n`` keeps
    only the first n tokens (small parity cases with a ragged tail).
    """
    ci = [s.name for s in SPECS].index(spec.name) + 1 if spec in SPECS else 0
    seed = 0xD17000 + ci if seed is None else seed
    wseed = 0xD17100 + ci if weight_seed is None else weight_seed
    rng = np.random.default_rng(seed)
    pos64, rows = layout_for(spec) if spec in SPECS else (None, None)
    nn = spec.n if n is None else n
    x = rng.standard_normal((nn, spec.D), dtype=np.float32)
    u = float(rng.uniform(0.0, 1.0))
    if spec.variant == "mmh3":
        if spec.name == "t2va":
            plan = [("value", u), ("remap", 0, 12.0, 3.0)]
        elif spec.name == "toy":
            plan = [("value", 1.0 - u)]  # t ~ U(0,1), sigma = 1 - t
        else:
            plan = [("value", u)] * spec.slots
        if rows_mode == "random":
            rows = rng.integers(0, spec.mod_rows, size=spec.n, dtype=np.int32)
    elif spec.variant == "zimage":
        plan = [("value", u)]  # t ~ U(0,1)
    else:
        plan = []
    pos = None if pos64 is None else pos64[:nn].astype(np.float32)
    if rows is not None:
        rows = np.ascontiguousarray(rows[:nn], dtype=np.int32)
    return Workload(spec, x, rows, pos, plan, make_weights(spec, wseed), seed)


def small_spec(spec: BlockSpec, **kw) -> BlockSpec:
    """A copy of ``spec`` with some fields replaced (small parity cases)."""
    return dataclasses.replace(spec, **kw)


def make_custom_workload(spec: BlockSpec, seed: int, pos: Optional[np.ndarray] = None,
                         rows: Optional[np.ndarray] = None, sigmas: Sequence[float] = ()) -> Workload:
    """Workload for an arbitrary (usually small) spec: x ~ N(0,1), positions
    and rows as given (random if None), explicit slot sigmas."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((spec.n, spec.D), dtype=np.float32)
    if spec.rope != "none" and pos is None:
        pos = rng.uniform(0.0, 64.0, size=(spec.n, 3)).astype(np.float32)
    if spec.mod_rows and rows is None:
        rows = rng.integers(0, spec.mod_rows, size=spec.n, dtype=np.int32)
    if not sigmas:
        sigmas = [float(v) for v in rng.uniform(0.0, 1.0, size=max(spec.slots, 1))]
    plan = [("value", float(s)) for s in sigmas]
    if spec.variant in ("siglip", "refiner", "zcontext"):
        plan = []
    return Workload(spec, x, rows, None if pos is None else np.asarray(pos, np.float32),
                    plan, make_weights(spec, seed + 1), seed)

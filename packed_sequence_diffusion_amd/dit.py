"""ctypes binding of libdit.so (the C ABI declared in include/dit.h).

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built, importing this module raises: there is no CPU
fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_size_t, c_void_p
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdit.so")

MMH3, SIGLIP, ZIMAGE, REFINER, FINAL, ZCONTEXT, ZFINAL = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1
ROPE_NONE, ROPE_SPLIT_HALF, ROPE_INTERLEAVED, ROPE_PARTIAL = 0, 1, 2, 3
NPHASES = 9

_VARIANTS = {"mmh3": MMH3, "siglip": SIGLIP, "zimage": ZIMAGE, "refiner": REFINER, "final": FINAL,
             "zcontext": ZCONTEXT, "zfinal": ZFINAL}
_DTYPES = {"f32": F32, "bf16": BF16}
_ROPES = {"none": ROPE_NONE, "split_half": ROPE_SPLIT_HALF, "interleaved": ROPE_INTERLEAVED,
          "partial": ROPE_PARTIAL}

STATUS = {0: "DIT_OK", -1: "DIT_EINVAL", -2: "DIT_ESHAPE", -3: "DIT_EDTYPE", -4: "DIT_EALIGN",
          -5: "DIT_EWORKSPACE", -6: "DIT_EUNSUPPORTED", -7: "DIT_EHIP"}


class DitConfig(ctypes.Structure):
    _fields_ = [("variant", c_int32), ("dtype", c_int32), ("D", c_int32), ("H", c_int32),
                ("hd", c_int32), ("F", c_int32), ("slots", c_int32), ("tags", c_int32),
                ("rank", c_int32), ("grid", c_int32), ("rope", c_int32),
                ("rope_axes", c_int32 * 3), ("rope_theta", c_double), ("eps", c_float),
                ("qk_eps", c_float), ("temb_freq", c_int32), ("temb_hidden", c_int32),
                ("t_scale", c_float), ("adaln_shared", c_int32)]


WEIGHT_FIELDS = ["norm1", "norm2", "ln1_b", "ln2_b", "post_attn_norm", "post_ffn_norm",
                 "w_qkv", "w_out", "w_fc1", "w_fc2", "b_qkv", "b_out", "b_fc1", "b_fc2",
                 "q_norm", "k_norm", "adaln_basis", "adaln_bias", "adaln_table",
                 "temb_w1", "temb_b1", "temb_w2", "temb_b2", "ada_w", "ada_b", "rope_freq"]


class DitWeights(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in WEIGHT_FIELDS]


class DitWsLayout(ctypes.Structure):
    _fields_ = [(f, c_size_t) for f in ("mods", "rope", "xn", "qkv", "q", "k", "vt", "o", "x1",
                                         "a", "y", "temb", "part", "total")] + [("ldn", c_int32)]


NONE_OFFSET = (1 << (8 * ctypes.sizeof(c_size_t))) - 1

SEG_KINDS = {"text": 0, "video": 1, "audio": 2, "cond": 3, "ref_image": 4, "ref_audio": 5}
SEG_NAMES = {v: k for k, v in SEG_KINDS.items()}


class DitSegment(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("start", c_int32), ("stop", c_int32)]


class DitMmh3Model(ctypes.Structure):
    _fields_ = [("block", POINTER(DitConfig)), ("blocks", POINTER(c_void_p)), ("n_blocks", c_int32),
                ("head_video", POINTER(DitConfig)), ("head_video_w", c_void_p),
                ("head_audio", POINTER(DitConfig)), ("head_audio_w", c_void_p),
                ("latent_c", c_int32), ("audio_c", c_int32),
                ("video_patch_w", c_void_p), ("video_patch_b", c_void_p),
                ("audio_patch_w", c_void_p), ("audio_patch_b", c_void_p),
                ("shift_video", c_double), ("shift_audio", c_double),
                ("cond_aug", c_double), ("cond_aug_audio", c_double),
                ("audio_slope_rescale", c_int32)]


class DitLayoutRef(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("latent_t", c_int32), ("lat_h", c_int32), ("lat_w", c_int32),
                ("audio_t", c_int32)]


class DitZimageModel(ctypes.Structure):
    _fields_ = [("block", POINTER(DitConfig)), ("layers", POINTER(c_void_p)), ("n_layers", c_int32),
                ("noise_refiners", POINTER(c_void_p)), ("n_noise_refiners", c_int32),
                ("context", POINTER(DitConfig)), ("context_refiners", POINTER(c_void_p)),
                ("n_context_refiners", c_int32), ("final_layer", POINTER(DitConfig)),
                ("final_w", c_void_p), ("in_channels", c_int32), ("cap_dim", c_int32),
                ("x_embed_w", c_void_p), ("x_embed_b", c_void_p), ("cap_norm", c_void_p),
                ("cap_eps", c_float), ("cap_embed_w", c_void_p), ("cap_embed_b", c_void_p)]


class DitZimageCache(ctypes.Structure):
    _fields_ = [("caption", c_void_p), ("shallow", c_void_p), ("layers", c_int32),
                ("interval", c_int32), ("caption_valid", c_int32), ("shallow_valid", c_int32)]


class DitError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run packed_sequence_diffusion_amd.build "
                          "(there is no CPU fallback)")
    # torch first: its bundled HIP runtime (soname libamdhip64.so.7, the library's
    # dependency) is then the one the library binds to.  Loaded the other way round,
    # the process would hold two HIP runtimes and torch's would see no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    sig = {
        "dit_abi_version": (c_int32, []),
        "dit_last_error": (ctypes.c_char_p, []),
        "dit_sigma_remap": (c_double, [c_double, c_double, c_double]),
        "dit_sigma_remap_slope": (c_double, [c_double, c_double, c_double]),
        "dit_mmh3_slots": (c_int32, [c_double, c_double, c_double, c_double, c_double, c_int32,
                                     c_int32, P(c_double), P(c_int32)]),
        "dit_validate_config": (c_int32, [P(DitConfig)]),
        "dit_prepared_size": (c_size_t, [P(DitConfig)]),
        "dit_prepare_weights": (c_int32, [P(DitConfig), P(DitWeights), c_void_p, c_size_t, c_void_p]),
        "dit_workspace_size": (c_size_t, [P(DitConfig), c_int32]),
        "dit_workspace_layout": (c_int32, [P(DitConfig), c_int32, P(DitWsLayout)]),
        "dit_adaln_eval": (c_int32, [P(DitConfig), c_void_p, P(c_double), c_int32, c_void_p,
                                     c_void_p, c_void_p]),
        "dit_adaln_eval_noalloc": (c_int32, [P(DitConfig), c_void_p, P(c_double), c_int32,
                                             c_void_p, c_void_p]),
        "dit_adaln_modulate": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_int32, c_void_p,
                                         P(c_double), c_int32, c_int32, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
        "dit_block_forward": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_int32, c_void_p,
                                        c_void_p, P(c_double), c_int32, c_void_p, c_void_p,
                                        c_size_t, c_void_p]),
        "dit_block_forward_packed": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_int32,
                                               c_void_p, c_void_p, P(c_double), c_int32,
                                               P(c_int32), c_int32, c_void_p, c_void_p, c_size_t,
                                               c_void_p]),
        "dit_block_forward_mods": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_int32, c_void_p,
                                             c_void_p, c_void_p, P(c_int32), c_int32, c_void_p,
                                             c_void_p, c_size_t, c_void_p]),
        "dit_final_forward": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_int32, c_void_p,
                                        P(c_double), c_int32, c_void_p, c_void_p, c_size_t,
                                        c_void_p]),
        "dit_linear": (c_int32, [c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_int32,
                                 c_void_p, c_float, c_void_p, c_void_p]),
        "dit_stack_forward": (c_int32, [P(DitConfig), P(c_void_p), c_int32, c_void_p, c_int32,
                                        c_void_p, c_void_p, P(c_double), c_int32, P(c_int32),
                                        c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
        "dit_patchify_video": (c_int32, [c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                         c_void_p, c_void_p]),
        "dit_unpatchify_video": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                           c_void_p]),
        "dit_pack_audio": (c_int32, [c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
        "dit_patchify_image": (c_int32, [c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                         c_void_p]),
        "dit_unpatchify_image": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                           c_void_p]),
        "dit_zimage_workspace_size": (c_size_t, [P(DitZimageModel), c_int32, c_int32, c_int32]),
        "dit_zimage_forward": (c_int32, [P(DitZimageModel), c_void_p, c_int32, c_int32, c_void_p,
                                         c_int32, c_void_p, c_double, c_int32, P(DitZimageCache),
                                         c_void_p, c_void_p, c_size_t, c_void_p]),
        "dit_unpack_audio": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
        "dit_rms_norm": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_float, c_void_p,
                                   c_void_p]),
        "dit_mmh3_layout": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, P(c_int32),
                                      c_int32, P(DitLayoutRef), c_int32, P(c_double), c_int32,
                                      P(DitSegment), c_int32, P(c_int32)]),
        "dit_mmh3_workspace_size": (c_size_t, [P(DitMmh3Model), P(DitSegment), c_int32]),
        "dit_mmh3_forward": (c_int32, [P(DitMmh3Model), P(DitSegment), c_int32, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                       c_void_p,
                                       c_int32, P(c_void_p), c_double, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
        "dit_attention": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                    c_float, c_void_p, c_void_p]),
        "dit_attention_packed": (c_int32, [P(DitConfig), c_void_p, c_void_p, c_void_p, c_int32,
                                           c_int32, P(c_int32), c_int32, c_float, c_void_p,
                                           c_void_p]),
        "dit_attention_shard_workspace_size": (c_size_t, [P(DitConfig)]),
        "dit_attention_shard": (c_int32, [P(DitConfig), c_void_p, c_int32, c_int32, c_int32,
                                          c_void_p, c_void_p, c_int32, c_int32, c_float, c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
        "dit_profile_begin": (c_int32, [c_int32]),
        "dit_profile_end": (c_int32, [P(c_double), P(c_int32)]),
        "dit_phase_name": (ctypes.c_char_p, [c_int32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise DitError(status, lib.dit_last_error().decode())


def last_error() -> str:
    return lib.dit_last_error().decode()


def sigma_remap(sigma: float, from_shift: float, to_shift: float) -> float:
    return lib.dit_sigma_remap(sigma, from_shift, to_shift)


def sigma_remap_slope(sigma: float, from_shift: float, to_shift: float) -> float:
    return lib.dit_sigma_remap_slope(sigma, from_shift, to_shift)


def mmh3_slots(sigma_v: float, shift_video: float = 12.0, shift_audio: float = 3.0,
               cond_aug: float = 0.999, cond_aug_audio: float = 1.0, has_cond: bool = False,
               has_ref_audio: bool = False):
    """(slot sigmas, {"video", "audio", "cond", "ref_audio"} -> slot or -1)
    through dit_mmh3_slots."""
    sg = (c_double * 4)()
    so = (c_int32 * 4)()
    k = lib.dit_mmh3_slots(sigma_v, shift_video, shift_audio, cond_aug, cond_aug_audio,
                           int(has_cond), int(has_ref_audio), sg, so)
    if k < 0:
        raise DitError(k, lib.dit_last_error().decode())
    return [sg[i] for i in range(k)], dict(zip(("video", "audio", "cond", "ref_audio"), so))


_REF_KINDS = {"image": SEG_KINDS["ref_image"], "audio": SEG_KINDS["ref_audio"], "video": SEG_KINDS["video"]}


def mmh3_layout(text_len: int, latent_t: int, lat_h: int, lat_w: int, audio_t: int,
                keyframes: Sequence[Sequence[int]] = (), refs: Sequence[tuple] = ()):
    """(segments [(kind name, start, stop)], positions float64 [n, 3]) through
    dit_mmh3_layout.  keyframes: (pixel_index, frame_count) pairs; refs:
    ("image", lat_h, lat_w), ("audio", t) or ("video", latent_t, lat_h, lat_w,
    audio_t)."""
    import numpy as np
    kf = (c_int32 * max(2 * len(keyframes), 1))(*[int(v) for k in keyframes for v in k])
    rr = (DitLayoutRef * max(len(refs), 1))()
    for i, r in enumerate(refs):
        f = rr[i]
        f.kind = _REF_KINDS[r[0]]
        if r[0] == "image":
            f.lat_h, f.lat_w = r[1], r[2]
        elif r[0] == "audio":
            f.audio_t = r[1]
        else:
            f.latent_t, f.lat_h, f.lat_w, f.audio_t = r[1:5]
    ns = c_int32()
    n = lib.dit_mmh3_layout(text_len, latent_t, lat_h, lat_w, audio_t, kf, len(keyframes), rr, len(refs),
                            None, 0, None, 0, ctypes.byref(ns))
    if n < 0:
        raise DitError(n, lib.dit_last_error().decode())
    pos = np.zeros((max(n, 1), 3), dtype=np.float64)
    segs = (DitSegment * max(ns.value, 1))()
    got = lib.dit_mmh3_layout(text_len, latent_t, lat_h, lat_w, audio_t, kf, len(keyframes), rr,
                              len(refs), pos.ctypes.data_as(POINTER(c_double)), n, segs, ns.value,
                              ctypes.byref(ns))
    if got < 0:
        raise DitError(got, lib.dit_last_error().decode())
    return [(SEG_NAMES[segs[i].kind], segs[i].start, segs[i].stop) for i in range(ns.value)], pos[:n]


def resolve_sigmas(plan: Sequence[tuple]) -> List[float]:
    """Slot sigmas from a slot plan; remapped slots go through the library's
    dit_sigma_remap."""
    out: List[float] = []
    for item in plan:
        if item[0] == "value":
            out.append(float(item[1]))
        else:
            _, src, a, b = item
            out.append(sigma_remap(out[src], a, b))
    return out


def make_config(spec) -> DitConfig:
    """DitConfig from any object with the block-shape attributes (variant,
    dtype, D, H, hd, F, slots, tags, rank, grid, rope, rope_axes, rope_theta,
    eps, qk_eps, temb_freq, temb_hidden, t_scale; optional adaln_shared)."""
    c = DitConfig()
    c.variant = _VARIANTS[spec.variant] if isinstance(spec.variant, str) else int(spec.variant)
    c.dtype = _DTYPES[spec.dtype] if isinstance(spec.dtype, str) else int(spec.dtype)
    c.D, c.H, c.hd, c.F = spec.D, spec.H, spec.hd, spec.F
    c.slots, c.tags, c.rank, c.grid = spec.slots, spec.tags, spec.rank, spec.grid
    c.rope = _ROPES[spec.rope] if isinstance(spec.rope, str) else int(spec.rope)
    for i in range(3):
        c.rope_axes[i] = spec.rope_axes[i]
    c.rope_theta = spec.rope_theta
    c.eps, c.qk_eps = spec.eps, spec.qk_eps
    c.temb_freq, c.temb_hidden, c.t_scale = spec.temb_freq, spec.temb_hidden, spec.t_scale
    c.adaln_shared = int(getattr(spec, "adaln_shared", 0))
    return c


def _ptr(t, strided: bool = False) -> Optional[int]:
    """Device address of a tensor the library reads as dense row-major memory
    (a row-strided matrix with ``strided``: unit stride inside rows)."""
    if t is None:
        return None
    if not (t.is_contiguous() or (strided and t.dim() == 2 and t.stride(1) == 1)):
        raise ValueError(f"tensor of shape {tuple(t.shape)} and strides {t.stride()} is not "
                         "row-major contiguous")
    return t.data_ptr()


_TORCH_DT = {}


def _tdt(name: str):
    """torch dtype by short name ("f32", "bf16", "i32", "u8")."""
    import torch
    if not _TORCH_DT:
        _TORCH_DT.update(f32=torch.float32, bf16=torch.bfloat16, i32=torch.int32, u8=torch.uint8)
    return _TORCH_DT[name]


def _act(cfg: "DitConfig") -> str:
    return "bf16" if cfg.dtype == BF16 else "f32"


def _arg(t, name: str, dtype: str, shape: Optional[Sequence[int]] = None,
         optional: bool = False, strided: bool = False, min_numel: int = 0) -> Optional[int]:
    """Device address of ``t`` after checking what the C ABI cannot: a CUDA
    tensor of the given dtype and shape (entries None are free), row-major
    (``strided``: unit stride inside rows), at least ``min_numel`` elements.
    Raises ValueError instead of handing the library a buffer it would read
    or write out of bounds."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype != _tdt(dtype):
        raise ValueError(f"{name} must be {_tdt(dtype)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w)
                                        for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                             f"{tuple('*' if w is None else int(w) for w in shape)}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    return _ptr(t, strided)


def weight_shapes(cfg: "DitConfig") -> Dict[str, tuple]:
    """{field: (dtype, shape)} of the raw weights a configuration reads
    (include/dit.h, dit_weights); GEMM weights in the config's dtype, the rest
    fp32."""
    D, H, hd, F, S, T, r, G = cfg.D, cfg.H, cfg.hd, cfg.F, cfg.slots, cfg.tags, cfg.rank, cfg.grid
    a, f = _act(cfg), "f32"
    v = cfg.variant
    out: Dict[str, tuple] = {}
    if v == FINAL:
        rows = (1 if cfg.adaln_shared else S) * T * 2 * D
        out.update(norm1=(f, (D,)), w_fc1=(a, (F, D)), b_fc1=(f, (F,)),
                   adaln_basis=(f, (rows, r)), adaln_bias=(f, (rows,)), adaln_table=(f, (G, r)))
        return out
    tf, th = cfg.temb_freq, cfg.temb_hidden
    temb = dict(temb_w1=(f, (th, tf)), temb_b1=(f, (th,)), temb_w2=(f, (tf, th)), temb_b2=(f, (tf,)))
    if v == ZFINAL:
        out.update(w_fc1=(a, (F, D)), b_fc1=(f, (F,)), ada_w=(f, (D, tf)), ada_b=(f, (D,)), **temb)
        return out
    swiglu = v != SIGLIP
    out.update(norm1=(f, (D,)), norm2=(f, (D,)), w_qkv=(a, (3 * D, D)), w_out=(a, (D, D)),
               w_fc1=(a, (2 * F if swiglu else F, D)), w_fc2=(a, (D, F)))
    if v != SIGLIP:
        out.update(q_norm=(f, (hd,)), k_norm=(f, (hd,)))
    if cfg.rope == ROPE_PARTIAL:
        out["rope_freq"] = (f, (cfg.rope_axes[0] // 2,))
    if v == SIGLIP:
        out.update(ln1_b=(f, (D,)), ln2_b=(f, (D,)), b_qkv=(f, (3 * D,)), b_out=(f, (D,)),
                   b_fc1=(f, (F,)), b_fc2=(f, (D,)))
    if v == MMH3:
        rows = (1 if cfg.adaln_shared else S) * T * 6 * D
        out.update(adaln_basis=(f, (rows, r)), adaln_bias=(f, (rows,)), adaln_table=(f, (G, r)))
    if v in (ZIMAGE, ZCONTEXT):
        out.update(post_attn_norm=(f, (D,)), post_ffn_norm=(f, (D,)))
    if v == ZIMAGE:
        out.update(ada_w=(f, (4 * D, tf)), ada_b=(f, (4 * D,)), **temb)
    return out


def mod_shape(cfg: "DitConfig") -> tuple:
    """Shape of the modulation rows [R, E*D] (dit_adaln_eval's output)."""
    if cfg.variant == MMH3:
        return (cfg.slots * cfg.tags, 6 * cfg.D)
    if cfg.variant == FINAL:
        return (cfg.slots * cfg.tags, 2 * cfg.D)
    if cfg.variant == ZIMAGE:
        return (1, 4 * cfg.D)
    if cfg.variant == ZFINAL:
        return (1, cfg.D)
    raise ValueError("the configuration has no modulation rows")


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dbl(vals: Sequence[float]):
    arr = (c_double * max(len(vals), 1))(*vals)
    return arr, len(vals)


def _starts(seq_starts: Sequence[int]):
    vals = [int(v) for v in seq_starts]
    arr = (c_int32 * max(len(vals), 1))(*vals)
    return arr, len(vals) - 1


def validate(cfg: DitConfig) -> None:
    _check(lib.dit_validate_config(ctypes.byref(cfg)))


def workspace_layout(cfg: DitConfig, n: int) -> DitWsLayout:
    L = DitWsLayout()
    _check(lib.dit_workspace_layout(ctypes.byref(cfg), n, ctypes.byref(L)))
    return L


class Block:
    """Prepared weights of one block on the current GPU.

    ``weights``: dict of device tensors named as in ``DitWeights`` (GEMM
    weights in the config's dtype, everything else fp32, all contiguous)."""

    def __init__(self, cfg: DitConfig, weights: Dict[str, "object"], stream=None):
        import torch
        validate(cfg)
        self.cfg = cfg
        shapes = weight_shapes(cfg)
        w = DitWeights()
        for f in WEIGHT_FIELDS:
            t = weights.get(f)
            if f in shapes:  # read by this variant: dtype and shape checked
                dt, shp = shapes[f]
                setattr(w, f, _arg(t, f"weight {f}", dt, shp, optional=True))
            else:  # not read by this variant
                setattr(w, f, None)
        nbytes = lib.dit_prepared_size(ctypes.byref(cfg))
        self.prepared = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        _check(lib.dit_prepare_weights(ctypes.byref(cfg), ctypes.byref(w), self.prepared.data_ptr(),
                                       nbytes, _stream(stream)))
        cur = torch.cuda.current_stream()
        if stream is not None and stream != cur:
            # preparation ran on another stream: order later use on the current
            # stream after it, and keep the raw weights alive until it has run
            cur.wait_stream(stream)
            self.prepared.record_stream(stream)
            for f in shapes:
                t = weights.get(f)
                if t is not None:
                    t.record_stream(stream)
        self._ws = None

    def workspace(self, n: int):
        import torch
        need = lib.dit_workspace_size(ctypes.byref(self.cfg), n)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def forward(self, x, rows, pos, sigmas: Sequence[float], out=None, workspace=None,
                stream=None, seq_starts: Optional[Sequence[int]] = None):
        """One block forward; ``seq_starts`` (host ints, [0, ..., n]) packs
        independent samples whose queries see only their own keys."""
        import torch
        n = int(x.shape[0])
        if out is None:
            out = torch.empty_like(x)
        ws = self.workspace(n) if workspace is None else workspace
        px, prow, ppos, pout, pws = self._io(x, rows, pos, out, ws)
        sg, ns = _dbl(sigmas)
        if seq_starts is None:
            _check(lib.dit_block_forward(ctypes.byref(self.cfg), self.prepared.data_ptr(), px,
                                         n, prow, ppos, sg, ns, pout,
                                         pws, ws.numel(), _stream(stream)))
        else:
            st, nseq = _starts(seq_starts)
            _check(lib.dit_block_forward_packed(ctypes.byref(self.cfg), self.prepared.data_ptr(),
                                                px, n, prow, ppos, sg, ns, st,
                                                nseq, pout, pws, ws.numel(),
                                                _stream(stream)))
        return out

    def _io(self, x, rows, pos, out, ws):
        """Checked addresses of a block call's x [n, D], rows int32 [n], pos
        fp32 [n, 3], out [n, D] (fp32) and workspace (uint8)."""
        D = self.cfg.D
        n = int(x.shape[0]) if hasattr(x, "shape") and len(x.shape) else -1
        px = _arg(x, "x", "f32", (None, D))
        prow = _arg(rows, "rows", "i32", (n,), optional=True)
        ppos = _arg(pos, "pos", "f32", (n, 3), optional=True)
        pout = _arg(out, "out", "f32", (n, D))
        pws = _arg(ws, "workspace", "u8", (None,))
        return px, prow, ppos, pout, pws

    def forward_mods(self, x, rows, pos, mods, out=None, workspace=None, stream=None,
                     seq_starts: Optional[Sequence[int]] = None):
        """Block forward with caller-supplied modulation rows ``mods`` (device
        fp32 [R, E*D])."""
        import torch
        n = int(x.shape[0])
        if out is None:
            out = torch.empty_like(x)
        ws = self.workspace(n) if workspace is None else workspace
        px, prow, ppos, pout, pws = self._io(x, rows, pos, out, ws)
        pm = _arg(mods, "mods", "f32", mod_shape(self.cfg))
        if seq_starts is None:
            st, nseq = None, 0
        else:
            st, nseq = _starts(seq_starts)
        _check(lib.dit_block_forward_mods(ctypes.byref(self.cfg), self.prepared.data_ptr(), px,
                                          n, prow, ppos, pm, st, nseq, pout,
                                          pws, ws.numel(), _stream(stream)))
        return out

    def adaln_modulate(self, x, rows, sigmas: Sequence[float], half: int, xn_out, mods_out=None,
                       temb_scratch=None, stream=None):
        n = int(x.shape[0])
        c = self.cfg
        px = _arg(x, "x", "f32", (n, c.D))
        prow = _arg(rows, "rows", "i32", (n,), optional=True)
        pxn = _arg(xn_out, "xn_out", _act(c), (n, c.D))
        pm = _arg(mods_out, "mods_out", "f32", mod_shape(c), optional=True) \
            if c.variant in (MMH3, ZIMAGE, FINAL, ZFINAL) else None
        pt = _arg(temb_scratch, "temb_scratch", "f32", None, optional=True,
                  min_numel=c.temb_hidden + c.temb_freq)
        sg, ns = _dbl(sigmas)
        _check(lib.dit_adaln_modulate(ctypes.byref(c), self.prepared.data_ptr(), px, n,
                                      prow, sg, ns, half, pxn, pm, pt, _stream(stream)))
        return xn_out

    def adaln_eval_noalloc(self, sigmas: Sequence[float], mods_out, stream=None):
        """dit_adaln_eval_noalloc: the modulation rows with the timestep MLP's
        scratch in the library's own device array (no scratch argument)."""
        pm = _arg(mods_out, "mods_out", "f32", mod_shape(self.cfg))
        sg, ns = _dbl(sigmas)
        _check(lib.dit_adaln_eval_noalloc(ctypes.byref(self.cfg), self.prepared.data_ptr(), sg, ns,
                                          pm, _stream(stream)))
        return mods_out

    def adaln_eval(self, sigmas: Sequence[float], mods_out, temb_scratch=None, stream=None):
        c = self.cfg
        pm = _arg(mods_out, "mods_out", "f32", mod_shape(c))
        pt = _arg(temb_scratch, "temb_scratch", "f32", None, optional=True,
                  min_numel=c.temb_hidden + c.temb_freq)
        sg, ns = _dbl(sigmas)
        _check(lib.dit_adaln_eval(ctypes.byref(c), self.prepared.data_ptr(), sg, ns,
                                  pm, pt, _stream(stream)))
        return mods_out


def attention(cfg: DitConfig, q, k, vt, n: int, ldn: int, score_scale: float, o, stream=None,
              seq_starts: Optional[Sequence[int]] = None):
    a = _act(cfg)
    pq = _arg(q, "q", a, (cfg.H, ldn, cfg.hd))
    pk = _arg(k, "k", a, (cfg.H, ldn, cfg.hd))
    pv = _arg(vt, "vt", a, (cfg.H, cfg.hd, ldn))
    po = _arg(o, "o", a, (n, cfg.D))
    if seq_starts is None:
        _check(lib.dit_attention(ctypes.byref(cfg), pq, pk, pv, n, ldn,
                                 score_scale, po, _stream(stream)))
    else:
        st, nseq = _starts(seq_starts)
        _check(lib.dit_attention_packed(ctypes.byref(cfg), pq, pk, pv, n, ldn, st,
                                        nseq, score_scale, po, _stream(stream)))
    return o


def attention_shard(cfg: DitConfig, q, ldq: int, qlo: int, qhi: int, k, vt, n: int, ldn: int,
                    score_scale: float, o, workspace=None, stream=None):
    """dit_attention_shard: the queries of tokens [qlo, qhi) (q rows 0..qhi-qlo)
    against all n keys; o [qhi - qlo, D].  The workspace (the split tail's
    partials) is allocated here when not given."""
    import torch
    a = _act(cfg)
    m = qhi - qlo
    pq = _arg(q, "q", a, (cfg.H, ldq, cfg.hd))
    pk = _arg(k, "k", a, (cfg.H, ldn, cfg.hd))
    pv = _arg(vt, "vt", a, (cfg.H, cfg.hd, ldn))
    po = _arg(o, "o", a, (m, cfg.D))
    need = lib.dit_attention_shard_workspace_size(ctypes.byref(cfg))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw = _arg(workspace, "workspace", "u8", None, optional=True, min_numel=need)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib.dit_attention_shard(ctypes.byref(cfg), pq, ldq, qlo, qhi, pk, pv, n, ldn,
                                   score_scale, po, pw, nbytes, _stream(stream)))
    return o


def profile_begin(max_calls: int) -> None:
    _check(lib.dit_profile_begin(max_calls))


def profile_end() -> Dict[str, float]:
    """Summed ms per phase over the recorded calls (plus "calls")."""
    ms = (c_double * NPHASES)()
    calls = c_int32(0)
    _check(lib.dit_profile_end(ms, ctypes.byref(calls)))
    out = {lib.dit_phase_name(i).decode(): ms[i] for i in range(NPHASES)}
    out["calls"] = calls.value
    return out


def final_forward(blk: "Block", h, rows, sigmas: Sequence[float], out=None, workspace=None,
                  stream=None):
    """Output head (a Block prepared with a DIT_FINAL config): out = -(W
    modulate(RMSNorm(h)) + b), fp32 [n, F]; with a DIT_ZFINAL config the
    Z-Image final layer (sigmas = [t])."""
    import torch
    n = int(h.shape[0])
    if out is None:
        out = torch.empty((n, blk.cfg.F), dtype=torch.float32, device=h.device)
    ws = blk.workspace(n) if workspace is None else workspace
    ph = _arg(h, "h", "f32", (n, blk.cfg.D))
    prow = _arg(rows, "rows", "i32", (n,), optional=True)
    pout = _arg(out, "out", "f32", (n, blk.cfg.F))
    pws = _arg(ws, "workspace", "u8", (None,))
    sg, ns = _dbl(sigmas)
    _check(lib.dit_final_forward(ctypes.byref(blk.cfg), blk.prepared.data_ptr(), ph, n,
                                 prow, sg, ns, pout, pws, ws.numel(),
                                 _stream(stream)))
    return out


def linear(a, w, bias=None, alpha: float = 1.0, out=None, stream=None):
    """out = alpha * (a @ w^T + bias) in fp32 on the block GEMM kernels; a and w
    share a dtype (bfloat16 or float32)."""
    import torch
    m, k = int(a.shape[0]), int(a.shape[1])
    nout = int(w.shape[0])
    dtype = BF16 if a.dtype == torch.bfloat16 else F32
    dn = "bf16" if dtype == BF16 else "f32"
    if out is None:
        out = torch.empty((m, nout), dtype=torch.float32, device=a.device)
    pa = _arg(a, "a", dn, (m, k), strided=True)
    pw = _arg(w, "w", dn, (nout, k))
    pb = _arg(bias, "bias", "f32", (nout,), optional=True)
    po = _arg(out, "out", "f32", (m, nout))
    _check(lib.dit_linear(dtype, pa, int(a.stride(0)), m, k, pw, nout, pb,
                          alpha, po, _stream(stream)))
    return out


def stack_forward(blocks: Sequence["Block"], x, rows, pos, sigmas: Sequence[float], out=None,
                  workspace=None, stream=None, seq_starts: Optional[Sequence[int]] = None):
    """Blocks of one configuration in order: out = blocks[-1](...blocks[0](x))."""
    import torch
    n = int(x.shape[0])
    if out is None:
        out = torch.empty_like(x)
    ws = blocks[0].workspace(n) if workspace is None else workspace
    px, prow, ppos, pout, pws = blocks[0]._io(x, rows, pos, out, ws)
    preps = (c_void_p * len(blocks))(*[b.prepared.data_ptr() for b in blocks])
    sg, ns = _dbl(sigmas)
    st, nseq = (None, 0) if seq_starts is None else _starts(seq_starts)
    _check(lib.dit_stack_forward(ctypes.byref(blocks[0].cfg), preps, len(blocks), px, n,
                                 prow, ppos, sg, ns, st, nseq, pout,
                                 pws, ws.numel(), _stream(stream)))
    return out


def patchify_video(x, dtype_out=None, stream=None):
    """[C, T, H, W] fp32 -> rows [T*(H/2)*(W/2), 4C] (bfloat16 or float32)."""
    import torch
    C, T, H, W = (int(v) for v in x.shape)
    td = torch.bfloat16 if dtype_out == "bf16" else torch.float32
    rows = torch.empty((T * (H // 2) * (W // 2), 4 * C), dtype=td, device=x.device)
    _check(lib.dit_patchify_video(BF16 if td == torch.bfloat16 else F32, _ptr(x), C, T, H, W,
                                  _ptr(rows), _stream(stream)))
    return rows


def unpatchify_video(rows, C: int, T: int, H: int, W: int, stream=None):
    import torch
    x = torch.empty((C, T, H, W), dtype=torch.float32, device=rows.device)
    _check(lib.dit_unpatchify_video(_ptr(rows), C, T, H, W, _ptr(x), _stream(stream)))
    return x


def pack_audio(x, dtype_out=None, stream=None):
    """[C, 2, T] fp32 -> rows [2T, C]."""
    import torch
    C, _, T = (int(v) for v in x.shape)
    td = torch.bfloat16 if dtype_out == "bf16" else torch.float32
    rows = torch.empty((2 * T, C), dtype=td, device=x.device)
    _check(lib.dit_pack_audio(BF16 if td == torch.bfloat16 else F32, _ptr(x), C, T, _ptr(rows),
                              _stream(stream)))
    return rows


def patchify_image(x, dtype_out=None, stream=None):
    """[C, H, W] fp32 -> rows [(H/2)*(W/2), 4C], channel-fastest columns."""
    import torch
    C, H, W = (int(v) for v in x.shape)
    td = torch.bfloat16 if dtype_out == "bf16" else torch.float32
    rows = torch.empty(((H // 2) * (W // 2), 4 * C), dtype=td, device=x.device)
    _check(lib.dit_patchify_image(BF16 if td == torch.bfloat16 else F32, _ptr(x), C, H, W,
                                  _ptr(rows), _stream(stream)))
    return rows


def unpatchify_image(rows, C: int, H: int, W: int, stream=None):
    import torch
    x = torch.empty((C, H, W), dtype=torch.float32, device=rows.device)
    _check(lib.dit_unpatchify_image(_ptr(rows), C, H, W, _ptr(x), _stream(stream)))
    return x


def unpack_audio(rows, C: int, T: int, stream=None):
    import torch
    x = torch.empty((C, 2, T), dtype=torch.float32, device=rows.device)
    _check(lib.dit_unpack_audio(_ptr(rows), C, T, _ptr(x), _stream(stream)))
    return x


def rms_norm(x, g, eps: float, out=None, stream=None):
    import torch
    n, D = (int(v) for v in x.shape)
    if out is None:
        out = torch.empty_like(x)
    _check(lib.dit_rms_norm(_ptr(x), n, D, _ptr(g), eps, _ptr(out), _stream(stream)))
    return out


class Mmh3Model:
    """The MMH3 denoise evaluation over prepared pieces: blocks (Block with a
    DIT_MMH3 config), video/audio heads (Block with DIT_FINAL configs) and the
    patch projections (device tensors [D, 4C] / [D, Ca] in the blocks' dtype).
    ``audio_slope_rescale`` returns the audio velocity multiplied by
    d(sigma_a)/d(sigma_v) instead of unscaled."""

    def __init__(self, blocks: Sequence["Block"], head_video: "Block", head_audio: Optional["Block"],
                 latent_c: int, audio_c: int, video_patch_w, video_patch_b=None,
                 audio_patch_w=None, audio_patch_b=None, shift_video: float = 12.0,
                 shift_audio: float = 3.0, cond_aug: float = 0.999, cond_aug_audio: float = 1.0,
                 audio_slope_rescale: bool = False):
        self.blocks, self.head_video, self.head_audio = list(blocks), head_video, head_audio
        self._preps = (c_void_p * len(self.blocks))(*[b.prepared.data_ptr() for b in self.blocks])
        self._keep = (video_patch_w, video_patch_b, audio_patch_w, audio_patch_b)
        m = DitMmh3Model()
        m.block = ctypes.pointer(self.blocks[0].cfg)
        m.blocks = self._preps
        m.n_blocks = len(self.blocks)
        m.head_video = ctypes.pointer(head_video.cfg)
        m.head_video_w = head_video.prepared.data_ptr()
        if head_audio is not None:
            m.head_audio = ctypes.pointer(head_audio.cfg)
            m.head_audio_w = head_audio.prepared.data_ptr()
        m.latent_c, m.audio_c = latent_c, audio_c
        m.video_patch_w, m.video_patch_b = _ptr(video_patch_w), _ptr(video_patch_b)
        m.audio_patch_w, m.audio_patch_b = _ptr(audio_patch_w), _ptr(audio_patch_b)
        m.shift_video, m.shift_audio = shift_video, shift_audio
        m.cond_aug, m.cond_aug_audio = cond_aug, cond_aug_audio
        m.audio_slope_rescale = int(bool(audio_slope_rescale))
        self._m = m
        self._ws = None

    def forward(self, segments, pos, text, video, audio=None, conds=(), sigma_v: float = 0.5,
                stream=None, text_tags=None):
        """segments: [(kind, start, stop)] with kinds text / video / audio / cond;
        text_tags: device int32 [text rows] per-token modality (None = text).
        Returns (video velocity [C, T, H, W], audio velocity [Ca, 2, Ta] or None)."""
        import torch
        segs = (DitSegment * len(segments))(*[DitSegment(SEG_KINDS[k], a, b) for k, a, b in segments])
        need = lib.dit_mmh3_workspace_size(ctypes.byref(self._m), segs, len(segments))
        if need == 0:
            raise DitError(-1, lib.dit_last_error().decode())
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        C, T, H, W = (int(v) for v in video.shape)
        vout = torch.empty_like(video)
        aout = None if audio is None else torch.empty_like(audio)
        Ta = 0 if audio is None else int(audio.shape[2])
        cp = (c_void_p * max(len(conds), 1))(*[c.data_ptr() for c in conds])
        _check(lib.dit_mmh3_forward(ctypes.byref(self._m), segs, len(segments), _ptr(pos), _ptr(text),
                                    _ptr(text_tags), _ptr(video), T, H, W, _ptr(audio), Ta, cp, sigma_v,
                                    _ptr(vout), _ptr(aout), self._ws.data_ptr(), self._ws.numel(),
                                    _stream(stream)))
        return vout, aout


class ZimageCache:
    """Step-level reuse state of ZimageModel.forward: device buffers for the
    refined caption and the stream after the first ``layers`` main layers,
    refreshed when step % interval == 0.  ``reset()`` starts a new generation."""

    def __init__(self, model: "ZimageModel", H: int, W: int, cap_len: int, layers: int,
                 interval: int):
        import torch
        D = model.D
        n = (H // 2) * (W // 2) + cap_len
        self.caption = torch.empty((max(cap_len, 1), D), dtype=torch.float32, device="cuda")
        self.shallow = torch.empty((n, D), dtype=torch.float32, device="cuda")
        c = DitZimageCache()
        c.caption, c.shallow = self.caption.data_ptr(), self.shallow.data_ptr()
        c.layers, c.interval = layers, interval
        self.c = c

    def reset(self) -> None:
        self.c.caption_valid = 0
        self.c.shallow_valid = 0


class ZimageModel:
    """The Z-Image transformer over prepared pieces: main layers and noise
    refiners (Blocks with a DIT_ZIMAGE config), context refiners (DIT_ZCONTEXT),
    the final layer (DIT_ZFINAL) and the embedders (device tensors: x_embed_w
    [D, 4C] and cap_embed_w [D, cap_dim] in the blocks' dtype, fp32 biases and
    the caption RMSNorm gain)."""

    def __init__(self, layers: Sequence["Block"], noise_refiners: Sequence["Block"],
                 context_refiners: Sequence["Block"], final: "Block", in_channels: int,
                 x_embed_w, x_embed_b, cap_norm, cap_embed_w, cap_embed_b, cap_eps: float = 1e-6,
                 block_cfg: Optional[DitConfig] = None, context_cfg: Optional[DitConfig] = None):
        self.layers, self.noise, self.context = list(layers), list(noise_refiners), list(context_refiners)
        self.final = final
        arr = lambda bl: (c_void_p * max(len(bl), 1))(*[b.prepared.data_ptr() for b in bl])  # noqa: E731
        self._arrs = (arr(self.layers), arr(self.noise), arr(self.context))
        self._keep = (x_embed_w, x_embed_b, cap_norm, cap_embed_w, cap_embed_b)
        if block_cfg is None and not (self.layers or self.noise):
            raise ValueError("ZimageModel needs a block config (block_cfg) when it has no blocks")
        bcfg = block_cfg or (self.layers or self.noise)[0].cfg
        ccfg = context_cfg or (self.context[0].cfg if self.context else None)
        self._cfgs = (bcfg, ccfg)
        m = DitZimageModel()
        m.block = ctypes.pointer(bcfg)
        m.layers, m.n_layers = self._arrs[0], len(self.layers)
        m.noise_refiners, m.n_noise_refiners = self._arrs[1], len(self.noise)
        m.context = ctypes.pointer(ccfg) if ccfg is not None else None
        m.context_refiners, m.n_context_refiners = self._arrs[2], len(self.context)
        m.final_layer = ctypes.pointer(final.cfg)
        m.final_w = final.prepared.data_ptr()
        m.in_channels, m.cap_dim = in_channels, int(cap_embed_w.shape[1])
        m.x_embed_w, m.x_embed_b = _ptr(x_embed_w), _ptr(x_embed_b)
        m.cap_norm, m.cap_eps = _ptr(cap_norm), cap_eps
        m.cap_embed_w, m.cap_embed_b = _ptr(cap_embed_w), _ptr(cap_embed_b)
        self._m = m
        self.D = bcfg.D
        self._ws = None

    def forward(self, latents, cap_feats, pos, t: float, step: int = 0,
                cache: Optional[ZimageCache] = None, stream=None):
        """latents [C, H, W] fp32, cap_feats [L, cap_dim] fp32, pos [(H/2)(W/2) + L, 3]
        (image first).  Returns the final layer's output as [C, H, W]."""
        import torch
        C, H, W = (int(v) for v in latents.shape)
        L = int(cap_feats.shape[0])
        need = lib.dit_zimage_workspace_size(ctypes.byref(self._m), H, W, L)
        if need == 0:
            raise DitError(-1, lib.dit_last_error().decode())
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(latents)
        cp = ctypes.byref(cache.c) if cache is not None else None
        _check(lib.dit_zimage_forward(ctypes.byref(self._m), _ptr(latents), H, W, _ptr(cap_feats), L,
                                      _ptr(pos), t, step, cp, _ptr(out), self._ws.data_ptr(),
                                      self._ws.numel(), _stream(stream)))
        return out

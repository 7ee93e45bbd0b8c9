"""Stage a seeded workload on the GPU: the same values the oracle reads, as
device tensors (GEMM weights in the block's dtype, everything else fp32)."""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

GEMM_WEIGHTS = ("w_qkv", "w_out", "w_fc1", "w_fc2")


@dataclasses.dataclass
class DeviceWorkload:
    x: "object"
    rows: Optional["object"]
    pos: Optional["object"]
    weights: Dict[str, "object"]


def to_device(wl, device: str = "cuda") -> DeviceWorkload:
    import torch
    wdt = torch.bfloat16 if wl.spec.dtype == "bf16" else torch.float32
    weights = {}
    for k, v in wl.weights.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in GEMM_WEIGHTS:
            t = t.to(wdt)  # values are already bf16-representable: exact
        weights[k] = t.to(device).contiguous()
    # the SigLIP LayerNorm gains travel in the norm1/norm2 slots
    if wl.spec.variant == "siglip":
        weights["norm1"] = weights.pop("ln1_w")
        weights["norm2"] = weights.pop("ln2_w")
    x = torch.from_numpy(np.ascontiguousarray(wl.x)).to(device)
    rows = None if wl.rows is None else torch.from_numpy(np.ascontiguousarray(wl.rows)).to(device)
    pos = None if wl.pos is None else torch.from_numpy(np.ascontiguousarray(wl.pos)).to(device)
    return DeviceWorkload(x, rows, pos, weights)

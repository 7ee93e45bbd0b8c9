"""The binding refuses tensors of the wrong dtype or shape with ValueError
before anything reaches the C ABI (an int64 rows tensor would otherwise be
read as int32 pairs; a bf16 x or a short pos would be read out of bounds)."""

import pytest

from synth import workloads as W
from tests.gpu_common import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from packed_sequence_diffusion_amd import dit as d
    return d


def test_wrong_dtypes_and_shapes_raise(dit):
    import torch
    from synth.device import to_device
    spec = W.BlockSpec("binding", "mmh3", "bf16", n=130, D=256, H=2, hd=128, F=384, slots=2,
                       rope="split_half", rope_axes=(32, 48, 48))
    wl = W.make_custom_workload(spec, 77)
    dev = to_device(wl)
    cfg = dit.make_config(spec)
    bad_w = dict(dev.weights)
    bad_w["w_qkv"] = bad_w["w_qkv"].float()
    with pytest.raises(ValueError, match="w_qkv"):
        dit.Block(cfg, bad_w)
    bad_w = dict(dev.weights)
    bad_w["w_out"] = bad_w["w_out"][:128].contiguous()
    with pytest.raises(ValueError, match="w_out"):
        dit.Block(cfg, bad_w)
    blk = dit.Block(cfg, dev.weights)
    sig = [0.4, 0.2]
    cases = {
        "rows int64": (dev.x, dev.rows.long(), dev.pos),
        "x bf16": (dev.x.bfloat16(), dev.rows, dev.pos),
        "pos [n, 2]": (dev.x, dev.rows, dev.pos[:, :2].contiguous()),
        "rows short": (dev.x, dev.rows[:-1].contiguous(), dev.pos),
        "x on the host": (dev.x.cpu(), dev.rows, dev.pos),
    }
    for why, (x, rows, pos) in cases.items():
        with pytest.raises(ValueError):
            blk.forward(x, rows, pos, sig)
        log(f"[case] binding refuses {why}")
    mods = torch.empty((6, 6 * 256), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="mods"):
        blk.forward_mods(dev.x, dev.rows, dev.pos, mods[:, :100].contiguous())
    with pytest.raises(ValueError, match="mods_out"):
        blk.adaln_eval(sig, mods.double())
    xn = torch.empty((spec.n, spec.D), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="xn_out"):  # the bf16 block writes bf16 rows
        blk.adaln_modulate(dev.x, dev.rows, sig, 0, xn, mods)
    # the checked call still runs
    out = blk.forward(dev.x, dev.rows, dev.pos, sig)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()

"""The ctypes binding's argument checks (CPU): the weight table it validates
against agrees with the seeded weights of every variant, and tensors that are
not on a GPU are refused before anything reaches the C ABI."""

import numpy as np
import pytest
import torch

from synth import workloads as W


@pytest.fixture(scope="module")
def dit():
    from packed_sequence_diffusion_amd import dit as d
    return d


def _variant_specs():
    toy = W.spec_by_name("toy")
    z = W.spec_by_name("zimage")
    return [
        toy,
        W.small_spec(toy, name="shared", slots=3, adaln_shared=1),
        W.small_spec(toy, name="partial", rope="partial", rope_axes=(16, 16, 16)),
        W.small_spec(W.spec_by_name("siglip"), D=256, H=4, F=512),
        W.small_spec(z, D=256, H=2, F=384, temb_hidden=64, temb_freq=32),
        W.small_spec(toy, name="refiner", variant="refiner", slots=1),
        W.small_spec(z, name="zcontext", variant="zcontext", D=256, H=2, F=384),
        W.BlockSpec("head", "final", "bf16", n=4, D=256, H=2, hd=128, F=64, slots=3, tags=1),
        W.small_spec(z, name="zfinal", variant="zfinal", D=256, H=2, F=64, temb_hidden=64,
                     temb_freq=32),
    ]


@pytest.mark.parametrize("spec", _variant_specs(), ids=lambda s: f"{s.variant}-{s.name}")
def test_weight_table_matches_the_seeded_weights(dit, spec):
    """Every weight a variant reads has the shape the binding checks it
    against (the GPU parity tests run on exactly these tensors)."""
    cfg = dit.make_config(spec)
    dit.validate(cfg)
    table = dit.weight_shapes(cfg)
    w = W.make_weights(spec, 11)
    if spec.variant == "siglip":  # the LayerNorm gains travel as norm1 / norm2
        w["norm1"], w["norm2"] = w.pop("ln1_w"), w.pop("ln2_w")
    for name, arr in w.items():
        assert name in table, f"{spec.variant}: seeded weight {name} is not in the binding's table"
        assert tuple(arr.shape) == tuple(table[name][1]), (name, arr.shape, table[name])
    gemm = {"w_qkv", "w_out", "w_fc1", "w_fc2"}
    for name, (dt, _) in table.items():
        assert dt == ((spec.dtype if name in gemm else "f32")), name


def test_cpu_tensors_are_refused(dit):
    """A host tensor handed where the library expects device memory raises
    ValueError in the binding (nothing is launched)."""
    spec = W.small_spec(W.spec_by_name("t2va"), D=256, H=2, F=384)
    cfg = dit.make_config(spec)
    n, ldn = 100, 128
    q = torch.zeros((2, ldn, 128), dtype=torch.bfloat16)
    o = torch.zeros((n, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA tensor"):
        dit.attention(cfg, q, q, q.transpose(1, 2).contiguous(), n, ldn, 1.0, o)
    with pytest.raises(ValueError, match="CUDA tensor"):
        dit.linear(torch.zeros((4, 64), dtype=torch.bfloat16), torch.zeros((32, 64), dtype=torch.bfloat16))


def test_mod_shapes(dit):
    t2va = W.spec_by_name("t2va")
    assert dit.mod_shape(dit.make_config(t2va)) == (6, 6 * 2688)
    z = W.spec_by_name("zimage")
    assert dit.mod_shape(dit.make_config(z)) == (1, 4 * 3072)
    with pytest.raises(ValueError):
        dit.mod_shape(dit.make_config(W.spec_by_name("siglip")))
    spec = W.small_spec(t2va, D=256, H=2, F=384)
    assert np.prod(dit.mod_shape(dit.make_config(spec))) == spec.mod_rows * spec.chunks * spec.D

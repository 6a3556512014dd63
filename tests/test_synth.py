"""The seeded input generator: same seed gives identical bytes; shapes, dtypes and
distribution moments follow each workload's recipe."""
import numpy as np
import torch

from gated_deltanet_recurrent_02_amd import synth


def _same(a, b):
    return all(torch.equal(a[k], b[k]) for k in a if isinstance(a[k], torch.Tensor))


def test_decode_inputs_deterministic():
    a = synth.decode_inputs(2, 3, 16, 2, seed=5)
    b = synth.decode_inputs(2, 3, 16, 2, seed=5)
    c = synth.decode_inputs(2, 3, 16, 2, seed=6)
    assert _same(a, b) and not torch.equal(a["q"], c["q"])


def test_fused_inputs_deterministic():
    a = synth.fused_inputs(2, 2, 16, 3, seed=1)
    b = synth.fused_inputs(2, 2, 16, 3, seed=1)
    assert _same(a, b)


def test_decode_recipe_shapes_and_moments():
    x = synth.decode_inputs(8, 48, 128, 1, seed=0)
    assert x["q"].dtype == torch.bfloat16 and x["state"].dtype == torch.float32
    assert x["q"].shape == (8, 1, 48, 128) and x["state"].shape == (8, 48, 128, 128)
    assert x["alpha"].shape == (8, 1, 48) and x["alpha"].dtype == torch.float32
    nq = x["q"].double().norm(dim=-1)
    assert float((nq - 1).abs().max()) < 2 ** -7          # unit length up to bf16 rounding
    s = x["state"].double()
    assert abs(float(s.std()) - 0.02) < 1e-3 and abs(float(s.mean())) < 1e-4
    assert float(x["v"].double().std()) > 0.9
    al, be = x["alpha"].double(), x["beta"].double()
    assert 0 < float(al.min()) and float(al.max()) < 1 and 0 < float(be.min()) and float(be.max()) < 1
    # alpha = exp(-softplus(z + 2)): median exp(-softplus(2)) ~ 0.119
    assert abs(float(al.median()) - 0.119) < 0.03


def test_tiny_workload_recipe():
    x = synth.workload_inputs("decode_b1_h2_d16_t8")
    assert x["q"].dtype == torch.float32 and x["state"].abs().max() == 0
    assert x["q"].shape == (1, 8, 2, 16)


def test_fused_recipe():
    x = synth.fused_inputs(4, 48, 128, 4, seed=0)
    assert x["qkv"].shape == (4, 4, 3 * 48 * 128) and x["qkv"].dtype == torch.bfloat16
    assert x["conv_state"].shape == (4, 3 * 48 * 128, 3)
    assert x["conv_w"].shape == (3 * 48 * 128, 4)
    assert abs(float(x["conv_w"].std()) - 0.5) < 0.01

"""Host logic of the input generator and the workload table (CPU only)."""
import json
import os

import numpy as np
import torch

from dynamic_convolution_cnn_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e-39,
                                  65504.0, -1.5e-5], np.float32)])
    bits = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = inputs.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generator_is_seeded_and_shaped():
    for key in inputs.ORDER:
        w = inputs.WORKLOADS[key]
        d = inputs.make_inputs(w, seed=0, B=2)
        L0 = w.layers[0]
        assert d["x"].shape == (2, L0.Cin, L0.H, L0.W)
        assert len(d["experts"]) == len(w.layers)
        for L, e in zip(w.layers, d["experts"]):
            assert e.shape == (w.n,) + L.expert_shape
            if w.dtype == "bf16":
                np.testing.assert_array_equal(inputs.bf16_round(e), e)
        assert d["fc_w"].shape == (w.n, L0.Cin)
        np.testing.assert_array_equal(d["fc_b"], 0)
        d2 = inputs.make_inputs(w, seed=0, B=2)
        np.testing.assert_array_equal(d["x"], d2["x"])
    x = inputs.make_inputs(inputs.WORKLOADS["resnet50_3x3"], B=2)["x"]
    assert x.min() == 0.0


def test_flop_convention_from_the_pages():
    """One multiply-add counts as two FLOPs (CondConv page: abstract vs Tasks table)."""
    g = json.load(open(os.path.join(GOLDEN, "condconv_flop_convention.json")))
    assert abs(2 * g["multiply_adds"] / 1e9 - g["gflops"]) < 1e-12
    w = inputs.WORKLOADS["resnet50_3x3"]
    L = w.layers[0]
    assert w.conv_flops() == 2 * w.B * L.Cout * L.Ho * L.Wo * L.Cin * L.k * L.k
    assert abs(w.conv_flops() / 1e9 - 59.190018048) < 1e-6


def test_workload_shapes():
    w = inputs.WORKLOADS["effnet_b0_mbconv"]
    assert [L.Ho for L in w.layers] == [28, 28, 28]
    assert w.layers[1].expert_shape == (240, 1, 5, 5)
    assert inputs.WORKLOADS["many_expert_softmax"].fc_std_value() == np.sqrt(784 / 128)

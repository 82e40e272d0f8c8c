"""GPU parity of many-expert banks (KernelWarehouse: Rethinking the Design of
Dynamic Convolution, abstract: n > 100) through the C ABI against the oracle.

bf16 layers with groups == 1 and more than 16 experts mix on the matrix cores
with the experts as the reduction dimension (a bank transposed once into the
convolution's weight order), then run the premix convolutions. Tolerances:
2e-2 normwise for the layer (R10); the standalone mix also elementwise, one
bf16 rounding of a float32 sum (the attentions enter as three exact bf16
parts).
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_convolution_cnn_amd import binding as bd
from dynamic_convolution_cnn_amd import inputs

from test_gpu_parity import ALPHA_TOL, TOL, check, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(device):
    bd.lib()
    yield


@pytest.mark.parametrize("n,B,wshape", [(65, 3, (16, 8, 3, 3)), (100, 33, (24, 16, 3, 3)),
                                        (128, 70, (40, 24, 1, 1)), (256, 5, (8, 8, 5, 5)),
                                        (129, 64, (16, 16, 3, 3)),
                                        # 576 weight tiles: 64 examples per workgroup
                                        (72, 65, (128, 128, 3, 3)), (67, 100, (128, 128, 3, 3))])
def test_mix_many_experts(n, B, wshape):
    rng = np.random.default_rng(70 + n)
    e = inputs.bf16_round(rng.standard_normal((n,) + wshape, dtype=np.float32))
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    say("mix wide", n, B, wshape)
    m = bd.dynconv_mix(to_dev(alpha, "f32"), to_dev(e, "bf16"))
    torch.cuda.synchronize()
    got, ref = from_dev(m), oracle.mix(alpha, e)
    check(got, ref, TOL["bf16"], f"mix n={n}")
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * oracle.mix(np.abs(alpha), np.abs(e))
    assert np.all(np.abs(got - ref) <= bound)


WIDE_FWD = [
    # B, Cin, Cout, H, W, k, pad, n
    (3, 40, 72, 16, 16, 3, 1, 24),     # 3x3, 24 experts (two chunks of 16, the second partial)
    (2, 64, 48, 12, 12, 3, 1, 128),    # 3x3, 128 experts
    (3, 40, 80, 14, 14, 1, 0, 101),    # 1x1, 101 experts
    (70, 16, 16, 8, 8, 3, 1, 200),     # two 64-example workgroups, 200 experts
]


@pytest.mark.parametrize("case", WIDE_FWD)
def test_forward_many_experts(case):
    B, Cin, Cout, H, W, k, p, n = case
    rng = np.random.default_rng(80 + n)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round((rng.standard_normal((n, Cout, Cin, k, k)) * np.sqrt(2.0 / (Cin * k * k)))
                          .astype(np.float32))
    a = (rng.random((B, n)) / n * 4).astype(np.float32)
    desc = bd.make_desc(B, Cin, H, W, Cout, k, k, 1, p, 1, n, bd.DYNCONV_BF16)
    assert bd.dynconv_forward_policy(desc) == bd.DYNCONV_POLICY_PREMIX
    say("forward wide", case)
    y = bd.dynconv_forward(to_dev(x, "bf16"), to_dev(e, "bf16"), to_dev(a, "f32"), 1, p, 1)
    torch.cuda.synchronize()
    check(from_dev(y), oracle.forward(x, e, a, 1, p, 1), TOL["bf16"], f"forward n={n} {case}")
    with pytest.raises(bd.DynconvError):
        bd.dynconv_forward(to_dev(x, "bf16"), to_dev(e, "bf16"), to_dev(a, "f32"), 1, p, 1,
                           policy=bd.DYNCONV_POLICY_FUSED)


@pytest.mark.parametrize("case", WIDE_FWD[:3])
def test_forward_packed_many_experts(case):
    """A bank of more than 16 experts packed once ([n][t][o][c']) and reused: the same result, bit for bit, as
    dynconv_forward, which packs on every call."""
    B, Cin, Cout, H, W, k, p, n = case
    rng = np.random.default_rng(90 + n)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round((rng.standard_normal((n, Cout, Cin, k, k)) * np.sqrt(2.0 / (Cin * k * k)))
                          .astype(np.float32))
    a = (rng.random((B, n)) / n * 4).astype(np.float32)
    desc = bd.make_desc(B, Cin, H, W, Cout, k, k, 1, p, 1, n, bd.DYNCONV_BF16)
    say("forward packed wide", case)
    xd, ed, ad = to_dev(x, "bf16"), to_dev(e, "bf16"), to_dev(a, "f32")
    pk = torch.empty(bd.dynconv_packed_experts_bytes(desc), dtype=torch.uint8, device=xd.device)
    bd.dynconv_pack_experts(desc, ed, pk)
    y1 = bd.dynconv_forward_packed(desc, xd, pk, ad)
    y2 = bd.dynconv_forward_packed(desc, xd, pk, ad)   # the bank is reused, not consumed
    y0 = bd.dynconv_forward(xd, ed, ad, 1, p, 1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(y2, y0)
    check(from_dev(y1), oracle.forward(x, e, a, 1, p, 1), TOL["bf16"], f"forward packed n={n} {case}")


def test_route_and_layer_at_kernelwarehouse_scale():
    """The n = 128 workload's routing (softmax(z/4)) and layer, on sampled examples."""
    w = inputs.WORKLOADS["kernelwarehouse_n128"]
    d = inputs.make_inputs(w, seed=0)
    L = w.layers[0]
    xd = to_dev(d["x"], "bf16")
    say("kernelwarehouse n=128 route + forward")
    alpha = bd.dynconv_route(xd, to_dev(d["fc_w"], "f32"), to_dev(d["fc_b"], "f32"), w.route_mode, w.temperature)
    y = bd.dynconv_forward(xd, to_dev(d["experts"][0], "bf16"), alpha, L.stride, L.pad, L.groups)
    torch.cuda.synchronize()
    ra, _, _ = oracle.route(d["x"], d["fc_w"], d["fc_b"], w.route_mode, w.temperature)
    check(from_dev(alpha), ra, ALPHA_TOL, "kernelwarehouse alpha")
    sel = np.array([0, 31, 63])
    ry = oracle.forward(d["x"][sel], d["experts"][0], from_dev(alpha)[sel], L.stride, L.pad, L.groups)
    check(from_dev(y)[sel], ry, TOL["bf16"], "kernelwarehouse layer (sampled examples)")


def test_backward_many_experts():
    """The gradients with a 100-expert bank (the input gradient runs the wide forward)."""
    B, Cin, Cout, H, W, n = 2, 16, 24, 8, 8, 100
    rng = np.random.default_rng(90)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round((rng.standard_normal((n, Cout, Cin, 3, 3)) * 0.1).astype(np.float32))
    a = rng.random((B, n)).astype(np.float32) / n
    dy = inputs.bf16_round(rng.standard_normal((B, Cout, H, W), dtype=np.float32))
    say("backward wide")
    xd, ed, ad, dyd = to_dev(x, "bf16"), to_dev(e, "bf16"), to_dev(a, "f32"), to_dev(dy, "bf16")
    dx = bd.dynconv_backward_data(dyd, ed, ad, H, W, 1, 1, 1)
    da, de = bd.dynconv_backward_weights(xd, dyd, ed, ad, 1, 1, 1)
    torch.cuda.synchronize()
    rx, ra, re = oracle.backward(x, e, a, dy, 1, 1, 1)
    check(from_dev(dx), rx, TOL["bf16"], "wide dx")
    check(from_dev(da), ra, 1e-4, "wide dalpha")
    check(from_dev(de), re, 1e-4, "wide dexperts")

"""GPU parity of FMDConv's multi-attention layer (FMDConv: Fast multi-attention
dynamic convolution, abstract: input, temperature-degraded kernel and output
attention) through the C ABI against the CPU oracle.

Reading (the page gives no formula): each attention is a head of its own on
the layer input's global average pool, and
y[b,o] = a_out[b,o] * conv(a_in[b,:] * x[b], sum_i alpha[b,i] E_i)[o].
Tolerances as the other parity tests: 2e-2 normwise for bf16 layers (the
input attention is folded into the mixed kernel before its bf16 rounding),
1e-5 for float32 layers and for the attentions themselves.
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


ROUTE_CASES = [
    # B, Cin, Cout, H, W, n, mode, T
    (3, 16, 24, 8, 8, 4, 0, 1.0),
    (70, 64, 80, 14, 14, 16, 1, 4.0),   # batch of the single-kernel router size, softmax(z/4)
    (2, 40, 240, 7, 9, 8, 0, 1.0),      # odd plane, Cout 240
]


@pytest.mark.parametrize("case", ROUTE_CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_attn_matches_three_oracle_heads(case, dtype):
    B, Cin, Cout, H, W, n, mode, T = case
    rng = np.random.default_rng(41 + Cin)
    x = rng.standard_normal((B, Cin, H, W), dtype=np.float32)
    if dtype == "bf16":
        x = inputs.bf16_round(x)
    heads = [(rng.standard_normal((m, Cin), dtype=np.float32) * 0.3,
              rng.standard_normal(m, dtype=np.float32) * 0.1) for m in (n, Cin, Cout)]
    say("route_attn", case, dtype)
    a, ai, ao = bd.dynconv_route_attn(to_dev(x, dtype), Cout, *(to_dev(t, "f32") for hw in heads for t in hw),
                                      mode=mode, temperature=T)
    torch.cuda.synchronize()
    for got, (w, b), m in zip((a, ai, ao), heads, (mode, 0, 0)):
        ref, _, _ = oracle.route(x, w, b, m, T if m == 1 else 1.0)
        check(from_dev(got), ref, ALPHA_TOL, f"route_attn {case} head {w.shape[0]}")


FWD_CASES = [
    # B, Cin, Cout, H, W, k, stride, pad, groups, n, dtype -- the kernel family they reach
    (3, 40, 72, 16, 16, 3, 1, 1, 1, 4, "bf16"),     # 3x3 premix on 32x32x16 MFMA, dot2 premix
    (5, 64, 48, 12, 12, 3, 1, 1, 1, 16, "bf16"),    # matrix-core premix (16 experts)
    (3, 40, 72, 24, 20, 1, 1, 0, 1, 8, "bf16"),     # 1x1, Cin <= 64 (x resident)
    (3, 96, 40, 12, 12, 1, 1, 0, 1, 2, "bf16"),     # 1x1, persistent three-chunk path
    (2, 24, 40, 13, 13, 5, 1, 2, 1, 7, "bf16"),     # 5x5 on 16x16x32 MFMA
    (2, 16, 16, 15, 15, 3, 2, 1, 1, 2, "bf16"),     # stride 2 on 16x16x32 MFMA
    (6, 24, 24, 28, 28, 5, 1, 2, 24, 8, "bf16"),    # depthwise, matrix-core kernel
    (3, 16, 16, 14, 14, 3, 1, 1, 16, 12, "bf16"),   # depthwise, matrix-core kernel on premixed taps (n > 8)
    (4, 16, 16, 16, 16, 3, 2, 1, 16, 6, "bf16"),    # depthwise stride 2, channel-major kernel
    (3, 16, 16, 14, 14, 3, 2, 1, 16, 12, "bf16"),   # depthwise, plane-per-wave kernel (n > 8)
    (2, 8, 8, 9, 7, 3, 1, 1, 8, 3, "bf16"),         # depthwise, odd W (general kernel)
    (2, 12, 20, 9, 9, 3, 1, 1, 1, 3, "f32"),        # float32 direct
    (2, 8, 8, 10, 10, 5, 1, 2, 8, 4, "f32"),        # float32 depthwise (strip kernel)
]


def _forward_case(case, which, policy=bd.DYNCONV_POLICY_AUTO):
    B, Cin, Cout, H, W, k, st, p, g, n, dtype = case
    rng = np.random.default_rng(abs(hash(case)) % 2**32)
    x = rng.standard_normal((B, Cin, H, W), dtype=np.float32)
    e = rng.standard_normal((n, Cout, Cin // g, k, k), dtype=np.float32)
    if dtype == "bf16":
        x, e = inputs.bf16_round(x), inputs.bf16_round(e)
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    a_in = rng.uniform(0.05, 1.0, (B, Cin)).astype(np.float32) if which in ("both", "in") else None
    a_out = rng.uniform(0.05, 1.0, (B, Cout)).astype(np.float32) if which in ("both", "out") else None
    say("forward_attn", case, which, "policy", policy)
    y = bd.dynconv_forward_attn(to_dev(x, dtype), to_dev(e, dtype), to_dev(alpha, "f32"),
                                None if a_in is None else to_dev(a_in, "f32"),
                                None if a_out is None else to_dev(a_out, "f32"), st, p, g, policy=policy)
    torch.cuda.synchronize()
    ref = oracle.forward_attn(x, e, alpha, a_in, a_out, st, p, g)
    check(from_dev(y), ref, TOL[dtype], f"forward_attn {case} {which} policy {policy}")


@pytest.mark.parametrize("case", FWD_CASES)
def test_forward_attn_matches_oracle(case):
    _forward_case(case, "both")


@pytest.mark.parametrize("which", ["in", "out"])
@pytest.mark.parametrize("case", [FWD_CASES[0], FWD_CASES[2], FWD_CASES[6], FWD_CASES[11]])
def test_forward_attn_one_side(case, which):
    _forward_case(case, which)


@pytest.mark.parametrize("case", [FWD_CASES[6], FWD_CASES[7], FWD_CASES[9]])
def test_forward_attn_depthwise_premixed_taps(case):
    """Depthwise with the taps materialised first (PREMIX) scales them the same way."""
    _forward_case(case, "both", bd.DYNCONV_POLICY_PREMIX)


# Layers the small-image 3x3 fused kernel takes: the attentions ride the fused path (a_in scales the mixed
# weights before their rounding, a_out the accumulators); ragged example quads and channel tiles.
FUSED_ATTN_CASES = [
    (6, 64, 96, 14, 14, 3, 1, 1, 1, 4, "bf16"),     # ResNet-50-shaped layer, 1.5 example quads, 1.5 channel tiles
    (5, 40, 64, 10, 12, 3, 1, 1, 1, 3, "bf16"),     # 3 experts, Cin padded 40 -> 64, H != W
]


@pytest.mark.parametrize("which", ["both", "in", "out"])
@pytest.mark.parametrize("policy", [bd.DYNCONV_POLICY_FUSED, bd.DYNCONV_POLICY_AUTO])
@pytest.mark.parametrize("case", FUSED_ATTN_CASES)
def test_forward_attn_fused(case, policy, which):
    _forward_case(case, which, policy)


@pytest.mark.parametrize("case", FUSED_ATTN_CASES)
def test_fused_attention_of_ones_is_bitwise_the_plain_fused_layer(case):
    B, Cin, Cout, H, W, k, st, p, g, n, dtype = case
    rng = np.random.default_rng(11)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round(rng.standard_normal((n, Cout, Cin, k, k), dtype=np.float32))
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    xd, ed, ad = to_dev(x, dtype), to_dev(e, dtype), to_dev(alpha, "f32")
    ones_in = torch.ones((B, Cin), dtype=torch.float32, device="cuda")
    ones_out = torch.ones((B, Cout), dtype=torch.float32, device="cuda")
    say("fused attention of ones", case)
    pol = bd.DYNCONV_POLICY_FUSED
    y1 = bd.dynconv_forward_attn(xd, ed, ad, ones_in, ones_out, st, p, g, policy=pol)
    y0 = bd.dynconv_forward(xd, ed, ad, st, p, g, policy=pol)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("case", [FWD_CASES[0], FWD_CASES[1], FWD_CASES[2], FWD_CASES[6]])
def test_attention_of_ones_is_bitwise_the_plain_layer(case):
    """a_in = a_out = 1 gives exactly dynconv_forward's result on the same policy."""
    B, Cin, Cout, H, W, k, st, p, g, n, dtype = case
    rng = np.random.default_rng(7)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round(rng.standard_normal((n, Cout, Cin // g, k, k), dtype=np.float32))
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    pol = bd.DYNCONV_POLICY_PREMIX if g == 1 else bd.DYNCONV_POLICY_AUTO
    xd, ed, ad = to_dev(x, dtype), to_dev(e, dtype), to_dev(alpha, "f32")
    ones_in = torch.ones((B, Cin), dtype=torch.float32, device="cuda")
    ones_out = torch.ones((B, Cout), dtype=torch.float32, device="cuda")
    say("attention of ones", case)
    y1 = bd.dynconv_forward_attn(xd, ed, ad, ones_in, ones_out, st, p, g, policy=pol)
    y0 = bd.dynconv_forward(xd, ed, ad, st, p, g, policy=pol)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_fmdconv_resnet50_layer_full_size_sampled():
    """The ResNet-50-shaped FMDConv layer at its full batch on the fused path (AUTO resolves there); sampled
    examples against the oracle, with uniform attentions so every example differs."""
    w = inputs.WORKLOADS["fmdconv_resnet50_3x3"]
    d = inputs.make_inputs(w)
    L, e = w.layers[0], d["experts"][0]
    rng = np.random.default_rng(21)
    alpha = inputs.forced_alpha(w.B, w.n, "uniform")
    a_in = rng.uniform(0.05, 1.0, (w.B, L.Cin)).astype(np.float32)
    a_out = rng.uniform(0.05, 1.0, (w.B, L.Cout)).astype(np.float32)
    say("fmdconv resnet50 full size")
    y = bd.dynconv_forward_attn(to_dev(d["x"], "bf16"), to_dev(e, "bf16"), to_dev(alpha, "f32"),
                                to_dev(a_in, "f32"), to_dev(a_out, "f32"), L.stride, L.pad, L.groups)
    torch.cuda.synchronize()
    got = from_dev(y)
    for b in (0, 1, 130, 255):
        ref = oracle.forward_attn(d["x"][b:b + 1], e, alpha[b:b + 1], a_in[b:b + 1], a_out[b:b + 1],
                                  L.stride, L.pad, L.groups)
        check(got[b:b + 1], ref, TOL["bf16"], f"fmdconv resnet50 example {b}")

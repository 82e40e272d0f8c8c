"""Pins of the CPU oracle to things other than itself (CPU only, no GPU).

Each test fixes the oracle against a library routine, a closed form, an
invariant of the method's definition or brute force on tiny inputs, so that
a dropped term, a wrong sign or index, or a transposed operand in
``oracle/dynconv_oracle.c`` fails at least one of them:

* convolution indexing (stride, padding, groups, kh != kw): the single-expert
  case equals torch's conv2d in float64;
* the mixture of n static kernels (KernelWarehouse, abstract): one-hot attentions select one expert; the layer is linear in the
  attentions, checked against a sum of separate library convolutions;
* one kernel per example (CondConv, abstract): permuting the batch permutes the outputs; every example uses its own row of
  attentions;
* routing: closed forms (zero FC, constant planes, sigmoid symmetry, softmax
  normalisation and shift invariance, large temperature) and a hand-worked
  example;
* a hand-worked convolution with an asymmetric kernel (catches a kernel flip).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _torch_conv(x, w, stride, pad, groups):
    return F.conv2d(torch.from_numpy(np.asarray(x, np.float64)),
                    torch.from_numpy(np.asarray(w, np.float64)),
                    stride=stride, padding=pad, groups=groups).numpy()


CONV_CASES = [
    # B, Cin, Cout, H, W, kh, kw, stride, pad, groups
    (2, 3, 4, 5, 6, 3, 3, 1, 1, 1),
    (1, 4, 6, 7, 5, 3, 3, 2, 1, 1),
    (2, 4, 4, 6, 6, 5, 5, 1, 2, 4),     # depthwise
    (1, 6, 4, 5, 5, 1, 1, 1, 0, 2),     # grouped 1x1
    (2, 2, 3, 6, 4, 3, 1, 1, 1, 1),     # kh != kw
    (1, 3, 2, 4, 4, 3, 3, 1, 0, 1),     # no padding
    (1, 2, 2, 3, 3, 3, 3, 3, 2, 1),     # stride larger than kernel reach
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_single_expert_equals_static_conv(case):
    """n = 1, alpha = 1: the dynamic layer is an ordinary convolution."""
    B, Cin, Cout, H, W, kh, kw, st, p, g = case
    x = _rand((B, Cin, H, W), 1)
    e = _rand((1, Cout, Cin // g, kh, kw), 2)
    alpha = np.ones((B, 1))
    got = oracle.forward(x, e, alpha, stride=st, pad=p, groups=g)
    ref = _torch_conv(x, e[0], st, p, g)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_with_given_kernels_matches_torch_per_example(case):
    B, Cin, Cout, H, W, kh, kw, st, p, g = case
    x = _rand((B, Cin, H, W), 3)
    wb = _rand((B, Cout, Cin // g, kh, kw), 4).astype(np.float64)
    got = oracle.conv(x, wb, stride=st, pad=p, groups=g)
    for b in range(B):
        ref = _torch_conv(x[b:b + 1], wb[b], st, p, g)
        np.testing.assert_allclose(got[b:b + 1], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CONV_CASES)
def test_linearity_in_attentions(case):
    """conv(x_b, sum_i a_bi E_i) == sum_i a_bi conv(x_b, E_i), brute force."""
    B, Cin, Cout, H, W, kh, kw, st, p, g = case
    n = 3
    x = _rand((B, Cin, H, W), 5)
    e = _rand((n, Cout, Cin // g, kh, kw), 6)
    alpha = np.random.default_rng(7).uniform(-1.5, 1.5, (B, n))
    got = oracle.forward(x, e, alpha, stride=st, pad=p, groups=g)
    ref = np.zeros_like(got)
    for b in range(B):
        for i in range(n):
            ref[b] += alpha[b, i] * _torch_conv(x[b:b + 1], e[i], st, p, g)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_one_hot_selects_each_expert():
    n, B = 4, 5
    x = _rand((B, 3, 6, 6), 8)
    e = _rand((n, 5, 3, 3, 3), 9)
    alpha = np.zeros((B, n))
    alpha[np.arange(B), np.arange(B) % n] = 1.0
    got = oracle.forward(x, e, alpha, stride=1, pad=1)
    for b in range(B):
        ref = _torch_conv(x[b:b + 1], e[b % n], 1, 1, 1)
        np.testing.assert_allclose(got[b:b + 1], ref, rtol=1e-12, atol=1e-12)
    mixed = oracle.mix(alpha, e)
    for b in range(B):
        np.testing.assert_array_equal(mixed[b], e[b % n].astype(np.float64))


def test_mix_identities():
    """Scaled one-hot, sum of experts, linearity in alpha, expert permutation."""
    n, B = 5, 3
    e = _rand((n, 4, 2, 3, 3), 10)
    m = oracle.mix(np.full((B, n), 1.0), e)
    np.testing.assert_allclose(m[1], e.astype(np.float64).sum(0), rtol=1e-13, atol=1e-13)
    a1 = np.random.default_rng(11).uniform(-1, 1, (B, n))
    a2 = np.random.default_rng(12).uniform(-1, 1, (B, n))
    lhs = oracle.mix(0.75 * a1 - 2.0 * a2, e)
    rhs = 0.75 * oracle.mix(a1, e) - 2.0 * oracle.mix(a2, e)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    perm = np.array([3, 0, 4, 1, 2])
    np.testing.assert_allclose(oracle.mix(a1[:, perm], e[perm]), oracle.mix(a1, e),
                               rtol=1e-13, atol=1e-13)
    for j in range(n):
        a = np.zeros((B, n))
        a[:, j] = -2.5
        np.testing.assert_array_equal(oracle.mix(a, e)[2], -2.5 * e[j].astype(np.float64))


def test_each_example_uses_its_own_attention_row():
    """alpha rows differ per example; B != n so a swapped index shows."""
    B, n = 3, 2
    x = _rand((B, 2, 4, 4), 13)
    e = _rand((n, 3, 2, 3, 3), 14)
    alpha = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, -2.0]])
    got = oracle.forward(x, e, alpha, stride=1, pad=1)
    for b in range(B):
        w = alpha[b, 0] * e[0].astype(np.float64) + alpha[b, 1] * e[1].astype(np.float64)
        np.testing.assert_allclose(got[b:b + 1], _torch_conv(x[b:b + 1], w, 1, 1, 1),
                                   rtol=1e-12, atol=1e-12)


def test_batch_permutation_permutes_outputs():
    B, n = 6, 3
    x = _rand((B, 4, 5, 5), 15)
    e = _rand((n, 3, 4, 3, 3), 16)
    fc_w = _rand((n, 4), 17)
    fc_b = _rand((n,), 18)
    alpha, _, _ = oracle.route(x, fc_w, fc_b, oracle.SIGMOID)
    y = oracle.forward(x, e, alpha, stride=1, pad=1)
    perm = np.random.default_rng(19).permutation(B)
    alpha_p, _, _ = oracle.route(x[perm], fc_w, fc_b, oracle.SIGMOID)
    np.testing.assert_array_equal(alpha_p, alpha[perm])
    y_p = oracle.forward(x[perm], e, alpha_p, stride=1, pad=1)
    np.testing.assert_array_equal(y_p, y[perm])


def test_hand_worked_convolution():
    """A 3x3 image, experts: centre tap, 3x3 box, right-neighbour tap.

    x = [[1,2,3],[4,5,6],[7,8,9]], alpha = (2, 0.5, -1), pad 1, stride 1:
    y = 2*x + 0.5*boxsum(x) - x[h, w+1]. Box sums with zero padding are
    [[12,21,16],[27,45,33],[24,39,28]]; right neighbours are
    [[2,3,0],[5,6,0],[8,9,0]]. A flipped kernel would pick the left
    neighbour instead and fail.
    """
    x = np.arange(1, 10, dtype=np.float32).reshape(1, 1, 3, 3)
    e = np.zeros((3, 1, 1, 3, 3), np.float32)
    e[0, 0, 0, 1, 1] = 1.0
    e[1] = 1.0
    e[2, 0, 0, 1, 2] = 1.0
    alpha = np.array([[2.0, 0.5, -1.0]])
    y = oracle.forward(x, e, alpha, stride=1, pad=1)
    expect = np.array([[6.0, 11.5, 14.0], [16.5, 26.5, 28.5], [18.0, 26.5, 32.0]])
    np.testing.assert_array_equal(y[0, 0], expect)
    y2 = oracle.forward(x, e, alpha, stride=2, pad=1)
    np.testing.assert_array_equal(y2[0, 0], np.array([[6.0, 14.0], [18.0, 32.0]]))


def test_route_hand_worked():
    """gap = (1, -2) from constant planes; z = (-0.75, 0.5)."""
    x = np.empty((1, 2, 3, 4), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -2.0
    fc_w = np.array([[1.0, 1.0], [0.5, 0.0]], np.float32)
    fc_b = np.array([0.25, 0.0], np.float32)
    a, g, z = oracle.route(x, fc_w, fc_b, oracle.SIGMOID)
    np.testing.assert_array_equal(g, [[1.0, -2.0]])
    np.testing.assert_array_equal(z, [[-0.75, 0.5]])
    np.testing.assert_allclose(a, [[1.0 / (1.0 + math.exp(0.75)), 1.0 / (1.0 + math.exp(-0.5))]],
                               rtol=1e-15)
    a, _, _ = oracle.route(x, fc_w, fc_b, oracle.SOFTMAX, 2.0)
    # softmax of z/2 = (-0.375, 0.25): first = 1 / (1 + e^0.625)
    p0 = 1.0 / (1.0 + math.exp(0.625))
    np.testing.assert_allclose(a, [[p0, 1.0 - p0]], rtol=1e-15)


def test_route_closed_forms():
    B, C, n = 4, 6, 5
    x = _rand((B, C, 5, 7), 20)
    zero_w = np.zeros((n, C), np.float32)
    a, _, _ = oracle.route(x, zero_w, None, oracle.SIGMOID)
    np.testing.assert_array_equal(a, np.full((B, n), 0.5))
    a, _, _ = oracle.route(x, zero_w, np.zeros(n, np.float32), oracle.SOFTMAX, 4.0)
    np.testing.assert_allclose(a, np.full((B, n), 1.0 / n), rtol=1e-15)
    fc_w = _rand((n, C), 21)
    # dyadic biases, so that adding 3 below is exact in float32
    fc_b = (np.round(_rand((n,), 22) * 1024) / 1024).astype(np.float32)
    # sigmoid symmetry: negating the FC maps alpha to 1 - alpha
    a1, _, z1 = oracle.route(x, fc_w, fc_b, oracle.SIGMOID)
    a2, _, z2 = oracle.route(x, -fc_w, -fc_b, oracle.SIGMOID)
    np.testing.assert_allclose(z2, -z1, rtol=0, atol=0)
    np.testing.assert_allclose(a1 + a2, 1.0, rtol=1e-15)
    # softmax: rows sum to 1, invariant to a shared shift of the logits
    s1, _, _ = oracle.route(x, fc_w, fc_b, oracle.SOFTMAX, 4.0)
    np.testing.assert_allclose(s1.sum(1), 1.0, rtol=1e-14)
    s2, _, _ = oracle.route(x, fc_w, fc_b + np.float32(3.0), oracle.SOFTMAX, 4.0)
    np.testing.assert_allclose(s2, s1, rtol=1e-13)
    # large temperature -> uniform
    s3, _, _ = oracle.route(x, fc_w, fc_b, oracle.SOFTMAX, 1e9)
    np.testing.assert_allclose(s3, 1.0 / n, rtol=1e-8)
    # large logits do not overflow the sigmoid
    a4, _, _ = oracle.route(x, fc_w * np.float32(1e4), None, oracle.SIGMOID)
    assert np.all(np.isfinite(a4)) and np.all((a4 >= 0) & (a4 <= 1))


def test_route_matches_library_ops():
    """GAP / FC / sigmoid and softmax(z/T) via torch's own routines in float64."""
    B, C, n = 3, 7, 4
    x = _rand((B, C, 6, 5), 23)
    fc_w = _rand((n, C), 24)
    fc_b = _rand((n,), 25)
    xt = torch.from_numpy(x.astype(np.float64))
    z = F.linear(F.adaptive_avg_pool2d(xt, 1).flatten(1),
                 torch.from_numpy(fc_w.astype(np.float64)),
                 torch.from_numpy(fc_b.astype(np.float64)))
    a, g, zz = oracle.route(x, fc_w, fc_b, oracle.SIGMOID)
    np.testing.assert_allclose(g, F.adaptive_avg_pool2d(xt, 1).flatten(1).numpy(), rtol=1e-13)
    np.testing.assert_allclose(zz, z.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a, torch.sigmoid(z).numpy(), rtol=1e-13)
    s, _, _ = oracle.route(x, fc_w, fc_b, oracle.SOFTMAX, 4.0)
    np.testing.assert_allclose(s, torch.softmax(z / 4.0, dim=1).numpy(), rtol=1e-13)


def test_gap_of_constant_planes():
    x = np.empty((2, 3, 4, 5), np.float32)
    vals = np.array([[1.5, -2.0, 0.25], [7.0, 0.0, -0.125]], np.float32)
    x[:] = vals[:, :, None, None]
    np.testing.assert_array_equal(oracle.gap(x), vals.astype(np.float64))


def test_forward_points_match_full_forward():
    B, n = 2, 3
    x = _rand((B, 4, 6, 6), 26)
    e = _rand((n, 5, 4, 3, 3), 27)
    alpha = np.random.default_rng(28).uniform(0, 1, (B, n))
    y = oracle.forward(x, e, alpha, stride=1, pad=1)
    rng = np.random.default_rng(29)
    idx = np.stack([rng.integers(0, s, 40) for s in y.shape], axis=1)
    pts = oracle.forward_points(x, e, alpha, idx, stride=1, pad=1)
    np.testing.assert_allclose(pts, y[tuple(idx.T)], rtol=1e-13, atol=1e-13)


def test_invalid_arguments_rejected():
    x = _rand((1, 3, 4, 4), 30)
    e = _rand((2, 4, 3, 3, 3), 31)
    with pytest.raises(ValueError):
        oracle.forward(x, e, np.ones((1, 2)), stride=0, pad=1)
    with pytest.raises(ValueError):
        oracle.forward(x, e, np.ones((1, 2)), stride=1, pad=-1)
    with pytest.raises(ValueError):
        oracle.route(x, np.ones((2, 3), np.float32), None, oracle.SOFTMAX, 0.0)


# ------------------------------------------------ FMDConv input / output attention
ATTN_CASES = [
    # B, Cin, Cout, H, W, k, stride, pad, groups, n
    (2, 6, 5, 7, 6, 3, 1, 1, 1, 3),
    (3, 4, 4, 6, 6, 5, 2, 2, 4, 2),   # depthwise
    (2, 8, 3, 5, 5, 1, 1, 0, 1, 1),   # 1x1
]


@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_of_ones_is_the_plain_layer(case):
    B, Cin, Cout, H, W, k, st, p, g, n = case
    rng = np.random.default_rng(31)
    x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
    e = rng.standard_normal((n, Cout, Cin // g, k, k)).astype(np.float32)
    alpha = rng.uniform(0, 1, (B, n))
    ones_in, ones_out = np.ones((B, Cin)), np.ones((B, Cout))
    ref = oracle.forward(x, e, alpha, st, p, g)
    np.testing.assert_allclose(oracle.forward_attn(x, e, alpha, ones_in, ones_out, st, p, g), ref,
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.forward_attn(x, e, alpha, None, None, st, p, g), ref,
                               rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("case", ATTN_CASES)
def test_output_attention_scales_output_channels(case):
    """a_out[b, o] multiplies output channel o of example b (and nothing else)."""
    B, Cin, Cout, H, W, k, st, p, g, n = case
    rng = np.random.default_rng(32)
    x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
    e = rng.standard_normal((n, Cout, Cin // g, k, k)).astype(np.float32)
    alpha = rng.uniform(0, 1, (B, n))
    a_out = rng.uniform(0.1, 1.0, (B, Cout))
    got = oracle.forward_attn(x, e, alpha, None, a_out, st, p, g)
    ref = oracle.forward(x, e, alpha, st, p, g) * a_out[:, :, None, None]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", ATTN_CASES)
def test_input_attention_scales_input_channels(case):
    """a_in[b, c] acts as a scale of input channel c of example b: the layer of
    the scaled input (power-of-two scales, so x * a_in is exact in float32)."""
    B, Cin, Cout, H, W, k, st, p, g, n = case
    rng = np.random.default_rng(33)
    x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
    e = rng.standard_normal((n, Cout, Cin // g, k, k)).astype(np.float32)
    alpha = rng.uniform(0, 1, (B, n))
    a_in = 2.0 ** rng.integers(-3, 2, (B, Cin))   # 1/8 .. 2: exact scaling
    got = oracle.forward_attn(x, e, alpha, a_in, None, st, p, g)
    xs = (x.astype(np.float64) * a_in[:, :, None, None]).astype(np.float32)
    np.testing.assert_allclose(got, oracle.forward(xs, e, alpha, st, p, g), rtol=1e-12, atol=1e-12)


def test_attention_layer_matches_torch_conv2d():
    """One expert with attention 1: a_out * conv2d(a_in * x, E_0) in float64 torch."""
    rng = np.random.default_rng(34)
    for (B, Cin, Cout, H, W, k, st, p, g, _) in ATTN_CASES:
        x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
        e = rng.standard_normal((1, Cout, Cin // g, k, k)).astype(np.float32)
        a_in = rng.uniform(0.1, 1.0, (B, Cin))
        a_out = rng.uniform(0.1, 1.0, (B, Cout))
        got = oracle.forward_attn(x, e, np.ones((B, 1)), a_in, a_out, st, p, g)
        xt = torch.from_numpy(x.astype(np.float64)) * torch.from_numpy(a_in)[:, :, None, None]
        ref = F.conv2d(xt, torch.from_numpy(e[0].astype(np.float64)), stride=st, padding=p, groups=g)
        ref = (ref * torch.from_numpy(a_out)[:, :, None, None]).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("n", [101, 128])
def test_many_experts_one_hot_and_linearity(n):
    """KernelWarehouse's n > 100 (KernelWarehouse, abstract): with one-hot
    attentions the layer equals one expert's ordinary convolution (torch conv2d
    in float64); and the layer is linear in the attentions across the whole bank."""
    B, Cin, Cout, H, W = 2, 3, 4, 5, 6
    x = _rand((B, Cin, H, W), 31)
    e = _rand((n, Cout, Cin, 3, 3), 32)
    for k in (0, n // 2, n - 1):
        a = np.zeros((B, n))
        a[:, k] = 1.0
        y = oracle.forward(x, e, a, 1, 1, 1)
        np.testing.assert_allclose(y, _torch_conv(x, e[k], 1, 1, 1), rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(33)
    a1, a2 = rng.random((B, n)), rng.random((B, n))
    y12 = oracle.forward(x, e, a1 + a2, 1, 1, 1)
    y1, y2 = oracle.forward(x, e, a1, 1, 1, 1), oracle.forward(x, e, a2, 1, 1, 1)
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-11, atol=1e-11)
    m = oracle.mix(a1, e)
    np.testing.assert_allclose(oracle.mix(a1 + a2, e), m + oracle.mix(a2, e), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("residual", [False, True])
def test_sparse_evaluation_special_cases(residual):
    """Gated evaluation (Dynamic Convolutions: Exploiting Spatial Sparsity for
    Faster Inference, abstract): an all-ones gate is the dense layer (plus the
    residual), an all-zero gate leaves only the residual; and each output is
    either the dense layer's value at that position or the residual alone."""
    B, C, H, W, n = 2, 4, 6, 5, 3
    x = _rand((B, C, H, W), 41)
    e = _rand((n, C, C, 3, 3), 42)
    a = np.random.default_rng(43).random((B, n))
    dense = _torch_conv(x[0:1], np.einsum("i,i...->...", a[0], e.astype(np.float64)), 1, 1, 1)
    ones = np.ones((B, H, W), np.uint8)
    zeros = np.zeros((B, H, W), np.uint8)
    res = x.astype(np.float64) if residual else 0.0
    y1 = oracle.forward_sparse(x, e, a, ones, 1, 1, 1, residual)
    np.testing.assert_allclose(y1[0:1], dense + (res[0:1] if residual else 0.0), rtol=1e-12, atol=1e-12)
    y0 = oracle.forward_sparse(x, e, a, zeros, 1, 1, 1, residual)
    np.testing.assert_array_equal(y0, np.zeros_like(y0) + res)
    m = (np.random.default_rng(44).random((B, H, W)) < 0.4).astype(np.uint8)
    ym = oracle.forward_sparse(x, e, a, m, 1, 1, 1, residual)
    full = oracle.forward(x, e, a, 1, 1, 1) + res
    on = np.broadcast_to(m[:, None] != 0, ym.shape)
    np.testing.assert_array_equal(ym[on], full[on])
    np.testing.assert_array_equal(ym[~on], (np.zeros_like(ym) + res)[~on])

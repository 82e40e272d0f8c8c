"""Pins of the oracle's gradients (CPU only, no GPU).

The pages train dynamic convolutions end to end but print no backward pass.
The oracle's ``backward`` and ``route_backward`` write out the derivative of
the forward definition. These tests fix them against things other than
themselves, so that a dropped term, a wrong sign or index, or a transposed
operand fails at least one test:

* torch autograd in float64 through a layer built from library routines
  (einsum mixing and ``conv2d`` per example), and through the routing
  (mean, linear map, sigmoid or softmax(z/T));
* brute force on tiny inputs: the layer is linear in x, in alpha and in
  each expert, so every gradient entry equals <dy, forward(unit input)>;
* Euler's identity for the bilinear layer:
  <dy, y> = <dx, x> = <dalpha, alpha> = <dE, E>;
* closed forms of the routing derivative (sigmoid at zero logits, softmax
  gradients that sum to zero, a constant attention gradient under softmax);
* for the layer with FMDConv's channel attentions (``backward_attn``): torch
  autograd through x * a_in, the mixed kernels, ``conv2d`` and * a_out,
  Euler's identity over all five gradients (the layer is linear in each of
  x, alpha, E, a_in and a_out), and the plain ``backward`` when both
  attentions are ones.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


BWD_CASES = [
    # B, Cin, Cout, H, W, kh, kw, stride, pad, groups, n
    (2, 3, 4, 5, 6, 3, 3, 1, 1, 1, 3),
    (2, 4, 6, 7, 5, 3, 3, 2, 1, 1, 2),
    (3, 4, 4, 6, 6, 5, 5, 1, 2, 4, 4),     # depthwise
    (2, 6, 4, 5, 5, 1, 1, 1, 0, 2, 2),     # grouped 1x1
    (2, 2, 3, 6, 4, 3, 1, 1, 1, 1, 2),     # kh != kw
    (1, 3, 2, 4, 4, 3, 3, 1, 0, 1, 3),     # no padding
    (2, 5, 3, 9, 7, 1, 1, 1, 0, 1, 4),     # 1x1
]


def _inputs(case, seed=0):
    B, Cin, Cout, H, W, kh, kw, st, p, g, n = case
    Ho, Wo = oracle.out_size(H, kh, st, p), oracle.out_size(W, kw, st, p)
    x = _rand((B, Cin, H, W), seed + 1)
    e = _rand((n, Cout, Cin // g, kh, kw), seed + 2)
    a = np.random.default_rng(seed + 3).random((B, n)) + 0.25
    dy = _rand((B, Cout, Ho, Wo), seed + 4)
    return x, e, a, dy


def _torch_grads(x, e, a, dy, st, p, g):
    """Reference gradients from torch autograd in float64 on the CPU."""
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    et = torch.tensor(np.asarray(e, np.float64), requires_grad=True)
    at = torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    wb = torch.einsum("bi,i...->b...", at, et)
    ys = [F.conv2d(xt[b:b + 1], wb[b], stride=st, padding=p, groups=g) for b in range(x.shape[0])]
    loss = (torch.cat(ys) * torch.from_numpy(np.asarray(dy, np.float64))).sum()
    loss.backward()
    return xt.grad.numpy(), at.grad.numpy(), et.grad.numpy()


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_matches_torch_autograd(case):
    *_, st, p, g, n = case
    x, e, a, dy = _inputs(case)
    dx, da, de = oracle.backward(x, e, a, dy, st, p, g)
    rx, ra, re = _torch_grads(x, e, a, dy, st, p, g)
    assert _rel(dx, rx) < 1e-12
    assert _rel(da, ra) < 1e-12
    assert _rel(de, re) < 1e-12


@pytest.mark.parametrize("case", BWD_CASES[:3])
def test_backward_brute_force_unit_inputs(case):
    """Each gradient entry is <dy, forward(...)> with one input set to a unit
    impulse, because the layer is linear in x, in alpha and in each expert."""
    B, Cin, Cout, H, W, kh, kw, st, p, g, n = case
    x, e, a, dy = _inputs(case, seed=10)
    dx, da, de = oracle.backward(x, e, a, dy, st, p, g)
    dyd = dy.astype(np.float64)
    # dx: unit impulses in x
    bx = np.empty_like(dx)
    for j in range(x.size):
        u = np.zeros(x.size, np.float32)
        u[j] = 1.0
        bx.flat[j] = np.sum(dyd * oracle.forward(u.reshape(x.shape), e, a, st, p, g))
    assert _rel(dx, bx) < 1e-12
    # dalpha: one-hot attentions
    ba = np.empty_like(da)
    for i in range(n):
        oh = np.zeros_like(a)
        oh[:, i] = 1.0
        yi = oracle.forward(x, e, oh, st, p, g)
        ba[:, i] = np.sum(dyd * yi, axis=(1, 2, 3))
    assert _rel(da, ba) < 1e-12
    # dexperts: unit impulses in the bank
    be = np.empty_like(de)
    for j in range(e.size):
        u = np.zeros(e.size, np.float32)
        u[j] = 1.0
        be.flat[j] = np.sum(dyd * oracle.forward(x, u.reshape(e.shape), a, st, p, g))
    assert _rel(de, be) < 1e-12


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_euler_identity(case):
    *_, st, p, g, n = case
    x, e, a, dy = _inputs(case, seed=20)
    dx, da, de = oracle.backward(x, e, a, dy, st, p, g)
    y = oracle.forward(x, e, a, st, p, g)
    ref = float(np.sum(dy.astype(np.float64) * y))
    scale = float(np.sum(np.abs(dy.astype(np.float64) * y)))
    for v in (np.sum(dx * x), np.sum(da * a), np.sum(de * e)):
        assert abs(float(v) - ref) <= 1e-12 * scale


def test_backward_partial_outputs_agree():
    case = BWD_CASES[0]
    *_, st, p, g, n = case
    x, e, a, dy = _inputs(case)
    full = oracle.backward(x, e, a, dy, st, p, g)
    only_da = oracle.backward(x, e, a, dy, st, p, g, want=("dalpha",))
    assert only_da[0] is None and only_da[2] is None
    np.testing.assert_array_equal(only_da[1], full[1])


ROUTE_CASES = [
    # B, C, H, W, n, mode, T
    (3, 5, 4, 6, 4, oracle.SIGMOID, 1.0),
    (2, 7, 3, 3, 6, oracle.SOFTMAX, 4.0),
    (4, 3, 5, 2, 3, oracle.SOFTMAX, 0.5),
]


def _route_inputs(case, seed=0):
    B, C, H, W, n, mode, T = case
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C, H, W)).astype(np.float32)
    fw = (rng.standard_normal((n, C)) * 0.7).astype(np.float32)
    fb = (rng.standard_normal(n) * 0.3).astype(np.float32)
    da = rng.standard_normal((B, n))
    return x, fw, fb, da


@pytest.mark.parametrize("case", ROUTE_CASES)
def test_route_backward_matches_torch_autograd(case):
    B, C, H, W, n, mode, T = case
    x, fw, fb, da = _route_inputs(case)
    dfw, dfb, dgap, dx = oracle.route_backward(x, fw, fb, da, mode, T)
    xt = torch.tensor(x.astype(np.float64), requires_grad=True)
    wt = torch.tensor(fw.astype(np.float64), requires_grad=True)
    bt = torch.tensor(fb.astype(np.float64), requires_grad=True)
    z = xt.mean(dim=(2, 3)) @ wt.T + bt
    alpha = torch.sigmoid(z) if mode == oracle.SIGMOID else torch.softmax(z / T, dim=1)
    (alpha * torch.from_numpy(da)).sum().backward()
    assert _rel(dfw, wt.grad.numpy()) < 1e-12
    assert _rel(dfb, bt.grad.numpy()) < 1e-12
    assert _rel(dx, xt.grad.numpy()) < 1e-12
    assert dgap.shape == (B, C)


def test_route_backward_closed_forms():
    B, C, H, W, n = 2, 4, 3, 3, 5
    x = _rand((B, C, H, W), 5)
    da = np.random.default_rng(6).standard_normal((B, n))
    zero_w = np.zeros((n, C), np.float32)
    # sigmoid at zero logits: alpha = 1/2, so dz = dalpha / 4
    _, dfb, _, _ = oracle.route_backward(x, zero_w, None, da, oracle.SIGMOID)
    np.testing.assert_allclose(dfb, da.sum(axis=0) / 4.0, rtol=0, atol=1e-15)
    # softmax: the logit gradients of each example sum to zero (shift invariance)
    fw = _rand((n, C), 7)
    dfw, dfb, _, _ = oracle.route_backward(x, fw, None, da, oracle.SOFTMAX, 2.0)
    assert abs(dfb.sum()) < 1e-14
    # softmax with zero FC: alpha = 1/n, dz_j = (dalpha_j - mean(dalpha)) / (n T)
    _, dfb, _, _ = oracle.route_backward(x, zero_w, None, da, oracle.SOFTMAX, 2.0)
    ref = ((da - da.mean(axis=1, keepdims=True)) / (n * 2.0)).sum(axis=0)
    np.testing.assert_allclose(dfb, ref, rtol=0, atol=1e-15)
    # a constant attention gradient changes nothing under softmax
    const = np.full((B, n), 3.0)
    dfw, dfb, dgap, dx = oracle.route_backward(x, fw, None, const, oracle.SOFTMAX, 2.0)
    for v in (dfw, dfb, dgap, dx):
        assert np.max(np.abs(v)) < 1e-14


# ---- FMDConv channel attentions -------------------------------------------------

def _attn_inputs(case, seed=0):
    B, Cin, Cout = case[0], case[1], case[2]
    x, e, a, dy = _inputs(case, seed)
    rng = np.random.default_rng(seed + 5)
    return x, e, a, dy, rng.random((B, Cin)) + 0.5, rng.random((B, Cout)) + 0.5


def _torch_attn_grads(x, e, a, dy, ai, ao, st, p, g):
    """Reference gradients of <dy, a_out * conv(a_in * x, W_b)> from torch
    autograd in float64 on the CPU."""
    f64 = lambda v: torch.tensor(np.asarray(v, np.float64), requires_grad=True)
    xt, et, at, it, ot = f64(x), f64(e), f64(a), f64(ai), f64(ao)
    wb = torch.einsum("bi,i...->b...", at, et)
    xs = xt * it[:, :, None, None]
    ys = [F.conv2d(xs[b:b + 1], wb[b], stride=st, padding=p, groups=g) for b in range(x.shape[0])]
    y = torch.cat(ys) * ot[:, :, None, None]
    (y * torch.from_numpy(np.asarray(dy, np.float64))).sum().backward()
    return xt.grad.numpy(), at.grad.numpy(), et.grad.numpy(), it.grad.numpy(), ot.grad.numpy()


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_attn_matches_torch_autograd(case):
    *_, st, p, g, n = case
    x, e, a, dy, ai, ao = _attn_inputs(case, seed=30)
    got = oracle.backward_attn(x, e, a, dy, ai, ao, st, p, g)
    ref = _torch_attn_grads(x, e, a, dy, ai, ao, st, p, g)
    for name, v, r in zip(("dx", "dalpha", "dexperts", "da_in", "da_out"), got, ref):
        assert _rel(v, r) < 1e-12, name


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_attn_euler_identity(case):
    *_, st, p, g, n = case
    x, e, a, dy, ai, ao = _attn_inputs(case, seed=40)
    dx, da, de, dai, dao = oracle.backward_attn(x, e, a, dy, ai, ao, st, p, g)
    y = oracle.forward_attn(x, e, a, ai, ao, st, p, g)
    ref = float(np.sum(dy.astype(np.float64) * y))
    scale = float(np.sum(np.abs(dy.astype(np.float64) * y)))
    for v in (np.sum(dx * x), np.sum(da * a), np.sum(de * e), np.sum(dai * ai), np.sum(dao * ao)):
        assert abs(float(v) - ref) <= 1e-12 * scale


@pytest.mark.parametrize("case", BWD_CASES[:4])
def test_backward_attn_with_unit_attentions_is_backward(case):
    *_, st, p, g, n = case
    B, Cin, Cout = case[0], case[1], case[2]
    x, e, a, dy = _inputs(case, seed=50)
    plain = oracle.backward(x, e, a, dy, st, p, g)
    none = oracle.backward_attn(x, e, a, dy, None, None, st, p, g)
    ones = oracle.backward_attn(x, e, a, dy, np.ones((B, Cin)), np.ones((B, Cout)), st, p, g)
    for u, v, w in zip(plain, none[:3], ones[:3]):
        assert np.array_equal(u, v) and np.array_equal(u, w)
    assert np.array_equal(none[3], ones[3]) and np.array_equal(none[4], ones[4])
    # with unit attentions, da_out[b,o] is <dy, y> over channel o
    y = oracle.forward(x, e, a, st, p, g)
    assert _rel(none[4], np.sum(dy.astype(np.float64) * y, axis=(2, 3))) < 1e-12

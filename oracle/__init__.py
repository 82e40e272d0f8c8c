"""CPU oracle for CondConv-style dynamic convolution (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package
imports nothing from the product.

The arithmetic lives in ``dynconv_oracle.c`` (plain C, double precision,
OpenMP over independent outputs). This module only builds that file with the
host compiler, loads it with ctypes and marshals numpy arrays. Each function
cites the passage of the pages it follows:

* routing - global average pool, FC with bias, sigmoid or softmax(z/T):
  attentions that depend on the input (KernelWarehouse: Rethinking the Design
  of Dynamic Convolution, abstract) and a kernel attention whose temperature
  is lowered over training (FMDConv: Fast multi-attention dynamic
  convolution, abstract). The pages
  give no formula for the router; the plainest reading is used.
* mixing - W_b = sum_i alpha_bi E_i: each example's kernel is a weighted sum
  of n static kernels, the weights being its attentions (KernelWarehouse,
  abstract).
* convolution - one ordinary convolution per example with its own kernel
  (CondConv: Conditionally Parameterized Convolutions, abstract).
* input and output attention - FMDConv's per-channel scales of the layer's
  input and output (FMDConv: Fast multi-attention dynamic convolution,
  abstract, which names them without a formula; the reading is stated at
  ``forward_attn``). Each head is a route (GAP -> FC -> sigmoid) of its own.
* spatially sparse evaluation - a small learned gate picks the output
  positions a residual block computes, executed by gathering and scattering
  those positions (Dynamic Convolutions: Exploiting Spatial Sparsity for
  Faster Inference, abstract). ``forward_sparse`` takes the gate as a
  given mask: the layer's output at the masked positions only, plus the
  block's input when the block is residual.
* gradients - the pages train these layers end to end (CondConv abstract;
  KernelWarehouse abstract) but print no backward pass. ``backward`` and
  ``route_backward`` write out the derivative of the forward definition.

Parity pins live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dynconv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

SIGMOID = 0
SOFTMAX = 1


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (gcc, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and (
        os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)
    ):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    i64 = ctypes.c_long
    lib.oracle_threads.restype = i32
    lib.oracle_gap.argtypes = [i32, i32, i32, i32, P, P]
    lib.oracle_route.argtypes = [i32, i32, i32, i32, i32, P, P, P, i32,
                                 ctypes.c_double, P, P, P]
    lib.oracle_mix.argtypes = [i32, i32, i64, P, P, P]
    lib.oracle_conv.argtypes = [i32] * 10 + [P, P, P]
    lib.oracle_forward.argtypes = [i32] * 11 + [P, P, P, P]
    lib.oracle_forward_points.argtypes = [i32] * 11 + [P, P, P, i64, P, P]
    lib.oracle_forward_attn.argtypes = [i32] * 11 + [P, P, P, P, P, P]
    lib.oracle_backward.argtypes = [i32] * 11 + [P, P, P, P, P, P, P]
    lib.oracle_backward_attn.argtypes = [i32] * 11 + [P] * 11
    for f in (lib.oracle_gap, lib.oracle_route, lib.oracle_mix, lib.oracle_conv,
              lib.oracle_forward, lib.oracle_forward_points, lib.oracle_forward_attn,
              lib.oracle_backward, lib.oracle_backward_attn):
        f.restype = i32
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_threads())


def out_size(n: int, k: int, stride: int, pad: int) -> int:
    if stride < 1 or pad < 0:
        raise ValueError("oracle: stride must be >= 1 and pad >= 0")
    return (n + 2 * pad - k) // stride + 1


def gap(x) -> np.ndarray:
    """Global average pool over H, W of x[B, C, H, W] (float64 result)."""
    x = _f32(x)
    B, C, H, W = x.shape
    out = np.empty((B, C), np.float64)
    _check(_load().oracle_gap(B, C, H, W, _ptr(x), _ptr(out)), "gap")
    return out


def route(x, fc_w, fc_b=None, mode: int = SIGMOID, temperature: float = 1.0):
    """Attentions alpha[B, n] from GAP -> FC(+bias) -> sigmoid | softmax(z/T).

    Returns (alpha, gap, z), all float64.
    """
    x = _f32(x)
    fc_w = _f32(fc_w)
    B, C, H, W = x.shape
    n = fc_w.shape[0]
    assert fc_w.shape == (n, C)
    fb = None if fc_b is None else _f32(fc_b)
    if fb is not None:
        assert fb.shape == (n,)
    alpha = np.empty((B, n), np.float64)
    g = np.empty((B, C), np.float64)
    z = np.empty((B, n), np.float64)
    rc = _load().oracle_route(B, C, H, W, n, _ptr(x), _ptr(fc_w),
                              None if fb is None else _ptr(fb), int(mode),
                              float(temperature), _ptr(g), _ptr(z), _ptr(alpha))
    _check(rc, "route")
    return alpha, g, z


def mix(alpha, experts) -> np.ndarray:
    """W_b = sum_i alpha[b, i] * E_i for experts[n, ...]; result [B, ...] float64."""
    alpha = _f64(alpha)
    experts = _f32(experts)
    B, n = alpha.shape
    assert experts.shape[0] == n
    wsize = int(np.prod(experts.shape[1:]))
    out = np.empty((B,) + experts.shape[1:], np.float64)
    _check(_load().oracle_mix(B, n, wsize, _ptr(alpha), _ptr(experts), _ptr(out)), "mix")
    return out


def conv(x, wb, stride: int = 1, pad: int = 0, groups: int = 1) -> np.ndarray:
    """Per-example convolution of x[B, Cin, H, W] with wb[B, Cout, Cin/g, kh, kw]."""
    x = _f32(x)
    wb = _f64(wb)
    B, Cin, H, W = x.shape
    _, Cout, cpg, kh, kw = wb.shape
    assert wb.shape[0] == B and cpg * groups == Cin
    Ho, Wo = out_size(H, kh, stride, pad), out_size(W, kw, stride, pad)
    y = np.empty((B, Cout, Ho, Wo), np.float64)
    rc = _load().oracle_conv(B, Cin, H, W, Cout, kh, kw, stride, pad, groups,
                             _ptr(x), _ptr(wb), _ptr(y))
    _check(rc, "conv")
    return y


def forward(x, experts, alpha, stride: int = 1, pad: int = 0, groups: int = 1) -> np.ndarray:
    """The dynamic convolution layer for given attentions (mix, then convolve)."""
    x = _f32(x)
    experts = _f32(experts)
    alpha = _f64(alpha)
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    assert alpha.shape == (B, n) and cpg * groups == Cin
    Ho, Wo = out_size(H, kh, stride, pad), out_size(W, kw, stride, pad)
    y = np.empty((B, Cout, Ho, Wo), np.float64)
    rc = _load().oracle_forward(B, Cin, H, W, Cout, kh, kw, stride, pad, groups, n,
                                _ptr(x), _ptr(experts), _ptr(alpha), _ptr(y))
    _check(rc, "forward")
    return y


def forward_points(x, experts, alpha, idx, stride: int = 1, pad: int = 0,
                   groups: int = 1) -> np.ndarray:
    """Selected outputs y[b, o, r, s] of the layer; idx is an int array [m, 4]."""
    x = _f32(x)
    experts = _f32(experts)
    alpha = _f64(alpha)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(-1, 4))
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    assert alpha.shape == (B, n) and cpg * groups == Cin
    out = np.empty(idx.shape[0], np.float64)
    rc = _load().oracle_forward_points(B, Cin, H, W, Cout, kh, kw, stride, pad, groups,
                                       n, _ptr(x), _ptr(experts), _ptr(alpha),
                                       idx.shape[0], _ptr(idx), _ptr(out))
    _check(rc, "forward_points")
    return out


def forward_attn(x, experts, alpha, a_in=None, a_out=None, stride: int = 1, pad: int = 0,
                 groups: int = 1) -> np.ndarray:
    """The layer with FMDConv's input and output attentions (FMDConv: Fast
    multi-attention dynamic convolution, abstract). Reading: a_in[b, c]
    scales input channel c of example b before the convolution, a_out[b, o]
    scales output channel o after it; None means all ones:
    y[b,o] = a_out[b,o] * conv(a_in[b,:] * x[b], W_b)[o]."""
    x = _f32(x)
    experts = _f32(experts)
    alpha = _f64(alpha)
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    assert alpha.shape == (B, n) and cpg * groups == Cin
    ai = None if a_in is None else _f64(a_in)
    ao = None if a_out is None else _f64(a_out)
    if ai is not None:
        assert ai.shape == (B, Cin)
    if ao is not None:
        assert ao.shape == (B, Cout)
    Ho, Wo = out_size(H, kh, stride, pad), out_size(W, kw, stride, pad)
    y = np.empty((B, Cout, Ho, Wo), np.float64)
    rc = _load().oracle_forward_attn(B, Cin, H, W, Cout, kh, kw, stride, pad, groups, n,
                                     _ptr(x), _ptr(experts), _ptr(alpha),
                                     None if ai is None else _ptr(ai),
                                     None if ao is None else _ptr(ao), _ptr(y))
    _check(rc, "forward_attn")
    return y


def backward(x, experts, alpha, dy, stride: int = 1, pad: int = 0, groups: int = 1,
             want=("dx", "dalpha", "dexperts")):
    """Gradients of the layer (``forward``) for the output gradient dy.

    Returns (dx [B,Cin,H,W], dalpha [B,n], dexperts [n,Cout,Cin/g,kh,kw]) in
    float64; an entry not named in ``want`` is None. Definitions (the
    derivative of the forward, written out in ``dynconv_oracle.c``):
    dW_b = sum_{r,s} dy * shifted x;  dalpha[b,i] = <dW_b, E_i>;
    dE_i = sum_b alpha[b,i] dW_b;  dx = the adjoint of the convolution
    with W_b applied to dy."""
    x = _f32(x)
    experts = _f32(experts)
    alpha = _f64(alpha)
    dy = _f32(dy)
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    assert alpha.shape == (B, n) and cpg * groups == Cin
    Ho, Wo = out_size(H, kh, stride, pad), out_size(W, kw, stride, pad)
    assert dy.shape == (B, Cout, Ho, Wo)
    dx = np.empty(x.shape, np.float64) if "dx" in want else None
    da = np.empty((B, n), np.float64) if "dalpha" in want else None
    de = np.empty(experts.shape, np.float64) if "dexperts" in want else None
    rc = _load().oracle_backward(B, Cin, H, W, Cout, kh, kw, stride, pad, groups, n,
                                 _ptr(x), _ptr(experts), _ptr(alpha), _ptr(dy),
                                 None if dx is None else _ptr(dx),
                                 None if da is None else _ptr(da),
                                 None if de is None else _ptr(de))
    _check(rc, "backward")
    return dx, da, de


def backward_attn(x, experts, alpha, dy, a_in=None, a_out=None, stride: int = 1, pad: int = 0,
                  groups: int = 1, want=("dx", "dalpha", "dexperts", "da_in", "da_out")):
    """Gradients of the layer with FMDConv's channel attentions
    (``forward_attn``; FMDConv: Fast multi-attention dynamic convolution,
    abstract) for the output gradient dy: returns (dx, dalpha, dexperts,
    da_in [B,Cin], da_out [B,Cout]) in float64, None where not in ``want``.
    The derivative of y = a_out * conv(a_in * x, W_b), written out term by
    term in ``dynconv_oracle.c``; a_in or a_out None means all ones."""
    x = _f32(x)
    experts = _f32(experts)
    alpha = _f64(alpha)
    dy = _f32(dy)
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    assert alpha.shape == (B, n) and cpg * groups == Cin
    ai = None if a_in is None else _f64(a_in)
    ao = None if a_out is None else _f64(a_out)
    if ai is not None:
        assert ai.shape == (B, Cin)
    if ao is not None:
        assert ao.shape == (B, Cout)
    Ho, Wo = out_size(H, kh, stride, pad), out_size(W, kw, stride, pad)
    assert dy.shape == (B, Cout, Ho, Wo)
    dx = np.empty(x.shape, np.float64) if "dx" in want else None
    da = np.empty((B, n), np.float64) if "dalpha" in want else None
    de = np.empty(experts.shape, np.float64) if "dexperts" in want else None
    dai = np.empty((B, Cin), np.float64) if "da_in" in want else None
    dao = np.empty((B, Cout), np.float64) if "da_out" in want else None
    p = lambda a: None if a is None else _ptr(a)
    rc = _load().oracle_backward_attn(B, Cin, H, W, Cout, kh, kw, stride, pad, groups, n,
                                      _ptr(x), _ptr(experts), _ptr(alpha), p(ai), p(ao), _ptr(dy),
                                      p(dx), p(da), p(de), p(dai), p(dao))
    _check(rc, "backward_attn")
    return dx, da, de, dai, dao


def route_backward(x, fc_w, fc_b, dalpha, mode: int = SIGMOID, temperature: float = 1.0):
    """Gradients of the routing (``route``: GAP -> FC(+bias) -> sigmoid or
    softmax(z/T)) for the attention gradient dalpha[B, n].

    The derivative of each routing step, in reverse order:
    sigmoid: dz = dalpha * alpha * (1 - alpha);
    softmax(z/T): dz_j = alpha_j * (dalpha_j - sum_k alpha_k dalpha_k) / T;
    dfc_w = dz^T gap, dfc_b = sum_b dz, dgap = dz fc_w, and every position
    of channel c receives dgap[b, c] / (H W).
    Returns (dfc_w [n,Cin], dfc_b [n], dgap [B,Cin], dx [B,Cin,H,W]) in float64.
    """
    alpha, g, _ = route(x, fc_w, fc_b, mode, temperature)
    da = _f64(dalpha)
    assert da.shape == alpha.shape
    if mode == SIGMOID:
        dz = da * alpha * (1.0 - alpha)
    else:
        inner = np.sum(alpha * da, axis=1, keepdims=True)
        dz = alpha * (da - inner) / float(temperature)
    fw = _f64(fc_w)
    dfc_w = dz.T @ g
    dfc_b = dz.sum(axis=0)
    dgap = dz @ fw
    B, C, H, W = np.shape(x)
    dx = np.broadcast_to((dgap / float(H * W))[:, :, None, None], (B, C, H, W)).copy()
    return dfc_w, dfc_b, dgap, dx


def forward_sparse(x, experts, alpha, mask, stride: int = 1, pad: int = 0, groups: int = 1,
                   residual: bool = False) -> np.ndarray:
    """The layer evaluated at the positions a gate selects (Dynamic
    Convolutions: Exploiting Spatial Sparsity for Faster Inference, abstract:
    a gating branch chooses the spatial positions to evaluate, inside a
    residual block). Reading: mask[b, r, s] (nonzero = evaluate) over the
    output positions;
        y[b, o, r, s] = (x[b, o, r, s] if residual else 0) + [mask[b, r, s] != 0] * layer(x)[b, o, r, s]
    where layer is ``forward``. A residual block needs Cin == Cout and an
    output the size of the input."""
    y = forward(x, experts, alpha, stride, pad, groups)
    m = (np.asarray(mask) != 0)
    assert m.shape == (y.shape[0],) + y.shape[2:]
    out = y * m[:, None, :, :]
    if residual:
        xv = _f32(x).astype(np.float64)
        assert xv.shape == out.shape, "a residual block needs the output the size of the input"
        out = out + xv
    return out

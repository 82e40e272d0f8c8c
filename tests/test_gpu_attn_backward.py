"""GPU parity of the gradients of the layer with FMDConv's channel attentions
(dynconv_backward_weights_attn, dynconv_backward_data_attn) against the CPU
oracle's backward_attn (FMDConv: Fast multi-attention dynamic convolution,
abstract: input and output channel attentions beside the kernel attention).

Tolerances, normwise as in test_gpu_backward.py:
* dx: 2e-2 for bf16 layers (the transposed layer mixes and rounds its
  attention-scaled kernels to bf16, as the forward does), 1e-5 for float32;
* dalpha, dexperts, da_in, da_out: 1e-4 for bf16 layers and 1e-5 for float32
  layers: float32 sums of exact products of the stored values, the kernels
  mixed and the attention factors applied in float32.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_convolution_cnn_amd import binding as bd

from test_gpu_backward import GRAD_TOL, _layer_inputs
from test_gpu_parity import TOL, check, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(device):
    bd.lib()
    yield


def _attn(case, seed):
    B, Cin, Cout = case[0], case[1], case[2]
    rng = np.random.default_rng(seed)
    return ((rng.random((B, Cin)) + 0.5).astype(np.float32), (rng.random((B, Cout)) + 0.5).astype(np.float32))


ATTN_CASES = [
    # B, Cin, Cout, H, W, k, stride, pad, groups, n, dtype
    (3, 40, 72, 16, 16, 3, 1, 1, 1, 4, "bf16"),     # ragged channel tiles
    (3, 64, 64, 14, 14, 3, 1, 1, 1, 4, "bf16"),     # the transposed layer fits the fused path
    (2, 24, 40, 13, 11, 5, 1, 2, 1, 7, "bf16"),     # 5x5, 7 experts
    (4, 24, 24, 14, 14, 5, 1, 2, 24, 8, "bf16"),    # depthwise 5x5
    (2, 12, 20, 9, 9, 3, 1, 1, 1, 3, "f32"),        # float32 groups == 1
    (2, 8, 8, 9, 7, 3, 1, 1, 8, 3, "f32"),          # depthwise float32
    (12, 24, 32, 10, 10, 3, 1, 1, 1, 4, "bf16"),    # 2 example groups in the contraction
]


@pytest.mark.parametrize("case", ATTN_CASES)
def test_backward_attn_matches_oracle(case):
    B, Cin, Cout, H, W, k, st, p, g, n, dtype = case
    x, e, a, dy = _layer_inputs(case, seed=300 + Cin + Cout)
    ai, ao = _attn(case, seed=301 + Cin)
    say("backward_attn", case)
    xd, ed, ad, dyd = to_dev(x, dtype), to_dev(e, dtype), to_dev(a, "f32"), to_dev(dy, dtype)
    aid, aod = to_dev(ai, "f32"), to_dev(ao, "f32")
    dx = bd.dynconv_backward_data_attn(dyd, ed, ad, aid, aod, H, W, st, p, g)
    da, de, dai, dao = bd.dynconv_backward_weights_attn(xd, dyd, ed, ad, aid, aod, st, p, g)
    torch.cuda.synchronize()
    rx, ra, re, rai, rao = oracle.backward_attn(x, e, a, dy, ai, ao, st, p, g)
    check(from_dev(dx), rx, TOL[dtype], f"dx {case}")
    check(from_dev(da), ra, GRAD_TOL[dtype], f"dalpha {case}")
    check(from_dev(de), re, GRAD_TOL[dtype], f"dexperts {case}")
    check(from_dev(dai), rai, GRAD_TOL[dtype], f"da_in {case}")
    check(from_dev(dao), rao, GRAD_TOL[dtype], f"da_out {case}")


@pytest.mark.parametrize("which", ["in", "out"])
def test_backward_attn_one_side(which):
    """One attention given, the other NULL (all ones)."""
    case = ATTN_CASES[0]
    B, Cin, Cout, H, W, k, st, p, g, n, dtype = case
    x, e, a, dy = _layer_inputs(case, seed=311)
    ai, ao = _attn(case, seed=312)
    ai, ao = (ai, None) if which == "in" else (None, ao)
    say("backward_attn one side", which)
    dev = lambda v: None if v is None else to_dev(v, "f32")
    xd, ed, ad, dyd = to_dev(x, dtype), to_dev(e, dtype), to_dev(a, "f32"), to_dev(dy, dtype)
    dx = bd.dynconv_backward_data_attn(dyd, ed, ad, dev(ai), dev(ao), H, W, st, p, g)
    da, de, dai, dao = bd.dynconv_backward_weights_attn(xd, dyd, ed, ad, dev(ai), dev(ao), st, p, g)
    torch.cuda.synchronize()
    rx, ra, re, rai, rao = oracle.backward_attn(x, e, a, dy, ai, ao, st, p, g)
    check(from_dev(dx), rx, TOL[dtype], f"dx a_{which}")
    for got, ref, name in ((da, ra, "dalpha"), (de, re, "dexperts"), (dai, rai, "da_in"), (dao, rao, "da_out")):
        check(from_dev(got), ref, GRAD_TOL[dtype], f"{name} a_{which}")


def test_backward_attn_partial_outputs_and_stride2():
    """Each output alone is bitwise the full call's; a stride-2 layer has the
    kernel and attention gradients but no transposed layer for dx."""
    case = (2, 16, 24, 15, 15, 3, 2, 1, 1, 2, "bf16")
    B, Cin, Cout, H, W, k, st, p, g, n, dtype = case
    x, e, a, dy = _layer_inputs(case, seed=321)
    ai, ao = _attn(case, seed=322)
    say("backward_attn partial outputs, stride 2")
    xd, ed, ad, dyd = to_dev(x, dtype), to_dev(e, dtype), to_dev(a, "f32"), to_dev(dy, dtype)
    aid, aod = to_dev(ai, "f32"), to_dev(ao, "f32")
    full = bd.dynconv_backward_weights_attn(xd, dyd, ed, ad, aid, aod, st, p, g)
    names = ("dalpha", "dexperts", "da_in", "da_out")
    for j, name in enumerate(names):
        part = bd.dynconv_backward_weights_attn(xd, dyd, ed, ad, aid, aod, st, p, g, want=(name,))
        torch.cuda.synchronize()
        assert all(part[m] is None for m in range(4) if m != j)
        assert torch.equal(part[j], full[j]), name
    _, ra, re, rai, rao = oracle.backward_attn(x, e, a, dy, ai, ao, st, p, g, want=names)
    for got, ref, name in zip(full, (ra, re, rai, rao), names):
        check(from_dev(got), ref, GRAD_TOL[dtype], f"{name} stride 2")
    with pytest.raises(bd.DynconvError):
        bd.dynconv_backward_data_attn(dyd, ed, ad, aid, aod, H, W, st, p, g)

"""GPU parity of gated (spatially sparse) evaluation through the C ABI
against the oracle (Dynamic Convolutions: Exploiting Spatial Sparsity for
Faster Inference, abstract: a gating branch picks the positions a residual
block evaluates; gather-scatter execution). The gate is a seeded mask.
Tolerance 2e-2 normwise (bf16 layer, R10); positions the gate leaves off must
hold exactly 0, or exactly x in a residual block.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_convolution_cnn_amd import binding as bd
from dynamic_convolution_cnn_amd import inputs

from test_gpu_parity import TOL, check, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(device):
    bd.lib()
    yield


SPARSE_CASES = [
    # B, Cin, Cout, H, W, k, stride, pad, n, density, residual
    (3, 40, 72, 13, 11, 3, 1, 1, 3, 0.3, False),    # ragged channels and plane
    (2, 64, 64, 20, 20, 3, 1, 1, 4, 0.25, True),    # residual block
    (2, 64, 64, 20, 20, 3, 1, 1, 4, 1.0, True),     # every position on
    (2, 32, 32, 9, 9, 3, 1, 1, 2, 0.0, True),       # every position off
    (3, 40, 80, 14, 14, 1, 1, 0, 8, 0.5, False),    # 1x1
    (2, 24, 40, 15, 15, 3, 2, 1, 3, 0.4, False),    # stride 2
    (2, 32, 32, 10, 10, 3, 1, 1, 20, 0.3, True),    # 20 experts (wide bank)
    (70, 16, 16, 9, 7, 3, 1, 1, 4, 0.05, False),    # many examples, few positions each
    # one-pass band kernel (3x3 stride 1 pad 1, W % 8 == 0, Cin and Cout <= 64)
    (40, 64, 64, 16, 16, 3, 1, 1, 4, 0.3, True),    # 3-row bands, the last one a single row
    (3, 40, 48, 12, 16, 3, 1, 1, 3, 0.5, False),    # Cin padded to 64, Cout 48 (zero rows to 64)
    (2, 24, 24, 8, 8, 3, 1, 1, 20, 0.6, True),      # 32-channel tiles, 20 experts (wide bank)
    (2, 64, 64, 16, 24, 3, 1, 1, 4, 1.0, True),     # every position on
    (2, 64, 64, 16, 24, 3, 1, 1, 4, 0.0, True),     # every position off
    (64, 16, 16, 24, 8, 3, 1, 1, 2, 0.1, False),    # 6-row bands, no residual
    (2, 32, 32, 12, 64, 3, 1, 1, 4, 0.4, True),     # 64-wide rows
]


@pytest.mark.parametrize("case", SPARSE_CASES)
def test_forward_sparse_matches_oracle(case):
    B, Cin, Cout, H, W, k, st, p, n, dens, res = case
    rng = np.random.default_rng(110 + Cin + n)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round((rng.standard_normal((n, Cout, Cin, k, k)) * np.sqrt(2.0 / (Cin * k * k)))
                          .astype(np.float32))
    a = rng.random((B, n)).astype(np.float32)
    Ho, Wo = oracle.out_size(H, k, st, p), oracle.out_size(W, k, st, p)
    m = (rng.random((B, Ho, Wo)) < dens).astype(np.uint8)
    say("forward_sparse", case, int(m.sum()))
    y = bd.dynconv_forward_sparse(to_dev(x, "bf16"), to_dev(e, "bf16"), to_dev(a, "f32"),
                                  torch.from_numpy(m).cuda(), st, p, 1, residual=res)
    torch.cuda.synchronize()
    ref = oracle.forward_sparse(x, e, a, m, st, p, 1, res)
    got = from_dev(y)
    off = np.broadcast_to(m[:, None] == 0, got.shape)
    np.testing.assert_array_equal(got[off], ref[off])   # gate off: exactly 0 or x
    if m.any():
        check(got, ref, TOL["bf16"], f"forward_sparse {case}")


@pytest.mark.parametrize("case", [SPARSE_CASES[0], SPARSE_CASES[6], SPARSE_CASES[8], SPARSE_CASES[10]])
def test_forward_sparse_packed_equals_unpacked(case):
    """A bank packed once gives bitwise the results of the packing entry point."""
    B, Cin, Cout, H, W, k, st, p, n, dens, res = case
    rng = np.random.default_rng(7 + Cin + n)
    x = to_dev(inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32)), "bf16")
    e = to_dev(inputs.bf16_round((rng.standard_normal((n, Cout, Cin, k, k)) * 0.1).astype(np.float32)), "bf16")
    a = to_dev(rng.random((B, n)).astype(np.float32), "f32")
    Ho, Wo = oracle.out_size(H, k, st, p), oracle.out_size(W, k, st, p)
    m = torch.from_numpy((rng.random((B, Ho, Wo)) < dens).astype(np.uint8)).cuda()
    say("forward_sparse_packed", case)
    desc = bd.layer_desc(x, e, st, p, 1)
    pk = bd.dynconv_pack_experts(desc, e)
    y1 = bd.dynconv_forward_sparse(x, e, a, m, st, p, 1, residual=res)
    y2 = bd.dynconv_forward_sparse_packed(desc, x, pk, a, m, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_forward_sparse_deterministic_and_full_size_sampled():
    w = inputs.WORKLOADS["sparse_resnet18_3x3"]
    d = inputs.make_inputs(w, seed=0)
    L = w.layers[0]
    rng = np.random.default_rng(3)
    a = rng.random((w.B, w.n)).astype(np.float32)
    xd, ed, ad = to_dev(d["x"], "bf16"), to_dev(d["experts"][0], "bf16"), to_dev(a, "f32")
    md = torch.from_numpy(d["mask"]).cuda()
    say("forward_sparse full size", w.key, float(d["mask"].mean()))
    y1 = bd.dynconv_forward_sparse(xd, ed, ad, md, L.stride, L.pad, 1, residual=True)
    y2 = bd.dynconv_forward_sparse(xd, ed, ad, md, L.stride, L.pad, 1, residual=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    sel = np.array([0, 17, 31])
    ref = oracle.forward_sparse(d["x"][sel], d["experts"][0], a[sel], d["mask"][sel], L.stride, L.pad, 1, True)
    check(from_dev(y1)[sel], ref, TOL["bf16"], "forward_sparse full size (sampled examples)")

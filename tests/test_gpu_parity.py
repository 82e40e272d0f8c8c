"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case runs the library on seeded inputs and compares with the oracle on
the same inputs. Tolerances (normwise: max |gpu - oracle| / max |oracle| per
output tensor): 1e-5 for float32 layers, 2e-2 for bf16 layers (float32
accumulation, mixed kernels and outputs rounded to bf16). Attentions are
float32 in both cases and are held to 1e-5.

At full workload sizes the whole output is computed on the GPU in the same
launch configuration the benchmark times; the oracle then checks every
output of a few examples (first, second, last, ...) plus a few thousand
sampled outputs spread over the whole batch.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dynamic_convolution_cnn_amd import binding as bd
from dynamic_convolution_cnn_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
ALPHA_TOL = 1e-5


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    a = np.ascontiguousarray(a, np.float32)
    if dtype == "bf16":
        bits = inputs.f32_to_bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def relerr(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def check(got, ref, tol, what):
    e = relerr(got, ref)
    say(f"{what}: rel err {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{what}: relative error {e:.3e} > {tol}"


def sample_idx(shape, m, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.integers(0, s, m) for s in shape], axis=1).astype(np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu(device):
    bd.lib()
    yield


# ----------------------------------------------------------------- routing
@pytest.mark.parametrize("key", inputs.ORDER)
def test_route_full_size(key):
    w = inputs.WORKLOADS[key]
    d = inputs.make_inputs(w)
    say("route", key)
    x = to_dev(d["x"], w.dtype)
    alpha = bd.dynconv_route(x, to_dev(d["fc_w"], "f32"), to_dev(d["fc_b"], "f32"),
                             w.route_mode, w.temperature)
    torch.cuda.synchronize()
    ref, _, _ = oracle.route(d["x"], d["fc_w"], d["fc_b"], w.route_mode, w.temperature)
    check(from_dev(alpha), ref, ALPHA_TOL, f"route {key}")


@pytest.mark.parametrize("shape", [(3, 5, 7, 9, 6), (2, 3, 1, 1, 300 // 2), (5, 33, 13, 11, 256),
                                   (1, 8, 56, 56, 17), (130, 7, 5, 3, 9), (128, 33, 8, 8, 40),
                                   (200, 3, 14, 14, 256), (70, 6, 2, 6, 5), (64, 130, 14, 14, 3),
                                   (3, 1100, 3, 3, 4),     # split router: 3 workgroups per example
                                   (63, 96, 14, 14, 256),  # split router, 16-byte loads, n = 256
                                   (1, 4096, 2, 2, 5),     # split router, Cin at its limit (8 workgroups)
                                   (40, 3, 90, 90, 7),     # planes past one pass: two kernels
                                   (2, 3, 100, 100, 5),    # planes too large for one pass: two kernels
                                   (256, 9, 8, 8, 5), (257, 3, 7, 7, 3)])  # one workgroup per example
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", [0, 1])
def test_route_ragged(shape, dtype, mode):
    B, C, H, W, n = shape
    rng = np.random.default_rng(B * 1000 + C)
    x = rng.standard_normal((B, C, H, W), dtype=np.float32) + np.float32(0.3)
    if dtype == "bf16":
        x = inputs.bf16_round(x)
    fc_w = rng.standard_normal((n, C), dtype=np.float32)
    fc_b = rng.standard_normal((n,), dtype=np.float32)
    say("route ragged", shape, dtype, mode)
    a = bd.dynconv_route(to_dev(x, dtype), to_dev(fc_w, "f32"), to_dev(fc_b, "f32"), mode, 2.5)
    torch.cuda.synchronize()
    ref, _, _ = oracle.route(x, fc_w, fc_b, mode, 2.5)
    check(from_dev(a), ref, ALPHA_TOL, f"route ragged {shape}")


@pytest.mark.parametrize("shape", [(32, 64, 56, 56, 4), (6, 40, 14, 14, 16), (5, 12, 9, 7, 3)])
def test_route_workspace_reuse(shape):
    """The split router's ticket counters go back to zero after each call:
    consecutive calls on one zero-filled workspace, on different inputs, all
    match the oracle, and the counters read zero afterwards."""
    B, C, H, W, n = shape
    rng = np.random.default_rng(B + C)
    fc_w = rng.standard_normal((n, C), dtype=np.float32)
    fc_b = rng.standard_normal((n,), dtype=np.float32)
    desc = bd.make_desc(B, C, H, W, n=n, dtype=bd.DYNCONV_BF16)
    nb = bd.dynconv_route_workspace_bytes(desc)
    assert nb >= 256 + B * C * 4
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    fw, fb = to_dev(fc_w, "f32"), to_dev(fc_b, "f32")
    for r in range(3):
        x = inputs.bf16_round(rng.standard_normal((B, C, H, W), dtype=np.float32) + np.float32(0.1 * r))
        say("route reuse", shape, r)
        a = bd.dynconv_route(to_dev(x, "bf16"), fw, fb, r % 2, 2.0, workspace=ws)
        torch.cuda.synchronize()
        ref, _, _ = oracle.route(x, fc_w, fc_b, r % 2, 2.0)
        check(from_dev(a), ref, ALPHA_TOL, f"route reuse {shape} call {r}")
        assert int(ws[: 4 * B].view(torch.int32).abs().sum().item()) == 0, "ticket counters not reset"


def test_route_without_bias():
    rng = np.random.default_rng(3)
    x = inputs.bf16_round(rng.standard_normal((4, 16, 8, 8), dtype=np.float32))
    fc_w = rng.standard_normal((4, 16), dtype=np.float32)
    say("route no bias")
    a = bd.dynconv_route(to_dev(x, "bf16"), to_dev(fc_w, "f32"), None, 0, 1.0)
    torch.cuda.synchronize()
    ref, _, _ = oracle.route(x, fc_w, None, 0)
    check(from_dev(a), ref, ALPHA_TOL, "route no bias")


# ------------------------------------------------------------------ mixing
@pytest.mark.parametrize("key", inputs.ORDER)
def test_mix_full_size(key):
    w = inputs.WORKLOADS[key]
    d = inputs.make_inputs(w)
    alpha = inputs.forced_alpha(w.B, w.n, "uniform")
    a_dev = to_dev(alpha, "f32")
    sel = sorted({0, 1, w.B // 2, w.B - 1})
    for li, (L, e) in enumerate(zip(w.layers, d["experts"])):
        say("mix", key, "layer", li)
        m = bd.dynconv_mix(a_dev, to_dev(e, w.dtype), groups=L.groups)
        torch.cuda.synchronize()
        got = from_dev(m[sel])
        ref = oracle.mix(alpha[sel], e)
        check(got, ref, TOL[w.dtype], f"mix {key} layer {li}")
        if w.dtype == "bf16":
            # element-wise: one bf16 rounding of a float32 sum
            bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * oracle.mix(np.abs(alpha[sel]), np.abs(e))
            assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mix_one_hot_is_bitwise(dtype):
    B, n = 7, 3
    rng = np.random.default_rng(5)
    e = rng.standard_normal((n, 24, 16, 3, 3), dtype=np.float32)
    if dtype == "bf16":
        e = inputs.bf16_round(e)
    alpha = inputs.forced_alpha(B, n, "onehot")
    say("mix one-hot", dtype)
    m = bd.dynconv_mix(to_dev(alpha, "f32"), to_dev(e, dtype))
    torch.cuda.synchronize()
    got = m.float().cpu().numpy()
    for b in range(B):
        np.testing.assert_array_equal(got[b], e[b % n])


@pytest.mark.parametrize("n,B", [(5, 11), (7, 11), (9, 11), (12, 11), (16, 11), (17, 11), (33, 11), (48, 11),
                                 (64, 11), (20, 70), (16, 129)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mix_vector_expert_counts(n, B, dtype):
    """Vector path (kernel size a multiple of 8, not of the 256-weight matrix
    tile) for expert counts below and above the single-pass limit and across
    the matrix-core groups of 16, with batches that are not multiples of 8 or
    span several 64-example chunks."""
    rng = np.random.default_rng(13 + n)
    e = rng.standard_normal((n, 16, 8, 3, 3), dtype=np.float32)
    if dtype == "bf16":
        e = inputs.bf16_round(e)
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    say("mix vector", n, dtype)
    m = bd.dynconv_mix(to_dev(alpha, "f32"), to_dev(e, dtype))
    torch.cuda.synchronize()
    check(from_dev(m), oracle.mix(alpha, e), TOL[dtype], f"mix n={n}")


@pytest.mark.parametrize("wshape", [(5, 3, 3, 3), (7, 1, 5, 5), (3, 2, 1, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mix_ragged(wshape, dtype):
    """Kernel sizes not divisible by 8 take the scalar path."""
    B, n = 9, 5
    rng = np.random.default_rng(11)
    e = rng.standard_normal((n,) + wshape, dtype=np.float32)
    if dtype == "bf16":
        e = inputs.bf16_round(e)
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    groups = 1 if wshape[1] != 1 else wshape[0]
    say("mix ragged", wshape, dtype)
    m = bd.dynconv_mix(to_dev(alpha, "f32"), to_dev(e, dtype), groups=groups)
    torch.cuda.synchronize()
    check(from_dev(m), oracle.mix(alpha, e), TOL[dtype], f"mix ragged {wshape}")


# ----------------------------------------------------------------- forward
def run_layer(x, e, alpha, L, dtype, policy=bd.DYNCONV_POLICY_AUTO):
    y = bd.dynconv_forward(to_dev(x, dtype), to_dev(e, dtype), to_dev(alpha, "f32"),
                           L.stride, L.pad, L.groups, policy=policy)
    torch.cuda.synchronize()
    return y


def compare_layer(y, x, e, alpha, L, dtype, what, full_limit=8):
    """Every output of up to `full_limit` examples, plus sampled outputs over the batch."""
    B = x.shape[0]
    sel = sorted({0, 1, B // 2, B - 1} | set(range(min(full_limit, B))))
    got = y.float().cpu().numpy().astype(np.float64)
    ref = oracle.forward(x[sel], e, alpha[sel], L.stride, L.pad, L.groups)
    check(got[sel], ref, TOL[dtype], what + " (whole examples)")
    idx = sample_idx(got.shape, 3000, seed=B)
    pts = oracle.forward_points(x, e, alpha, idx, L.stride, L.pad, L.groups)
    den = np.max(np.abs(ref))
    err = float(np.max(np.abs(got[tuple(idx.T)] - pts)) / den)
    say(f"{what} (sampled): rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("key", inputs.ORDER)
@pytest.mark.parametrize("akind", ["routed", "uniform", "onehot"])
def test_forward_full_size(key, akind):
    w = inputs.WORKLOADS[key]
    d = inputs.make_inputs(w)
    if akind == "routed":
        alpha, _, _ = oracle.route(d["x"], d["fc_w"], d["fc_b"], w.route_mode, w.temperature)
        alpha = alpha.astype(np.float32)
    else:
        alpha = inputs.forced_alpha(w.B, w.n, akind)
    for li, (L, e) in enumerate(zip(w.layers, d["experts"])):
        x = d["x"] if li == 0 else inputs.layer_input(L, w.B, w.dtype, seed=100 + li)
        say("forward", key, akind, "layer", li)
        y = run_layer(x, e, alpha, L, w.dtype)
        compare_layer(y, x, e, alpha, L, w.dtype, f"forward {key} {akind} layer {li}")


def test_headline_layer_both_policies_and_determinism():
    w = inputs.WORKLOADS["resnet50_3x3"]
    d = inputs.make_inputs(w)
    L, e = w.layers[0], d["experts"][0]
    alpha = inputs.forced_alpha(w.B, w.n, "uniform")
    outs = {}
    for pol in (bd.DYNCONV_POLICY_FUSED, bd.DYNCONV_POLICY_PREMIX):
        say("headline policy", pol)
        y1 = run_layer(d["x"], e, alpha, L, w.dtype, pol)
        y2 = run_layer(d["x"], e, alpha, L, w.dtype, pol)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"
        compare_layer(y1, d["x"], e, alpha, L, w.dtype, f"headline policy {pol}", full_limit=4)
        outs[pol] = y1.float().cpu().numpy()
    # both paths round the same float32 sums only differently in order
    assert relerr(outs[bd.DYNCONV_POLICY_FUSED], outs[bd.DYNCONV_POLICY_PREMIX].astype(np.float64)) < 2e-2


RAGGED = [
    # B, Cin, Cout, H, W, k(h,w), stride, pad, n
    (3, 40, 24, 9, 11, (3, 3), 1, 1, 3),     # odd W, channel tail, Cout tail
    (5, 64, 80, 14, 14, (3, 3), 1, 1, 4),    # B not a multiple of 4
    (2, 16, 16, 15, 15, (3, 3), 2, 1, 2),    # stride 2, odd sizes
    (2, 33, 17, 10, 8, (3, 1), 1, 1, 5),     # kh != kw
    (4, 32, 48, 12, 12, (1, 1), 1, 0, 1),    # 1x1, single expert
    (2, 24, 40, 13, 13, (5, 5), 1, 2, 7),    # 5x5
    (1, 8, 8, 1, 1, (3, 3), 1, 1, 2),        # 1x1 image
    (3, 96, 64, 7, 9, (3, 3), 1, 0, 16),     # no padding, 16 experts
    (2, 64, 32, 40, 40, (3, 3), 1, 1, 4),    # several position tiles
    (6, 40, 100, 16, 16, (3, 3), 1, 1, 3),   # 256 positions, channel and Cout tails
    (3, 256, 64, 10, 12, (5, 5), 1, 2, 2),   # 5x5 on a non-square image
    (5, 32, 32, 20, 20, (3, 3), 2, 1, 4),    # stride 2
    (3, 48, 40, 13, 14, (3, 3), 1, 1, 3),    # 16-wide padded rows, odd Ho, tails
    (2, 256, 24, 6, 6, (3, 3), 1, 1, 16),    # expert slab too big for the LDS packing path
    (7, 64, 64, 6, 6, (3, 3), 1, 1, 4),      # small image: fewer rows than blocks
    (3, 40, 72, 24, 20, (1, 1), 1, 0, 8),    # 1x1: two chunks (tail), two channel tiles, partial position tile
    (2, 48, 64, 30, 56, (3, 3), 1, 1, 2),    # wide rows: several 256-position tiles spanning rows
    (2, 64, 130, 18, 16, (1, 1), 1, 0, 4),   # 1x1, Cin <= 64: three output tiles (tail 2), position tail 32
    (3, 20, 33, 10, 8, (1, 1), 1, 0, 3),     # 1x1, one partial chunk, odd Cout
    (3, 96, 40, 12, 12, (1, 1), 1, 0, 2),    # 1x1, three chunks (odd count) on the persistent path
    (3, 96, 90, 12, 12, (1, 1), 1, 0, 3),    # 1x1 persistent path, one 96-channel tile (Cout tail 6)
    (2, 80, 270, 9, 8, (1, 1), 1, 0, 2),     # 1x1, three 96-channel tiles, partial position tile
    # 3x3 pad-1 layers up to 14x14 with n <= 4 (the fused path's one-wave-per-example kernel)
    (1, 20, 70, 14, 12, (3, 3), 1, 1, 2),    # one example, 16-channel chunk tail, Cout tail, two experts
    (6, 256, 256, 14, 14, (3, 3), 1, 1, 1),  # one expert
    (9, 32, 64, 14, 14, (3, 3), 1, 1, 4),    # 9 examples: a quad with one live example
    (4, 16, 64, 2, 2, (3, 3), 1, 1, 3),      # 2x2 image
]


@pytest.mark.parametrize("case", RAGGED)
@pytest.mark.parametrize("policy", [bd.DYNCONV_POLICY_PREMIX, bd.DYNCONV_POLICY_FUSED])
def test_forward_ragged_bf16(case, policy):
    B, Cin, Cout, H, W, (kh, kw), st, p, n = case
    Ho, Wo = (H + 2 * p - kh) // st + 1, (W + 2 * p - kw) // st + 1
    if policy == bd.DYNCONV_POLICY_FUSED and Ho * Wo > 256:
        pytest.skip("fused path covers at most 256 output positions")
    rng = np.random.default_rng(hash(case) % 2**32)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round(rng.standard_normal((n, Cout, Cin, kh, kw), dtype=np.float32))
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    say("ragged", case, "policy", policy)
    try:
        y = bd.dynconv_forward(to_dev(x, "bf16"), to_dev(e, "bf16"), to_dev(alpha, "f32"), st, p,
                               1, policy=policy)
    except bd.DynconvError as err:
        if err.status == bd.DYNCONV_ERR_UNSUPPORTED and policy == bd.DYNCONV_POLICY_FUSED:
            pytest.skip(f"fused path declines this layer: {err}")
        raise
    torch.cuda.synchronize()
    ref = oracle.forward(x, e, alpha, st, p, 1)
    check(from_dev(y), ref, TOL["bf16"], f"ragged {case} policy {policy}")


@pytest.mark.parametrize("case", RAGGED[:6])
def test_forward_ragged_f32(case):
    B, Cin, Cout, H, W, (kh, kw), st, p, n = case
    rng = np.random.default_rng(7 + hash(case) % 1000)
    x = rng.standard_normal((B, Cin, H, W), dtype=np.float32)
    e = rng.standard_normal((n, Cout, Cin, kh, kw), dtype=np.float32)
    alpha = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    say("ragged f32", case)
    y = bd.dynconv_forward(to_dev(x, "f32"), to_dev(e, "f32"), to_dev(alpha, "f32"), st, p, 1)
    torch.cuda.synchronize()
    check(from_dev(y), oracle.forward(x, e, alpha, st, p, 1), TOL["f32"], f"ragged f32 {case}")


DW = [(3, 16, 9, 11, 5, 1, 2, 4), (2, 24, 28, 28, 3, 2, 1, 3), (4, 8, 7, 7, 7, 1, 3, 9),
      (1, 5, 1, 1, 3, 1, 1, 2),
      # even W (bf16 dot2 kernels): 2-element rows, n > 8, stride 2 with odd pad,
      # batch not a multiple of 16, a plane past the lanes' prefetched pieces, pad 0
      (3, 12, 10, 10, 5, 1, 2, 4), (2, 8, 14, 14, 3, 1, 1, 12), (2, 10, 16, 16, 5, 2, 2, 5),
      (2, 6, 12, 12, 7, 1, 3, 8), (5, 7, 28, 28, 5, 1, 2, 8), (1, 2, 56, 56, 3, 1, 1, 4),
      (2, 4, 12, 12, 3, 2, 0, 4), (17, 3, 8, 8, 7, 2, 3, 2),
      # matrix-core kernel (stride 1, output planes up to 32 x 32): 32 output
      # rows, pad 0, 7x7 with 24-wide rows, rows not a multiple of 4, a batch
      # of 19 (one wave of the second example group busy), pad beyond K - 1,
      # planes of 84 elements (8-byte pieces)
      (3, 5, 32, 28, 5, 1, 2, 6), (2, 4, 18, 18, 3, 1, 0, 3), (2, 3, 32, 24, 7, 1, 3, 5),
      (4, 6, 14, 6, 3, 1, 1, 7), (19, 3, 16, 16, 5, 1, 2, 8), (2, 3, 4, 4, 7, 1, 5, 2),
      (2, 5, 7, 12, 3, 1, 1, 4)]


@pytest.mark.parametrize("case", DW)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("policy", [bd.DYNCONV_POLICY_FUSED, bd.DYNCONV_POLICY_PREMIX])
def test_depthwise_ragged(case, dtype, policy):
    B, C, H, W, k, st, p, n = case
    rng = np.random.default_rng(C * 31 + k)
    x = rng.standard_normal((B, C, H, W), dtype=np.float32)
    e = rng.standard_normal((n, C, 1, k, k), dtype=np.float32)
    if dtype == "bf16":
        x, e = inputs.bf16_round(x), inputs.bf16_round(e)
    alpha = rng.uniform(0, 1, (B, n)).astype(np.float32)
    say("depthwise", case, dtype, policy)
    y = bd.dynconv_forward(to_dev(x, dtype), to_dev(e, dtype), to_dev(alpha, "f32"), st, p, C,
                           policy=policy)
    torch.cuda.synchronize()
    check(from_dev(y), oracle.forward(x, e, alpha, st, p, C), TOL[dtype], f"depthwise {case}")


def test_mbconv_block_chained():
    """Route once on the block input, then expand -> depthwise -> project, bf16 between layers."""
    w = inputs.WORKLOADS["effnet_b0_mbconv"]
    d = inputs.make_inputs(w, B=16)
    say("mbconv chained")
    x = to_dev(d["x"], "bf16")
    alpha = bd.dynconv_route(x, to_dev(d["fc_w"], "f32"), to_dev(d["fc_b"], "f32"), 0, 1.0)
    h = x
    for L, e in zip(w.layers, d["experts"]):
        h = bd.dynconv_forward(h, to_dev(e, "bf16"), alpha, L.stride, L.pad, L.groups)
    torch.cuda.synchronize()
    a_ref, _, _ = oracle.route(d["x"], d["fc_w"], d["fc_b"], 0)
    check(from_dev(alpha), a_ref, ALPHA_TOL, "mbconv alpha")
    r = d["x"]
    for L, e in zip(w.layers, d["experts"]):
        r = oracle.forward(r, e, a_ref, L.stride, L.pad, L.groups)
    check(from_dev(h), r, TOL["bf16"], "mbconv block output")


def test_permuted_batch_permutes_output():
    w = inputs.WORKLOADS["resnet50_3x3"]
    d = inputs.make_inputs(w, B=12)
    L, e = w.layers[0], d["experts"][0]
    alpha = inputs.forced_alpha(12, w.n, "uniform")
    perm = np.random.default_rng(2).permutation(12)
    say("permutation")
    y = run_layer(d["x"], e, alpha, L, "bf16").cpu()
    yp = run_layer(d["x"][perm], e, alpha[perm], L, "bf16").cpu()
    assert torch.equal(yp.view(torch.int16), y[perm].view(torch.int16))


@pytest.mark.parametrize("key,B", [("resnet50_3x3", 8), ("many_expert_softmax", 3),
                                   ("resnet18_3x3", 2)])
def test_packed_api_matches_forward(key, B):
    """pack once + forward_packed gives bitwise the same y as forward (both policies)."""
    w = inputs.WORKLOADS[key]
    d = inputs.make_inputs(w, B=B)
    L, e = w.layers[0], d["experts"][0]
    alpha = to_dev(inputs.forced_alpha(B, w.n, "uniform"), "f32")
    x, ed = to_dev(d["x"], "bf16"), to_dev(e, "bf16")
    desc = bd.layer_desc(x, ed, L.stride, L.pad, L.groups)
    say("packed api", key)
    packed = bd.dynconv_pack_experts(desc, ed)
    for pol in (bd.DYNCONV_POLICY_PREMIX, bd.DYNCONV_POLICY_FUSED):
        if pol == bd.DYNCONV_POLICY_FUSED and (L.Ho * L.Wo > 256 or w.n > 4):
            continue
        y1 = bd.dynconv_forward_packed(desc, x, packed, alpha, policy=pol)
        y2 = bd.dynconv_forward(x, ed, alpha, L.stride, L.pad, L.groups, policy=pol)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("key,B", [("resnet50_3x3", 8), ("many_expert_softmax", 4)])
def test_graph_replay_matches_eager(key, B):
    """A HIP graph holding route + pack + forward (as the benchmark replays it)
    gives bitwise the eager results on every replay, with other eager work and
    host synchronisations between the replays."""
    w = inputs.WORKLOADS[key]
    d = inputs.make_inputs(w, B=B)
    L, e = w.layers[0], d["experts"][0]
    x, ed = to_dev(d["x"], "bf16"), to_dev(e, "bf16")
    fw, fb = to_dev(d["fc_w"], "f32"), to_dev(d["fc_b"], "f32")
    desc = bd.layer_desc(x, ed, L.stride, L.pad, L.groups)
    pol = bd.dynconv_forward_policy(desc)
    alpha = torch.empty((B, w.n), dtype=torch.float32, device="cuda")
    packed = torch.empty(bd.dynconv_packed_experts_bytes(desc), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(bd.dynconv_forward_packed_workspace_bytes(desc, pol), 16), dtype=torch.uint8,
                     device="cuda")
    rws = torch.zeros(max(bd.dynconv_route_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((B, L.Cout, L.Ho, L.Wo), dtype=torch.bfloat16, device="cuda")

    def step():
        bd.dynconv_route(x, fw, fb, w.route_mode, w.temperature, alpha=alpha, workspace=rws)
        bd.dynconv_pack_experts(desc, ed, packed)
        bd.dynconv_forward_packed(desc, x, packed, alpha, policy=pol, y=y, workspace=ws)

    say("graph replay", key, "policy", pol)
    step()
    torch.cuda.synchronize()
    a_ref, y_ref = alpha.clone(), y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    x2 = torch.flip(x, dims=[0]).contiguous()
    for r in range(3):
        alpha.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(alpha, a_ref), f"replay {r}: alpha differs"
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"replay {r}: y differs"
        # unrelated eager work between replays
        bd.dynconv_forward(x2, ed, a_ref, L.stride, L.pad, L.groups)
        torch.cuda.synchronize()

"""dynconv_forward_noalloc (the forward with the library's fixed per-GPU
scratch as its workspace) against dynconv_forward through the C ABI: bitwise
equal outputs on consecutive calls, the second smaller than the first (the
scratch keeps the previous call's contents), on the fused and the premix
policies; a layer whose workspace exceeds the scratch is refused before
anything runs."""
import numpy as np
import pytest
import torch

from dynamic_convolution_cnn_amd import binding as bd
from dynamic_convolution_cnn_amd import inputs

pytestmark = pytest.mark.gpu


def _layer(B, Cin, Cout, H, W, k, n, seed):
    rng = np.random.default_rng(seed)
    x = inputs.bf16_round(rng.standard_normal((B, Cin, H, W), dtype=np.float32))
    e = inputs.bf16_round((rng.standard_normal((n, Cout, Cin, k, k)) * np.sqrt(2.0 / (Cin * k * k)))
                          .astype(np.float32))
    a = rng.uniform(0.05, 0.95, (B, n)).astype(np.float32)

    def dev(t, bf16=True):
        t = np.ascontiguousarray(t, np.float32)
        if bf16:
            return torch.from_numpy(inputs.f32_to_bf16_bits(t).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(t).cuda()
    return dev(x), dev(e), dev(a, bf16=False)


def _same(u, v):
    return torch.equal(u.view(torch.int16), v.view(torch.int16))


# (B, Cin, Cout, H, W, k, n, policy): each pair is a larger call, then a smaller one
SEQUENCES = [
    [(64, 256, 256, 14, 14, 3, 4, bd.DYNCONV_POLICY_FUSED), (6, 64, 48, 10, 10, 3, 3, bd.DYNCONV_POLICY_FUSED)],
    [(12, 128, 128, 28, 28, 3, 16, bd.DYNCONV_POLICY_PREMIX), (3, 40, 24, 9, 12, 3, 5, bd.DYNCONV_POLICY_PREMIX)],
    [(32, 64, 64, 56, 56, 3, 4, bd.DYNCONV_POLICY_AUTO), (5, 64, 80, 14, 14, 3, 4, bd.DYNCONV_POLICY_AUTO)],
]


@pytest.mark.parametrize("seq", SEQUENCES)
def test_noalloc_matches_forward_on_consecutive_calls(seq, device):
    for i, (B, Cin, Cout, H, W, k, n, pol) in enumerate(seq):
        x, e, a = _layer(B, Cin, Cout, H, W, k, n, seed=40 + i + B)
        print(f"[case] noalloc call {i}: B={B} {Cin}->{Cout} {H}x{W} k={k} n={n} policy={pol}", flush=True)
        y_ref = bd.dynconv_forward(x, e, a, 1, k // 2, 1, policy=pol)
        y = torch.full_like(y_ref, float("nan"))
        bd.dynconv_forward_noalloc(x, e, a, 1, k // 2, 1, policy=pol, y=y)
        torch.cuda.synchronize()
        assert _same(y, y_ref), f"call {i}: dynconv_forward_noalloc differs from dynconv_forward"


def test_noalloc_refuses_a_workspace_beyond_the_scratch(device):
    # the ResNet-50-shaped layer on the premix policy needs the bank plus 302 MB of mixed kernels
    x, e, a = _layer(256, 256, 256, 14, 14, 3, 4, seed=3)
    desc = bd.layer_desc(x, e, 1, 1, 1)
    assert bd.dynconv_forward_workspace_bytes(desc, bd.DYNCONV_POLICY_PREMIX) > bd.DYNCONV_NOALLOC_MAX_BYTES
    y = torch.zeros((256, 256, 14, 14), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bd.DynconvError) as err:
        bd.dynconv_forward_noalloc(x, e, a, 1, 1, 1, policy=bd.DYNCONV_POLICY_PREMIX, y=y)
    assert err.value.status == bd.DYNCONV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y.view(torch.int16))) == 0  # nothing written

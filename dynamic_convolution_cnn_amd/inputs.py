"""Seeded synthetic inputs and the workload table.

This module is shared by the tests, the benchmark and the smoke check. It
holds no arithmetic of the method (no pooling, routing, mixing or
convolution): only the shapes of the five workloads, the random draws that
fill them, and the round-to-nearest-even conversion of float32 draws to
bfloat16 storage.

The pages describe the method on networks trained on ImageNet, CIFAR and
COCO (CondConv: Conditionally Parameterized Convolutions, abstract;
FMDConv, abstract; KernelWarehouse, abstract). Neither those datasets nor
trained weights are used; every tensor here is a seeded draw with the shape
of one layer of the networks the pages name (ResNet-18/50, EfficientNet-B0).

Draw order per workload (numpy ``default_rng(seed)``, float32 draws):
    x, then the expert banks layer by layer, then fc_w; fc_b is zero.
Distributions:
    x            ~ N(0, 1)            (ReLU(N(0, 1)) for the ResNet-50 layer)
    experts      ~ N(0, 2 / fan_in),  fan_in = (Cin / groups) * k * k, each
                   expert drawn independently (Kaiming-normal, untruncated)
    fc_w         ~ N(0, 0.1^2); for the many-expert softmax layer the std is
                   sqrt(H*W / Cin), so that the routing logits are ~N(0, 1)
    fc_b         = 0
bf16 workloads round each float32 draw to bf16 (RNE); the oracle and the GPU
both consume the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

SIGMOID = 0
SOFTMAX = 1


@dataclasses.dataclass(frozen=True)
class Layer:
    Cin: int
    Cout: int
    H: int
    W: int
    k: int
    stride: int = 1
    pad: int = 0
    groups: int = 1

    @property
    def Ho(self) -> int:
        return (self.H + 2 * self.pad - self.k) // self.stride + 1

    @property
    def Wo(self) -> int:
        return (self.W + 2 * self.pad - self.k) // self.stride + 1

    @property
    def expert_shape(self):
        return (self.Cout, self.Cin // self.groups, self.k, self.k)

    @property
    def fan_in(self) -> int:
        return (self.Cin // self.groups) * self.k * self.k

    def macs_per_example(self) -> int:
        """Multiply-adds of one example's convolution."""
        return self.Cout * self.Ho * self.Wo * (self.Cin // self.groups) * self.k * self.k


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    title: str
    B: int
    n: int
    dtype: str                  # "f32" or "bf16"
    layers: tuple               # Layer, ...; routing uses layers[0]'s input
    route_mode: int = SIGMOID
    temperature: float = 1.0
    x_relu: bool = False
    fc_std: Optional[float] = 0.1
    attention: bool = False     # FMDConv input and output attention heads as well
    mask_density: float = 0.0   # > 0: a gate evaluates this fraction of output positions (residual block)

    @property
    def route_layer(self) -> Layer:
        return self.layers[0]

    def fc_std_value(self) -> float:
        if self.fc_std is not None:
            return self.fc_std
        L = self.route_layer
        return math.sqrt(L.H * L.W / L.Cin)

    def conv_flops(self) -> int:
        """Useful FLOPs of the convolutions, one multiply-add counted as 2."""
        return sum(2 * self.B * L.macs_per_example() for L in self.layers)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        key="tiny", title="tiny CondConv 3x3, B=2, 16->16, 8x8, n=4, fp32",
        B=2, n=4, dtype="f32",
        layers=(Layer(16, 16, 8, 8, 3, 1, 1),)),
    "resnet18_3x3": Workload(
        key="resnet18_3x3", title="ResNet-18-shaped 3x3, B=32, 64->64, 56x56, n=4, bf16",
        B=32, n=4, dtype="bf16",
        layers=(Layer(64, 64, 56, 56, 3, 1, 1),)),
    "effnet_b0_mbconv": Workload(
        key="effnet_b0_mbconv",
        title="EfficientNet-B0-shaped MBConv block, B=128, 40->240 1x1, dw 5x5, 240->80 1x1, 28x28, n=8, bf16",
        B=128, n=8, dtype="bf16",
        layers=(Layer(40, 240, 28, 28, 1, 1, 0),
                Layer(240, 240, 28, 28, 5, 1, 2, groups=240),
                Layer(240, 80, 28, 28, 1, 1, 0))),
    "resnet50_3x3": Workload(
        key="resnet50_3x3", title="ResNet-50-shaped 3x3, B=256, 256->256, 14x14, n=4, bf16",
        B=256, n=4, dtype="bf16", x_relu=True,
        layers=(Layer(256, 256, 14, 14, 3, 1, 1),)),
    "many_expert_softmax": Workload(
        key="many_expert_softmax",
        title="many-expert 3x3, B=64, 128->128, 28x28, n=16, softmax(z/4), bf16",
        B=64, n=16, dtype="bf16", route_mode=SOFTMAX, temperature=4.0, fc_std=None,
        layers=(Layer(128, 128, 28, 28, 3, 1, 1),)),
    # FMDConv's multi-attention layer (input, temperature-scaled kernel and
    # output attention) on the ResNet-18-shaped 3x3 layer; not one of the
    # five configurations of the method's hot path
    "fmdconv_resnet18_3x3": Workload(
        key="fmdconv_resnet18_3x3",
        title="FMDConv multi-attention on the ResNet-18-shaped 3x3, B=32, 64->64, 56x56, n=4, softmax(z/4), bf16",
        B=32, n=4, dtype="bf16", route_mode=SOFTMAX, temperature=4.0, attention=True,
        layers=(Layer(64, 64, 56, 56, 3, 1, 1),)),
    # the same attentions on the ResNet-50-shaped layer, where they ride the
    # fused path (W_b never in memory)
    "fmdconv_resnet50_3x3": Workload(
        key="fmdconv_resnet50_3x3",
        title="FMDConv multi-attention on the ResNet-50-shaped 3x3, B=256, 256->256, 14x14, n=4, softmax(z/4), bf16",
        B=256, n=4, dtype="bf16", route_mode=SOFTMAX, temperature=4.0, attention=True, x_relu=True,
        layers=(Layer(256, 256, 14, 14, 3, 1, 1),)),
    # spatially sparse evaluation: a gate selects a quarter of the positions of
    # a residual ResNet-18-shaped layer; not one of the five configurations
    "sparse_resnet18_3x3": Workload(
        key="sparse_resnet18_3x3",
        title="gated residual 3x3, 25% of positions, B=32, 64->64, 56x56, n=4, bf16",
        B=32, n=4, dtype="bf16", mask_density=0.25,
        layers=(Layer(64, 64, 56, 56, 3, 1, 1),)),
    # KernelWarehouse's setting of more than 100 experts (n > 100) on the
    # many-expert layer's shape; not one of the five configurations
    "kernelwarehouse_n128": Workload(
        key="kernelwarehouse_n128",
        title="KernelWarehouse-scale bank: 3x3, B=64, 128->128, 28x28, n=128, softmax(z/4), bf16",
        B=64, n=128, dtype="bf16", route_mode=SOFTMAX, temperature=4.0, fc_std=None,
        layers=(Layer(128, 128, 28, 28, 3, 1, 1),)),
}

# The order the workloads are listed in: the tiny parity case first, the
# headline ResNet-50 layer fourth.
ORDER: List[str] = ["tiny", "resnet18_3x3", "effnet_b0_mbconv", "resnet50_3x3",
                    "many_expert_softmax"]


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 result."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round to nearest even.

    Inputs here are finite; NaN and overflow handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def make_inputs(w: Workload, seed: int = 0, B: Optional[int] = None) -> dict:
    """Seeded inputs of a workload.

    Returns a dict with float32 arrays (values already representable in the
    workload's storage type): ``x`` [B, Cin, H, W], ``experts`` (a list, one
    [n, Cout, Cin/g, k, k] bank per layer), ``fc_w`` [n, Cin], ``fc_b`` [n].
    ``B`` overrides the batch (the draws of the first B' examples of a
    larger batch are NOT the same as a smaller batch's draws).
    """
    rng = np.random.default_rng(seed)
    Bn = w.B if B is None else B
    L0 = w.route_layer
    x = rng.standard_normal((Bn, L0.Cin, L0.H, L0.W), dtype=np.float32)
    if w.x_relu:
        x = np.maximum(x, np.float32(0.0))
    banks = []
    for L in w.layers:
        std = math.sqrt(2.0 / L.fan_in)
        e = rng.standard_normal((w.n,) + L.expert_shape, dtype=np.float32) * np.float32(std)
        banks.append(_store(e, w.dtype))
    fc_w = rng.standard_normal((w.n, L0.Cin), dtype=np.float32) * np.float32(w.fc_std_value())
    fc_b = np.zeros((w.n,), np.float32)
    out = {"x": _store(x, w.dtype), "experts": banks, "fc_w": fc_w.astype(np.float32), "fc_b": fc_b}
    if w.attention:
        # input and output attention heads (FC on the same pooled input), drawn
        # after everything else so the other draws match a plain workload's
        Cout = w.layers[-1].Cout
        for name, m in (("in", L0.Cin), ("out", Cout)):
            out[f"fc_w_{name}"] = (rng.standard_normal((m, L0.Cin), dtype=np.float32) *
                                   np.float32(w.fc_std_value())).astype(np.float32)
            out[f"fc_b_{name}"] = np.zeros((m,), np.float32)
    if w.mask_density > 0:
        # the gate: each output position of each example on with probability
        # mask_density (drawn last, so the other draws match a dense workload's)
        L = w.layers[0]
        out["mask"] = (rng.random((Bn, L.Ho, L.Wo)) < w.mask_density).astype(np.uint8)
    return out


def layer_input(L: Layer, B: int, dtype: str, seed: int) -> np.ndarray:
    """A stand-alone N(0, 1) input for one layer (used to check layers one by one)."""
    rng = np.random.default_rng(seed)
    return _store(rng.standard_normal((B, L.Cin, L.H, L.W), dtype=np.float32), dtype)


def forced_alpha(B: int, n: int, kind: str, seed: int = 1) -> np.ndarray:
    """Attentions that differ strongly between examples (float32 [B, n]).

    ``uniform``: U(0, 1) per (b, i), seed 1; ``onehot``: alpha_b = e_{b mod n}.
    Under the workloads' own initialisation the routed attentions hardly vary
    between examples, so a wrong example index could hide inside the bf16
    tolerance; these inputs close that gap.
    """
    if kind == "uniform":
        return np.random.default_rng(seed).random((B, n), dtype=np.float32)
    if kind == "onehot":
        a = np.zeros((B, n), np.float32)
        a[np.arange(B), np.arange(B) % n] = 1.0
        return a
    raise ValueError(kind)


def random_layer_inputs(L: Layer, B: int, n: int, dtype: str, seed: int) -> dict:
    """x, experts and fc weights of arbitrary shape for the ragged-shape parity cases."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L.Cin, L.H, L.W), dtype=np.float32)
    e = rng.standard_normal((n,) + L.expert_shape, dtype=np.float32) * np.float32(
        math.sqrt(2.0 / L.fan_in))
    fc_w = rng.standard_normal((n, L.Cin), dtype=np.float32) * np.float32(0.5)
    fc_b = rng.standard_normal((n,), dtype=np.float32) * np.float32(0.1)
    return {"x": _store(x, dtype), "experts": _store(e, dtype), "fc_w": fc_w, "fc_b": fc_b}

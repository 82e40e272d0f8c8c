"""ctypes binding of libdynconv.so (the C ABI in include/dynconv.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
The library is loaded on first use; if it is missing this module raises
(there is no CPU fallback).

The functions carry the C entry points' names. Tensors must be contiguous,
on the GPU, bf16 or float32 (attentions and router weights float32).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdynconv.so")

DYNCONV_OK = 0
DYNCONV_ERR_INVALID_ARG = 1
DYNCONV_ERR_UNSUPPORTED = 2
DYNCONV_ERR_WORKSPACE = 3
DYNCONV_ERR_HIP = 4

DYNCONV_F32 = 0
DYNCONV_BF16 = 1

DYNCONV_SIGMOID = 0
DYNCONV_SOFTMAX = 1

DYNCONV_POLICY_AUTO = 0
DYNCONV_POLICY_PREMIX = 1
DYNCONV_POLICY_FUSED = 2

# Every symbol include/dynconv.h declares.
EXPORTED = (
    "dynconv_route", "dynconv_route_workspace_bytes", "dynconv_mix", "dynconv_forward",
    "dynconv_forward_workspace_bytes", "dynconv_forward_policy", "dynconv_status_string",
    "dynconv_last_error", "dynconv_abi_version", "dynconv_packed_experts_bytes",
    "dynconv_pack_experts", "dynconv_forward_packed", "dynconv_forward_packed_workspace_bytes",
    "dynconv_route_attn", "dynconv_route_attn_workspace_bytes", "dynconv_forward_attn",
    "dynconv_forward_attn_workspace_bytes", "dynconv_backward_data",
    "dynconv_backward_data_workspace_bytes", "dynconv_backward_weights",
    "dynconv_backward_weights_workspace_bytes", "dynconv_route_backward",
    "dynconv_route_backward_workspace_bytes", "dynconv_forward_sparse",
    "dynconv_forward_sparse_workspace_bytes", "dynconv_forward_noalloc",
    "dynconv_forward_sparse_packed", "dynconv_forward_sparse_packed_workspace_bytes",
    "dynconv_backward_weights_attn", "dynconv_backward_weights_attn_workspace_bytes",
    "dynconv_backward_data_attn", "dynconv_backward_data_attn_workspace_bytes",
)


class dynconv_desc_t(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("B", "Cin", "H", "W", "Cout", "kh", "kw", "stride", "pad", "groups", "n",
                 "dtype")]


class DynconvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)} ({detail})")
        self.status = status


_lib = None


def lib():
    """The loaded library with typed entry points (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m dynamic_convolution_cnn_amd.build` "
            "(the dynamic convolution has no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(dynconv_desc_t)
    i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.dynconv_route.argtypes = [D, P, P, P, i32, f32, P, P, sz, P]
    L.dynconv_route.restype = i32
    L.dynconv_route_workspace_bytes.argtypes = [D]
    L.dynconv_route_workspace_bytes.restype = sz
    L.dynconv_mix.argtypes = [D, P, P, P, P]
    L.dynconv_mix.restype = i32
    L.dynconv_forward.argtypes = [D, i32, P, P, P, P, P, sz, P]
    L.dynconv_forward.restype = i32
    L.dynconv_forward_workspace_bytes.argtypes = [D, i32]
    L.dynconv_forward_workspace_bytes.restype = sz
    L.dynconv_forward_policy.argtypes = [D]
    L.dynconv_forward_policy.restype = i32
    L.dynconv_status_string.argtypes = [i32]
    L.dynconv_status_string.restype = ctypes.c_char_p
    L.dynconv_last_error.argtypes = []
    L.dynconv_last_error.restype = ctypes.c_char_p
    L.dynconv_abi_version.argtypes = []
    L.dynconv_abi_version.restype = i32
    L.dynconv_packed_experts_bytes.argtypes = [D]
    L.dynconv_packed_experts_bytes.restype = sz
    L.dynconv_pack_experts.argtypes = [D, P, P, sz, P]
    L.dynconv_pack_experts.restype = i32
    L.dynconv_forward_packed.argtypes = [D, i32, P, P, P, P, P, sz, P]
    L.dynconv_forward_packed.restype = i32
    L.dynconv_forward_packed_workspace_bytes.argtypes = [D, i32]
    L.dynconv_forward_packed_workspace_bytes.restype = sz
    L.dynconv_route_attn.argtypes = [D, P, P, P, i32, f32, P, P, P, P, P, P, P, P, sz, P]
    L.dynconv_route_attn.restype = i32
    L.dynconv_route_attn_workspace_bytes.argtypes = [D]
    L.dynconv_route_attn_workspace_bytes.restype = sz
    L.dynconv_forward_attn.argtypes = [D, i32, P, P, P, P, P, P, P, sz, P]
    L.dynconv_forward_attn.restype = i32
    L.dynconv_forward_attn_workspace_bytes.argtypes = [D, i32]
    L.dynconv_forward_attn_workspace_bytes.restype = sz
    L.dynconv_backward_data.argtypes = [D, i32, P, P, P, P, P, sz, P]
    L.dynconv_backward_data.restype = i32
    L.dynconv_backward_data_workspace_bytes.argtypes = [D, i32]
    L.dynconv_backward_data_workspace_bytes.restype = sz
    L.dynconv_backward_weights.argtypes = [D, P, P, P, P, P, P, P, sz, P]
    L.dynconv_backward_weights.restype = i32
    L.dynconv_backward_weights_workspace_bytes.argtypes = [D]
    L.dynconv_backward_weights_workspace_bytes.restype = sz
    L.dynconv_route_backward.argtypes = [D, P, P, i32, f32, P, P, P, P, P, P, sz, P]
    L.dynconv_route_backward.restype = i32
    L.dynconv_route_backward_workspace_bytes.argtypes = [D]
    L.dynconv_route_backward_workspace_bytes.restype = sz
    L.dynconv_forward_sparse.argtypes = [D, P, P, P, P, i32, P, P, sz, P]
    L.dynconv_forward_sparse.restype = i32
    L.dynconv_forward_sparse_workspace_bytes.argtypes = [D]
    L.dynconv_forward_sparse_workspace_bytes.restype = sz
    L.dynconv_forward_sparse_packed.argtypes = [D, P, P, P, P, i32, P, P, sz, P]
    L.dynconv_forward_sparse_packed.restype = i32
    L.dynconv_forward_sparse_packed_workspace_bytes.argtypes = [D]
    L.dynconv_forward_sparse_packed_workspace_bytes.restype = sz
    L.dynconv_forward_noalloc.argtypes = [D, i32, P, P, P, P, P]
    L.dynconv_forward_noalloc.restype = i32
    L.dynconv_backward_weights_attn.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    L.dynconv_backward_weights_attn.restype = i32
    L.dynconv_backward_weights_attn_workspace_bytes.argtypes = [D]
    L.dynconv_backward_weights_attn_workspace_bytes.restype = sz
    L.dynconv_backward_data_attn.argtypes = [D, i32, P, P, P, P, P, P, P, sz, P]
    L.dynconv_backward_data_attn.restype = i32
    L.dynconv_backward_data_attn_workspace_bytes.argtypes = [D, i32]
    L.dynconv_backward_data_attn_workspace_bytes.restype = sz
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dynconv_status_string(int(status)).decode()


def last_error() -> str:
    return lib().dynconv_last_error().decode()


def make_desc(B, Cin, H, W, Cout=1, kh=1, kw=1, stride=1, pad=0, groups=1, n=1,
              dtype=DYNCONV_BF16) -> dynconv_desc_t:
    return dynconv_desc_t(B, Cin, H, W, Cout, kh, kw, stride, pad, groups, n, dtype)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DYNCONV_BF16
    if t.dtype == torch.float32:
        return DYNCONV_F32
    raise ValueError(f"unsupported dtype {t.dtype}: activations and experts are bfloat16 or float32")


F32 = torch.float32


def _need(t: Optional[torch.Tensor], name: str, shape, dtype=None, optional: bool = False):
    """Check one tensor argument against what the call will read or write:
    its exact shape, its dtype and a dense layout. The C ABI takes raw
    pointers and sizes from the descriptor, so a tensor that does not match
    would be read or written out of bounds; mismatches raise ValueError
    before the library is called."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_bytes(t: Optional[torch.Tensor], name: str, nbytes: int):
    """A byte buffer (packed bank, workspace): dense and at least nbytes long."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, {nbytes} needed")


def _same_gpu(**tensors):
    """Every given tensor on one GPU (the device the call's pointers belong to)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} is on {t.device}; the library takes device memory only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
    return dev


def _out_hw(H, W, kh, kw, stride, pad):
    Ho = (H + 2 * pad - kh) // stride + 1
    Wo = (W + 2 * pad - kw) // stride + 1
    if Ho < 1 or Wo < 1:
        raise ValueError(f"kernel {kh}x{kw} does not fit the padded {H}x{W} input")
    return Ho, Wo


def _layer_tensors(x, experts, groups):
    """Shapes implied by x [B, Cin, H, W] and experts [n, Cout, Cin/groups, kh, kw]."""
    if x.dim() != 4:
        raise ValueError(f"x must be [B, Cin, H, W] (got {tuple(x.shape)})")
    if experts.dim() != 5:
        raise ValueError(f"experts must be [n, Cout, Cin/groups, kh, kw] (got {tuple(experts.shape)})")
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    if groups < 1 or Cin % groups or cpg != Cin // groups:
        raise ValueError(f"experts.shape[2] = {cpg} must be Cin / groups = {Cin} / {groups}")
    if experts.dtype != x.dtype:
        raise ValueError(f"experts dtype {experts.dtype} differs from x dtype {x.dtype}")
    _dtype_code(x)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != DYNCONV_OK:
        raise DynconvError(status, where, last_error())


def _workspace(nbytes: int, device, given: Optional[torch.Tensor], zeroed: bool = False):
    if given is not None:
        _need_bytes(given, "workspace", nbytes)
        _same_gpu(workspace=given)
        if given.device != device:
            raise ValueError(f"workspace is on {given.device}, the call's tensors on {device}")
    if nbytes == 0:
        return given, 0
    if given is not None:
        return given, given.numel() * given.element_size()
    alloc = torch.zeros if zeroed else torch.empty
    return alloc(nbytes, dtype=torch.uint8, device=device), nbytes


def layer_desc(x: torch.Tensor, experts: torch.Tensor, stride: int, pad: int,
               groups: int) -> dynconv_desc_t:
    _layer_tensors(x, experts, groups)
    B, Cin, H, W = x.shape
    n, Cout, cpg, kh, kw = experts.shape
    return make_desc(B, Cin, H, W, Cout, kh, kw, stride, pad, groups, n, _dtype_code(x))


def dynconv_route_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_route_workspace_bytes(ctypes.byref(desc)))


def dynconv_forward_workspace_bytes(desc: dynconv_desc_t, policy: int = DYNCONV_POLICY_AUTO) -> int:
    return int(lib().dynconv_forward_workspace_bytes(ctypes.byref(desc), int(policy)))


def dynconv_forward_policy(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_forward_policy(ctypes.byref(desc)))


def dynconv_status_string(status: int) -> str:
    return status_string(status)


def dynconv_last_error() -> str:
    return last_error()


def dynconv_abi_version() -> int:
    return int(lib().dynconv_abi_version())


def dynconv_route(x: torch.Tensor, fc_w: torch.Tensor, fc_b: Optional[torch.Tensor],
                  mode: int = DYNCONV_SIGMOID, temperature: float = 1.0,
                  alpha: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """alpha[B, n] (float32) from GAP -> FC(+bias) -> sigmoid | softmax(z / T)."""
    if x.dim() != 4 or fc_w.dim() != 2:
        raise ValueError("x must be [B, Cin, H, W] and fc_w [n, Cin]")
    B, Cin, H, W = x.shape
    n = fc_w.shape[0]
    desc = make_desc(B, Cin, H, W, n=n, dtype=_dtype_code(x))
    _need(fc_w, "fc_w", (n, Cin), F32)
    _need(fc_b, "fc_b", (n,), F32, optional=True)
    _need(alpha, "alpha", (B, n), F32, optional=True)
    _same_gpu(x=x, fc_w=fc_w, fc_b=fc_b, alpha=alpha)
    if alpha is None:
        alpha = torch.empty((B, n), dtype=torch.float32, device=x.device)
    # a workspace made here starts zero-filled, as the router's ticket
    # counters need; one passed in must have been zero-filled once (each call
    # leaves the counters zero)
    ws, ws_bytes = _workspace(dynconv_route_workspace_bytes(desc), x.device, workspace, zeroed=True)
    _check(lib().dynconv_route(ctypes.byref(desc), _ptr(x), _ptr(fc_w), _ptr(fc_b), int(mode),
                               float(temperature), _ptr(alpha), _ptr(ws), ws_bytes,
                               _stream(stream)), "dynconv_route")
    return alpha


def dynconv_mix(alpha: torch.Tensor, experts: torch.Tensor, groups: int = 1,
                mixed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mixed[b] = sum_i alpha[b, i] experts[i]; experts [n, Cout, Cin/g, kh, kw]."""
    if alpha.dim() != 2 or experts.dim() != 5:
        raise ValueError("alpha must be [B, n] and experts [n, Cout, Cin/groups, kh, kw]")
    B = alpha.shape[0]
    n, Cout, cpg, kh, kw = experts.shape
    # H = W = kh, kw-sized input keeps the descriptor valid; mixing reads only the kernel shape
    desc = make_desc(B, cpg * groups, kh, kw, Cout, kh, kw, 1, 0, groups, n, _dtype_code(experts))
    _need(alpha, "alpha", (B, n), F32)
    _need(experts, "experts", (n, Cout, cpg, kh, kw))
    _need(mixed, "mixed", (B, Cout, cpg, kh, kw), experts.dtype, optional=True)
    _same_gpu(alpha=alpha, experts=experts, mixed=mixed)
    if mixed is None:
        mixed = torch.empty((B, Cout, cpg, kh, kw), dtype=experts.dtype, device=experts.device)
    _check(lib().dynconv_mix(ctypes.byref(desc), _ptr(alpha), _ptr(experts), _ptr(mixed),
                             _stream(stream)), "dynconv_mix")
    return mixed


def dynconv_forward(x: torch.Tensor, experts: torch.Tensor, alpha: torch.Tensor,
                    stride: int = 1, pad: int = 0, groups: int = 1,
                    policy: int = DYNCONV_POLICY_AUTO, y: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[b] = conv(x[b], sum_i alpha[b, i] experts[i]) for every example."""
    desc = layer_desc(x, experts, stride, pad, groups)
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, stride, pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W))
    _need(experts, "experts", tuple(experts.shape))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(y, "y", (desc.B, desc.Cout, Ho, Wo), x.dtype, optional=True)
    _same_gpu(x=x, experts=experts, alpha=alpha, y=y)
    if y is None:
        y = torch.empty((desc.B, desc.Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    ws, ws_bytes = _workspace(dynconv_forward_workspace_bytes(desc, policy), x.device, workspace)
    _check(lib().dynconv_forward(ctypes.byref(desc), int(policy), _ptr(x), _ptr(experts),
                                 _ptr(alpha), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "dynconv_forward")
    return y


DYNCONV_NOALLOC_MAX_BYTES = 64 << 20


def dynconv_forward_noalloc(x: torch.Tensor, experts: torch.Tensor, alpha: torch.Tensor,
                            stride: int = 1, pad: int = 0, groups: int = 1,
                            policy: int = DYNCONV_POLICY_AUTO, y: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """dynconv_forward with the library's fixed per-GPU scratch as workspace (no
    device allocation in the call; pass y to keep the call allocation-free)."""
    desc = layer_desc(x, experts, stride, pad, groups)
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, stride, pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W))
    _need(experts, "experts", tuple(experts.shape))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(y, "y", (desc.B, desc.Cout, Ho, Wo), x.dtype, optional=True)
    _same_gpu(x=x, experts=experts, alpha=alpha, y=y)
    if y is None:
        y = torch.empty((desc.B, desc.Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    _check(lib().dynconv_forward_noalloc(ctypes.byref(desc), int(policy), _ptr(x), _ptr(experts),
                                         _ptr(alpha), _ptr(y), _stream(stream)), "dynconv_forward_noalloc")
    return y


def dynconv_route_attn_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_route_attn_workspace_bytes(ctypes.byref(desc)))


def dynconv_route_attn(x: torch.Tensor, Cout: int, fc_w: torch.Tensor, fc_b: Optional[torch.Tensor],
                       fc_w_in: torch.Tensor, fc_b_in: Optional[torch.Tensor], fc_w_out: torch.Tensor,
                       fc_b_out: Optional[torch.Tensor], mode: int = DYNCONV_SIGMOID,
                       temperature: float = 1.0, alpha: Optional[torch.Tensor] = None,
                       a_in: Optional[torch.Tensor] = None, a_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """FMDConv's three attentions from one pooling of x: (alpha [B, n], a_in [B, Cin],
    a_out [B, Cout]), float32."""
    if x.dim() != 4 or fc_w.dim() != 2:
        raise ValueError("x must be [B, Cin, H, W] and fc_w [n, Cin]")
    B, Cin, H, W = x.shape
    n = fc_w.shape[0]
    desc = make_desc(B, Cin, H, W, Cout, 1, 1, 1, 0, 1, n, _dtype_code(x))
    _need(fc_w, "fc_w", (n, Cin), F32)
    _need(fc_b, "fc_b", (n,), F32, optional=True)
    _need(fc_w_in, "fc_w_in", (Cin, Cin), F32)
    _need(fc_b_in, "fc_b_in", (Cin,), F32, optional=True)
    _need(fc_w_out, "fc_w_out", (Cout, Cin), F32)
    _need(fc_b_out, "fc_b_out", (Cout,), F32, optional=True)
    _need(alpha, "alpha", (B, n), F32, optional=True)
    _need(a_in, "a_in", (B, Cin), F32, optional=True)
    _need(a_out, "a_out", (B, Cout), F32, optional=True)
    _same_gpu(x=x, fc_w=fc_w, fc_b=fc_b, fc_w_in=fc_w_in, fc_b_in=fc_b_in, fc_w_out=fc_w_out,
              fc_b_out=fc_b_out, alpha=alpha, a_in=a_in, a_out=a_out)
    if alpha is None:
        alpha = torch.empty((B, n), dtype=torch.float32, device=x.device)
    if a_in is None:
        a_in = torch.empty((B, Cin), dtype=torch.float32, device=x.device)
    if a_out is None:
        a_out = torch.empty((B, Cout), dtype=torch.float32, device=x.device)
    ws, ws_bytes = _workspace(dynconv_route_attn_workspace_bytes(desc), x.device, workspace)
    _check(lib().dynconv_route_attn(ctypes.byref(desc), _ptr(x), _ptr(fc_w), _ptr(fc_b), int(mode),
                                    float(temperature), _ptr(fc_w_in), _ptr(fc_b_in), _ptr(fc_w_out),
                                    _ptr(fc_b_out), _ptr(alpha), _ptr(a_in), _ptr(a_out), _ptr(ws),
                                    ws_bytes, _stream(stream)), "dynconv_route_attn")
    return alpha, a_in, a_out


def dynconv_forward_attn_workspace_bytes(desc: dynconv_desc_t, policy: int = DYNCONV_POLICY_AUTO) -> int:
    return int(lib().dynconv_forward_attn_workspace_bytes(ctypes.byref(desc), int(policy)))


def dynconv_forward_attn(x: torch.Tensor, experts: torch.Tensor, alpha: torch.Tensor,
                         a_in: Optional[torch.Tensor], a_out: Optional[torch.Tensor],
                         stride: int = 1, pad: int = 0, groups: int = 1,
                         policy: int = DYNCONV_POLICY_AUTO, y: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[b, o] = a_out[b, o] * conv(a_in[b, :] x[b], sum_i alpha[b, i] experts[i])[o]."""
    desc = layer_desc(x, experts, stride, pad, groups)
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, stride, pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W))
    _need(experts, "experts", tuple(experts.shape))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(a_in, "a_in", (desc.B, desc.Cin), F32, optional=True)
    _need(a_out, "a_out", (desc.B, desc.Cout), F32, optional=True)
    _need(y, "y", (desc.B, desc.Cout, Ho, Wo), x.dtype, optional=True)
    _same_gpu(x=x, experts=experts, alpha=alpha, a_in=a_in, a_out=a_out, y=y)
    if y is None:
        y = torch.empty((desc.B, desc.Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    ws, ws_bytes = _workspace(dynconv_forward_attn_workspace_bytes(desc, policy), x.device, workspace)
    _check(lib().dynconv_forward_attn(ctypes.byref(desc), int(policy), _ptr(x), _ptr(experts),
                                      _ptr(alpha), _ptr(a_in), _ptr(a_out), _ptr(y), _ptr(ws), ws_bytes,
                                      _stream(stream)), "dynconv_forward_attn")
    return y


def dynconv_packed_experts_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_packed_experts_bytes(ctypes.byref(desc)))


def dynconv_forward_packed_workspace_bytes(desc: dynconv_desc_t,
                                           policy: int = DYNCONV_POLICY_AUTO) -> int:
    return int(lib().dynconv_forward_packed_workspace_bytes(ctypes.byref(desc), int(policy)))


def dynconv_pack_experts(desc: dynconv_desc_t, experts: torch.Tensor,
                         packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The expert bank in the layout the bf16 MFMA convolution reads (uint8 bytes)."""
    nbytes = dynconv_packed_experts_bytes(desc)
    _need(experts, "experts", (desc.n, desc.Cout, desc.Cin // max(desc.groups, 1), desc.kh, desc.kw),
          torch.bfloat16)
    _need_bytes(packed, "packed", nbytes)
    _same_gpu(experts=experts, packed=packed)
    if packed is None:
        packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=experts.device)
    _check(lib().dynconv_pack_experts(ctypes.byref(desc), _ptr(experts), _ptr(packed),
                                      packed.numel() * packed.element_size(), _stream(stream)),
           "dynconv_pack_experts")
    return packed


def dynconv_forward_packed(desc: dynconv_desc_t, x: torch.Tensor, packed: torch.Tensor,
                           alpha: torch.Tensor, policy: int = DYNCONV_POLICY_AUTO,
                           y: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dynconv_forward with a bank packed by dynconv_pack_experts."""
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, desc.stride, desc.pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W), torch.bfloat16)
    _need_bytes(packed, "packed", dynconv_packed_experts_bytes(desc))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(y, "y", (desc.B, desc.Cout, Ho, Wo), torch.bfloat16, optional=True)
    _same_gpu(x=x, packed=packed, alpha=alpha, y=y)
    if y is None:
        y = torch.empty((desc.B, desc.Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    ws, ws_bytes = _workspace(dynconv_forward_packed_workspace_bytes(desc, policy), x.device,
                              workspace)
    _check(lib().dynconv_forward_packed(ctypes.byref(desc), int(policy), _ptr(x), _ptr(packed),
                                        _ptr(alpha), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "dynconv_forward_packed")
    return y


def dynconv_backward_data_workspace_bytes(desc: dynconv_desc_t, policy: int = DYNCONV_POLICY_AUTO) -> int:
    return int(lib().dynconv_backward_data_workspace_bytes(ctypes.byref(desc), int(policy)))


def dynconv_backward_data(dy: torch.Tensor, experts: torch.Tensor, alpha: torch.Tensor, H: int, W: int,
                          stride: int = 1, pad: int = 0, groups: int = 1,
                          policy: int = DYNCONV_POLICY_AUTO, dx: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Input gradient dx [B, Cin, H, W] of the layer for the output gradient dy."""
    if dy.dim() != 4 or experts.dim() != 5:
        raise ValueError("dy must be [B, Cout, Ho, Wo] and experts [n, Cout, Cin/groups, kh, kw]")
    B = dy.shape[0]
    n, Cout, cpg, kh, kw = experts.shape
    desc = make_desc(B, cpg * groups, H, W, Cout, kh, kw, stride, pad, groups, n, _dtype_code(dy))
    Ho, Wo = _out_hw(H, W, kh, kw, stride, pad)
    _need(dy, "dy", (B, Cout, Ho, Wo))
    _need(experts, "experts", (n, Cout, cpg, kh, kw), dy.dtype)
    _need(alpha, "alpha", (B, n), F32)
    _need(dx, "dx", (B, cpg * groups, H, W), dy.dtype, optional=True)
    _same_gpu(dy=dy, experts=experts, alpha=alpha, dx=dx)
    if dx is None:
        dx = torch.empty((B, cpg * groups, H, W), dtype=dy.dtype, device=dy.device)
    ws, ws_bytes = _workspace(dynconv_backward_data_workspace_bytes(desc, policy), dy.device, workspace)
    _check(lib().dynconv_backward_data(ctypes.byref(desc), int(policy), _ptr(dy), _ptr(experts),
                                       _ptr(alpha), _ptr(dx), _ptr(ws), ws_bytes, _stream(stream)),
           "dynconv_backward_data")
    return dx


def dynconv_backward_weights_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_backward_weights_workspace_bytes(ctypes.byref(desc)))


def dynconv_backward_weights(x: torch.Tensor, dy: torch.Tensor, experts: torch.Tensor,
                             alpha: torch.Tensor, stride: int = 1, pad: int = 0, groups: int = 1,
                             dalpha: Optional[torch.Tensor] = None,
                             dexperts: Optional[torch.Tensor] = None, want=("dalpha", "dexperts"),
                             workspace: Optional[torch.Tensor] = None, stream=None):
    """(dalpha [B, n], dexperts [n, Cout, Cin/g, kh, kw]), float32; an entry not in
    ``want`` (and not given) is None."""
    desc = layer_desc(x, experts, stride, pad, groups)
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, stride, pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W))
    _need(dy, "dy", (desc.B, desc.Cout, Ho, Wo), x.dtype)
    _need(experts, "experts", tuple(experts.shape))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(dalpha, "dalpha", (desc.B, desc.n), F32, optional=True)
    _need(dexperts, "dexperts", tuple(experts.shape), F32, optional=True)
    _same_gpu(x=x, dy=dy, experts=experts, alpha=alpha, dalpha=dalpha, dexperts=dexperts)
    if dalpha is None and "dalpha" in want:
        dalpha = torch.empty((desc.B, desc.n), dtype=torch.float32, device=x.device)
    if dexperts is None and "dexperts" in want:
        dexperts = torch.empty(tuple(experts.shape), dtype=torch.float32, device=x.device)
    ws, ws_bytes = _workspace(dynconv_backward_weights_workspace_bytes(desc), x.device, workspace)
    _check(lib().dynconv_backward_weights(ctypes.byref(desc), _ptr(x), _ptr(dy), _ptr(experts),
                                          _ptr(alpha), _ptr(dalpha), _ptr(dexperts), _ptr(ws), ws_bytes,
                                          _stream(stream)), "dynconv_backward_weights")
    return dalpha, dexperts


def dynconv_backward_weights_attn_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_backward_weights_attn_workspace_bytes(ctypes.byref(desc)))


def dynconv_backward_weights_attn(x: torch.Tensor, dy: torch.Tensor, experts: torch.Tensor,
                                  alpha: torch.Tensor, a_in: Optional[torch.Tensor],
                                  a_out: Optional[torch.Tensor], stride: int = 1, pad: int = 0,
                                  groups: int = 1, want=("dalpha", "dexperts", "da_in", "da_out"),
                                  workspace: Optional[torch.Tensor] = None, stream=None):
    """(dalpha [B, n], dexperts, da_in [B, Cin], da_out [B, Cout]), float32, of the layer
    with channel attentions; an entry not in ``want`` is None."""
    desc = layer_desc(x, experts, stride, pad, groups)
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, stride, pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W))
    _need(dy, "dy", (desc.B, desc.Cout, Ho, Wo), x.dtype)
    _need(experts, "experts", tuple(experts.shape))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(a_in, "a_in", (desc.B, desc.Cin), F32, optional=True)
    _need(a_out, "a_out", (desc.B, desc.Cout), F32, optional=True)
    _same_gpu(x=x, dy=dy, experts=experts, alpha=alpha, a_in=a_in, a_out=a_out)
    mk = lambda name, shape: (torch.empty(shape, dtype=torch.float32, device=x.device)
                              if name in want else None)
    dalpha = mk("dalpha", (desc.B, desc.n))
    dexperts = mk("dexperts", tuple(experts.shape))
    da_in = mk("da_in", (desc.B, desc.Cin))
    da_out = mk("da_out", (desc.B, desc.Cout))
    ws, ws_bytes = _workspace(dynconv_backward_weights_attn_workspace_bytes(desc), x.device, workspace)
    _check(lib().dynconv_backward_weights_attn(ctypes.byref(desc), _ptr(x), _ptr(dy), _ptr(experts),
                                               _ptr(alpha), _ptr(a_in), _ptr(a_out), _ptr(dalpha),
                                               _ptr(dexperts), _ptr(da_in), _ptr(da_out), _ptr(ws),
                                               ws_bytes, _stream(stream)), "dynconv_backward_weights_attn")
    return dalpha, dexperts, da_in, da_out


def dynconv_backward_data_attn_workspace_bytes(desc: dynconv_desc_t, policy: int = DYNCONV_POLICY_AUTO) -> int:
    return int(lib().dynconv_backward_data_attn_workspace_bytes(ctypes.byref(desc), int(policy)))


def dynconv_backward_data_attn(dy: torch.Tensor, experts: torch.Tensor, alpha: torch.Tensor,
                               a_in: Optional[torch.Tensor], a_out: Optional[torch.Tensor], H: int, W: int,
                               stride: int = 1, pad: int = 0, groups: int = 1,
                               policy: int = DYNCONV_POLICY_AUTO, dx: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Input gradient dx [B, Cin, H, W] of the layer with channel attentions."""
    if dy.dim() != 4 or experts.dim() != 5:
        raise ValueError("dy must be [B, Cout, Ho, Wo] and experts [n, Cout, Cin/groups, kh, kw]")
    B = dy.shape[0]
    n, Cout, cpg, kh, kw = experts.shape
    desc = make_desc(B, cpg * groups, H, W, Cout, kh, kw, stride, pad, groups, n, _dtype_code(dy))
    Ho, Wo = _out_hw(H, W, kh, kw, stride, pad)
    _need(dy, "dy", (B, Cout, Ho, Wo))
    _need(experts, "experts", (n, Cout, cpg, kh, kw), dy.dtype)
    _need(alpha, "alpha", (B, n), F32)
    _need(a_in, "a_in", (B, cpg * groups), F32, optional=True)
    _need(a_out, "a_out", (B, Cout), F32, optional=True)
    _need(dx, "dx", (B, cpg * groups, H, W), dy.dtype, optional=True)
    _same_gpu(dy=dy, experts=experts, alpha=alpha, a_in=a_in, a_out=a_out, dx=dx)
    if dx is None:
        dx = torch.empty((B, cpg * groups, H, W), dtype=dy.dtype, device=dy.device)
    ws, ws_bytes = _workspace(dynconv_backward_data_attn_workspace_bytes(desc, policy), dy.device, workspace)
    _check(lib().dynconv_backward_data_attn(ctypes.byref(desc), int(policy), _ptr(dy), _ptr(experts),
                                            _ptr(alpha), _ptr(a_in), _ptr(a_out), _ptr(dx), _ptr(ws), ws_bytes,
                                            _stream(stream)), "dynconv_backward_data_attn")
    return dx


def dynconv_route_backward_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_route_backward_workspace_bytes(ctypes.byref(desc)))


def dynconv_route_backward(x: torch.Tensor, fc_w: torch.Tensor, alpha: torch.Tensor,
                           dalpha: torch.Tensor, mode: int = DYNCONV_SIGMOID,
                           temperature: float = 1.0, dx: Optional[torch.Tensor] = None,
                           dfc_w: Optional[torch.Tensor] = None, dfc_b: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """(dfc_w [n, Cin], dfc_b [n]) of the routing; when dx is given, the pooling's
    share dgap / (H W) is added to it in place."""
    if x.dim() != 4 or fc_w.dim() != 2:
        raise ValueError("x must be [B, Cin, H, W] and fc_w [n, Cin]")
    B, Cin, H, W = x.shape
    n = fc_w.shape[0]
    desc = make_desc(B, Cin, H, W, n=n, dtype=_dtype_code(x))
    _need(fc_w, "fc_w", (n, Cin), F32)
    _need(alpha, "alpha", (B, n), F32)
    _need(dalpha, "dalpha", (B, n), F32)
    _need(dx, "dx", (B, Cin, H, W), x.dtype, optional=True)
    _need(dfc_w, "dfc_w", (n, Cin), F32, optional=True)
    _need(dfc_b, "dfc_b", (n,), F32, optional=True)
    _same_gpu(x=x, fc_w=fc_w, alpha=alpha, dalpha=dalpha, dx=dx, dfc_w=dfc_w, dfc_b=dfc_b)
    if dfc_w is None:
        dfc_w = torch.empty((n, Cin), dtype=torch.float32, device=x.device)
    if dfc_b is None:
        dfc_b = torch.empty((n,), dtype=torch.float32, device=x.device)
    ws, ws_bytes = _workspace(dynconv_route_backward_workspace_bytes(desc), x.device, workspace)
    _check(lib().dynconv_route_backward(ctypes.byref(desc), _ptr(x), _ptr(fc_w), int(mode),
                                        float(temperature), _ptr(alpha), _ptr(dalpha), _ptr(dfc_w),
                                        _ptr(dfc_b), _ptr(dx), _ptr(ws), ws_bytes, _stream(stream)),
           "dynconv_route_backward")
    return dfc_w, dfc_b


def dynconv_forward_sparse_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_forward_sparse_workspace_bytes(ctypes.byref(desc)))


def dynconv_forward_sparse(x: torch.Tensor, experts: torch.Tensor, alpha: torch.Tensor, mask: torch.Tensor,
                           stride: int = 1, pad: int = 0, groups: int = 1, residual: bool = False,
                           y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """y = (x if residual else 0) + mask * layer(x); mask [B, Ho, Wo] uint8 (nonzero = evaluate)."""
    desc = layer_desc(x, experts, stride, pad, groups)
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, stride, pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W))
    _need(experts, "experts", tuple(experts.shape))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(mask, "mask", (desc.B, Ho, Wo), torch.uint8)
    _need(y, "y", (desc.B, desc.Cout, Ho, Wo), x.dtype, optional=True)
    _same_gpu(x=x, experts=experts, alpha=alpha, mask=mask, y=y)
    if y is None:
        y = torch.empty((desc.B, desc.Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    ws, ws_bytes = _workspace(dynconv_forward_sparse_workspace_bytes(desc), x.device, workspace)
    _check(lib().dynconv_forward_sparse(ctypes.byref(desc), _ptr(x), _ptr(experts), _ptr(alpha), _ptr(mask),
                                        int(bool(residual)), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "dynconv_forward_sparse")
    return y


def dynconv_forward_sparse_packed_workspace_bytes(desc: dynconv_desc_t) -> int:
    return int(lib().dynconv_forward_sparse_packed_workspace_bytes(ctypes.byref(desc)))


def dynconv_forward_sparse_packed(desc: dynconv_desc_t, x: torch.Tensor, packed: torch.Tensor,
                                  alpha: torch.Tensor, mask: torch.Tensor, residual: bool = False,
                                  y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                  stream=None) -> torch.Tensor:
    """dynconv_forward_sparse with a bank packed by dynconv_pack_experts."""
    Ho, Wo = _out_hw(desc.H, desc.W, desc.kh, desc.kw, desc.stride, desc.pad)
    _need(x, "x", (desc.B, desc.Cin, desc.H, desc.W), torch.bfloat16)
    _need_bytes(packed, "packed", dynconv_packed_experts_bytes(desc))
    _need(alpha, "alpha", (desc.B, desc.n), F32)
    _need(mask, "mask", (desc.B, Ho, Wo), torch.uint8)
    _need(y, "y", (desc.B, desc.Cout, Ho, Wo), x.dtype, optional=True)
    _same_gpu(x=x, packed=packed, alpha=alpha, mask=mask, y=y)
    if y is None:
        y = torch.empty((desc.B, desc.Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    ws, ws_bytes = _workspace(dynconv_forward_sparse_packed_workspace_bytes(desc), x.device, workspace)
    _check(lib().dynconv_forward_sparse_packed(ctypes.byref(desc), _ptr(x), _ptr(packed), _ptr(alpha), _ptr(mask),
                                               int(bool(residual)), _ptr(y), _ptr(ws), ws_bytes,
                                               _stream(stream)),
           "dynconv_forward_sparse_packed")
    return y

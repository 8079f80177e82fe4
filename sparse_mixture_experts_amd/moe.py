"""Thin ctypes binding of libsmoe.so (declared in include/moe.h).

Argument marshalling only: torch tensors provide device memory and the current HIP
stream; every step of the layer runs in the library's kernels.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTE_SOFTMAX_TOPK_RENORM, MOE_ROUTE_TOPK_SOFTMAX = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_SWIGLU_OAI = 0, 1
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_GROUPED = 0, 1, 2
MOE_EXPERTS_DENSE, MOE_EXPERTS_MXFP4, MOE_EXPERTS_Q4K = 0, 1, 2

_ROUTE = {"softmax_topk_renorm": MOE_ROUTE_SOFTMAX_TOPK_RENORM, "topk_softmax": MOE_ROUTE_TOPK_SOFTMAX}
_ACT = {"swiglu": MOE_ACT_SWIGLU, "swiglu_oai": MOE_ACT_SWIGLU_OAI}
_PATH = {"auto": MOE_PATH_AUTO, "decode": MOE_PATH_DECODE, "grouped": MOE_PATH_GROUPED}
_EXPERTS = {"dense": MOE_EXPERTS_DENSE, "mxfp4": MOE_EXPERTS_MXFP4, "q4k": MOE_EXPERTS_Q4K}

_P = ctypes.c_void_p


class MoeLayer(ctypes.Structure):
    """Mirror of ``moe_layer`` (9 int32, 3 float, 12 pointers at byte offset 48, then 2
    int32 and 2 pointers at offset 144)."""
    _fields_ = [
        ("d", ctypes.c_int32), ("n_expert", ctypes.c_int32), ("ff", ctypes.c_int32),
        ("k", ctypes.c_int32), ("shared_ff", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("route", ctypes.c_int32), ("act", ctypes.c_int32), ("path", ctypes.c_int32),
        ("route_scale", ctypes.c_float), ("oai_alpha", ctypes.c_float), ("oai_limit", ctypes.c_float),
        ("w_router", _P), ("b_router", _P), ("w_gate", _P), ("w_up", _P),
        ("w_gate_up", _P), ("b_gate_up", _P), ("w_down", _P), ("b_down", _P),
        ("ws_gate", _P), ("ws_up", _P), ("ws_down", _P), ("ws_gate_inp", _P),
        ("expert_format", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("w_gate_up_scales", _P), ("w_down_scales", _P), ("grouped_pack", _P),
    ]


POINTER_FIELDS = [f for f, t in MoeLayer._fields_ if t is _P]
ABI_VERSION = 4
EXPORTS = ["moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_route",
           "moe_permute_workspace_size", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_shell", "moe_forward_noalloc", "moe_grouped_pack_size",
           "moe_grouped_pack"]
# Bytes of the library's fixed scratch array behind moe_forward_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        pl = ctypes.POINTER(MoeLayer)
        L.moe_abi_version.restype = i32
        L.moe_abi_version.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_workspace_size.restype = i32
        L.moe_workspace_size.argtypes = [pl, i32, ctypes.POINTER(sz)]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [pl, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_permute_workspace_size.restype = i32
        L.moe_permute_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_permute.restype = i32
        L.moe_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn.restype = i32
        L.moe_expert_ffn.argtypes = [pl, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [pl, vp, vp, vp, vp, i32, vp, vp]
        L.moe_forward.restype = i32
        L.moe_forward.argtypes = [pl, vp, i32, vp, vp, sz, vp]
        L.moe_forward_shell.restype = i32
        L.moe_forward_shell.argtypes = [pl, vp, i32, vp, ctypes.c_float, vp, vp, sz, vp]
        L.moe_forward_noalloc.restype = i32
        L.moe_forward_noalloc.argtypes = [pl, vp, i32, vp, vp]
        L.moe_grouped_pack_size.restype = i32
        L.moe_grouped_pack_size.argtypes = [pl, ctypes.POINTER(sz)]
        L.moe_grouped_pack.restype = i32
        L.moe_grouped_pack.argtypes = [pl, vp, sz, vp]
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError("libsmoe.so ABI version mismatch")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


# ----------------------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _want(t, name, dtype, shape=None, numel=None):
    """Reject a tensor argument the kernels would read or write out of bounds: wrong
    dtype, shape or element count, a non-contiguous view, or memory that is not on the
    current HIP device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda" or t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, expected the current device "
                         f"cuda:{torch.cuda.current_device()}")
    return t


def _want_ws(ws, layer, T):
    torch = _torch()
    return _want(ws, "ws", torch.uint8, numel=workspace_size(layer, T) if T > 0 else None)


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def to_device(a: np.ndarray | None, device="cuda"):
    """A stored numpy tensor (uint16 bf16 bits or float32) as a torch tensor on device."""
    if a is None:
        return None
    torch = _torch()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class Layer:
    """A layer's parameters resident on the device plus the ``moe_layer`` struct that
    points at them.  Holds references so the tensors outlive the struct."""

    def __init__(self, d, n_expert, ff, k, shared_ff, dtype, route, act, route_scale=1.0,
                 oai_alpha=1.702, oai_limit=7.0, path="auto", expert_format="dense", **tensors):
        self.tensors = dict(tensors)
        self.d, self.n_expert, self.ff, self.k, self.shared_ff = d, n_expert, ff, k, shared_ff
        self.dtype = dtype
        s = MoeLayer()
        s.d, s.n_expert, s.ff, s.k, s.shared_ff = d, n_expert, ff, k, shared_ff
        s.dtype = MOE_BF16 if dtype == "bf16" else MOE_F32
        s.route, s.act, s.path = _ROUTE[route], _ACT[act], _PATH[path]
        s.route_scale, s.oai_alpha, s.oai_limit = route_scale, oai_alpha, oai_limit
        s.expert_format = _EXPERTS[expert_format]
        self.expert_format = expert_format
        for name in POINTER_FIELDS:
            setattr(s, name, _ptr(self.tensors.get(name)))
        self.struct = s

    @classmethod
    def from_arrays(cls, L: dict, device="cuda", path="auto"):
        """From a layer dict of the input generator (numpy storage arrays)."""
        tensors = {n: to_device(L.get(n), device) for n in POINTER_FIELDS}
        return cls(L["d"], L["n_expert"], L["ff"], L["k"], L["shared_ff"], L["dtype"], L["route"],
                   L["act"], L.get("route_scale", 1.0), L.get("oai_alpha", 1.702),
                   L.get("oai_limit", 7.0), path=path, expert_format=L.get("expert_format", "dense"),
                   **tensors)

    def with_grouped_pack(self) -> "Layer":
        """A copy of this bf16 layer whose grouped kernels read the grouped copy of the
        expert weights (moe_grouped_pack), written now on the current stream into a new
        device buffer that the returned layer holds."""
        torch = _torch()
        n = ctypes.c_size_t(0)
        _check(lib().moe_grouped_pack_size(self.ref(), ctypes.byref(n)), "moe_grouped_pack_size")
        dev = self.tensors["w_down"].device
        buf = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
        _check(lib().moe_grouped_pack(self.ref(), _ptr(buf), n.value, _stream()), "moe_grouped_pack")
        other = Layer.__new__(Layer)
        other.__dict__.update(self.__dict__)
        other.tensors = dict(self.tensors, grouped_pack=buf)
        other.struct = MoeLayer.from_buffer_copy(self.struct)
        other.struct.grouped_pack = _ptr(buf)
        return other

    def with_path(self, path: str) -> "Layer":
        other = Layer.__new__(Layer)
        other.__dict__.update(self.__dict__)
        other.struct = MoeLayer.from_buffer_copy(self.struct)
        other.struct.path = _PATH[path]
        return other

    @property
    def torch_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def ref(self):
        return ctypes.byref(self.struct)


def workspace_size(layer: Layer, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(layer.ref(), int(T), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def workspace(layer: Layer, T: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(workspace_size(layer, T), 1), dtype=torch.uint8, device=device)


def route(layer: Layer, x, ws=None):
    """(topk_idx int32 [T,k], topk_w fp32 [T,k], shared_gate fp32 [T] or None)."""
    torch = _torch()
    T = x.shape[0]
    _want(x, "x", layer.torch_dtype, (T, layer.d))
    ws = workspace(layer, T, x.device) if ws is None else _want_ws(ws, layer, T)
    idx = torch.empty((T, layer.k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, layer.k), dtype=torch.float32, device=x.device)
    sg = torch.empty(T, dtype=torch.float32, device=x.device) if layer.shared_ff else None
    _check(lib().moe_route(layer.ref(), _ptr(x), T, _ptr(idx), _ptr(w), _ptr(sg), _ptr(ws),
                           ws.numel(), _stream()), "moe_route")
    return idx, w, sg


def permute(topk_idx, n_expert: int):
    """(expert_offsets [E+1], perm_token [T*k], perm_inv [T*k]) int32."""
    torch = _torch()
    T, k = topk_idx.shape
    _want(topk_idx, "topk_idx", torch.int32, (T, k))
    n = ctypes.c_size_t(0)
    _check(lib().moe_permute_workspace_size(T, k, n_expert, ctypes.byref(n)), "moe_permute_workspace_size")
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=topk_idx.device)
    off = torch.empty(n_expert + 1, dtype=torch.int32, device=topk_idx.device)
    pt = torch.empty(T * k, dtype=torch.int32, device=topk_idx.device)
    pi = torch.empty(T * k, dtype=torch.int32, device=topk_idx.device)
    _check(lib().moe_permute(_ptr(topk_idx), T, k, n_expert, _ptr(off), _ptr(pt), _ptr(pi),
                             _ptr(ws), ws.numel(), _stream()), "moe_permute")
    return off, pt, pi


def expert_ffn(layer: Layer, x, expert_offsets, perm_token, ws=None):
    """y_perm fp32 [T*k (+T), d]."""
    torch = _torch()
    T = x.shape[0]
    rows = T * layer.k + (T if layer.shared_ff else 0)
    _want(x, "x", layer.torch_dtype, (T, layer.d))
    _want(expert_offsets, "expert_offsets", torch.int32, (layer.n_expert + 1,))
    _want(perm_token, "perm_token", torch.int32, (T * layer.k,))
    ws = workspace(layer, T, x.device) if ws is None else _want_ws(ws, layer, T)
    y = torch.empty((rows, layer.d), dtype=torch.float32, device=x.device)
    _check(lib().moe_expert_ffn(layer.ref(), _ptr(x), T, _ptr(expert_offsets), _ptr(perm_token),
                                _ptr(y), _ptr(ws), ws.numel(), _stream()), "moe_expert_ffn")
    return y


def combine(layer: Layer, y_perm, perm_inv, topk_w, shared_gate):
    torch = _torch()
    T = topk_w.shape[0]
    rows = T * layer.k + (T if layer.shared_ff else 0)
    _want(topk_w, "topk_w", torch.float32, (T, layer.k))
    _want(y_perm, "y_perm", torch.float32, (rows, layer.d))
    _want(perm_inv, "perm_inv", torch.int32, (T * layer.k,))
    if shared_gate is not None:
        _want(shared_gate, "shared_gate", torch.float32, (T,))
    y = torch.empty((T, layer.d), dtype=layer.torch_dtype, device=topk_w.device)
    _check(lib().moe_combine(layer.ref(), _ptr(y_perm), _ptr(perm_inv), _ptr(topk_w), _ptr(shared_gate),
                             T, _ptr(y), _stream()), "moe_combine")
    return y


def forward(layer: Layer, x, ws=None, out=None):
    """The whole layer: y [T, d] in the layer dtype."""
    torch = _torch()
    T = x.shape[0]
    _want(x, "x", layer.torch_dtype, (T, layer.d))
    ws = workspace(layer, T, x.device) if ws is None else _want_ws(ws, layer, T)
    y = torch.empty((T, layer.d), dtype=layer.torch_dtype, device=x.device) if out is None else out
    _want(y, "out", layer.torch_dtype, (T, layer.d))
    _check(lib().moe_forward(layer.ref(), _ptr(x), T, _ptr(y), _ptr(ws), ws.numel(), _stream()),
           "moe_forward")
    return y


def forward_shell(layer: Layer, h, norm_w, eps: float = 1e-5, ws=None, out=None):
    """out = h + MoE(RMSNorm(h) * norm_w) [T, d] in the layer dtype; ``out`` may be ``h``
    itself (in-place residual update)."""
    torch = _torch()
    T = h.shape[0]
    _want(h, "h", layer.torch_dtype, (T, layer.d))
    _want(norm_w, "norm_w", layer.torch_dtype, (layer.d,))
    ws = workspace(layer, T, h.device) if ws is None else _want_ws(ws, layer, T)
    y = torch.empty((T, layer.d), dtype=layer.torch_dtype, device=h.device) if out is None else out
    _want(y, "out", layer.torch_dtype, (T, layer.d))
    _check(lib().moe_forward_shell(layer.ref(), _ptr(h), T, _ptr(norm_w), float(eps), _ptr(y), _ptr(ws),
                                   ws.numel(), _stream()), "moe_forward_shell")
    return y


def forward_noalloc(layer: Layer, x, out=None):
    """moe_forward_noalloc: the whole layer with the library's fixed scratch array as the
    workspace (no workspace argument, nothing allocated by the call beyond ``out`` when
    it is not given).  Raises MoeError (MOE_ERR_WORKSPACE) when the batch needs more than
    NOALLOC_SCRATCH_BYTES of workspace."""
    torch = _torch()
    T = x.shape[0]
    _want(x, "x", layer.torch_dtype, (T, layer.d))
    y = torch.empty((T, layer.d), dtype=layer.torch_dtype, device=x.device) if out is None else out
    _want(y, "out", layer.torch_dtype, (T, layer.d))
    _check(lib().moe_forward_noalloc(layer.ref(), _ptr(x), T, _ptr(y), _stream()), "moe_forward_noalloc")
    return y

"""ctypes binding of libmoe_mi355x.so: the C ABI's entry points under the same
names, taking torch tensors.  Argument marshalling only -- every step of the
layer runs in the library's HIP kernels.  There is no fallback: if the library
is missing the import of this module's functions raises."""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_FFN_AUTO, MOE_FFN_TILED, MOE_FFN_STREAM = 0, 1, 2
MOE_H_AUTO, MOE_H_BF16, MOE_H_SPLIT = 0, 1, 2
MOE_CAPACITY_DROP, MOE_CAPACITY_REROUTE = 0, 1
_POLICIES = {"drop": MOE_CAPACITY_DROP, "reroute": MOE_CAPACITY_REROUTE}

ENTRY_POINTS = ("moe_status_string", "moe_last_error", "moe_workspace_size", "moe_query_plan",
                "moe_route", "moe_permute", "moe_ffn_up", "moe_ffn_up_gather", "moe_ffn_down", "moe_grouped_ffn",
                "moe_shared_ffn", "moe_combine", "moe_forward", "moe_forward_noalloc",
                "moe_read_probe")


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class CDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("tokens", "d_model", "d_ff", "n_experts", "top_k", "renormalize", "capacity",
                 "dtype", "has_expert_bias", "ffn_path", "h_mode", "d_ff_shared",
                 "capacity_policy")]


class CPlan(ctypes.Structure):
    _fields_ = [("ffn_path", ctypes.c_int32), ("h_mode", ctypes.c_int32),
                ("h_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]


class CWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "b_router", "w1", "b1", "w2", "b2",
                                               "b_select", "w1_shared", "b1_shared", "w2_shared",
                                               "b2_shared")]


class CRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "counts", "offsets", "dest", "src", "top1_count",
                 "prob_mean", "z_loss", "reroute_rounds")]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_mixture_experts_49_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    pd, pw, pr = ctypes.POINTER(CDesc), ctypes.POINTER(CWeights), ctypes.POINTER(CRouting)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [I]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_workspace_size": (I, [pd, ctypes.POINTER(S)]),
        "moe_query_plan": (I, [pd, ctypes.POINTER(CPlan)]),
        "moe_route": (I, [pd, P, pw, pr, P, P, S, P]),
        "moe_permute": (I, [pd, P, pr, P, P, S, P]),
        "moe_ffn_up": (I, [pd, P, P, pw, P, P, S, P]),
        "moe_ffn_up_gather": (I, [pd, P, P, P, pw, P, P, S, P]),
        "moe_ffn_down": (I, [pd, P, P, pw, P, P, S, P]),
        "moe_grouped_ffn": (I, [pd, P, P, pw, P, P, P, S, P]),
        "moe_shared_ffn": (I, [pd, P, pw, P, P, S, P]),
        "moe_combine": (I, [pd, P, P, P, P, P, P]),
        "moe_forward": (I, [pd, P, pw, P, P, pr, P, S, P]),
        "moe_forward_noalloc": (I, [pd, P, pw, P, P, pr, P]),
        "moe_read_probe": (I, [P, S, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


@dataclasses.dataclass
class Desc:
    tokens: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    renormalize: bool = True
    capacity: int = 0
    dtype: str = "bf16"          # "bf16" or "f32"
    has_expert_bias: bool = True
    ffn_path: int = MOE_FFN_AUTO
    h_mode: int = MOE_H_AUTO
    d_ff_shared: int = 0          # shared expert width, 0 = none
    capacity_policy: str = "drop"  # "drop" or "reroute": what happens past the capacity

    def to_c(self) -> CDesc:
        return CDesc(self.tokens, self.d_model, self.d_ff, self.n_experts, self.top_k,
                     int(bool(self.renormalize)), self.capacity,
                     MOE_DTYPE_BF16 if self.dtype == "bf16" else MOE_DTYPE_F32,
                     int(bool(self.has_expert_bias)), self.ffn_path, self.h_mode, self.d_ff_shared,
                     _POLICIES.get(self.capacity_policy, -1))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


@dataclasses.dataclass
class Weights:
    w_router: torch.Tensor
    w1: torch.Tensor
    w2: torch.Tensor
    b_router: Optional[torch.Tensor] = None
    b1: Optional[torch.Tensor] = None
    b2: Optional[torch.Tensor] = None
    b_select: Optional[torch.Tensor] = None
    w1_shared: Optional[torch.Tensor] = None
    b1_shared: Optional[torch.Tensor] = None
    w2_shared: Optional[torch.Tensor] = None
    b2_shared: Optional[torch.Tensor] = None

    def to_c(self) -> CWeights:
        return CWeights(*(_ptr(getattr(self, n)) for n, _ in CWeights._fields_))


@dataclasses.dataclass
class Routing:
    topk_idx: Optional[torch.Tensor] = None
    topk_w: Optional[torch.Tensor] = None
    counts: Optional[torch.Tensor] = None
    offsets: Optional[torch.Tensor] = None
    dest: Optional[torch.Tensor] = None
    src: Optional[torch.Tensor] = None
    top1_count: Optional[torch.Tensor] = None
    prob_mean: Optional[torch.Tensor] = None
    z_loss: Optional[torch.Tensor] = None
    reroute_rounds: Optional[torch.Tensor] = None

    @classmethod
    def allocate(cls, desc: Desc, device) -> "Routing":
        T, k, E = desc.tokens, desc.top_k, desc.n_experts
        i32 = dict(dtype=torch.int32, device=device)
        return cls(topk_idx=torch.empty(T, k, **i32),
                   topk_w=torch.empty(T, k, dtype=torch.float32, device=device),
                   counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                   dest=torch.empty(T, k, **i32), src=torch.empty(T * k, **i32),
                   top1_count=torch.empty(E, **i32),
                   prob_mean=torch.empty(E, dtype=torch.float32, device=device),
                   z_loss=torch.empty(1, dtype=torch.float32, device=device),
                   reroute_rounds=torch.empty(1, **i32))

    def to_c(self) -> CRouting:
        return CRouting(*(_ptr(getattr(self, f.name)) for f in dataclasses.fields(self)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _expected(desc: "Desc") -> dict:
    """(dtype, element count) of every array the C ABI sizes from the descriptor,
    by argument name (the same shapes the library's alias and bounds logic uses)."""
    T, d, F, E, k, Fs = (desc.tokens, desc.d_model, desc.d_ff, desc.n_experts, desc.top_k,
                         desc.d_ff_shared)
    dt, f32, i32 = desc.torch_dtype, torch.float32, torch.int32
    return {"x": (dt, T * d), "w_router": (dt, E * d), "b_router": (f32, E), "b_select": (f32, E),
            "w1": (dt, E * F * d), "b1": (dt, E * F), "w2": (dt, E * d * F), "b2": (dt, E * d),
            "w1_shared": (dt, Fs * d), "b1_shared": (dt, Fs), "w2_shared": (dt, d * Fs),
            "b2_shared": (dt, d),
            "topk_idx": (i32, T * k), "topk_w": (f32, T * k), "counts": (i32, E),
            "offsets": (i32, E + 1), "dest": (i32, T * k), "src": (i32, T * k),
            "top1_count": (i32, E), "prob_mean": (f32, E), "z_loss": (f32, 1),
            "reroute_rounds": (i32, 1),
            "x_perm": (dt, T * k * d), "o": (f32, T * k * d), "y": (f32, T * d),
            "o_shared": (f32, T * d), "aux": (f32, 1)}


def check_tensor(t, name: str, dtype, numel: int, device) -> None:
    """Refuse, before any call into the library, a tensor the library would read or
    write out of bounds or misinterpret: not on `device` (a GPU), wrong dtype, fewer
    than `numel` elements, or not contiguous.  Raw integer pointers are the
    caller's responsibility and pass unchecked."""
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise MoeError(MOE_ERR_INVALID, f"{name} must be a torch tensor, an int pointer or None")
    if (t.device != device) if device is not None else (t.device.type != "cuda"):
        raise MoeError(MOE_ERR_INVALID, f"{name} is on {t.device}, expected {device or 'a GPU'}")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(MOE_ERR_INVALID, f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() < numel:
        raise MoeError(MOE_ERR_INVALID, f"{name} has {t.numel()} elements, needs {numel}")
    if not t.is_contiguous():
        raise MoeError(MOE_ERR_INVALID, f"{name} must be contiguous")


def _device_of(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor):
            return t.device
    return None


class _Args:
    """Checks the tensors of one call against the descriptor (see check_tensor)."""

    def __init__(self, desc: "Desc", *anchor):
        self.desc = desc
        self.want = _expected(desc)
        self.device = _device_of(*anchor)
        if self.device is not None and self.device.type != "cuda":
            raise MoeError(MOE_ERR_INVALID, f"tensors are on {self.device}, expected a GPU")

    def t(self, t, name, key=None):
        dtype, n = self.want[key or name]
        check_tensor(t, name, dtype, n, self.device)
        return _ptr(t)

    def weights(self, w: "Weights", router: bool, experts: bool):
        names = (("w_router", "b_router", "b_select") if router else ()) + \
                (("w1", "b1", "w2", "b2", "w1_shared", "b1_shared", "w2_shared", "b2_shared")
                 if experts else ())
        for n in names:
            self.t(getattr(w, n), "weights." + n, n)
        return ctypes.byref(w.to_c())

    def routing(self, r: "Routing"):
        for f in dataclasses.fields(r):
            self.t(getattr(r, f.name), "routing." + f.name, f.name)
        return ctypes.byref(r.to_c())

    def h(self, t):
        if t is None or isinstance(t, int):
            return _ptr(t)
        plan = moe_query_plan(self.desc)
        check_tensor(t, "h", self.desc.torch_dtype, 0, self.device)
        if t.numel() * t.element_size() < plan["h_bytes"]:
            raise MoeError(MOE_ERR_INVALID, f"h has {t.numel() * t.element_size()} bytes, "
                                            f"needs {plan['h_bytes']}")
        return _ptr(t)

    def ws(self, t):
        """(pointer, bytes) of the workspace; None allocates one of the right size."""
        if t is None:
            t = alloc_workspace(self.desc, self.device)
        if isinstance(t, int):
            raise MoeError(MOE_ERR_INVALID, "pass the workspace as a tensor (its size is needed)")
        check_tensor(t, "workspace", None, 0, self.device)
        self._ws_keep = t
        return _ptr(t), t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(status: int):
    if status != MOE_OK:
        lib = load_library()
        raise MoeError(status, lib.moe_last_error().decode() or lib.moe_status_string(status).decode())


def moe_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(ctypes.byref(desc.to_c()), ctypes.byref(n)))
    return n.value


def moe_query_plan(desc: Desc) -> dict:
    """Resolved kernel path, h storage mode, h buffer bytes and workspace bytes."""
    p = CPlan()
    _check(load_library().moe_query_plan(ctypes.byref(desc.to_c()), ctypes.byref(p)))
    return {"ffn_path": p.ffn_path, "h_mode": p.h_mode, "h_bytes": p.h_bytes,
            "workspace_bytes": p.workspace_bytes}


def alloc_h(desc: Desc, device) -> torch.Tensor:
    """A buffer for the post-GELU activations as moe_ffn_up writes them."""
    plan = moe_query_plan(desc)
    rows = desc.tokens * desc.top_k
    if desc.dtype == "f32":
        return torch.empty(rows, desc.d_ff, dtype=torch.float32, device=device)
    if plan["h_mode"] == MOE_H_SPLIT:
        return torch.empty(2, rows, desc.d_ff, dtype=torch.bfloat16, device=device)
    return torch.empty(rows, desc.d_ff, dtype=torch.bfloat16, device=device)


def alloc_workspace(desc: Desc, device) -> torch.Tensor:
    return torch.empty(moe_workspace_size(desc), dtype=torch.uint8, device=device)


def moe_route(desc, x, weights, routing, aux=None, workspace=None, stream=None):
    a = _Args(desc, x)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_route(ctypes.byref(desc.to_c()), a.t(x, "x"), a.weights(weights, True, False),
                                    a.routing(routing), a.t(aux, "aux"), ws, nb, _stream(stream)))


def moe_permute(desc, x, routing, x_perm, workspace=None, stream=None):
    a = _Args(desc, x)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_permute(ctypes.byref(desc.to_c()), a.t(x, "x"), a.routing(routing),
                                      a.t(x_perm, "x_perm"), ws, nb, _stream(stream)))


def moe_ffn_up(desc, x_perm, offsets, weights, h, workspace=None, stream=None):
    a = _Args(desc, x_perm)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_ffn_up(ctypes.byref(desc.to_c()), a.t(x_perm, "x_perm"),
                                     a.t(offsets, "offsets"), a.weights(weights, False, True), a.h(h),
                                     ws, nb, _stream(stream)))


def moe_ffn_up_gather(desc, x, src, offsets, weights, h, workspace=None, stream=None):
    a = _Args(desc, x)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_ffn_up_gather(ctypes.byref(desc.to_c()), a.t(x, "x"), a.t(src, "src"),
                                            a.t(offsets, "offsets"), a.weights(weights, False, True),
                                            a.h(h), ws, nb, _stream(stream)))


def moe_ffn_down(desc, h, offsets, weights, o, workspace=None, stream=None):
    a = _Args(desc, h)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_ffn_down(ctypes.byref(desc.to_c()), a.h(h), a.t(offsets, "offsets"),
                                       a.weights(weights, False, True), a.t(o, "o"), ws, nb,
                                       _stream(stream)))


def moe_grouped_ffn(desc, x_perm, offsets, weights, h, o, workspace=None, stream=None):
    a = _Args(desc, x_perm)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_grouped_ffn(ctypes.byref(desc.to_c()), a.t(x_perm, "x_perm"),
                                          a.t(offsets, "offsets"), a.weights(weights, False, True),
                                          a.h(h), a.t(o, "o"), ws, nb, _stream(stream)))


def moe_shared_ffn(desc, x, weights, o_shared, workspace=None, stream=None):
    a = _Args(desc, x)
    ws, nb = a.ws(workspace)
    _check(load_library().moe_shared_ffn(ctypes.byref(desc.to_c()), a.t(x, "x"),
                                         a.weights(weights, False, True),
                                         a.t(o_shared, "o_shared"), ws, nb, _stream(stream)))


def moe_combine(desc, o, dest, topk_w, y, o_shared=None, stream=None):
    a = _Args(desc, o)
    _check(load_library().moe_combine(ctypes.byref(desc.to_c()), a.t(o, "o"), a.t(dest, "dest"),
                                      a.t(topk_w, "topk_w"), a.t(o_shared, "o_shared"), a.t(y, "y"),
                                      _stream(stream)))


def moe_forward(desc, x, weights, y, aux=None, routing=None, workspace=None, stream=None):
    a = _Args(desc, x)
    ws, nb = a.ws(workspace)
    r = a.routing(routing) if routing is not None else None
    _check(load_library().moe_forward(ctypes.byref(desc.to_c()), a.t(x, "x"),
                                      a.weights(weights, True, True), a.t(y, "y"), a.t(aux, "aux"), r,
                                      ws, nb, _stream(stream)))


def moe_forward_noalloc(desc, x, weights, y, aux=None, routing=None, stream=None):
    """moe_forward on the library's own device scratch (no workspace, no allocation)."""
    a = _Args(desc, x)
    r = a.routing(routing) if routing is not None else None
    _check(load_library().moe_forward_noalloc(ctypes.byref(desc.to_c()), a.t(x, "x"),
                                              a.weights(weights, True, True), a.t(y, "y"),
                                              a.t(aux, "aux"), r, _stream(stream)))


def moe_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """One plain streaming read of buf (a measurement aid, not part of the layer)."""
    check_tensor(buf, "buf", None, 0, None)
    check_tensor(sink, "sink", torch.int32, 1, buf.device)
    _check(load_library().moe_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                         _stream(stream)))


def forward(x: torch.Tensor, weights: Weights, desc: Desc, workspace=None, stream=None):
    """The layer's module-style call: returns (y [T, d] fp32, aux fp32 scalar tensor)."""
    y = torch.empty(desc.tokens, desc.d_model, dtype=torch.float32, device=x.device)
    aux = torch.empty((), dtype=torch.float32, device=x.device)
    moe_forward(desc, x, weights, y, aux, None, workspace, stream)
    return y, aux

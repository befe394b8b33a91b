"""Python binding of libmoe.so, the C ABI declared in include/moe.h.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors supply device memory and streams; their data
pointers and the current HIP stream are passed through ctypes.  There is no
CPU fallback: if libmoe.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL = 1
MOE_ERR_SHAPE = 2
MOE_ERR_FORMAT = 3
MOE_ERR_ALIGN = 4
MOE_ERR_ROWS = 5
MOE_ERR_WORKSPACE = 6
MOE_ERR_ALIAS = 7
MOE_ERR_HIP = 8

MOE_DEVERR_NONFINITE_SCORE = 0x1
MOE_DEVERR_NONFINITE_MID = 0x2
MOE_DEVERR_WAIT_TIMEOUT = 0x4

MOE_FMT_FP8_B128 = 0
MOE_FMT_MXFP4 = 1
MOE_BIAS_F32 = 0
MOE_BIAS_BF16 = 1


class MoeConfig(C.Structure):
    _fields_ = [("hidden", C.c_int), ("inter", C.c_int), ("shared_inter", C.c_int),
                ("n_experts", C.c_int), ("top_k", C.c_int), ("n_group", C.c_int),
                ("topk_group", C.c_int), ("n_shared", C.c_int), ("routed_scale", C.c_float),
                ("routed_fmt", C.c_int), ("shared_fmt", C.c_int), ("bias_dtype", C.c_int),
                ("max_rows", C.c_int)]


class MoeWeights(C.Structure):
    _fields_ = [("router_w", C.c_void_p), ("bias", C.c_void_p),
                ("w_gate_up", C.c_void_p), ("s_gate_up", C.c_void_p),
                ("w_down", C.c_void_p), ("s_down", C.c_void_p),
                ("sh_w_gate_up", C.c_void_p), ("sh_s_gate_up", C.c_void_p),
                ("sh_w_down", C.c_void_p), ("sh_s_down", C.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} (code {code})")


_lib = None


def lib() -> C.CDLL:
    """The loaded libmoe.so (raises if it is missing: no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_decode_sigmoid_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I, Z = C.c_void_p, C.c_int, C.c_size_t
        L.moe_workspace_size.argtypes = [C.POINTER(MoeConfig), C.POINTER(C.c_size_t)]
        L.moe_workspace_init.argtypes = [P, Z, P]
        L.moe_route.argtypes = [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, P, Z, P]
        L.moe_groups.argtypes = [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, Z, P]
        L.moe_forward.argtypes = [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, Z, P]
        L.moe_forward_residual.argtypes = [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, P, Z, P]
        L.moe_read_error.argtypes = [P, P, C.POINTER(C.c_uint32)]
        L.moe_strerror.argtypes = [I]
        L.moe_strerror.restype = C.c_char_p
        L.moe_last_hip_error.argtypes = []
        for f in ("moe_workspace_size", "moe_workspace_init", "moe_route", "moe_groups",
                  "moe_forward", "moe_forward_residual", "moe_read_error", "moe_last_hip_error"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


EXPORTS = ("moe_workspace_size", "moe_workspace_init", "moe_route", "moe_groups",
           "moe_forward", "moe_forward_residual", "moe_read_error", "moe_strerror", "moe_last_hip_error")


def strerror(code: int) -> str:
    return lib().moe_strerror(int(code)).decode()


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def make_config(spec: dict, max_rows: int) -> MoeConfig:
    """spec: the layer's sizes and routing parameters (see fixtures.SPECS)."""
    return MoeConfig(int(spec["hidden"]), int(spec["inter"]), int(spec["shared_inter"]),
                     int(spec["n_experts"]), int(spec["top_k"]), int(spec["n_group"]),
                     int(spec["topk_group"]), int(spec["n_shared"]), float(spec["routed_scale"]),
                     int(spec["routed_fmt"]), MOE_FMT_FP8_B128,
                     MOE_BIAS_BF16 if spec["bias_bf16"] else MOE_BIAS_F32, int(max_rows))


def make_weights(case: dict) -> MoeWeights:
    """case: device tensors named as in fixtures.make_case."""
    g = case.get
    return MoeWeights(_ptr(g("router_w")), _ptr(g("bias")), _ptr(g("w_gate_up")), _ptr(g("s_gate_up")),
                      _ptr(g("w_down")), _ptr(g("s_down")), _ptr(g("sh_w_gate_up")),
                      _ptr(g("sh_s_gate_up")), _ptr(g("sh_w_down")), _ptr(g("sh_s_down")))


def moe_workspace_size(cfg: MoeConfig) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_workspace_size(C.byref(cfg), C.byref(n)), "moe_workspace_size")
    return int(n.value)


def moe_workspace_init(ws: torch.Tensor, stream=None):
    _check(lib().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_workspace_init")


def new_workspace(cfg: MoeConfig, device="cuda", stream=None) -> torch.Tensor:
    """Allocates (torch) and initialises a workspace for cfg."""
    ws = torch.empty(moe_workspace_size(cfg), dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream)
    return ws


def moe_route(cfg, w, x, ids, wts, ws, stream=None):
    """ids: [rows, K] int32, wts: [rows, K] float32 (device, written)."""
    _check(lib().moe_route(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(ids), _ptr(wts),
                           _ptr(ws), ws.numel(), _stream(stream)), "moe_route")


def moe_groups(cfg, w, x, out, ws, stream=None):
    """out: int32 device buffer of at least 4 + 3*(1 + rows*K) + rows*(K+1) entries."""
    _check(lib().moe_groups(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(out),
                            _ptr(ws), ws.numel(), _stream(stream)), "moe_groups")


def moe_forward(cfg, w, x, out, ws, stream=None):
    """x: [rows, H] bf16, out: [rows, H] bf16 (device)."""
    _check(lib().moe_forward(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(out),
                             _ptr(ws), ws.numel(), _stream(stream)), "moe_forward")


def moe_forward_residual(cfg, w, x, residual, out, ws, stream=None):
    """x, residual, out: [rows, H] bf16 (device); residual may be out."""
    _check(lib().moe_forward_residual(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(residual),
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "moe_forward_residual")


def moe_read_error(ws, stream=None) -> int:
    bits = C.c_uint32(0)
    _check(lib().moe_read_error(_ptr(ws), _stream(stream), C.byref(bits)), "moe_read_error")
    return int(bits.value)


def moe_last_hip_error() -> int:
    return int(lib().moe_last_hip_error())


# ---------------------------------------------------------------- convenience

class Layer:
    """Holds a config, weight pointers and a workspace for one device."""

    def __init__(self, spec: dict, case: dict, max_rows: int, device="cuda"):
        self.spec = spec
        self.case = case
        self.cfg = make_config(spec, max_rows)
        self.w = make_weights(case)
        self.ws = new_workspace(self.cfg, device)

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None, stream=None,
                residual: torch.Tensor | None = None) -> torch.Tensor:
        if out is None:
            out = torch.empty_like(x)
        if residual is None:
            moe_forward(self.cfg, self.w, x, out, self.ws, stream)
        else:
            moe_forward_residual(self.cfg, self.w, x, residual, out, self.ws, stream)
        return out

    def route(self, x: torch.Tensor, stream=None):
        K = self.spec["top_k"]
        ids = torch.empty(x.shape[0], K, dtype=torch.int32, device=x.device)
        wts = torch.empty(x.shape[0], K, dtype=torch.float32, device=x.device)
        moe_route(self.cfg, self.w, x, ids, wts, self.ws, stream)
        return ids, wts

    def groups(self, x: torch.Tensor, stream=None):
        T, K = x.shape[0], self.spec["top_k"]
        n = 4 + 3 * (1 + T * K) + T * (K + 1)
        buf = torch.full((n,), -7, dtype=torch.int32, device=x.device)
        moe_groups(self.cfg, self.w, x, buf, self.ws, stream)
        b = buf.cpu().tolist()
        G = b[0]
        ge, gn, gs = b[4:4 + G], b[4 + G:4 + 2 * G], b[4 + 2 * G:4 + 3 * G]
        ncol = T * (K + (1 if self.spec["n_shared"] else 0))
        cols = b[4 + 3 * G:4 + 3 * G + ncol]
        return ge, gn, gs, cols

    def read_error(self, stream=None) -> int:
        return moe_read_error(self.ws, stream)

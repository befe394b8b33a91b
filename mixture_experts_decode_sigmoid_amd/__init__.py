"""Python binding of libmoe.so, the C ABI declared in include/moe.h.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors supply device memory and streams; their data
pointers and the current HIP stream are passed through ctypes.  There is no
CPU fallback: if libmoe.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import contextlib
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
MOE_ERR_LAUNCH = 9

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
                ("max_rows", C.c_int), ("expert_first", C.c_int), ("expert_count", C.c_int)]


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
_lib_path = LIB_PATH


def use_library(path: str) -> None:
    """Load another build of the same library (e.g. the phase-stamp build)
    instead of libmoe.so; must be called before the first call."""
    global _lib_path
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    _lib_path = path


def load_library(path: str, strict: bool = True) -> C.CDLL:
    """Loads the build of the library at `path` with its argument types set.
    Several builds can be loaded side by side, each with its own kernels (the
    A/B tool does so).  strict=False skips entry points a build lacks."""
    L = C.CDLL(path)
    P, I, Z = C.c_void_p, C.c_int, C.c_size_t
    sig = {
        "moe_workspace_size": [C.POINTER(MoeConfig), C.POINTER(C.c_size_t)],
        "moe_workspace_init": [P, Z, P],
        "moe_route": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, P, Z, P],
        "moe_groups": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, Z, P],
        "moe_forward": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, Z, P],
        "moe_forward_residual": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, P, Z, P],
        "moe_read_error": [P, P, C.POINTER(C.c_uint32)],
        "moe_strerror": [I],
        "moe_last_hip_error": [],
        "moe_probe_stream_read": [P, Z, P, I, P],
        "moe_pack_mxfp4_scales": [P, P, I, I, P],
        "moe_forward_noalloc": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P],
        "moe_forward_prefill": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, Z, P],
        "moe_forward_unfused": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, P, P, Z, P],
        "moe_forward_after": [C.POINTER(MoeConfig), C.POINTER(MoeWeights), P, I, P, P, P, Z, P,
                              C.c_uint32, C.c_uint32, P],
    }
    for name, args in sig.items():
        try:
            f = getattr(L, name)
        except AttributeError:
            if strict:
                raise
            continue
        f.argtypes = args
        f.restype = C.c_char_p if name == "moe_strerror" else C.c_int
    return L


def lib() -> C.CDLL:
    """The loaded libmoe.so (raises if it is missing: no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_lib_path):
            raise RuntimeError(f"{_lib_path} is missing: build it with "
                               "`python -m mixture_experts_decode_sigmoid_amd.build`")
        _lib = load_library(_lib_path)
    return _lib


@contextlib.contextmanager
def using(L: C.CDLL):
    """Routes this module's calls to the loaded build L while the block runs."""
    global _lib
    prev = _lib
    _lib = L
    try:
        yield L
    finally:
        _lib = prev


EXPORTS = ("moe_workspace_size", "moe_workspace_init", "moe_route", "moe_groups",
           "moe_forward", "moe_forward_residual", "moe_read_error", "moe_strerror", "moe_last_hip_error",
           "moe_probe_stream_read", "moe_pack_mxfp4_scales", "moe_forward_noalloc", "moe_forward_after", "moe_forward_unfused",
           "moe_forward_prefill")


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
                     MOE_BIAS_BF16 if spec["bias_bf16"] else MOE_BIAS_F32, int(max_rows),
                     int(spec.get("expert_first", 0)), int(spec.get("expert_count", 0)))


def make_weights(case: dict) -> MoeWeights:
    """case: device tensors named as in fixtures.make_case."""
    g = case.get
    return MoeWeights(_ptr(g("router_w")), _ptr(g("bias")), _ptr(g("w_gate_up")), _ptr(g("s_gate_up")),
                      _ptr(g("w_down")), _ptr(g("s_down")), _ptr(g("sh_w_gate_up")),
                      _ptr(g("sh_s_gate_up")), _ptr(g("sh_w_down")), _ptr(g("sh_s_down")))


def moe_pack_mxfp4_scales(src: torch.Tensor, dst: torch.Tensor, rows: int, k: int, stream=None):
    """E8M0 scale bytes of `rows` rows of k elements from the [rows][k/32]
    grid (src) into the tiled layout the layer reads (dst, same size)."""
    _check(lib().moe_pack_mxfp4_scales(_ptr(src), _ptr(dst), int(rows), int(k), _stream(stream)),
           "moe_pack_mxfp4_scales")


def packed_weights(spec: dict, case: dict) -> dict:
    """The weight tensors the layer takes: case itself, or for MXFP4 routed
    experts a copy of case whose scale bytes are packed into the tiled layout
    (new device tensors; case keeps the [rows][k/32] grids)."""
    if int(spec["routed_fmt"]) != MOE_FMT_MXFP4 or case.get("s_gate_up") is None:
        return case
    out = dict(case)
    H, I = int(spec["hidden"]), int(spec["inter"])
    for key, k in (("s_gate_up", H), ("s_down", I)):
        src = case[key]
        dst = torch.empty_like(src)
        moe_pack_mxfp4_scales(src, dst, src.numel() // (k // 32), k)
        out[key] = dst
    return out


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


def moe_forward_noalloc(cfg, w, x, out, stream=None):
    """moe_forward with the library's static per-device workspace (no
    workspace argument, nothing allocated)."""
    _check(lib().moe_forward_noalloc(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(out),
                                     _stream(stream)), "moe_forward_noalloc")


def moe_forward_prefill(cfg, w, x, out, ws, stream=None):
    """Any number of rows: the fused pass over chunks of cfg.max_rows rows."""
    _check(lib().moe_forward_prefill(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(out), _ptr(ws),
                                     ws.numel(), _stream(stream)), "moe_forward_prefill")


def moe_forward_unfused(cfg, w, x, out, tmp_routed, tmp_shared, ws, stream=None):
    """The four-launch unfused layout of the same layer (routed MoE, shared
    gate/up, shared down, add); tmp_routed and tmp_shared: [rows, H] bf16."""
    _check(lib().moe_forward_unfused(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(out), _ptr(tmp_routed),
                                     _ptr(tmp_shared), _ptr(ws), ws.numel(), _stream(stream)), "moe_forward_unfused")


def moe_forward_after(cfg, w, x, out, ws, x_ready, x_ready_value: int, residual=None, max_polls: int = 0,
                      stream=None):
    """moe_forward (or with a residual) reading x only once the device word
    x_ready (int32/uint32 tensor, element 0) reaches x_ready_value."""
    _check(lib().moe_forward_after(C.byref(cfg), C.byref(w), _ptr(x), int(x.shape[0]), _ptr(residual), _ptr(out),
                                   _ptr(ws), ws.numel(), _ptr(x_ready), C.c_uint32(x_ready_value & 0xFFFFFFFF),
                                   C.c_uint32(max_polls), _stream(stream)), "moe_forward_after")


def moe_read_error(ws, stream=None) -> int:
    bits = C.c_uint32(0)
    _check(lib().moe_read_error(_ptr(ws), _stream(stream), C.byref(bits)), "moe_read_error")
    return int(bits.value)


def moe_last_hip_error() -> int:
    return int(lib().moe_last_hip_error())


def moe_probe_stream_read(buf, sink, blocks: int, stream=None):
    """buf: device tensor read once (bytes a multiple of 16); sink: int32
    device tensor of at least `blocks` entries (written)."""
    _check(lib().moe_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(blocks),
                                       _stream(stream)), "moe_probe_stream_read")


# ---------------------------------------------------------------- convenience

class Layer:
    """Holds a config, weight pointers and a workspace for one device."""

    def __init__(self, spec: dict, case: dict, max_rows: int, device="cuda", ws_extra: int = 0):
        self.spec = spec
        self.case = case
        self.cfg = make_config(spec, max_rows)
        # MXFP4 scales are packed once here (later changes to case's scale
        # tensors do not reach the layer)
        self.weights = packed_weights(spec, case)
        self.w = make_weights(self.weights)
        self.ws_bytes = moe_workspace_size(self.cfg)
        self.ws = torch.empty(self.ws_bytes + ws_extra, dtype=torch.uint8, device=device)
        moe_workspace_init(self.ws)

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
        cols = b[4 + 3 * G:4 + 3 * G + sum(gn)]
        return ge, gn, gs, cols

    def read_error(self, stream=None) -> int:
        return moe_read_error(self.ws, stream)

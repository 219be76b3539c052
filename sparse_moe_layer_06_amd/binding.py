"""ctypes binding of liblatentmoe.so (include/latentmoe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
torch supplies device memory and the stream.  There is no fallback: if the
library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from .synth import LayerDims

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblatentmoe.so")

LMOE_OK = 0
LMOE_ERR_NULL = -1
LMOE_ERR_SHAPE = -2
LMOE_ERR_DTYPE = -3
LMOE_ERR_ALIGN = -4
LMOE_ERR_WORKSPACE = -5
LMOE_ERR_HIP = -6

LMOE_F32, LMOE_BF16, LMOE_NVFP4, LMOE_BF16_TILED, LMOE_FP8_E4M3, LMOE_NVFP4_2D, LMOE_MXFP8 = 0, 1, 2, 3, 4, 5, 6
DTYPE_CODE = {"f32": LMOE_F32, "bf16": LMOE_BF16, "nvfp4": LMOE_NVFP4, "bf16_tiled": LMOE_BF16_TILED,
              "fp8": LMOE_FP8_E4M3, "nvfp4_2d": LMOE_NVFP4_2D, "mxfp8": LMOE_MXFP8}

EXPORTED = ["lmoe_workspace_bytes", "lmoe_validate_dims", "lmoe_strerror", "lmoe_last_hip_error",
            "latentmoe_forward", "lmoe_project_route", "lmoe_permute", "lmoe_experts_ffn",
            "lmoe_combine_up", "lmoe_timing_start", "lmoe_timing_stop", "lmoe_pack_expert_weights",
            "lmoe_quantize_rows_fp8", "lmoe_quantize_rows_mxfp8", "lmoe_create", "lmoe_destroy",
            "lmoe_ctx_reserve", "lmoe_ctx_workspace_bytes", "lmoe_ctx_forward", "lmoe_static_forward"]
LMOE_STATIC_SCRATCH_BYTES = 128 << 20


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("l", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64), ("f", ctypes.c_int64),
                ("f_s", ctypes.c_int64), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32), ("router_latent", ctypes.c_int32),
                ("shared_dtype", ctypes.c_int32), ("standard_moe", ctypes.c_int32),
                ("proj_dtype", ctypes.c_int32)]


class Fp8Matrix(ctypes.Structure):
    """lmoe_fp8_matrix: E4M3 codes [rows][cols] and fp32 scales [rows] (device);
    also lmoe_mxfp8_matrix (codes, E8M0 scale bytes [rows][cols/32]): the
    same two pointers."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("W1", "W2", "W1_codes", "W1_scales", "W1_ts", "W2_codes", "W2_scales", "W2_ts")]


class Shared(ctypes.Structure):
    _fields_ = [("W_s1", ctypes.c_void_p), ("W_s2", ctypes.c_void_p), ("W_s1_scale", ctypes.c_void_p),
                ("W_s2_scale", ctypes.c_void_p)]


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("z", "logits", "topk_idx", "topk_gate", "counts", "offsets", "perm", "inv", "c")]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", ctypes.c_float)]


class LatentMoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status} ({_strerror(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_moe_layer_06_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        pd = ctypes.POINTER(Dims)
        L.lmoe_workspace_bytes.argtypes = [pd]
        L.lmoe_workspace_bytes.restype = sz
        L.lmoe_validate_dims.argtypes = [pd]
        L.lmoe_validate_dims.restype = ctypes.c_int
        L.lmoe_strerror.argtypes = [ctypes.c_int]
        L.lmoe_strerror.restype = ctypes.c_char_p
        L.lmoe_last_hip_error.argtypes = []
        L.lmoe_last_hip_error.restype = ctypes.c_int
        L.latentmoe_forward.argtypes = [pd, vp, vp, vp, vp, ctypes.POINTER(Experts), vp,
                                        ctypes.POINTER(Shared), ctypes.c_int, vp, vp, sz,
                                        ctypes.POINTER(Debug), vp]
        L.lmoe_project_route.argtypes = [pd, vp, vp, vp, vp, ctypes.POINTER(Shared), vp, vp, vp, vp,
                                         vp, vp, sz, vp]
        L.lmoe_permute.argtypes = [pd, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmoe_experts_ffn.argtypes = [pd, vp, vp, vp, ctypes.POINTER(Experts), vp, vp, sz, vp]
        L.lmoe_combine_up.argtypes = [pd, vp, vp, vp, vp, ctypes.POINTER(Shared), vp, vp, vp, vp, sz, vp]
        L.lmoe_timing_start.argtypes = [ctypes.c_int]
        L.lmoe_timing_start.restype = ctypes.c_int
        L.lmoe_timing_stop.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        L.lmoe_timing_stop.restype = ctypes.c_int
        L.lmoe_pack_expert_weights.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
        L.lmoe_pack_expert_weights.restype = ctypes.c_int
        L.lmoe_quantize_rows_fp8.argtypes = [ctypes.c_int64, ctypes.c_int64, vp, vp, vp, vp]
        L.lmoe_quantize_rows_mxfp8.argtypes = [ctypes.c_int64, ctypes.c_int64, vp, vp, vp, vp]
        L.lmoe_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int]
        L.lmoe_destroy.argtypes = [vp]
        L.lmoe_ctx_reserve.argtypes = [vp, pd]
        L.lmoe_ctx_workspace_bytes.argtypes = [vp]
        L.lmoe_ctx_workspace_bytes.restype = sz
        L.lmoe_ctx_forward.argtypes = [vp, pd, vp, vp, vp, vp, ctypes.POINTER(Experts), vp,
                                       ctypes.POINTER(Shared), ctypes.c_int, vp, ctypes.POINTER(Debug), vp]
        L.lmoe_static_forward.argtypes = [pd, vp, vp, vp, vp, ctypes.POINTER(Experts), vp,
                                          ctypes.POINTER(Shared), ctypes.c_int, vp, ctypes.POINTER(Debug), vp]
        L.lmoe_static_forward.restype = ctypes.c_int
        L.lmoe_quantize_rows_fp8.restype = ctypes.c_int
        for n in ("latentmoe_forward", "lmoe_project_route", "lmoe_permute", "lmoe_experts_ffn",
                  "lmoe_combine_up"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _strerror(status: int) -> str:
    try:
        return lib().lmoe_strerror(status).decode()
    except ImportError:
        return "?"


def _check(status: int, what: str):
    if status != LMOE_OK:
        raise LatentMoEError(status, what)


def dims_of(cfg: LayerDims, T: Optional[int] = None) -> Dims:
    return Dims(T if T is not None else cfg.T, cfg.d, cfg.l, cfg.E, cfg.k, cfg.f, cfg.f_s,
                DTYPE_CODE[cfg.act], DTYPE_CODE[cfg.experts], 1 if cfg.router_latent else 0,
                DTYPE_CODE["fp8" if cfg.shared_fp8 else cfg.act], 1 if cfg.standard_moe else 0,
                DTYPE_CODE["mxfp8" if cfg.proj_mxfp8 else "fp8" if cfg.proj_fp8 else cfg.act])


class _Proj:
    """The W_down / W_up argument: the tensor's address, or with FP8
    projections a pointer to an lmoe_fp8_matrix (kept alive here)."""

    def __init__(self, cfg: LayerDims, inp, name: str):
        self.m = None
        if cfg.proj_fp8 or cfg.proj_mxfp8:
            self.m = Fp8Matrix(_p(inp[name]), _p(inp[name + ("_mxscale" if cfg.proj_mxfp8 else "_scale")]))
            self.arg = ctypes.cast(ctypes.pointer(self.m), ctypes.c_void_p)
        else:
            self.arg = _p(inp.get(name))


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def workspace_bytes(cfg: LayerDims, T: Optional[int] = None) -> int:
    d = dims_of(cfg, T)
    return int(lib().lmoe_workspace_bytes(ctypes.byref(d)))


def validate_dims(d: Dims) -> int:
    return int(lib().lmoe_validate_dims(ctypes.byref(d)))


def alloc_workspace(cfg: LayerDims, device="cuda", T: Optional[int] = None) -> torch.Tensor:
    n = workspace_bytes(cfg, T)
    if n == 0:
        raise LatentMoEError(LMOE_ERR_SHAPE, "workspace size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def experts_struct(inp: Dict[str, Optional[torch.Tensor]]) -> Experts:
    g = inp.get
    return Experts(_p(g("W1")), _p(g("W2")), _p(g("W1_codes")), _p(g("W1_scales")), _p(g("W1_ts")),
                   _p(g("W2_codes")), _p(g("W2_scales")), _p(g("W2_ts")))


def pack_expert_weights(W: torch.Tensor, stream=None) -> torch.Tensor:
    """The LMOE_BF16_TILED image of one bf16 expert stack W [E][rows][cols]."""
    if W.dtype != torch.bfloat16 or W.dim() != 3 or not W.is_contiguous():
        raise LatentMoEError(LMOE_ERR_DTYPE, "pack_expert_weights needs a contiguous [E][rows][cols] bf16 stack")
    P = torch.empty_like(W)
    E, rows, cols = W.shape
    _check(lib().lmoe_pack_expert_weights(E, rows, cols, _p(W), _p(P), _stream(stream)),
           "lmoe_pack_expert_weights")
    return P


def pack_experts(cfg: LayerDims, inp, stream=None):
    """(cfg, inputs) of the same layer with W1 and W2 in the tiled layout: the
    config says experts='bf16_tiled' and the inputs hold the packed stacks."""
    if cfg.experts != "bf16":
        raise LatentMoEError(LMOE_ERR_DTYPE, "only bf16 expert stacks are packed")
    out = dict(inp)
    out["W1"] = pack_expert_weights(inp["W1"], stream)
    out["W2"] = pack_expert_weights(inp["W2"], stream)
    return cfg.with_(experts="bf16_tiled"), out


def shared_struct(inp) -> Optional[Shared]:
    if inp.get("W_s1") is None:
        return None
    return Shared(_p(inp["W_s1"]), _p(inp["W_s2"]), _p(inp.get("W_s1_scale")), _p(inp.get("W_s2_scale")))


def quantize_rows_fp8(src: torch.Tensor, stream=None):
    """(codes uint8 [rows][cols], scales fp32 [rows]) of a contiguous bf16
    matrix, per row: scale = max|v| / 448, code = E4M3(v / scale)."""
    if src.dtype != torch.bfloat16 or src.dim() != 2 or not src.is_contiguous():
        raise LatentMoEError(LMOE_ERR_DTYPE, "quantize_rows_fp8 needs a contiguous [rows][cols] bf16 matrix")
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty(rows, dtype=torch.float32, device=src.device)
    _check(lib().lmoe_quantize_rows_fp8(rows, cols, _p(src), _p(codes), _p(scales), _stream(stream)),
           "lmoe_quantize_rows_fp8")
    return codes, scales


def _byref_opt(s):
    return ctypes.byref(s) if s is not None else None


def act_dtype(cfg: LayerDims) -> torch.dtype:
    return torch.bfloat16 if cfg.act == "bf16" else torch.float32


class Context:
    """An lmoe_ctx: a workspace the library owns (grown by reserve, outside
    any forward call)."""

    def __init__(self, device: int = 0):
        self.h = ctypes.c_void_p()
        _check(lib().lmoe_create(ctypes.byref(self.h), device), "lmoe_create")

    def reserve(self, cfg: LayerDims, T: Optional[int] = None):
        d = dims_of(cfg, T)
        _check(lib().lmoe_ctx_reserve(self.h, ctypes.byref(d)), "lmoe_ctx_reserve")

    def workspace_bytes(self) -> int:
        return int(lib().lmoe_ctx_workspace_bytes(self.h))

    def forward(self, cfg: LayerDims, inp, out: torch.Tensor, debug=None, stream=None) -> torch.Tensor:
        d = dims_of(cfg, inp["x"].shape[0])
        ex, sh = experts_struct(inp), shared_struct(inp)
        wd, wu = _Proj(cfg, inp, "W_down"), _Proj(cfg, inp, "W_up")
        dbg = Debug(**{n: _p(debug.get(n)) for n, _ in Debug._fields_}) if debug else None
        _check(lib().lmoe_ctx_forward(self.h, ctypes.byref(d), _p(inp["x"]), wd.arg, _p(inp["W_r"]),
                                      _p(inp.get("b_r")), ctypes.byref(ex), wu.arg, _byref_opt(sh), cfg.k,
                                      _p(out), _byref_opt(dbg), _stream(stream)), "lmoe_ctx_forward")
        return out

    def close(self):
        if self.h:
            _check(lib().lmoe_destroy(self.h), "lmoe_destroy")
            self.h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def quantize_rows_mxfp8(src: torch.Tensor, stream=None):
    """(codes uint8 [rows][cols], E8M0 scales uint8 [rows][cols/32]) of a
    contiguous bf16 matrix, per 32-element block (OCP MXFP8)."""
    if src.dtype != torch.bfloat16 or src.dim() != 2 or not src.is_contiguous():
        raise LatentMoEError(LMOE_ERR_DTYPE, "quantize_rows_mxfp8 needs a contiguous [rows][cols] bf16 matrix")
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=src.device)
    _check(lib().lmoe_quantize_rows_mxfp8(rows, cols, _p(src), _p(codes), _p(scales), _stream(stream)),
           "lmoe_quantize_rows_mxfp8")
    return codes, scales


class Call:
    """A prepared forward call: argument structs built once, so timing loops
    only pay for the ctypes call and the kernels."""

    def __init__(self, cfg: LayerDims, inp, out: torch.Tensor, workspace: torch.Tensor,
                 debug: Optional[Dict[str, torch.Tensor]] = None, stream=None):
        self.cfg = cfg
        self.dims = dims_of(cfg, inp["x"].shape[0])
        self.ex = experts_struct(inp)
        self.sh = shared_struct(inp)
        self.dbg = None
        if debug:
            self.dbg = Debug(**{n: _p(debug.get(n)) for n, _ in Debug._fields_})
        self.wd, self.wu = _Proj(cfg, inp, "W_down"), _Proj(cfg, inp, "W_up")
        self.args = (ctypes.byref(self.dims), _p(inp["x"]), self.wd.arg, _p(inp["W_r"]),
                     _p(inp.get("b_r")), ctypes.byref(self.ex), self.wu.arg, _byref_opt(self.sh),
                     cfg.k, _p(out), _p(workspace), workspace.numel(), _byref_opt(self.dbg),
                     _stream(stream))
        self._keep = (inp, out, workspace, debug)

    def __call__(self):
        _check(lib().latentmoe_forward(*self.args), "latentmoe_forward")


def forward(cfg: LayerDims, inp, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, debug=None, stream=None) -> torch.Tensor:
    """out [T][d] = LatentMoE(inp['x']) on the current (or given) stream."""
    x = inp["x"]
    if out is None:
        out = torch.empty((x.shape[0], cfg.d), dtype=act_dtype(cfg), device=x.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, x.device, x.shape[0])
    Call(cfg, inp, out, workspace, debug, stream)()
    return out


def static_forward(cfg: LayerDims, inp, out: Optional[torch.Tensor] = None, debug=None,
                   stream=None) -> torch.Tensor:
    """out [T][d] = LatentMoE(inp['x']) through lmoe_static_forward: the
    library's own per-GPU scratch array as workspace (no allocation by the
    library; out is allocated here when not given)."""
    x = inp["x"]
    if out is None:
        out = torch.empty((x.shape[0], cfg.d), dtype=act_dtype(cfg), device=x.device)
    d = dims_of(cfg, x.shape[0])
    ex, sh = experts_struct(inp), shared_struct(inp)
    wd, wu = _Proj(cfg, inp, "W_down"), _Proj(cfg, inp, "W_up")
    dbg = Debug(**{n: _p(debug.get(n)) for n, _ in Debug._fields_}) if debug else None
    _check(lib().lmoe_static_forward(ctypes.byref(d), _p(x), wd.arg, _p(inp["W_r"]), _p(inp.get("b_r")),
                                     ctypes.byref(ex), wu.arg, _byref_opt(sh), cfg.k, _p(out), _byref_opt(dbg),
                                     _stream(stream)), "lmoe_static_forward")
    return out


class KernelTimer:
    """Per-kernel durations of the library's own launches (hipEvents on the
    launch stream), as a list of (kernel name, ms)."""

    def __init__(self, capacity: int = 4096):
        self.capacity = capacity
        self.records = []

    def __enter__(self):
        _check(lib().lmoe_timing_start(self.capacity), "lmoe_timing_start")
        return self

    def __exit__(self, *exc):
        buf = (KernelTime * self.capacity)()
        n = ctypes.c_int(0)
        _check(lib().lmoe_timing_stop(buf, self.capacity, ctypes.byref(n)), "lmoe_timing_stop")
        self.records = [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n.value)]
        return False

    def by_kernel(self):
        out = {}
        for name, ms in self.records:
            out.setdefault(name, []).append(ms)
        return out


# ---- staged entry points ------------------------------------------------

def project_route(cfg: LayerDims, inp, workspace, stream=None):
    x = inp["x"]
    T, dev = x.shape[0], x.device
    dt = act_dtype(cfg)
    z = torch.empty((T, cfg.l), dtype=dt, device=dev)
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    sh = shared_struct(inp)
    hs = torch.empty((T, cfg.f_s), dtype=dt, device=dev) if sh is not None else None
    d = dims_of(cfg, T)
    wd = _Proj(cfg, inp, "W_down")
    _check(lib().lmoe_project_route(ctypes.byref(d), _p(x), wd.arg, _p(inp["W_r"]),
                                    _p(inp.get("b_r")), _byref_opt(sh), _p(z), _p(logits), _p(idx),
                                    _p(gate), _p(hs), _p(workspace), workspace.numel(),
                                    _stream(stream)), "lmoe_project_route")
    return dict(z=z, logits=logits, idx=idx, gate=gate, hs=hs)


def permute(cfg: LayerDims, idx: torch.Tensor, workspace, stream=None):
    T, dev = idx.shape[0], idx.device
    n = T * cfg.k
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    inv = torch.empty(n, dtype=torch.int32, device=dev)
    d = dims_of(cfg, T)
    _check(lib().lmoe_permute(ctypes.byref(d), _p(idx), _p(counts), _p(offsets), _p(perm), _p(inv),
                              _p(workspace), workspace.numel(), _stream(stream)), "lmoe_permute")
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv)


def experts_ffn(cfg: LayerDims, inp, z, offsets, perm, workspace, stream=None):
    T, dev = z.shape[0], z.device
    Y = torch.empty((T * cfg.k, cfg.l), dtype=act_dtype(cfg), device=dev)
    ex = experts_struct(inp)
    d = dims_of(cfg, T)
    _check(lib().lmoe_experts_ffn(ctypes.byref(d), _p(z), _p(offsets), _p(perm),
                                  ctypes.byref(ex), _p(Y), _p(workspace), workspace.numel(),
                                  _stream(stream)), "lmoe_experts_ffn")
    return Y


def combine_up(cfg: LayerDims, inp, Y, inv, gate, hs, workspace, T: int, stream=None):
    dev = Y.device
    dt = act_dtype(cfg)
    c = torch.empty((T, cfg.l), dtype=dt, device=dev)
    out = torch.empty((T, cfg.d), dtype=dt, device=dev)
    sh = shared_struct(inp)
    d = dims_of(cfg, T)
    wu = _Proj(cfg, inp, "W_up")
    _check(lib().lmoe_combine_up(ctypes.byref(d), _p(Y), _p(inv), _p(gate), wu.arg, _byref_opt(sh),
                                 _p(hs), _p(c), _p(out), _p(workspace), workspace.numel(),
                                 _stream(stream)), "lmoe_combine_up")
    return dict(c=c, out=out)

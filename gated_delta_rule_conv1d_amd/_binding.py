"""ctypes binding of libgdn.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
F32, BF16 = 0, 1
_STATUS = {0: "GDN_OK", -1: "GDN_ERR_INVALID_ARG", -2: "GDN_ERR_UNSUPPORTED", -3: "GDN_ERR_WORKSPACE",
           -4: "GDN_ERR_HIP"}

#: every symbol include/gdn.h declares
SYMBOLS = ("gdn_status_string", "gdn_max_chunks", "gdn_chunk_index", "gdn_conv1d", "gdn_conv1d_bwd_workspace",
           "gdn_conv1d_bwd", "gdn_chunk_fwd_workspace", "gdn_chunk_fwd", "gdn_chunk_bwd_workspace",
           "gdn_chunk_bwd", "gdn_chunk_fwd_save", "gdn_chunk_bwd_saved", "gdn_chunk_fwd_fp8", "gdn_chunk_fwd_gated",
           "gdn_chunk_fwd_save_gated", "gdn_chunk_bwd_gated", "gdn_chunk_bwd_saved_gated", "gdn_norm_gate",
           "gdn_norm_gate_bwd_workspace", "gdn_norm_gate_bwd", "gdn_norm_gate_bwd_noalloc", "gdn_gates",
           "gdn_gates_bwd_workspace",
           "gdn_gates_bwd", "gdn_recurrent_step", "gdn_conv1d_step", "gdn_conv1d_window", "gdn_conv1d_prefill",
           "gdn_profile_enable", "gdn_profile_report", "gdn_probe_copy", "gdn_probe_mfma")


class GdnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code} ({_STATUS.get(code, 'unknown')})")
        self.code = code


class _Shape(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class _GateInputs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


class _GateGrads(ctypes.Structure):
    _fields_ = [("da", ctypes.c_void_p), ("db", ctypes.c_void_p), ("dA_log", ctypes.c_void_p),
                ("ddt_bias", ctypes.c_void_p)]


@dataclass(frozen=True)
class Shape:
    n_seqs: int
    total_tokens: int
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    chunk: int = 64
    dtype: int = BF16
    scale: float = 1.0

    @property
    def channels(self) -> int:
        return 2 * self.h_qk * self.d_k + self.h_v * self.d_v

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == BF16 else torch.float32

    def c(self) -> _Shape:
        return _Shape(self.n_seqs, self.total_tokens, self.h_qk, self.h_v, self.d_k, self.d_v, self.chunk,
                      self.dtype, self.scale)


def lib_path() -> str:
    return os.path.join(_HERE, "libgdn.so")


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libgdn.so (built by gated_delta_rule_conv1d_amd.build)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_conv1d_amd.build` "
                               "(there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        S = ctypes.POINTER(_Shape)
        GI, GG = ctypes.POINTER(_GateInputs), ctypes.POINTER(_GateGrads)
        sig = {
            "gdn_status_string": (ctypes.c_char_p, [I32]),
            "gdn_max_chunks": (I64, [S]),
            "gdn_chunk_index": (I32, [S, P, P, P, P]),
            "gdn_conv1d": (I32, [S, P, P, I32, F, P, P, P]),
            "gdn_conv1d_bwd_workspace": (SZ, [S, I32]),
            "gdn_conv1d_bwd": (I32, [S, P, P, P, I32, F, P, P, P, P, SZ, P]),
            "gdn_chunk_fwd_workspace": (SZ, [S]),
            "gdn_chunk_fwd": (I32, [S, P, P, P, I64, I64, P, P, P, P, P, P, P, SZ, P]),
            "gdn_chunk_bwd_workspace": (SZ, [S]),
            "gdn_chunk_bwd": (I32, [S, P, P, P, I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "gdn_chunk_fwd_save": (I32, [S, P, P, P, I64, I64, P, P, P, P, P, P, P, SZ, P]),
            "gdn_chunk_bwd_saved": (I32, [S, P, P, P, I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "gdn_chunk_fwd_fp8": (I32, [S, P, P, P, I64, I64, F, F, F, P, P, P, P, P, P, P, SZ, P]),
            "gdn_chunk_fwd_gated": (I32, [S, P, P, P, I64, I64, GI, P, P, P, P, P, SZ, P]),
            "gdn_chunk_fwd_save_gated": (I32, [S, P, P, P, I64, I64, GI, P, P, P, P, P, SZ, P]),
            "gdn_chunk_bwd_gated": (I32, [S, P, P, P, I64, I64, GI, P, P, P, P, P, P, P, GG, P, P, SZ, P]),
            "gdn_chunk_bwd_saved_gated": (I32, [S, P, P, P, I64, I64, GI, P, P, P, P, P, P, P, GG, P, P, SZ, P]),
            "gdn_norm_gate": (I32, [S, P, P, P, F, P, P]),
            "gdn_norm_gate_bwd_workspace": (SZ, [S]),
            "gdn_norm_gate_bwd": (I32, [S, P, P, P, P, F, P, P, P, P, SZ, P]),
            "gdn_norm_gate_bwd_noalloc": (I32, [S, P, P, P, P, F, P, P, P, P]),
            "gdn_gates": (I32, [S, P, P, P, P, P, P, P]),
            "gdn_gates_bwd_workspace": (SZ, [S]),
            "gdn_gates_bwd": (I32, [S, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "gdn_recurrent_step": (I32, [S, P, P, P, I64, I64, P, P, P, P, P, P]),
            "gdn_conv1d_step": (I32, [S, P, P, I32, F, P, P, P]),
            "gdn_conv1d_window": (I32, [S, P, I32, P, P, P, P]),
            "gdn_conv1d_prefill": (I32, [S, P, P, I32, F, P, P, P, P, P]),
            "gdn_profile_enable": (None, [ctypes.c_int]),
            "gdn_profile_report": (SZ, [ctypes.c_char_p, SZ]),
            "gdn_probe_copy": (I32, [P, P, SZ, P]),
            "gdn_probe_mfma": (I32, [P, I32, I32, I32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, code: int):
    if code != 0:
        raise GdnError(fn, code)


def _need(t: torch.Tensor, name: str, dtype, shape=None, inner_contig=True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if inner_contig and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _tok_view(t: torch.Tensor, name: str, rows: int, width: int) -> int:
    """Token stride of a [T, width] (possibly strided-row) view with unit inner stride."""
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] != width or (width > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a [{rows}, {width}] view with unit inner stride")
    return t.stride(0)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- chunk index
def max_chunks(shape: Shape) -> int:
    return int(load().gdn_max_chunks(ctypes.byref(shape.c())))


def chunk_index(cu_seqlens: torch.Tensor, shape: Shape) -> Tuple[torch.Tensor, torch.Tensor]:
    _need(cu_seqlens, "cu_seqlens", torch.int32, (shape.n_seqs + 1,))
    M = max_chunks(shape)
    table = torch.empty((M, 4), dtype=torch.int32, device=cu_seqlens.device)
    first = torch.empty((shape.n_seqs + 1,), dtype=torch.int32, device=cu_seqlens.device)
    _check("gdn_chunk_index", load().gdn_chunk_index(ctypes.byref(shape.c()), _ptr(cu_seqlens), _ptr(table),
                                                     _ptr(first), _stream(cu_seqlens.device)))
    return table, first


# ----------------------------------------------------------------------------- conv
def conv1d(x: torch.Tensor, w_conv: torch.Tensor, cu_seqlens: torch.Tensor, shape: Shape, l2_eps: float = 1e-6,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dt = shape.torch_dtype
    T, Cch = shape.total_tokens, shape.channels
    _need(x, "x", dt, (T, Cch))
    _need(w_conv, "w_conv", dt)
    if w_conv.dim() != 2 or w_conv.shape[0] != Cch:
        raise ValueError("w_conv must be [Cch, width]")
    _need(cu_seqlens, "cu_seqlens", torch.int32, (shape.n_seqs + 1,))
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dt, (T, Cch))
    _check("gdn_conv1d", load().gdn_conv1d(ctypes.byref(shape.c()), _ptr(x), _ptr(w_conv), int(w_conv.shape[1]),
                                           float(l2_eps), _ptr(cu_seqlens), _ptr(y), _stream(x.device)))
    return y


def conv1d_bwd_workspace(shape: Shape, width: int) -> int:
    return int(load().gdn_conv1d_bwd_workspace(ctypes.byref(shape.c()), int(width)))


def conv1d_bwd(dy: torch.Tensor, x: torch.Tensor, w_conv: torch.Tensor, cu_seqlens: torch.Tensor, shape: Shape,
               l2_eps: float = 1e-6, ws: Optional[torch.Tensor] = None):
    dt = shape.torch_dtype
    T, Cch = shape.total_tokens, shape.channels
    _need(dy, "dy", dt, (T, Cch))
    _need(x, "x", dt, (T, Cch))
    _need(w_conv, "w_conv", dt)
    width = int(w_conv.shape[1])
    dx = torch.empty_like(x)
    dw = torch.empty((Cch, width), dtype=torch.float32, device=x.device)
    nb = conv1d_bwd_workspace(shape, width)
    ws = _workspace(nb, x.device, ws)
    _check("gdn_conv1d_bwd", load().gdn_conv1d_bwd(ctypes.byref(shape.c()), _ptr(dy), _ptr(x), _ptr(w_conv), width,
                                                   float(l2_eps), _ptr(cu_seqlens), _ptr(dx), _ptr(dw), _ptr(ws),
                                                   ws.numel(), _stream(x.device)))
    return dx, dw


# ----------------------------------------------------------------------------- chunked recurrence
def chunk_fwd_workspace(shape: Shape) -> int:
    return int(load().gdn_chunk_fwd_workspace(ctypes.byref(shape.c())))


def chunk_bwd_workspace(shape: Shape) -> int:
    return int(load().gdn_chunk_bwd_workspace(ctypes.byref(shape.c())))


def _qkv_strides(q, k, v, shape: Shape):
    T = shape.total_tokens
    sq = _tok_view(q, "q", T, shape.h_qk * shape.d_k)
    sk = _tok_view(k, "k", T, shape.h_qk * shape.d_k)
    sv = _tok_view(v, "v", T, shape.h_v * shape.d_v)
    if sq != sk:
        raise ValueError("q and k must share one token stride")
    return sq, sv


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              cu_seqlens: torch.Tensor, shape: Shape, h0: Optional[torch.Tensor] = None, want_ht: bool = True,
              ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, save: bool = False,
              ht_out: Optional[torch.Tensor] = None):
    """q, k: [T, Hk*dk] views; v: [T, Hv*dv] view; g, beta: fp32 [T, Hv].
    Returns (o [T, Hv, dv], ht [N, Hv, dk, dv] fp32 or None).  With save=True
    (gdn_chunk_fwd_save) ws must be a backward-sized workspace, which then
    holds what chunk_bwd(..., saved=True) reads.  out / ht_out: contiguous
    views of the caller's tensors to receive o / ht."""
    dt = shape.torch_dtype
    T, N, Hv, dk, dv = shape.total_tokens, shape.n_seqs, shape.h_v, shape.d_k, shape.d_v
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, dt, inner_contig=False)
    sqk, sv = _qkv_strides(q, k, v, shape)
    _need(g, "g", torch.float32, (T, Hv))
    _need(beta, "beta", torch.float32, (T, Hv))
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, Hv, dk, dv))
    if out is None:
        out = torch.empty((T, Hv, dv), dtype=dt, device=q.device)
    _need(out, "out", dt, (T, Hv, dv))
    o = out
    ht = None
    if want_ht:
        ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=q.device) if ht_out is None else ht_out
        _need(ht, "ht", torch.float32, (N, Hv, dk, dv))
    if save and ws is None:
        raise ValueError("save=True needs the caller's backward workspace (it carries state to chunk_bwd)")
    ws = _workspace(chunk_bwd_workspace(shape) if save else chunk_fwd_workspace(shape), q.device, ws)
    name = "gdn_chunk_fwd_save" if save else "gdn_chunk_fwd"
    _check(name, getattr(load(), name)(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), sqk, sv,
                                       _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht),
                                       _ptr(ws), ws.numel(), _stream(q.device)))
    return o, ht


def chunk_bwd(q, k, v, g, beta, cu_seqlens, shape: Shape, d_o, h0=None, dht=None, dq=None, dk=None, dv=None,
              want_dh0: bool = True, ws: Optional[torch.Tensor] = None, saved: bool = False,
              dg: Optional[torch.Tensor] = None, dbeta: Optional[torch.Tensor] = None,
              dh0: Optional[torch.Tensor] = None):
    """Returns dict dq, dk, dv (like q, k, v: [T, H*d]), dg, dbeta [T, Hv] fp32, dh0 (or None).
    saved=True (gdn_chunk_bwd_saved): ws is the workspace a chunk_fwd(..., save=True)
    with the same inputs just filled.  dq, dk, dv, dg, dbeta, dh0 may be given
    (contiguous views of the caller's tensors) to receive the results."""
    dt = shape.torch_dtype
    T, N, Hk, Hv, dkk, dvv = shape.total_tokens, shape.n_seqs, shape.h_qk, shape.h_v, shape.d_k, shape.d_v
    sqk, sv = _qkv_strides(q, k, v, shape)
    _need(d_o, "d_o", dt, (T, Hv, dvv))
    if dq is None:
        dq = torch.empty((T, Hk * dkk), dtype=dt, device=q.device)
    if dk is None:
        dk = torch.empty((T, Hk * dkk), dtype=dt, device=q.device)
    if dv is None:
        dv = torch.empty((T, Hv * dvv), dtype=dt, device=q.device)
    if _tok_view(dq, "dq", T, Hk * dkk) != sqk or _tok_view(dk, "dk", T, Hk * dkk) != sqk \
            or _tok_view(dv, "dv", T, Hv * dvv) != sv:
        raise ValueError("dq/dk/dv must use the token strides of q/k/v")
    if dht is not None:
        _need(dht, "dht", torch.float32, (N, Hv, dkk, dvv))
    if dg is None:
        dg = torch.empty((T, Hv), dtype=torch.float32, device=q.device)
    if dbeta is None:
        dbeta = torch.empty((T, Hv), dtype=torch.float32, device=q.device)
    db = dbeta
    _need(dg, "dg", torch.float32, (T, Hv))
    _need(db, "dbeta", torch.float32, (T, Hv))
    if not want_dh0:
        dh0 = None
    elif dh0 is None:
        dh0 = torch.empty((N, Hv, dkk, dvv), dtype=torch.float32, device=q.device)
    else:
        _need(dh0, "dh0", torch.float32, (N, Hv, dkk, dvv))
    if saved and ws is None:
        raise ValueError("saved=True needs the workspace filled by chunk_fwd(..., save=True)")
    ws = _workspace(chunk_bwd_workspace(shape), q.device, ws)
    name = "gdn_chunk_bwd_saved" if saved else "gdn_chunk_bwd"
    _check(name, getattr(load(), name)(
        ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), sqk, sv, _ptr(g), _ptr(beta), _ptr(cu_seqlens),
        _ptr(h0), _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dh0), _ptr(ws),
        ws.numel(), _stream(q.device)))
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=db, dh0=dh0)


def chunk_fwd_fp8(q8, k8, v8, scales, g, beta, cu_seqlens, shape: Shape, h0=None, want_ht: bool = True,
                  ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """gdn_chunk_fwd_fp8: q8, k8 [T, Hk*dk] and v8 [T, Hv*dv] views of
    torch.float8_e4m3fn (or uint8) tensors with unit inner stride; scales =
    (scale_q, scale_k, scale_v), powers of two.  shape.dtype is BF16 (o)."""
    T, N, Hv, dk, dv = shape.total_tokens, shape.n_seqs, shape.h_v, shape.d_k, shape.d_v
    for t, nm in ((q8, "q"), (k8, "k"), (v8, "v")):
        if t.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)) or not t.is_cuda:
            raise ValueError(f"{nm} must be a GPU float8_e4m3fn (or uint8) tensor")
    sqk, sv = _qkv_strides(q8, k8, v8, shape)
    _need(g, "g", torch.float32, (T, Hv))
    _need(beta, "beta", torch.float32, (T, Hv))
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, Hv, dk, dv))
    o = torch.empty((T, Hv, dv), dtype=torch.bfloat16, device=q8.device) if out is None else out
    ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=q8.device) if want_ht else None
    ws = _workspace(chunk_fwd_workspace(shape), q8.device, ws)
    sq, sk, svs = (float(x) for x in scales)
    _check("gdn_chunk_fwd_fp8", load().gdn_chunk_fwd_fp8(
        ctypes.byref(shape.c()), _ptr(q8), _ptr(k8), _ptr(v8), sqk, sv, sq, sk, svs, _ptr(g), _ptr(beta),
        _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht), _ptr(ws), ws.numel(), _stream(q8.device)))
    return o, ht


def _gate_inputs(gates, shape: Shape):
    a, b, A_log, dt_bias = gates
    _need(a, "a", torch.float32, (shape.total_tokens, shape.h_v))
    _need(b, "b", torch.float32, (shape.total_tokens, shape.h_v))
    _need(A_log, "A_log", torch.float32, (shape.h_v,))
    _need(dt_bias, "dt_bias", torch.float32, (shape.h_v,))
    return _GateInputs(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias))


def chunk_fwd_gated(q, k, v, gates, cu_seqlens, shape: Shape, h0=None, want_ht: bool = True,
                    ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, save: bool = False):
    """gdn_chunk_fwd_gated / gdn_chunk_fwd_save_gated: as chunk_fwd, with g and
    beta computed inside the kernels from gates = (a, b, A_log, dt_bias)."""
    dt = shape.torch_dtype
    T, N, Hv, dk, dv = shape.total_tokens, shape.n_seqs, shape.h_v, shape.d_k, shape.d_v
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, dt, inner_contig=False)
    sqk, sv = _qkv_strides(q, k, v, shape)
    gi = _gate_inputs(gates, shape)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, Hv, dk, dv))
    o = torch.empty((T, Hv, dv), dtype=dt, device=q.device) if out is None else out
    ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=q.device) if want_ht else None
    if save and ws is None:
        raise ValueError("save=True needs the caller's backward workspace (it carries state to chunk_bwd)")
    ws = _workspace(chunk_bwd_workspace(shape) if save else chunk_fwd_workspace(shape), q.device, ws)
    name = "gdn_chunk_fwd_save_gated" if save else "gdn_chunk_fwd_gated"
    _check(name, getattr(load(), name)(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), sqk, sv,
                                       ctypes.byref(gi), _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht),
                                       _ptr(ws), ws.numel(), _stream(q.device)))
    return o, ht


def chunk_bwd_gated(q, k, v, gates, cu_seqlens, shape: Shape, d_o, h0=None, dht=None, dq=None, dk=None, dv=None,
                    want_dh0: bool = True, ws: Optional[torch.Tensor] = None, saved: bool = False):
    """gdn_chunk_bwd_gated / gdn_chunk_bwd_saved_gated.  Returns dict dq, dk, dv,
    da, db [T, Hv], dA_log, ddt_bias [Hv] and dh0 (or None)."""
    dt = shape.torch_dtype
    T, N, Hk, Hv, dkk, dvv = shape.total_tokens, shape.n_seqs, shape.h_qk, shape.h_v, shape.d_k, shape.d_v
    sqk, sv = _qkv_strides(q, k, v, shape)
    gi = _gate_inputs(gates, shape)
    _need(d_o, "d_o", dt, (T, Hv, dvv))
    dq = torch.empty((T, Hk * dkk), dtype=dt, device=q.device) if dq is None else dq
    dk = torch.empty((T, Hk * dkk), dtype=dt, device=q.device) if dk is None else dk
    dv = torch.empty((T, Hv * dvv), dtype=dt, device=q.device) if dv is None else dv
    if _tok_view(dq, "dq", T, Hk * dkk) != sqk or _tok_view(dk, "dk", T, Hk * dkk) != sqk \
            or _tok_view(dv, "dv", T, Hv * dvv) != sv:
        raise ValueError("dq/dk/dv must use the token strides of q/k/v")
    if dht is not None:
        _need(dht, "dht", torch.float32, (N, Hv, dkk, dvv))
    da = torch.empty((T, Hv), dtype=torch.float32, device=q.device)
    db = torch.empty((T, Hv), dtype=torch.float32, device=q.device)
    dA = torch.empty((Hv,), dtype=torch.float32, device=q.device)
    ddt = torch.empty((Hv,), dtype=torch.float32, device=q.device)
    gg = _GateGrads(_ptr(da), _ptr(db), _ptr(dA), _ptr(ddt))
    dh0 = torch.empty((N, Hv, dkk, dvv), dtype=torch.float32, device=q.device) if want_dh0 else None
    if saved and ws is None:
        raise ValueError("saved=True needs the workspace filled by chunk_fwd_gated(..., save=True)")
    ws = _workspace(chunk_bwd_workspace(shape), q.device, ws)
    name = "gdn_chunk_bwd_saved_gated" if saved else "gdn_chunk_bwd_gated"
    _check(name, getattr(load(), name)(
        ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), sqk, sv, ctypes.byref(gi), _ptr(cu_seqlens),
        _ptr(h0), _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), ctypes.byref(gg), _ptr(dh0), _ptr(ws),
        ws.numel(), _stream(q.device)))
    return dict(dq=dq, dk=dk, dv=dv, da=da, db=db, dA_log=dA, ddt_bias=ddt, dh0=dh0)


# ----------------------------------------------------------------------------- norm gate
def norm_gate(o: torch.Tensor, z: torch.Tensor, w_norm: torch.Tensor, shape: Shape, eps: float = 1e-6,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dt = shape.torch_dtype
    sh = (shape.total_tokens, shape.h_v, shape.d_v)
    _need(o, "o", dt, sh)
    _need(z, "z", dt, sh)
    _need(w_norm, "w_norm", dt, (shape.d_v,))
    y = torch.empty_like(o) if out is None else out
    _check("gdn_norm_gate", load().gdn_norm_gate(ctypes.byref(shape.c()), _ptr(o), _ptr(z), _ptr(w_norm), float(eps),
                                                 _ptr(y), _stream(o.device)))
    return y


def norm_gate_bwd_workspace(shape: Shape) -> int:
    return int(load().gdn_norm_gate_bwd_workspace(ctypes.byref(shape.c())))


def norm_gate_bwd(dy, o, z, w_norm, shape: Shape, eps: float = 1e-6, ws: Optional[torch.Tensor] = None):
    dt = shape.torch_dtype
    sh = (shape.total_tokens, shape.h_v, shape.d_v)
    for t, nm in ((dy, "dy"), (o, "o"), (z, "z")):
        _need(t, nm, dt, sh)
    _need(w_norm, "w_norm", dt, (shape.d_v,))
    d_o = torch.empty_like(o)
    dz = torch.empty_like(z)
    dw = torch.empty((shape.d_v,), dtype=torch.float32, device=o.device)
    ws = _workspace(norm_gate_bwd_workspace(shape), o.device, ws)
    _check("gdn_norm_gate_bwd", load().gdn_norm_gate_bwd(ctypes.byref(shape.c()), _ptr(dy), _ptr(o), _ptr(z),
                                                         _ptr(w_norm), float(eps), _ptr(d_o), _ptr(dz), _ptr(dw),
                                                         _ptr(ws), ws.numel(), _stream(o.device)))
    return d_o, dz, dw


def norm_gate_bwd_noalloc(dy, o, z, w_norm, shape: Shape, eps: float = 1e-6, d_o=None, dz=None, dw=None):
    """gdn_norm_gate_bwd_noalloc: the same backward with the library's own
    device scratch instead of a workspace (outputs may be passed in, so that a
    caller that cannot allocate can reuse them)."""
    dt = shape.torch_dtype
    sh = (shape.total_tokens, shape.h_v, shape.d_v)
    for t, nm in ((dy, "dy"), (o, "o"), (z, "z")):
        _need(t, nm, dt, sh)
    _need(w_norm, "w_norm", dt, (shape.d_v,))
    d_o = torch.empty_like(o) if d_o is None else d_o
    dz = torch.empty_like(z) if dz is None else dz
    dw = torch.empty((shape.d_v,), dtype=torch.float32, device=o.device) if dw is None else dw
    _need(d_o, "d_o", dt, sh)
    _need(dz, "dz", dt, sh)
    _need(dw, "dw", torch.float32, (shape.d_v,))
    _check("gdn_norm_gate_bwd_noalloc", load().gdn_norm_gate_bwd_noalloc(
        ctypes.byref(shape.c()), _ptr(dy), _ptr(o), _ptr(z), _ptr(w_norm), float(eps), _ptr(d_o), _ptr(dz),
        _ptr(dw), _stream(o.device)))
    return d_o, dz, dw


# ----------------------------------------------------------------------------- gates
def gates(a: torch.Tensor, b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor, shape: Shape):
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); a, b float32 [T, Hv]."""
    sh = (shape.total_tokens, shape.h_v)
    _need(a, "a", torch.float32, sh)
    _need(b, "b", torch.float32, sh)
    _need(A_log, "A_log", torch.float32, (shape.h_v,))
    _need(dt_bias, "dt_bias", torch.float32, (shape.h_v,))
    g = torch.empty_like(a)
    beta = torch.empty_like(b)
    _check("gdn_gates", load().gdn_gates(ctypes.byref(shape.c()), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                         _ptr(g), _ptr(beta), _stream(a.device)))
    return g, beta


def gates_bwd_workspace(shape: Shape) -> int:
    return int(load().gdn_gates_bwd_workspace(ctypes.byref(shape.c())))


def gates_bwd(a, b, A_log, dt_bias, dg, dbeta, shape: Shape, ws: Optional[torch.Tensor] = None):
    """Gradients of gates(): dict(da, db [T, Hv], dA_log, ddt_bias [Hv])."""
    sh = (shape.total_tokens, shape.h_v)
    for t, nm in ((a, "a"), (b, "b"), (dg, "dg"), (dbeta, "dbeta")):
        _need(t, nm, torch.float32, sh)
    _need(A_log, "A_log", torch.float32, (shape.h_v,))
    _need(dt_bias, "dt_bias", torch.float32, (shape.h_v,))
    da = torch.empty_like(a)
    db = torch.empty_like(b)
    dA = torch.empty_like(A_log)
    ddt = torch.empty_like(dt_bias)
    ws = _workspace(gates_bwd_workspace(shape), a.device, ws)
    _check("gdn_gates_bwd", load().gdn_gates_bwd(ctypes.byref(shape.c()), _ptr(a), _ptr(b), _ptr(A_log),
                                                 _ptr(dt_bias), _ptr(dg), _ptr(dbeta), _ptr(da), _ptr(db), _ptr(dA),
                                                 _ptr(ddt), _ptr(ws), ws.numel(), _stream(a.device)))
    return dict(da=da, db=db, dA_log=dA, ddt_bias=ddt)


# ----------------------------------------------------------------------------- decode
def recurrent_step(q, k, v, g, beta, shape: Shape, state_in=None, state_out=None, o=None):
    """One new token per sequence (shape.total_tokens == shape.n_seqs): the gated
    delta rule step.  state_out defaults to a new tensor; pass state_out=state_in
    to update in place.  Returns (o, state_out)."""
    N = shape.n_seqs
    sqk, sv = _qkv_strides(q, k, v, shape)
    _need(g, "g", torch.float32, (N, shape.h_v))
    _need(beta, "beta", torch.float32, (N, shape.h_v))
    st_shape = (N, shape.h_v, shape.d_k, shape.d_v)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, st_shape)
    if state_out is None:
        state_out = torch.empty(st_shape, dtype=torch.float32, device=q.device)
    _need(state_out, "state_out", torch.float32, st_shape)
    if o is None:
        o = torch.empty((N, shape.h_v, shape.d_v), dtype=shape.torch_dtype, device=q.device)
    _check("gdn_recurrent_step", load().gdn_recurrent_step(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), sqk,
                                                           sv, _ptr(g), _ptr(beta), _ptr(state_in), _ptr(state_out),
                                                           _ptr(o), _stream(q.device)))
    return o, state_out


def conv1d_step(x, w_conv, conv_window, shape: Shape, l2_eps: float = 1e-6):
    """Conv1d + SiLU + L2 of one new token per sequence; advances conv_window
    [N, width-1, Cch] in place.  Returns y [N, Cch]."""
    dt = shape.torch_dtype
    C = shape.channels
    W = int(w_conv.shape[1])
    _need(x, "x", dt, (shape.n_seqs, C))
    _need(w_conv, "w_conv", dt, (C, W))
    _need(conv_window, "conv_window", dt, (shape.n_seqs, W - 1, C))
    y = torch.empty_like(x)
    _check("gdn_conv1d_step", load().gdn_conv1d_step(ctypes.byref(shape.c()), _ptr(x), _ptr(w_conv), W,
                                                     float(l2_eps), _ptr(conv_window), _ptr(y), _stream(x.device)))
    return y


def conv1d_window(x, cu_seqlens, shape: Shape, width: int, window_in=None):
    """The conv window [N, width-1, Cch] after a prefill of x [T, Cch]."""
    dt = shape.torch_dtype
    C = shape.channels
    _need(x, "x", dt, (shape.total_tokens, C))
    _need(cu_seqlens, "cu_seqlens", torch.int32, (shape.n_seqs + 1,))
    if window_in is not None:
        _need(window_in, "window_in", dt, (shape.n_seqs, width - 1, C))
    out = torch.empty((shape.n_seqs, width - 1, C), dtype=dt, device=x.device)
    _check("gdn_conv1d_window", load().gdn_conv1d_window(ctypes.byref(shape.c()), _ptr(x), int(width),
                                                         _ptr(cu_seqlens), _ptr(window_in), _ptr(out),
                                                         _stream(x.device)))
    return out


def conv1d_prefill(x, w_conv, cu_seqlens, shape: Shape, window_in=None, want_window=True, l2_eps: float = 1e-6):
    """gdn_conv1d continuing from carried windows (None: fresh sequences).
    Returns (y [T, Cch], window_out [N, width-1, Cch] or None)."""
    dt = shape.torch_dtype
    C = shape.channels
    W = int(w_conv.shape[1])
    _need(x, "x", dt, (shape.total_tokens, C))
    _need(w_conv, "w_conv", dt, (C, W))
    _need(cu_seqlens, "cu_seqlens", torch.int32, (shape.n_seqs + 1,))
    if window_in is not None:
        _need(window_in, "window_in", dt, (shape.n_seqs, W - 1, C))
    y = torch.empty_like(x)
    win = torch.empty((shape.n_seqs, W - 1, C), dtype=dt, device=x.device) if want_window else None
    _check("gdn_conv1d_prefill", load().gdn_conv1d_prefill(ctypes.byref(shape.c()), _ptr(x), _ptr(w_conv), W,
                                                           float(l2_eps), _ptr(cu_seqlens), _ptr(window_in), _ptr(y),
                                                           _ptr(win), _stream(x.device)))
    return y, win


# ----------------------------------------------------------------------------- diagnostics
def profile_enable(on: bool) -> None:
    """Bracket every later kernel launch with HIP events (True) or stop (False)."""
    load().gdn_profile_enable(1 if on else 0)


def profile_report() -> dict:
    """{kernel name: (launches, total ms)} for the launches since profile_enable(True)."""
    lib = load()
    n = int(lib.gdn_profile_report(None, 0))
    buf = ctypes.create_string_buffer(n + 1)
    lib.gdn_profile_report(buf, n + 1)
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


# ----------------------------------------------------------------------------- achievable-peak probes
def probe_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """gdn_probe_copy of src's bytes into dst (contiguous GPU tensors)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("dst must be contiguous and at least as large as src")
    _check("gdn_probe_copy", load().gdn_probe_copy(_ptr(src), _ptr(dst), n, _stream(src.device)))


def probe_mfma(out: torch.Tensor, blocks: int, iters: int, shape: int = 0) -> int:
    """gdn_probe_mfma; out: float32 [blocks * 256]; shape 0: 16x16x32, 1: 32x32x16
    bf16 products.  Returns the flops it performs."""
    _need(out, "out", torch.float32, (blocks * 256,))
    _check("gdn_probe_mfma", load().gdn_probe_mfma(_ptr(out), int(blocks), int(iters), int(shape),
                                                   _stream(out.device)))
    return blocks * 4 * iters * 8 * 16384

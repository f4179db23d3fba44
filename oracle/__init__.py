"""CPU oracle for the GatedDeltaNet layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library (``gated_delta_rule_conv1d_amd``)
never does, and this package imports nothing from it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64; an fp32 build exists
only to show the fp32 tolerance is reachable).  This module loads it through
ctypes, adds the integer chunk table, and composes the layer:

    conv1d + SiLU + L2(q, k)  ->  gated delta rule  ->  RMSNormGated

Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (GatedDeltaNet,
RMSNormGated, depthwise conv1d, naive fallback); "Support Qwen35 SFT", XTuner
changes (varlen mode); "feat(models): dense Qwen3.5 custom attention", Summary
(cu_seqlens for one packed row).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIBS = {64: os.path.join(_HERE, "liboracle64.so"), 32: os.path.join(_HERE, "liboracle32.so")}
_loaded: Dict[int, ctypes.CDLL] = {}

L2_EPS = 1e-6
NORM_EPS = 1e-6


def build(force: bool = True) -> None:
    """Compile the oracle with gcc (fp64 and fp32 builds)."""
    for bits, out in _LIBS.items():
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
            continue
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-o", out + ".tmp", _SRC, "-lm"]
        if bits == 32:
            cmd.insert(1, "-DREAL=float")
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)


def _lib(bits: int = 64) -> ctypes.CDLL:
    if bits not in _loaded:
        if not os.path.exists(_LIBS[bits]) or os.path.getmtime(_LIBS[bits]) < os.path.getmtime(_SRC):
            build(force=False)
        lib = ctypes.CDLL(_LIBS[bits])
        _loaded[bits] = lib
    return _loaded[bits]


def threads() -> int:
    return int(_lib(64).oracle_threads())


def set_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (both builds)."""
    for bits in (64, 32):
        _lib(bits).oracle_set_threads(ctypes.c_int(int(n)))


def _dt(bits):
    return np.float64 if bits == 64 else np.float32


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, bits):
    return None if a is None else np.ascontiguousarray(a, dtype=_dt(bits))


def _real(bits):
    return ctypes.c_double if bits == 64 else ctypes.c_float


# ---------------------------------------------------------------------------
# A0: the chunk table (integers).  Chunks restart at every sequence start and
# never straddle two sequences; the last chunk of a sequence may be partial.
# ---------------------------------------------------------------------------
def chunk_table(cu: np.ndarray, chunk: int) -> Tuple[np.ndarray, np.ndarray]:
    """Return (table [n_chunks, 3] = (seq, first token, length), seq_chunk0 [N+1])."""
    cu = [int(c) for c in cu]
    rows: List[Tuple[int, int, int]] = []
    first = [0]
    for n in range(len(cu) - 1):
        t = cu[n]
        while t < cu[n + 1]:
            ln = min(chunk, cu[n + 1] - t)
            rows.append((n, t, ln))
            t += ln
        first.append(len(rows))
    return np.array(rows, dtype=np.int32).reshape(-1, 3), np.array(first, dtype=np.int32)


# ---------------------------------------------------------------------------
# Steps of the layer.
# ---------------------------------------------------------------------------
def conv1d(x, w, cu, n_qk_ch, d_k, eps=L2_EPS, bits=64):
    """Causal depthwise conv + SiLU + per-head L2 of the first n_qk_ch channels."""
    x = _c(x, bits); w = _c(w, bits); cu = np.ascontiguousarray(cu, dtype=np.int32)
    T, Cch = x.shape
    y = np.empty_like(x)
    _lib(bits).oracle_conv1d(ctypes.c_int(len(cu) - 1), _p(cu), ctypes.c_int(Cch),
                             ctypes.c_int(w.shape[1]), ctypes.c_int(n_qk_ch), ctypes.c_int(d_k),
                             _real(bits)(eps), _p(x), _p(w), _p(y))
    return y


def conv1d_bwd(x, w, cu, n_qk_ch, d_k, dy, eps=L2_EPS, bits=64):
    x = _c(x, bits); w = _c(w, bits); dy = _c(dy, bits); cu = np.ascontiguousarray(cu, dtype=np.int32)
    T, Cch = x.shape
    dx = np.empty_like(x)
    dw = np.empty_like(w)
    _lib(bits).oracle_conv1d_bwd(ctypes.c_int(len(cu) - 1), _p(cu), ctypes.c_int(Cch),
                                 ctypes.c_int(w.shape[1]), ctypes.c_int(n_qk_ch), ctypes.c_int(d_k),
                                 _real(bits)(eps), _p(x), _p(w), _p(dy), _p(dx), _p(dw))
    return dx, dw


def recurrence(q, k, v, g, beta, cu, h0=None, scale=1.0, bits=64):
    """Gated delta rule.  q, k: [T, Hk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv];
    h0: [N, Hv, dk, dv] or None.  Returns (o [T, Hv, dv], ht [N, Hv, dk, dv])."""
    q = _c(q, bits); k = _c(k, bits); v = _c(v, bits)
    g = _c(g, bits); beta = _c(beta, bits); h0 = _c(h0, bits)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T, Hk, dk = q.shape
    _, Hv, dv = v.shape
    N = len(cu) - 1
    o = np.empty((T, Hv, dv), dtype=_dt(bits))
    ht = np.empty((N, Hv, dk, dv), dtype=_dt(bits))
    _lib(bits).oracle_recurrence(ctypes.c_int(N), _p(cu), ctypes.c_int(Hk), ctypes.c_int(Hv),
                                 ctypes.c_int(dk), ctypes.c_int(dv), _real(bits)(scale),
                                 _p(q), _p(k), ctypes.c_long(Hk * dk), _p(v), ctypes.c_long(Hv * dv),
                                 _p(g), _p(beta), _p(h0), _p(o), _p(ht))
    return o, ht


def recurrence_bwd(q, k, v, g, beta, cu, d_o, h0=None, dht=None, scale=1.0, bits=64):
    """Reverse mode of `recurrence`.  Returns dict dq, dk, dv, dg, dbeta, dh0."""
    q = _c(q, bits); k = _c(k, bits); v = _c(v, bits)
    g = _c(g, bits); beta = _c(beta, bits); h0 = _c(h0, bits)
    d_o = _c(d_o, bits); dht = _c(dht, bits)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T, Hk, dk = q.shape
    _, Hv, dv = v.shape
    N = len(cu) - 1
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v),
               dg=np.empty((T, Hv), dtype=_dt(bits)), dbeta=np.empty((T, Hv), dtype=_dt(bits)),
               dh0=np.empty((N, Hv, dk, dv), dtype=_dt(bits)))
    _lib(bits).oracle_recurrence_bwd(
        ctypes.c_int(N), _p(cu), ctypes.c_int(Hk), ctypes.c_int(Hv), ctypes.c_int(dk), ctypes.c_int(dv),
        _real(bits)(scale), _p(q), _p(k), ctypes.c_long(Hk * dk), _p(v), ctypes.c_long(Hv * dv),
        _p(g), _p(beta), _p(h0), _p(d_o), _p(dht),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dg"]), _p(out["dbeta"]), _p(out["dh0"]))
    return out


def norm_gate(o, z, w, eps=NORM_EPS, bits=64):
    """RMSNormGated over the last axis: o * rsqrt(mean(o^2)+eps) * w * silu(z)."""
    o = _c(o, bits); z = _c(z, bits); w = _c(w, bits)
    dv = o.shape[-1]
    y = np.empty_like(o)
    _lib(bits).oracle_norm_gate(ctypes.c_long(o.size // dv), ctypes.c_int(dv), _real(bits)(eps),
                                _p(o), _p(z), _p(w), _p(y))
    return y


def norm_gate_bwd(o, z, w, dy, eps=NORM_EPS, bits=64):
    o = _c(o, bits); z = _c(z, bits); w = _c(w, bits); dy = _c(dy, bits)
    dv = o.shape[-1]
    d_o = np.empty_like(o); dz = np.empty_like(z); dw = np.empty_like(w)
    _lib(bits).oracle_norm_gate_bwd(ctypes.c_long(o.size // dv), ctypes.c_int(dv), _real(bits)(eps),
                                    _p(dy), _p(o), _p(z), _p(w), _p(d_o), _p(dz), _p(dw))
    return d_o, dz, dw


def gates(a, b, A_log, dt_bias, bits=64):
    """g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b); a, b [T, Hv]."""
    a = _c(a, bits); b = _c(b, bits); A_log = _c(A_log, bits); dt_bias = _c(dt_bias, bits)
    T, Hv = a.shape
    g = np.empty_like(a); beta = np.empty_like(b)
    _lib(bits).oracle_gates(ctypes.c_long(T), ctypes.c_int(Hv), _p(a), _p(b), _p(A_log), _p(dt_bias),
                            _p(g), _p(beta))
    return g, beta


def gates_bwd(a, b, A_log, dt_bias, dg, dbeta, bits=64):
    """Gradients of gates(): da, db [T, Hv]; dA_log, ddt_bias [Hv]."""
    a = _c(a, bits); b = _c(b, bits); A_log = _c(A_log, bits); dt_bias = _c(dt_bias, bits)
    dg = _c(dg, bits); dbeta = _c(dbeta, bits)
    T, Hv = a.shape
    da = np.empty_like(a); db = np.empty_like(b)
    dA = np.empty_like(A_log); ddt = np.empty_like(dt_bias)
    _lib(bits).oracle_gates_bwd(ctypes.c_long(T), ctypes.c_int(Hv), _p(a), _p(b), _p(A_log), _p(dt_bias),
                                _p(dg), _p(dbeta), _p(da), _p(db), _p(dA), _p(ddt))
    return dict(da=da, db=db, dA_log=dA, ddt_bias=ddt)


# ---------------------------------------------------------------------------
# The whole layer.
# ---------------------------------------------------------------------------
def split_qkv(y, Hk, Hv, dk, dv):
    T = y.shape[0]
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    return q, k, v


def _store(a, storage):
    """Round a tensor that crosses a call boundary to its storage format.

    With storage="bf16" the layer is computed as the four calls of the library
    compose it: the conv output and the recurrence output (and, backward, the
    gradients handed from one call to the next) are stored as bf16 between
    calls, so the oracle rounds exactly those tensors, to nearest-even, and
    computes everything else in full precision."""
    if storage == "bf16":
        import synth  # the seeded-input module; only its rounding helper is used
        return synth.round_bf16(np.asarray(a, dtype=np.float32)).astype(np.float64)
    return a


def layer_fwd(cfg, inp, bits=64, scale=1.0, storage=None):
    """Forward of the layer on one workload's inputs (see synth.make_inputs).

    Returns dict: y_conv [T, Cch], o [T, Hv, dv], ht [N, Hv, dk, dv] and, when
    the workload has the norm, y [T, Hv, dv].  y_conv and o are the values the
    next step consumes (rounded to the storage format); y_conv_exact and
    o_exact are the same tensors before that rounding."""
    Hk, Hv, dk, dv = cfg.h_qk, cfg.h_v, cfg.d_k, cfg.d_v
    yc_exact = conv1d(inp["x"], inp["w_conv"], inp["cu"], 2 * Hk * dk, dk, bits=bits)
    yc = _store(yc_exact, storage)
    q, k, v = split_qkv(yc, Hk, Hv, dk, dv)
    o_exact, ht = recurrence(q, k, v, inp["g"], inp["beta"], inp["cu"], h0=inp.get("h0"), scale=scale, bits=bits)
    o = _store(o_exact, storage)
    out = dict(y_conv=yc, o=o, ht=ht, y_conv_exact=yc_exact, o_exact=o_exact)
    if cfg.norm:
        out["y"] = norm_gate(o, inp["z"], inp["w_norm"], bits=bits)
    return out


def layer_bwd(cfg, inp, fwd, dy, bits=64, scale=1.0, dht=None, storage=None):
    """Backward of the layer given the upstream gradient dy on its output
    (the norm output if present, else o).  Returns dict with dx, dw_conv, dg,
    dbeta, dh0, and dz, dw_norm when the norm is present; also the gradients
    at the recurrence inputs (dq, dk, dv) and d_o (rounded to the storage
    format, as the recurrence's backward consumes it; d_o_exact before)."""
    Hk, Hv, dk, dv = cfg.h_qk, cfg.h_v, cfg.d_k, cfg.d_v
    res = {}
    if cfg.norm:
        d_o_exact, dz, dwn = norm_gate_bwd(fwd["o"], inp["z"], inp["w_norm"], dy, bits=bits)
        d_o = _store(d_o_exact, storage)
        res.update(dz=dz, dw_norm=dwn)
    else:
        d_o = d_o_exact = dy
    res["d_o"] = d_o
    res["d_o_exact"] = d_o_exact
    q, k, v = split_qkv(fwd["y_conv"], Hk, Hv, dk, dv)
    r = recurrence_bwd(q, k, v, inp["g"], inp["beta"], inp["cu"], d_o, h0=inp.get("h0"), dht=dht,
                       scale=scale, bits=bits)
    res.update(dq=r["dq"], dk=r["dk"], dv=r["dv"], dg=r["dg"], dbeta=r["dbeta"], dh0=r["dh0"])
    T = q.shape[0]
    dyc = _store(np.concatenate([r["dq"].reshape(T, Hk * dk), r["dk"].reshape(T, Hk * dk),
                                 r["dv"].reshape(T, Hv * dv)], axis=1), storage)
    dx, dwc = conv1d_bwd(inp["x"], inp["w_conv"], inp["cu"], 2 * Hk * dk, dk, dyc, bits=bits)
    res.update(dx=dx, dw_conv=dwc)
    return res


def subset(cfg, inp, seqs, kheads):
    """Restrict a workload to some sequences and k-heads (with their v-heads).

    Every step of the layer is independent across sequences and across
    k-head groups, except the weight-gradient sums, so the oracle can check
    sampled outputs of a full-size run by recomputing only a subset.
    Returns (cfg', inp', token index array, v-head index array)."""
    cu = inp["cu"]
    G = cfg.h_v // cfg.h_qk
    Hk, Hv, dk, dv = cfg.h_qk, cfg.h_v, cfg.d_k, cfg.d_v
    toks = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]).astype(np.int64)
    vheads = np.array([j * G + i for j in kheads for i in range(G)], dtype=np.int64)
    qch = np.concatenate([np.arange(j * dk, (j + 1) * dk) for j in kheads])
    kch = qch + Hk * dk
    vch = np.concatenate([2 * Hk * dk + np.arange(h * dv, (h + 1) * dv) for h in vheads])
    ch = np.concatenate([qch, kch, vch])
    lens = [int(cu[n + 1] - cu[n]) for n in seqs]
    sub = {"cu": np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
           "x": inp["x"][toks][:, ch], "w_conv": inp["w_conv"][ch],
           "g": inp["g"][toks][:, vheads], "beta": inp["beta"][toks][:, vheads]}
    if "z" in inp:
        sub["z"] = inp["z"][toks][:, vheads]
        sub["w_norm"] = inp["w_norm"]
    if "h0" in inp:
        sub["h0"] = inp["h0"][np.asarray(seqs)][:, vheads]
    if "dy" in inp:
        sub["dy"] = inp["dy"][toks][:, vheads]
    c2 = cfg.replace(h_qk=len(kheads), h_v=len(vheads), lengths=tuple(lens), varlen_rule=None)
    return c2, sub, toks, vheads

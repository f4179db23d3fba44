"""Seeded synthetic inputs for the GatedDeltaNet layer over packed varlen rows.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It only draws random numbers and rounds them to the storage precision; it holds
none of the layer's arithmetic (conv, normalisation, recurrence, gating norm).

The gate values ``g`` and ``beta`` are *inputs* of the library: the workloads
define their distribution as ``g = -exp(A_log) * softplus(a + dt_bias)`` and
``beta = sigmoid(b)``, so the transform that shapes that distribution lives here
next to the other draws.  (Pages: "[Qwen3.5 MoE] Add hybrid decoder model",
Summary, names the softplus gate; "feat(models): dense Qwen3.5 custom
attention", Summary, names cu_seqlens as the varlen boundary.)

Draw order for one workload (one ``numpy.random.default_rng(seed)`` stream):
  1. sequence lengths (varlen workload only)
  2. x_q [T, Hk*dk], x_k [T, Hk*dk], x_v [T, Hv*dv]   ~ N(0, 1)
  3. w_conv [Cch, width]                              ~ N(0, 0.25)  (std)
  4. A_log [Hv] ~ U(0, 2);  dt_bias [Hv] = 0
  5. a [T, Hv] ~ N(0, 1);  b [T, Hv] ~ N(0, 1)
  6. g, beta (fp32, from 4-5)
  7. z [T, Hv, dv] ~ N(0, 1)                          (workloads with the norm)
  8. w_norm [dv] = 1 + N(0, 0.02)                     (workloads with the norm)
  9. h0 [N, Hv, dk, dv] ~ N(0, 0.1)                   (workloads with h0)
 10. dy [T, Hv, dv] ~ N(0, 1)                         (workloads with backward)
 11. window [N, width-1, Cch] ~ N(0, 1)               (the decode workload: the
     previous width-1 inputs of each continuing sequence)
Large arrays are drawn directly in float32; bf16 workloads then round every
bf16 tensor to bf16 with round-to-nearest-even, and both sides get exactly
those values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "make_inputs", "cu_from_lengths",
    "varlen_lengths", "bf16_bits", "bf16_value", "round_bf16",
]


@dataclass(frozen=True)
class Config:
    name: str
    lengths: tuple            # per-sequence token counts (sum = T)
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str                # "f32" or "bf16"
    norm: bool                # RMSNormGated epilogue present
    h0: bool                  # random initial states supplied
    bwd: bool                 # backward pass part of the workload
    seed: int
    width: int = 4            # depthwise causal conv taps
    weak_decay: bool = False  # A_log = -6: g ~ -0.0025 per token (long-range carry)
    varlen_rule: Optional[tuple] = None  # (n_seqs, total, lo, hi) when lengths are drawn
    decode: bool = False      # one token per sequence continuing from a state and a conv window

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def channels(self) -> int:
        return 2 * self.h_qk * self.d_k + self.h_v * self.d_v

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _base(name, lengths, seed, **kw):
    d = dict(h_qk=16, h_v=32, d_k=128, d_v=128, chunk=64, dtype="bf16",
             norm=True, h0=False, bwd=False)
    d.update(kw)
    return Config(name=name, lengths=tuple(lengths), seed=seed, **d)


#: The five workloads: tiny fp32 check, dense batch, varlen packed row with
#: states, long single sequence, and the training step (forward + backward).
CONFIGS: List[Config] = [
    Config(name="tiny", lengths=(64,), h_qk=2, h_v=2, d_k=16, d_v=16, chunk=16,
           dtype="f32", norm=False, h0=False, bwd=False, seed=0),
    _base("dense", [2048] * 4, seed=1),
    _base("varlen", [], seed=2, h0=True, varlen_rule=(20, 32768, 64, 8192)),
    _base("long", [65536], seed=3),
    _base("train", [8192] * 8, seed=4, bwd=True),
    # continuation: 256 sequences advance by one token each, from states and
    # conv windows (the previous width-1 inputs) drawn like h0 and x
    _base("decode", [1] * 256, seed=5, h0=True, decode=True),
]


def config(name: str) -> Config:
    """Return a workload by name, with drawn lengths resolved."""
    for c in CONFIGS:
        if c.name == name:
            if c.varlen_rule is not None and not c.lengths:
                rng = np.random.default_rng(c.seed)
                return c.replace(lengths=tuple(int(x) for x in varlen_lengths(rng, *c.varlen_rule)))
            return c
    raise KeyError(name)


def varlen_lengths(rng: np.random.Generator, n: int, total: int, lo: int, hi: int) -> np.ndarray:
    """Draw n lengths log-uniform in [lo, hi] whose total reaches `total`.

    The last length is cut so the sum is exactly `total`.  A draw whose first
    n-1 lengths already reach `total`, or whose n lengths fall short, is
    discarded and the next n lengths are drawn from the same stream.
    """
    while True:
        lens = np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))).astype(np.int64)
        head = int(lens[:-1].sum())
        if head < total <= head + int(lens[-1]):
            lens[-1] = total - head
            return lens


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 20  # blocks that stay in cache
    for i in range(0, u.size, step):
        ub = u[i:i + step]
        r = (ub >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += ub
        r >>= np.uint32(16)
        out[i:i + step] = r
    return out.reshape(a.shape)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact float32 values they encode."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_value(bf16_bits(a))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def make_inputs(cfg: Config, *, keep_raw: bool = False) -> Dict[str, np.ndarray]:
    """Draw every input of one workload.

    Returns float32 arrays holding the exact values both sides consume (for
    bf16 workloads these are bf16-representable), plus ``*_bits`` uint16 bf16
    patterns for the bf16 tensors.  Keys: cu, x, w_conv, g, beta and, where the
    workload has them, z, w_norm, h0, dy.  With keep_raw the gate parameters
    A_log, dt_bias, a, b are returned too.
    """
    rng = np.random.default_rng(cfg.seed)
    lengths = cfg.lengths
    if cfg.varlen_rule is not None:
        drawn = tuple(int(x) for x in varlen_lengths(rng, *cfg.varlen_rule))
        if lengths and tuple(lengths) != drawn:
            raise ValueError("lengths of a drawn-length workload cannot be overridden")
        lengths = drawn
    T = int(sum(lengths))
    Hk, Hv, dk, dv, W = cfg.h_qk, cfg.h_v, cfg.d_k, cfg.d_v, cfg.width
    Cch = 2 * Hk * dk + Hv * dv
    out: Dict[str, np.ndarray] = {"cu": cu_from_lengths(lengths)}

    x = np.empty((T, Cch), dtype=np.float32)
    x[:, : Hk * dk] = rng.standard_normal((T, Hk * dk), dtype=np.float32)
    x[:, Hk * dk: 2 * Hk * dk] = rng.standard_normal((T, Hk * dk), dtype=np.float32)
    x[:, 2 * Hk * dk:] = rng.standard_normal((T, Hv * dv), dtype=np.float32)
    w_conv = (0.25 * rng.standard_normal((Cch, W))).astype(np.float32)
    A_log = rng.uniform(0.0, 2.0, size=Hv)
    if cfg.weak_decay:
        A_log = np.full(Hv, -6.0)
    dt_bias = np.zeros(Hv)
    a = rng.standard_normal((T, Hv))
    b = rng.standard_normal((T, Hv))
    g = (-np.exp(A_log)[None, :] * _softplus(a + dt_bias[None, :])).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
    out.update(g=g, beta=beta)
    if keep_raw:
        out.update(A_log=A_log, dt_bias=dt_bias, a=a, b=b)
    if cfg.norm:
        out["z"] = rng.standard_normal((T, Hv, dv), dtype=np.float32)
        out["w_norm"] = (1.0 + 0.02 * rng.standard_normal(dv)).astype(np.float32)
    if cfg.h0:
        out["h0"] = (0.1 * rng.standard_normal((len(lengths), Hv, dk, dv))).astype(np.float32)
    if cfg.bwd:
        out["dy"] = rng.standard_normal((T, Hv, dv), dtype=np.float32)
    if cfg.decode:
        out["window"] = rng.standard_normal((len(lengths), W - 1, Cch), dtype=np.float32)
    out["x"] = x
    out["w_conv"] = w_conv

    if cfg.dtype == "bf16":
        for key in ("x", "w_conv", "z", "w_norm", "dy", "window"):
            if key in out:
                bits = bf16_bits(out[key])
                out[key + "_bits"] = bits
                out[key] = bf16_value(bits)
    elif cfg.dtype != "f32":
        raise ValueError(cfg.dtype)
    return out

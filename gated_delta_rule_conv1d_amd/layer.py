"""The whole GatedDeltaNet layer (conv1d+SiLU+L2 -> chunked gated delta rule ->
RMSNormGated) and its backward, composed from the C-ABI calls.

Workspaces are allocated once per layer object and reused, so a timed loop
allocates nothing.  Pages: "[Qwen3.5 MoE] Add hybrid decoder model",
Summary (GatedDeltaNet with RMSNormGated); "Support Qwen35 SFT", XTuner
changes (varlen mode).
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _binding as B


class GatedDeltaNetLayer:
    """Holds the shape and reusable workspaces of one layer configuration."""

    def __init__(self, shape: B.Shape, width: int = 4, device="cuda", norm: bool = True,
                 l2_eps: float = 1e-6, norm_eps: float = 1e-6):
        self.shape, self.width, self.norm = shape, width, norm
        self.l2_eps, self.norm_eps = l2_eps, norm_eps
        self.device = torch.device(device)
        self._ws: Dict[str, torch.Tensor] = {}
        self._saved = False  # the backward workspace holds a forward's products

    def _buf(self, name: str, nbytes: int) -> torch.Tensor:
        t = self._ws.get(name)
        if t is None or t.numel() < nbytes:
            t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._ws[name] = t
        return t

    def split(self, y: torch.Tensor):
        s = self.shape
        nq = s.h_qk * s.d_k
        return y[:, :nq], y[:, nq:2 * nq], y[:, 2 * nq:]

    def gates(self, a, b, A_log, dt_bias):
        """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b) (gdn_gates)."""
        return B.gates(a, b, A_log, dt_bias, self.shape)

    def gates_backward(self, a, b, A_log, dt_bias, dg, dbeta):
        """da, db, dA_log, ddt_bias from the dg, dbeta of backward() (gdn_gates_bwd)."""
        return B.gates_bwd(a, b, A_log, dt_bias, dg, dbeta, self.shape,
                           ws=self._buf("gates", B.gates_bwd_workspace(self.shape)))

    def forward(self, x, w_conv, g, beta, cu_seqlens, z=None, w_norm=None, h0=None, want_ht=True,
                for_backward=False, gates=None):
        """With for_backward=True the chunked recurrence keeps its per-chunk
        products in this layer's backward workspace (gdn_chunk_fwd_save), and
        the next backward() with the same inputs reads them instead of
        recomputing them.  gates = (a, b, A_log, dt_bias) instead of g, beta
        (both None): the chunk kernels compute the gates themselves
        (gdn_chunk_fwd_gated)."""
        s = self.shape
        yc = B.conv1d(x, w_conv, cu_seqlens, s, self.l2_eps)
        q, k, v = self.split(yc)
        ws = (self._buf("bwd", B.chunk_bwd_workspace(s)) if for_backward
              else self._buf("fwd", B.chunk_fwd_workspace(s)))
        if gates is not None:
            if g is not None or beta is not None:
                raise ValueError("pass either g, beta or gates")
            o, ht = B.chunk_fwd_gated(q, k, v, gates, cu_seqlens, s, h0=h0, want_ht=want_ht, ws=ws,
                                      save=for_backward)
        else:
            o, ht = B.chunk_fwd(q, k, v, g, beta, cu_seqlens, s, h0=h0, want_ht=want_ht, ws=ws, save=for_backward)
        self._saved = for_backward
        out = dict(y_conv=yc, o=o, ht=ht)
        if self.norm:
            out["y"] = B.norm_gate(o, z, w_norm, s, self.norm_eps)
        return out

    def backward(self, dy, x, w_conv, g, beta, cu_seqlens, fwd, z=None, w_norm=None, h0=None, dht=None,
                 gates=None):
        """dy: gradient w.r.t. the layer output (norm output if present, else o).
        Recomputes nothing of the conv except inside its own backward.  With
        gates = (a, b, A_log, dt_bias) (as in forward) the result holds da, db,
        dA_log, ddt_bias instead of dg, dbeta."""
        s = self.shape
        res = {}
        if self.norm:
            d_o, dz, dwn = B.norm_gate_bwd(dy, fwd["o"], z, w_norm, s, self.norm_eps,
                                           ws=self._buf("norm", B.norm_gate_bwd_workspace(s)))
            res.update(dz=dz, dw_norm=dwn)
        else:
            d_o = dy
        q, k, v = self.split(fwd["y_conv"])
        dyc = torch.empty_like(fwd["y_conv"])
        dq, dk, dv = self.split(dyc)
        ws = self._buf("bwd", B.chunk_bwd_workspace(s))
        if gates is not None:
            r = B.chunk_bwd_gated(q, k, v, gates, cu_seqlens, s, d_o, h0=h0, dht=dht, dq=dq, dk=dk, dv=dv,
                                  want_dh0=h0 is not None, ws=ws, saved=self._saved)
            res.update({key: r[key] for key in ("da", "db", "dA_log", "ddt_bias")})
        else:
            r = B.chunk_bwd(q, k, v, g, beta, cu_seqlens, s, d_o, h0=h0, dht=dht, dq=dq, dk=dk, dv=dv,
                            want_dh0=h0 is not None, ws=ws, saved=self._saved)
            res.update(dg=r["dg"], dbeta=r["dbeta"])
        self._saved = False  # the saved products are consumed
        dx, dwc = B.conv1d_bwd(dyc, x, w_conv, cu_seqlens, s, self.l2_eps,
                               ws=self._buf("conv", B.conv1d_bwd_workspace(s, self.width)))
        res.update(d_o=d_o, dy_conv=dyc, dh0=r["dh0"], dx=dx, dw_conv=dwc)
        return res


def layer_forward(shape: B.Shape, x, w_conv, g, beta, cu_seqlens, z=None, w_norm=None, h0=None, norm=True):
    return GatedDeltaNetLayer(shape, int(w_conv.shape[1]), x.device, norm).forward(
        x, w_conv, g, beta, cu_seqlens, z, w_norm, h0)


def layer_backward(shape: B.Shape, dy, x, w_conv, g, beta, cu_seqlens, fwd, z=None, w_norm=None, h0=None,
                   norm=True, dht=None):
    return GatedDeltaNetLayer(shape, int(w_conv.shape[1]), x.device, norm).backward(
        dy, x, w_conv, g, beta, cu_seqlens, fwd, z, w_norm, h0, dht)

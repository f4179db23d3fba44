"""The whole GatedDeltaNet layer (conv1d+SiLU+L2 -> chunked gated delta rule ->
RMSNormGated) and its backward, composed from the C-ABI calls.

Workspaces are allocated once per layer object and reused, so a timed loop
allocates nothing.  Pages: "[Qwen3.5 MoE] Add hybrid decoder model",
Summary (GatedDeltaNet with RMSNormGated); "Support Qwen35 SFT", XTuner
changes (varlen mode).
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Tuple, TypeVar

import torch

from . import _binding as B


def token_segments(cu: List[int], chunk: int, max_tokens: int) -> List[Tuple[int, int, int, int, Optional[Tuple[int, int]]]]:
    """Split a packed row (host cu_seqlens) into token segments of at most
    P = max(chunk, max_tokens rounded down to whole chunks) tokens, in token
    order: runs of whole sequences, or pieces of one sequence longer than P
    cut at multiples of P from its start (so the pieces' chunks are the
    sequence's own chunks).  Each entry is (t0, t1, n0, n1, piece): tokens
    [t0, t1) hold sequences n0 .. n1-1, and piece = (index, count) for a piece
    of sequence n0, else None."""
    P = max(chunk, (max_tokens // chunk) * chunk)
    segs = []
    n, N = 0, len(cu) - 1
    while n < N:
        L = cu[n + 1] - cu[n]
        if L > P:
            count = -(-L // P)
            for i in range(count):
                segs.append((cu[n] + i * P, min(cu[n] + (i + 1) * P, cu[n + 1]), n, n + 1, (i, count)))
            n += 1
            continue
        n1 = n + 1
        while n1 < N and cu[n1 + 1] - cu[n] <= P:
            n1 += 1
        segs.append((cu[n], cu[n1], n, n1, None))
        n = n1
    return segs


class GatedDeltaNetLayer:
    """Holds the shape and reusable workspaces of one layer configuration."""

    def __init__(self, shape: B.Shape, width: int = 4, device="cuda", norm: bool = True,
                 l2_eps: float = 1e-6, norm_eps: float = 1e-6):
        self.shape, self.width, self.norm = shape, width, norm
        self.l2_eps, self.norm_eps = l2_eps, norm_eps
        self.device = torch.device(device)
        self._ws: Dict[str, torch.Tensor] = {}
        self._saved = False  # the backward workspace holds a forward's products
        self._segs = None    # a segmented forward's segments, for the backward (max_tokens)

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
                for_backward=False, gates=None, max_tokens: Optional[int] = None):
        """With for_backward=True the chunked recurrence keeps its per-chunk
        products in this layer's backward workspace (gdn_chunk_fwd_save), and
        the next backward() with the same inputs reads them instead of
        recomputing them.  gates = (a, b, A_log, dt_bias) instead of g, beta
        (both None): the chunk kernels compute the gates themselves
        (gdn_chunk_fwd_gated).  max_tokens bounds the chunk workspaces to one
        token segment of that size (see token_segments): the recurrence runs
        segment by segment, carrying each long sequence's state from piece to
        piece, and the next backward() recomputes per segment (cu_seqlens is
        read on the host once)."""
        s = self.shape
        yc = B.conv1d(x, w_conv, cu_seqlens, s, self.l2_eps)
        if max_tokens is not None:
            if gates is not None or for_backward:
                raise ValueError("max_tokens runs the recomputing pair with g, beta")
            o, ht = self._chunk_fwd_segmented(yc, g, beta, cu_seqlens, h0, want_ht, max_tokens)
            self._saved = False
            out = dict(y_conv=yc, o=o, ht=ht)
            if self.norm:
                out["y"] = B.norm_gate(o, z, w_norm, s, self.norm_eps)
            return out
        self._segs = None
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
        if getattr(self, "_segs", None) is not None:
            if gates is not None:
                raise ValueError("the segmented pass takes g, beta")
            r = self._chunk_bwd_segmented(q, k, v, g, beta, d_o, h0, dht, dq, dk, dv)
            res.update(dg=r["dg"], dbeta=r["dbeta"])
            dx, dwc = B.conv1d_bwd(dyc, x, w_conv, cu_seqlens, s, self.l2_eps,
                                   ws=self._buf("conv", B.conv1d_bwd_workspace(s, self.width)))
            res.update(d_o=d_o, dy_conv=dyc, dh0=r["dh0"], dx=dx, dw_conv=dwc)
            return res
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


    # ---- bounded-memory mode: the chunk calls segment by segment ----
    def _seg_shape(self, n, T) -> B.Shape:
        s = self.shape
        return B.Shape(n, T, s.h_qk, s.h_v, s.d_k, s.d_v, s.chunk, s.dtype, s.scale)

    def _chunk_fwd_segmented(self, yc, g, beta, cu_seqlens, h0, want_ht, max_tokens):
        s = self.shape
        cu = [int(c) for c in cu_seqlens.cpu().tolist()]
        segs = token_segments(cu, s.chunk, max_tokens)
        dev = yc.device
        # every segment's own cu_seqlens (offsets from its first token), in one transfer
        flat = []
        for t0, t1, n0, n1, piece in segs:
            flat += [0, t1 - t0] if piece is not None else [c - t0 for c in cu[n0:n1 + 1]]
        cu_all = torch.tensor(flat, dtype=torch.int32).to(dev)
        cu_segs, o_ = [], 0
        for t0, t1, n0, n1, piece in segs:
            m = 2 if piece is not None else n1 - n0 + 1
            cu_segs.append(cu_all[o_:o_ + m])
            o_ += m
        q, k, v = self.split(yc)
        o = torch.empty((s.total_tokens, s.h_v, s.d_v), dtype=s.torch_dtype, device=dev)
        ht = torch.empty((s.n_seqs, s.h_v, s.d_k, s.d_v), dtype=torch.float32, device=dev) if want_ht else None
        fwd_ws = max(B.chunk_fwd_workspace(self._seg_shape(n1 - n0, t1 - t0)) for t0, t1, n0, n1, _ in segs) \
            if segs else 0
        bwd_ws = max(B.chunk_bwd_workspace(self._seg_shape(n1 - n0, t1 - t0)) for t0, t1, n0, n1, _ in segs) \
            if segs else 0
        ws = self._buf("seg_fwd", fwd_ws)
        entering = {}  # segment index -> state entering that piece of its sequence
        carry = None
        for i, (t0, t1, n0, n1, piece) in enumerate(segs):
            sh = self._seg_shape(n1 - n0, t1 - t0)
            inner = piece is not None and piece[0] > 0
            h0s = carry if inner else (h0[n0:n1] if h0 is not None else None)
            if inner:
                entering[i] = h0s
            more = piece is not None and piece[0] + 1 < piece[1]  # a later piece takes this state
            dst = None if (more or not want_ht) else ht[n0:n1]
            _, hs = B.chunk_fwd(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1], cu_segs[i], sh, h0=h0s,
                                want_ht=more or want_ht, ws=ws, out=o[t0:t1], ht_out=dst)
            carry = hs if more else None
        self._segs = (segs, cu_segs, entering, bwd_ws)
        return o, ht

    def _chunk_bwd_segmented(self, q, k, v, g, beta, d_o, h0, dht, dq, dk, dv):
        s = self.shape
        segs, cu_segs, entering, bwd_ws = self._segs
        dev = q.device
        dg = torch.empty((s.total_tokens, s.h_v), dtype=torch.float32, device=dev)
        db = torch.empty((s.total_tokens, s.h_v), dtype=torch.float32, device=dev)
        dh0 = torch.empty((s.n_seqs, s.h_v, s.d_k, s.d_v), dtype=torch.float32, device=dev) if h0 is not None else None
        ws = self._buf("seg_bwd", bwd_ws)
        carry = None  # gradient w.r.t. the state leaving the current piece, from the piece after it
        for i in reversed(range(len(segs))):
            t0, t1, n0, n1, piece = segs[i]
            sh = self._seg_shape(n1 - n0, t1 - t0)
            last = piece is None or piece[0] + 1 == piece[1]
            first = piece is None or piece[0] == 0
            dhts = (dht[n0:n1] if dht is not None else None) if last else carry
            h0s = (h0[n0:n1] if h0 is not None else None) if first else entering[i]
            r = B.chunk_bwd(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1], cu_segs[i], sh, d_o[t0:t1],
                            h0=h0s, dht=dhts, dq=dq[t0:t1], dk=dk[t0:t1], dv=dv[t0:t1],
                            want_dh0=(not first) or dh0 is not None, ws=ws, dg=dg[t0:t1], dbeta=db[t0:t1],
                            dh0=dh0[n0:n1] if (first and dh0 is not None) else None)
            carry = None if first else r["dh0"]
        self._segs = None
        return dict(dg=dg, dbeta=db, dh0=dh0)


R = TypeVar("R")


def capture(step: Callable[[], R]) -> Tuple["torch.cuda.CUDAGraph", R]:
    """Record one call of `step` into a HIP graph; return (graph, what step
    returned).  graph.replay() then re-issues every kernel of that call as one
    graph launch, without the per-launch host work.

    step() enqueues this library's calls on the current stream.  The entry
    points it may use launch kernels only (no HIP allocation, memset, copy or
    host synchronisation), so their launches record as plain kernel nodes.
    Not capturable: the bounded-memory mode (forward(max_tokens=...)), which
    reads cu_seqlens on the host, and per-kernel timing (profile_enable), whose
    HIP events are not graph nodes: switch it off before capturing.  Run
    step() once before capturing, so that the layers' workspaces already exist
    (a workspace first allocated during capture comes from the graph's memory
    pool and stays there).  Tensors that step allocates come from the graph's
    private pool: each replay rewrites them in place, and reads whatever the
    captured input tensors hold at that moment (copy new inputs into them)."""
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    return graph, out


def layer_forward(shape: B.Shape, x, w_conv, g, beta, cu_seqlens, z=None, w_norm=None, h0=None, norm=True):
    return GatedDeltaNetLayer(shape, int(w_conv.shape[1]), x.device, norm).forward(
        x, w_conv, g, beta, cu_seqlens, z, w_norm, h0)


def layer_backward(shape: B.Shape, dy, x, w_conv, g, beta, cu_seqlens, fwd, z=None, w_norm=None, h0=None,
                   norm=True, dht=None):
    return GatedDeltaNetLayer(shape, int(w_conv.shape[1]), x.device, norm).backward(
        dy, x, w_conv, g, beta, cu_seqlens, fwd, z, w_norm, h0, dht)

"""Chunked (WY) form of the gated delta rule in plain NumPy fp64, forward and
backward.  Test helper only: it checks that the chunked algebra the GPU kernels
use reproduces the token-by-token oracle for any chunk size, and that the
chunk-local gradient identities are right.  It is neither the oracle nor the
GPU path, and imports neither.

Per chunk (rows r, s inside the chunk, state H = S^T entering it):
  gamma_r = sum_{s<=r} g_s,  Gam = e^gamma,  D_rs = e^{gamma_r - gamma_s} (r >= s)
  A  = strict_lower(diag(beta) (D * K K^T)),  T = (I + A)^-1
  U  = T diag(beta) V,   Wk = T diag(beta Gam) K,   W = U - Wk H
  P  = lower_incl(D * Q K^T)
  O  = scale (diag(Gam) Q H + P W)
  H' = Gam_last H + K^T diag(e^{gamma_last - gamma}) W
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _chunks(cu, C):
    for n in range(len(cu) - 1):
        t = int(cu[n])
        while t < cu[n + 1]:
            L = min(C, int(cu[n + 1]) - t)
            yield n, t, L
            t += L


def _local(Q, K, V, g, b):
    L = len(g)
    gam = np.cumsum(g)
    Gam = np.exp(gam)
    diff = gam[:, None] - gam[None, :]
    incl = np.tril(np.ones((L, L), dtype=bool))
    strict = np.tril(np.ones((L, L), dtype=bool), -1)
    D = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
    Skk = K @ K.T
    A = np.where(strict, b[:, None] * D * Skk, 0.0)
    Tm = solve_triangular(np.eye(L) + A, np.eye(L), lower=True, unit_diagonal=True)
    U = Tm @ (b[:, None] * V)
    Wk = Tm @ ((b * Gam)[:, None] * K)
    P = np.where(incl, D * (Q @ K.T), 0.0)
    e = np.exp(gam[-1] - gam)
    return dict(gam=gam, Gam=Gam, D=D, Skk=Skk, A=A, Tm=Tm, U=U, Wk=Wk, P=P, e=e,
                incl=incl, strict=strict)


def chunk_fwd(q, k, v, g, beta, cu, C, h0=None, scale=1.0, return_states=False, round_wk=None):
    """round_wk: optional rounding applied to each chunk's Wk before it
    multiplies the state (to model an implementation that stores Wk in a
    narrower format)."""
    T, Hk, dk = q.shape
    _, Hv, dv = v.shape
    G = Hv // Hk
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    ht = np.zeros((N, Hv, dk, dv))
    states = {}
    for h in range(Hv):
        j = h // G
        cur = {n: (np.array(h0[n, h], dtype=np.float64) if h0 is not None else np.zeros((dk, dv)))
               for n in range(N)}
        for n, t0, L in _chunks(cu, C):
            sl = slice(t0, t0 + L)
            Q, K, V = q[sl, j].astype(np.float64), k[sl, j].astype(np.float64), v[sl, h].astype(np.float64)
            loc = _local(Q, K, V, g[sl, h].astype(np.float64), beta[sl, h].astype(np.float64))
            H = cur[n]
            states[(h, t0)] = H
            Wk = loc["Wk"] if round_wk is None else round_wk(loc["Wk"])
            W = loc["U"] - Wk @ H
            o[sl, h] = scale * (loc["Gam"][:, None] * (Q @ H) + loc["P"] @ W)
            cur[n] = loc["Gam"][-1] * H + K.T @ (loc["e"][:, None] * W)
        for n in range(N):
            ht[n, h] = cur[n]
    if return_states:
        return o, ht, states
    return o, ht


def chunk_bwd(q, k, v, g, beta, cu, C, d_o, h0=None, dht=None, scale=1.0, round_wk=None):
    """Gradients of <d_o, o> + <dht, ht> through the chunked form.  round_wk
    (as in chunk_fwd) models a narrower Wk in the forward state chain only:
    the entering states and W the gradients are formed from."""
    T, Hk, dk = q.shape
    _, Hv, dv = v.shape
    G = Hv // Hk
    N = len(cu) - 1
    _, _, states = chunk_fwd(q, k, v, g, beta, cu, C, h0=h0, scale=scale, return_states=True, round_wk=round_wk)
    dq = np.zeros((T, Hk, dk)); dk_ = np.zeros((T, Hk, dk)); dv_ = np.zeros((T, Hv, dv))
    dg = np.zeros((T, Hv)); db = np.zeros((T, Hv)); dh0 = np.zeros((N, Hv, dk, dv))
    chunks = list(_chunks(cu, C))
    for h in range(Hv):
        j = h // G
        dcur = {n: (np.array(dht[n, h], dtype=np.float64) if dht is not None else np.zeros((dk, dv)))
                for n in range(N)}
        for n, t0, L in reversed(chunks):
            sl = slice(t0, t0 + L)
            Q, K, V = q[sl, j].astype(np.float64), k[sl, j].astype(np.float64), v[sl, h].astype(np.float64)
            bb = beta[sl, h].astype(np.float64)
            loc = _local(Q, K, V, g[sl, h].astype(np.float64), bb)
            Gam, D, Tm, P, e, A = loc["Gam"], loc["D"], loc["Tm"], loc["P"], loc["e"], loc["A"]
            H = states[(h, t0)]
            W = loc["U"] - (loc["Wk"] if round_wk is None else round_wk(loc["Wk"])) @ H
            dOs = scale * d_o[sl, h].astype(np.float64)
            dHn = dcur[n]
            # state pass, reversed
            dW = P.T @ dOs + (e[:, None] * K) @ dHn
            dcur[n] = Gam[-1] * dHn + (Gam[:, None] * Q).T @ dOs - loc["Wk"].T @ dW
            # contractions over d_v
            dWk = -dW @ H.T
            dQ = Gam[:, None] * (dOs @ H.T)
            dgam = np.sum(dQ * Q, axis=1)
            dgam[-1] += Gam[-1] * np.sum(dHn * H)
            dKhn = e[:, None] * (W @ dHn.T)
            dK = dKhn.copy()
            tk = np.sum(dKhn * K, axis=1)
            dgam -= tk
            dgam[-1] += tk.sum()
            dP = np.where(loc["incl"], dOs @ W.T, 0.0)
            dS = dP * D
            dQ += dS @ K
            dK += dS.T @ Q
            PdP = dP * P
            dgam += PdP.sum(1) - PdP.sum(0)
            # through the WY representation
            Xu = bb[:, None] * V
            Xw = (bb * Gam)[:, None] * K
            dT = dW @ Xu.T + dWk @ Xw.T
            dXu = Tm.T @ dW
            dXw = Tm.T @ dWk
            dV = bb[:, None] * dXu
            dbeta = np.sum(dXu * V, 1) + Gam * np.sum(dXw * K, 1)
            dK += (bb * Gam)[:, None] * dXw
            dgam += np.sum(dXw * Xw, 1)
            dA = np.where(loc["strict"], -(Tm.T @ dT @ Tm.T), 0.0)
            dbeta += np.sum(dA * D * loc["Skk"], 1)
            At = dA * bb[:, None] * D
            dK += At @ K + At.T @ K
            AdA = dA * A
            dgam += AdA.sum(1) - AdA.sum(0)
            dq[sl, j] += dQ
            dk_[sl, j] += dK
            dv_[sl, h] = dV
            db[sl, h] = dbeta
            dg[sl, h] = np.cumsum(dgam[::-1])[::-1]
        for n in range(N):
            dh0[n, h] = dcur[n]
    return dict(dq=dq, dk=dk_, dv=dv_, dg=dg, dbeta=db, dh0=dh0)

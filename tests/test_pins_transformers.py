"""Pins of the oracle against an independent implementation of the same layer:
the plain-PyTorch fallbacks that transformers ships for Qwen3.5's GatedDeltaNet
(the "naive fallback" the hybrid-decoder page names next to the optional FLA
kernels: "[Qwen3.5 MoE] Add hybrid decoder model", Summary).

These are third-party code, written independently of this repository, so
agreement with them pins the readings the pages leave open:
  R3  the decay multiplies the whole S_{t-1}(I - b k k^T) (the prediction uses
      the decayed state)          -> torch_recurrent_gated_delta_rule
  R2  the state is stored [d_k][d_v] (H = S^T)   -> the same, final state
  R5  L2 norm x / sqrt(|x|^2 + 1e-6)              -> l2norm
  R6  causal depthwise conv, last tap on the current token, SiLU after
                                                  -> causal_conv1d_fn
  R11 RMSNormGated: normalise, multiply by w, then by silu(z)
                                                  -> Qwen3_5RMSNormGated
  and the chunked form against torch_chunk_gated_delta_rule.

The fallbacks compute in float32 and fold the query scale d_k^-1/2 into q; the
oracle takes the scale as an argument (R4 reads the pages as scale = 1), so
these pins pass scale = d_k^-1/2.  The fallbacks have no GQA and no varlen
(one sequence per batch row), so the cases use Hk = Hv and one sequence.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

m = pytest.importorskip("transformers.models.qwen3_5.modeling_qwen3_5")

F32_REL = 2e-5   # float32 arithmetic over at most a few hundred terms


def _problem(seed, T, H, d, g_scale=1.0, h0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, d))
    g = -g_scale * rng.random((T, H))
    beta = rng.random((T, H))
    S0 = 0.3 * rng.standard_normal((1, H, d, d)) if h0 else None
    return q, k, v, g, beta, S0


def _rel(a, b):
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - b)) / np.sqrt(np.mean(b * b)))


@pytest.mark.parametrize("T,H,d,g_scale,h0", [(37, 2, 16, 1.0, True), (80, 3, 32, 0.05, True),
                                              (5, 1, 8, 0.0, False)])
def test_recurrence_matches_transformers_recurrent(T, H, d, g_scale, h0):
    q, k, v, g, beta, S0 = _problem(T + d, T, H, d, g_scale, h0)
    scale = d ** -0.5
    o, ht = oracle.recurrence(q, k, v, g, beta, np.array([0, T], np.int32), h0=S0, scale=scale)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))[None]
    ro, rs = m.torch_recurrent_gated_delta_rule(t(q), t(k), t(v), t(g), t(beta),
                                                None if S0 is None else torch.from_numpy(S0.astype(np.float32)),
                                                True)
    assert _rel(o, ro[0].double().numpy()) < F32_REL
    assert _rel(ht, rs.double().numpy()) < F32_REL


def test_decay_placement_distinguishes_readings():
    """The pin above can tell R3 from the other reading (decay applied after
    the delta-rule write): with that variant the transformers result is far
    off, so agreement is not an accident of small decays."""
    T, H, d = 20, 1, 8
    q, k, v, g, beta, S0 = _problem(3, T, H, d, 2.0, True)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))[None]
    ro, _ = m.torch_recurrent_gated_delta_rule(t(q), t(k), t(v), t(g), t(beta),
                                               torch.from_numpy(S0.astype(np.float32)), True)
    # the other reading, written out: predict with the undecayed state, then decay
    S = S0[0, 0].copy()
    out = np.empty((T, d))
    for i in range(T):
        p = S.T @ k[i, 0]
        S = S + np.outer(k[i, 0], beta[i, 0] * (v[i, 0] - p))
        S = np.exp(g[i, 0]) * S
        out[i] = d ** -0.5 * (S.T @ q[i, 0])
    assert _rel(out, ro[0, :, 0].double().numpy()) > 1e-2


@pytest.mark.parametrize("T,chunk", [(64, 16), (100, 64), (7, 4)])
def test_recurrence_matches_transformers_chunked(T, chunk):
    H, d = 2, 16
    q, k, v, g, beta, S0 = _problem(T, T, H, d, 0.3, True)
    scale = d ** -0.5
    o, ht = oracle.recurrence(q, k, v, g, beta, np.array([0, T], np.int32), h0=S0, scale=scale)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))[None]
    ro, rs = m.torch_chunk_gated_delta_rule(t(q), t(k), t(v), t(g), t(beta), chunk_size=chunk,
                                            initial_state=torch.from_numpy(S0.astype(np.float32)),
                                            output_final_state=True)
    assert _rel(o, ro[0].double().numpy()) < 1e-4
    assert _rel(ht, rs.double().numpy()) < 1e-4


def test_l2_and_conv_match_transformers():
    """Conv + SiLU (v channels, no L2) against causal_conv1d_fn, and the L2
    step of the q/k heads against l2norm applied to that conv output."""
    rng = np.random.default_rng(11)
    T, d, Hk, Hv = 29, 8, 2, 3
    Cch = 2 * Hk * d + Hv * d
    x = rng.standard_normal((T, Cch))
    w = 0.5 * rng.standard_normal((Cch, 4))
    y = oracle.conv1d(x, w, np.array([0, T], np.int32), 2 * Hk * d, d)
    xt = torch.from_numpy(x.astype(np.float32)).T[None]            # [1, Cch, T]
    ref = m.causal_conv1d_fn(xt, torch.from_numpy(w.astype(np.float32)), None, activation="silu")[0].T
    ref = ref.double().numpy()
    assert _rel(y[:, 2 * Hk * d:], ref[:, 2 * Hk * d:]) < F32_REL
    qk = torch.from_numpy(ref[:, :2 * Hk * d].reshape(T, 2 * Hk, d))
    ref_l2 = m.l2norm(qk, dim=-1, eps=1e-6).reshape(T, -1).numpy()
    assert _rel(y[:, :2 * Hk * d], ref_l2) < F32_REL


def test_norm_gate_matches_transformers():
    rng = np.random.default_rng(12)
    rows, d = 50, 32
    o = rng.standard_normal((rows, d)) * np.exp(rng.standard_normal((rows, 1)))
    z = rng.standard_normal((rows, d))
    w = 1 + 0.02 * rng.standard_normal(d)
    y = oracle.norm_gate(o, z, w)
    mod = m.Qwen3_5RMSNormGated(d, eps=1e-6)
    with torch.no_grad():
        mod.weight.copy_(torch.from_numpy(w))
    # the module computes in float32 internally (float64 in, float64 out)
    ref = mod(torch.from_numpy(o), torch.from_numpy(z)).detach().numpy()
    np.testing.assert_allclose(y, ref, rtol=F32_REL, atol=1e-9)
    # the flagged alternative (gate before the norm) does not match
    alt = oracle.norm_gate(o * (z / (1 + np.exp(-z))), np.full_like(z, 50.0), w)
    assert _rel(alt, ref) > 1e-2

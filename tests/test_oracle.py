"""Pins for the CPU oracle: each check ties it to something other than itself
(a library routine, a brute-force expansion, a closed form, an invariant,
finite differences, or an independent autograd transcription)."""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth
from chunk_model import chunk_bwd, chunk_fwd

torch.set_default_dtype(torch.float64)


def rnd_problem(seed, lengths, Hk=2, Hv=2, dk=8, dv=6, g_scale=0.5, h0=True, unit=True):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = synth.cu_from_lengths(lengths)
    q = rng.standard_normal((T, Hk, dk))
    k = rng.standard_normal((T, Hk, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, dv))
    g = -g_scale * rng.random((T, Hv))
    beta = rng.random((T, Hv))
    H0 = 0.3 * rng.standard_normal((len(lengths), Hv, dk, dv)) if h0 else None
    return q, k, v, g, beta, cu, H0


# ---------------------------------------------------------------- conv + L2
def torch_conv_silu(x, w, cu):
    """Depthwise causal conv via torch.nn.functional.conv1d, per sequence."""
    outs = []
    W = w.shape[1]
    for n in range(len(cu) - 1):
        xs = torch.from_numpy(x[cu[n]:cu[n + 1]]).T[None]            # [1, C, L]
        y = F.conv1d(xs, torch.from_numpy(w)[:, None, :], padding=W - 1, groups=w.shape[0])
        outs.append(F.silu(y[0, :, : cu[n + 1] - cu[n]]).T)
    return torch.cat(outs).numpy()


def test_conv_matches_torch_conv1d():
    rng = np.random.default_rng(1)
    lengths = [1, 2, 3, 4, 9, 17]
    cu = synth.cu_from_lengths(lengths)
    x = rng.standard_normal((sum(lengths), 40))
    w = 0.5 * rng.standard_normal((40, 4))
    y = oracle.conv1d(x, w, cu, n_qk_ch=0, d_k=8)
    ref = torch_conv_silu(x, w, cu)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_conv_l2_heads():
    rng = np.random.default_rng(2)
    lengths = [5, 11]
    cu = synth.cu_from_lengths(lengths)
    x = rng.standard_normal((16, 48))
    w = 0.5 * rng.standard_normal((48, 4))
    y = oracle.conv1d(x, w, cu, n_qk_ch=32, d_k=8)
    a = torch_conv_silu(x, w, cu)
    for h in range(4):
        blk = a[:, 8 * h: 8 * h + 8]
        ss = (blk ** 2).sum(1)
        got = y[:, 8 * h: 8 * h + 8]
        # squared norm of the normalised head is ss / (ss + eps), same direction
        np.testing.assert_allclose((got ** 2).sum(1), ss / (ss + 1e-6), rtol=1e-13)
        np.testing.assert_allclose(got * np.sqrt(ss + 1e-6)[:, None], blk, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(y[:, 32:], a[:, 32:], rtol=1e-13)


def test_conv_impulse_weights():
    rng = np.random.default_rng(3)
    lengths = [2, 6, 4]
    cu = synth.cu_from_lengths(lengths)
    x = rng.standard_normal((12, 5))
    silu = lambda t: t / (1 + np.exp(-t))
    w = np.zeros((5, 4)); w[:, 3] = 1.0      # tap 3 multiplies the current token
    np.testing.assert_allclose(oracle.conv1d(x, w, cu, 0, 1), silu(x), rtol=1e-15)
    w = np.zeros((5, 4)); w[:, 0] = 1.0      # tap 0 reaches back 3 tokens
    exp = np.zeros_like(x)
    for n in range(3):
        for t in range(cu[n] + 3, cu[n + 1]):
            exp[t] = silu(x[t - 3])
    np.testing.assert_allclose(oracle.conv1d(x, w, cu, 0, 1), exp, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- recurrence
def brute_force(q, k, v, g, beta, h0):
    """S_t = S_0 P_1..P_t + sum_s b_s v_s k_s^T P_{s+1}..P_t, P_r = e^{g_r}(I - b_r k_r k_r^T),
    built from explicit d_k x d_k matrices; one sequence, one head."""
    L, dk = k.shape
    dv = v.shape[1]
    P = [np.exp(g[r]) * (np.eye(dk) - beta[r] * np.outer(k[r], k[r])) for r in range(L)]
    S0 = h0.T if h0 is not None else np.zeros((dv, dk))
    outs = []
    for t in range(L):
        prod = np.eye(dk)
        for r in range(t + 1):
            prod = prod @ P[r]
        S = S0 @ prod
        for s in range(t + 1):
            tail = np.eye(dk)
            for r in range(s + 1, t + 1):
                tail = tail @ P[r]
            S = S + beta[s] * np.outer(v[s], k[s]) @ tail
        outs.append(S @ q[t])
    return np.array(outs), S.T


@pytest.mark.parametrize("G", [1, 2])
def test_recurrence_brute_force(G):
    q, k, v, g, beta, cu, H0 = rnd_problem(4, [7, 1, 12], Hk=2, Hv=2 * G, dk=5, dv=3, g_scale=1.0)
    o, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0, scale=1.0)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        for h in range(2 * G):
            ob, Sb = brute_force(q[sl, h // G], k[sl, h // G], v[sl, h], g[sl, h], beta[sl, h], H0[n, h])
            np.testing.assert_allclose(o[sl, h], ob, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(ht[n, h], Sb, rtol=1e-12, atol=1e-12)


def test_scale_multiplies_output():
    q, k, v, g, beta, cu, H0 = rnd_problem(5, [9])
    o1, h1 = oracle.recurrence(q, k, v, g, beta, cu, h0=H0, scale=1.0)
    o2, h2 = oracle.recurrence(q, k, v, g, beta, cu, h0=H0, scale=0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-15)
    np.testing.assert_array_equal(h1, h2)


def test_closed_form_beta_zero():
    q, k, v, g, beta, cu, H0 = rnd_problem(6, [10], g_scale=0.7)
    beta[:] = 0
    o, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    csum = np.cumsum(g, axis=0)
    for h in range(2):
        exp_o = np.exp(csum[:, h])[:, None] * (q[:, h] @ H0[0, h])
        np.testing.assert_allclose(o[:, h], exp_o, rtol=1e-13)
        np.testing.assert_allclose(ht[0, h], np.exp(csum[-1, h]) * H0[0, h], rtol=1e-13)
    g[:] = 0
    o, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    np.testing.assert_array_equal(ht, H0)              # state stays exactly at h0
    for h in range(2):
        np.testing.assert_allclose(o[:, h], q[:, h] @ H0[0, h], rtol=1e-13, atol=1e-15)


def test_closed_form_single_token():
    q, k, v, g, beta, cu, _ = rnd_problem(7, [1], unit=True)
    g[:] = 0; beta[:] = 1
    o, _ = oracle.recurrence(q, k, v, g, beta, cu, h0=None)
    for h in range(2):
        np.testing.assert_allclose(o[0, h], v[0, h] * (k[0, h] @ q[0, h]), rtol=1e-14)
    # with an initial state: o = S0 (I - k k^T) q + v (k^T q)
    H0 = np.random.default_rng(8).standard_normal((1, 2, 8, 6))
    o, _ = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    for h in range(2):
        S0 = H0[0, h].T
        exp_o = S0 @ (q[0, h] - k[0, h] * (k[0, h] @ q[0, h])) + v[0, h] * (k[0, h] @ q[0, h])
        np.testing.assert_allclose(o[0, h], exp_o, rtol=1e-13)


def test_delta_rule_writes_value_exactly_for_unit_key():
    q, k, v, g, beta, cu, H0 = rnd_problem(9, [6], unit=True)
    g[:] = 0; beta[:] = 1
    q = k.copy()                       # read back at the key just written
    o, _ = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-13)


def test_orthonormal_keys_superpose():
    rng = np.random.default_rng(10)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :n].T[:, None, :]
    v = rng.standard_normal((n, 1, dv))
    q = rng.standard_normal((n, 1, dk))
    g = np.zeros((n, 1)); beta = np.ones((n, 1))
    _, ht = oracle.recurrence(q, k, v, g, beta, synth.cu_from_lengths([n]))
    np.testing.assert_allclose(ht[0, 0], k[:, 0].T @ v[:, 0], rtol=1e-13, atol=1e-14)


def test_full_decay_is_memoryless():
    q, k, v, g, beta, cu, H0 = rnd_problem(11, [8])
    g[:] = -1e4                        # e^g underflows to exactly 0
    o, _ = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    exp_o = beta[:, :, None] * v * np.einsum("thi,thi->th", k, q)[:, :, None]
    np.testing.assert_allclose(o, exp_o, rtol=1e-14, atol=1e-15)


def test_one_step_is_lms_gradient_step():
    # g = 0: S_t = S_{t-1} - b grad_S 1/2 |S k - v|^2  (Widrow-Hoff)
    q, k, v, g, beta, cu, H0 = rnd_problem(12, [1])
    g[:] = 0
    _, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    for h in range(2):
        S = H0[0, h].T
        grad = np.outer(S @ k[0, h] - v[0, h], k[0, h])
        np.testing.assert_allclose(ht[0, h].T, S - beta[0, h] * grad, rtol=1e-14, atol=1e-15)


def test_linearity_in_v_and_h0():
    q, k, v, g, beta, cu, H0 = rnd_problem(13, [11, 4])
    _, _, v2, _, _, _, H02 = rnd_problem(14, [11, 4])
    o1, h1 = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    o2, h2 = oracle.recurrence(q, k, v2, g, beta, cu, h0=H02)
    o3, h3 = oracle.recurrence(q, k, 2.5 * v - v2, g, beta, cu, h0=2.5 * H0 - H02)
    np.testing.assert_allclose(o3, 2.5 * o1 - o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h3, 2.5 * h1 - h2, rtol=1e-11, atol=1e-12)


def test_segment_split_and_packing_bit_exact():
    q, k, v, g, beta, cu, H0 = rnd_problem(15, [13, 7, 20], Hk=1, Hv=2)
    o, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    # each sequence alone
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        on, hn = oracle.recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl],
                                   synth.cu_from_lengths([cu[n + 1] - cu[n]]), h0=H0[n:n + 1])
        np.testing.assert_array_equal(on, o[sl])
        np.testing.assert_array_equal(hn[0], ht[n])
    # sequence 2 split at 6 and 15, carrying the state across calls
    a, b = int(cu[2]), int(cu[3])
    state = H0[2:3]
    parts = []
    for s, e in [(a, a + 6), (a + 6, a + 15), (a + 15, b)]:
        op, state = oracle.recurrence(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e],
                                      synth.cu_from_lengths([e - s]), h0=state)
        parts.append(op)
    np.testing.assert_array_equal(np.concatenate(parts), o[a:b])
    np.testing.assert_array_equal(state[0], ht[2])


def test_zero_length_sequence_passes_state_through():
    q, k, v, g, beta, _, H0 = rnd_problem(16, [3, 0, 2])
    cu = synth.cu_from_lengths([3, 0, 2])
    _, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0)
    np.testing.assert_array_equal(ht[1], H0[1])


def test_empty_row_layer():
    """T = 0: states pass through (ht = h0), their gradient is dht (here 0
    when none is given), and the weight gradients are zero sums."""
    cfg = synth.config("varlen").replace(lengths=(0, 0), varlen_rule=None, h_qk=1, h_v=2, d_k=16, d_v=16,
                                         chunk=16, bwd=True)
    inp = synth.make_inputs(cfg)
    fwd = oracle.layer_fwd(cfg, inp)
    np.testing.assert_array_equal(fwd["ht"], inp["h0"])
    dht = np.random.default_rng(5).standard_normal(inp["h0"].shape)
    b = oracle.layer_bwd(cfg, inp, fwd, inp["dy"], dht=dht)
    np.testing.assert_array_equal(b["dh0"], dht)
    assert b["dx"].shape == (0, inp["x"].shape[1])
    assert not np.any(b["dw_conv"]) and not np.any(b["dw_norm"])


@pytest.mark.parametrize("C", [1, 2, 4, 16, 64, 100])
def test_chunk_size_invariance(C):
    q, k, v, g, beta, cu, H0 = rnd_problem(17, [70, 1, 33, 64], Hk=2, Hv=4, dk=8, dv=6, g_scale=0.3)
    o, ht = oracle.recurrence(q, k, v, g, beta, cu, h0=H0, scale=0.7)
    oc, htc = chunk_fwd(q, k, v, g, beta, cu, C, h0=H0, scale=0.7)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(htc, ht, rtol=1e-10, atol=1e-12)


def test_chunk_inverse_is_triangular_solve():
    from scipy.linalg import solve_triangular
    rng = np.random.default_rng(18)
    A = np.tril(rng.standard_normal((16, 16)) * 0.3, -1)
    Tm = np.eye(16)
    for r in range(16):                 # forward substitution, row by row
        Tm[r] = np.eye(16)[r] - A[r, :r] @ Tm[:r]
    np.testing.assert_allclose(Tm, solve_triangular(np.eye(16) + A, np.eye(16), lower=True), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [1, 4, 16])
def test_chunk_backward_identities(C):
    q, k, v, g, beta, cu, H0 = rnd_problem(19, [37, 5, 16], Hk=2, Hv=4, dk=8, dv=6, g_scale=0.3)
    rng = np.random.default_rng(20)
    d_o = rng.standard_normal(v.shape)
    dht = rng.standard_normal(H0.shape)
    ref = oracle.recurrence_bwd(q, k, v, g, beta, cu, d_o, h0=H0, dht=dht, scale=0.7)
    got = chunk_bwd(q, k, v, g, beta, cu, C, d_o, h0=H0, dht=dht, scale=0.7)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-9, atol=1e-10, err_msg=key)


# ---------------------------------------------------------------- norm gate
def test_norm_gate_matches_torch_rms_norm():
    rng = np.random.default_rng(21)
    o = rng.standard_normal((7, 3, 16)); z = rng.standard_normal((7, 3, 16))
    w = 1 + 0.02 * rng.standard_normal(16)
    y = oracle.norm_gate(o, z, w, eps=1e-6)
    ref = F.rms_norm(torch.from_numpy(o), [16], eps=1e-6) * torch.from_numpy(w) * F.silu(torch.from_numpy(z))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)
    # exact scale invariance when eps scales with the square of the input
    y2 = oracle.norm_gate(1e3 * o, z, w, eps=1e-6 * 1e6)
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- backward
def torch_layer(x, wc, g, beta, z, wn, h0, cu, Hk, Hv, dk, dv, scale, eps=1e-6):
    """Independent PyTorch transcription of the layer (conv via F.conv1d,
    recurrence in S orientation), used only through autograd."""
    ys = []
    W = wc.shape[1]
    for n in range(len(cu) - 1):
        xs = x[cu[n]:cu[n + 1]].T[None]
        ys.append(F.silu(F.conv1d(xs, wc[:, None, :], padding=W - 1, groups=wc.shape[0])[0, :, : cu[n + 1] - cu[n]]).T)
    y = torch.cat(ys)
    T = y.shape[0]
    qk = y[:, : 2 * Hk * dk].reshape(T, 2 * Hk, dk)
    qk = qk / torch.sqrt((qk * qk).sum(-1, keepdim=True) + eps)
    q, k = qk[:, :Hk], qk[:, Hk:]
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    G = Hv // Hk
    outs = []
    for n in range(len(cu) - 1):
        o_seq = []
        for h in range(Hv):
            S = h0[n, h].T if h0 is not None else torch.zeros(dv, dk)
            col = []
            for t in range(cu[n], cu[n + 1]):
                kt, qt, vt = k[t, h // G], q[t, h // G], v[t, h]
                S = torch.exp(g[t, h]) * (S - beta[t, h] * torch.outer(S @ kt, kt)) + beta[t, h] * torch.outer(vt, kt)
                col.append(scale * (S @ qt))
            o_seq.append(torch.stack(col))
        outs.append(torch.stack(o_seq, 1))
    o = torch.cat(outs)
    r = torch.rsqrt((o * o).mean(-1, keepdim=True) + 1e-6)
    return o * r * wn * F.silu(z)


def test_layer_backward_matches_autograd_transcription():
    cfg = synth.config("tiny").replace(norm=True, h0=True, bwd=True, lengths=(9, 14), h_qk=1, h_v=2, d_k=4, d_v=4)
    inp = synth.make_inputs(cfg)
    fwd = oracle.layer_fwd(cfg, inp, scale=0.8)
    got = oracle.layer_bwd(cfg, inp, fwd, inp["dy"], scale=0.8)
    tx = {key: torch.tensor(inp[key], dtype=torch.float64, requires_grad=True)
          for key in ("x", "w_conv", "g", "beta", "z", "w_norm", "h0")}
    y = torch_layer(tx["x"], tx["w_conv"], tx["g"], tx["beta"], tx["z"], tx["w_norm"], tx["h0"],
                    [int(c) for c in inp["cu"]], 1, 2, 4, 4, 0.8)
    np.testing.assert_allclose(y.detach().numpy(), fwd["y"], rtol=1e-12, atol=1e-14)
    (y * torch.from_numpy(inp["dy"].astype(np.float64))).sum().backward()
    pairs = dict(x="dx", w_conv="dw_conv", g="dg", beta="dbeta", z="dz", w_norm="dw_norm", h0="dh0")
    for key, gk in pairs.items():
        np.testing.assert_allclose(got[gk], tx[key].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=gk)


def _loss(cfg, inp, dy):
    f = oracle.layer_fwd(cfg, inp)
    return float(np.sum(f["y"] * dy))


def _fd(cfg, inp, key, d, h):
    """Central difference of the loss along d, Richardson-extrapolated (O(h^4))."""
    def cd(step):
        plus = dict(inp); plus[key] = inp[key] + step * d
        minus = dict(inp); minus[key] = inp[key] - step * d
        return (_loss(cfg, plus, inp["dy"]) - _loss(cfg, minus, inp["dy"])) / (2 * step)
    return (4 * cd(h / 2) - cd(h)) / 3


def test_layer_backward_finite_differences():
    cfg = synth.config("tiny").replace(norm=True, h0=True, bwd=True)
    inp = synth.make_inputs(cfg)
    inp = {k: (v.astype(np.float64) if v.dtype == np.float32 else v) for k, v in inp.items()}
    fwd = oracle.layer_fwd(cfg, inp)
    got = oracle.layer_bwd(cfg, inp, fwd, inp["dy"])
    rng = np.random.default_rng(22)
    h = 1e-4
    pairs = dict(x="dx", w_conv="dw_conv", g="dg", beta="dbeta", z="dz", w_norm="dw_norm", h0="dh0")
    for key, gk in pairs.items():
        gscale = float(np.sqrt(np.sum(got[gk] ** 2)))
        for trial in range(3):
            d = rng.standard_normal(inp[key].shape)
            fd = _fd(cfg, inp, key, d, h)
            an = float(np.sum(got[gk] * d))
            assert abs(fd - an) <= 1e-7 * max(abs(an), gscale), (gk, fd, an)
        flat = inp[key].reshape(-1)
        for idx in rng.choice(flat.size, size=min(5, flat.size), replace=False):
            d = np.zeros(flat.size); d[idx] = 1
            fd = _fd(cfg, inp, key, d.reshape(inp[key].shape), h)
            an = float(got[gk].reshape(-1)[idx])
            assert abs(fd - an) <= 1e-7 * max(abs(an), gscale), (gk, idx, fd, an)


# ---------------------------------------------------------------- precision
def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def test_fp32_oracle_meets_fp32_tolerance():
    cfg = synth.config("tiny")
    inp = synth.make_inputs(cfg)
    f64 = oracle.layer_fwd(cfg, inp, bits=64)
    f32 = oracle.layer_fwd(cfg, inp, bits=32)
    for key in ("o", "ht"):
        assert np.max(np.abs(f32[key] - f64[key])) <= 1e-4 * rms(f64[key]), key


def test_chunk_table_rules():
    cu = synth.cu_from_lengths([5, 0, 16, 17, 1])
    tab, first = oracle.chunk_table(cu, 16)
    assert tab.tolist() == [[0, 0, 5], [2, 5, 16], [3, 21, 16], [3, 37, 1], [4, 38, 1]]
    assert first.tolist() == [0, 1, 1, 2, 4, 5]


# ---------------------------------------------------------------- gates
def test_gates_closed_forms_and_library_softplus():
    """softplus against numpy's logaddexp(0, x) and sigmoid against scipy's
    expit (library routines) over the whole float range the gates meet; g(A_log = 0, a + dt_bias = 0) = -ln 2;
    beta(0) = 1/2 and beta(b) + beta(-b) = 1; g < 0 wherever softplus > 0."""
    x = np.concatenate([np.linspace(-60, 60, 4001), [-700.0, -300.0, 300.0, 700.0]])
    T = x.size
    a = x[:, None]
    b = x[:, None]
    g, beta = oracle.gates(a, b, np.zeros(1), np.zeros(1))
    np.testing.assert_allclose(-g[:, 0], np.logaddexp(0.0, x), rtol=1e-14, atol=0)
    np.testing.assert_allclose(beta[:, 0], scipy.special.expit(x), rtol=1e-14, atol=0)
    gz, bz = oracle.gates(np.zeros((1, 3)), np.zeros((1, 3)), np.zeros(3), np.zeros(3))
    np.testing.assert_allclose(gz, -np.log(2.0), rtol=1e-15)
    np.testing.assert_array_equal(bz, 0.5)
    _, bn = oracle.gates(a, -b, np.zeros(1), np.zeros(1))
    np.testing.assert_allclose(beta + bn, 1.0, rtol=1e-15)
    assert np.all(g[np.abs(x) < 700] < 0)
    # the decay rate scales exactly by exp(A_log), and dt_bias shifts a
    rng = np.random.default_rng(3)
    a2 = rng.standard_normal((17, 4)); A = rng.uniform(0, 2, 4); dt = rng.standard_normal(4)
    g1, _ = oracle.gates(a2, a2, A, dt)
    g0, _ = oracle.gates(a2 + dt, a2, np.zeros(4), np.zeros(4))
    np.testing.assert_allclose(g1, g0 * np.exp(A), rtol=1e-14)
    assert T == g.shape[0]


def test_gates_backward_finite_differences():
    """Every gradient of the gates against central differences of
    L = sum(wg * g + wb * beta)."""
    rng = np.random.default_rng(5)
    T, Hv = 7, 3
    a = rng.standard_normal((T, Hv)); b = rng.standard_normal((T, Hv))
    A = rng.uniform(0, 2, Hv); dt = rng.standard_normal(Hv)
    wg = rng.standard_normal((T, Hv)); wb = rng.standard_normal((T, Hv))
    r = oracle.gates_bwd(a, b, A, dt, wg, wb)

    def loss(a_, b_, A_, dt_):
        g, beta = oracle.gates(a_, b_, A_, dt_)
        return float(np.sum(wg * g) + np.sum(wb * beta))

    eps = 1e-6
    for name, arr, key in (("a", a, "da"), ("b", b, "db"), ("A_log", A, "dA_log"), ("dt_bias", dt, "ddt_bias")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = {"a": a.copy(), "b": b.copy(), "A_log": A.copy(), "dt_bias": dt.copy()}
            args[name][idx] += eps
            lp = loss(args["a"], args["b"], args["A_log"], args["dt_bias"])
            args[name][idx] -= 2 * eps
            lm = loss(args["a"], args["b"], args["A_log"], args["dt_bias"])
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(r[key], fd, rtol=1e-7, atol=1e-9, err_msg=name)

"""GPU parity: every C-ABI call and the whole layer against the CPU oracle,
element by element, on seeded inputs spanning several chunks and ragged
tails.  Tolerance: max|gpu - oracle| <= tol * RMS(oracle), tol = 1e-4 (fp32
storage) or 2e-2 (bf16 storage, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_conv1d_amd as gdn
import oracle
import synth
from gpu_util import (TOL, TOL_F32_OUT, assert_close, f32, host, layer_gpu, qkv_inputs, shape_of, small_cfg, to_dev)

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# ----------------------------------------------------------------------------- A0 chunk index
@pytest.mark.parametrize("lengths,chunk", [((64,), 16), ((5, 0, 16, 17, 1), 16), ((2048,) * 4, 64),
                                           ((0, 0, 3), 32), ((1,) * 300, 64), ((4097, 0, 63, 65, 64), 64)])
def test_chunk_index_bit_exact(lengths, chunk):
    _print_case("chunk_index", lengths=len(lengths), chunk=chunk)
    cfg = small_cfg(lengths=lengths, chunk=chunk)
    s = shape_of(cfg)
    cu = synth.cu_from_lengths(lengths)
    table, first = gdn.chunk_index(torch.from_numpy(cu).cuda(), s)
    torch.cuda.synchronize()
    ref_tab, ref_first = oracle.chunk_table(cu, chunk)
    tab = table.cpu().numpy()
    n = len(ref_tab)
    np.testing.assert_array_equal(first.cpu().numpy(), ref_first)
    np.testing.assert_array_equal(tab[:n, :3], ref_tab)
    assert np.all(tab[n:, 0] == -1)


# ----------------------------------------------------------------------------- A1 conv
@pytest.mark.parametrize("dtype,d,lengths", [("f32", 16, (64,)), ("f32", 32, (1, 2, 3, 70, 9)),
                                             ("bf16", 128, (1, 3, 64, 130, 2, 77)), ("bf16", 64, (200,)),
                                             ("bf16", 16, (5, 0, 40))])
@pytest.mark.parametrize("width", [4, 3])
def test_conv1d_fwd_bwd(dtype, d, lengths, width):
    _print_case("conv1d", dtype=dtype, d=d, lengths=lengths, width=width)
    cfg = small_cfg(dtype=dtype, lengths=lengths, d=d).replace(width=width)
    inp = synth.make_inputs(cfg)
    s = shape_of(cfg)
    nqk = 2 * cfg.h_qk * cfg.d_k
    x, w, cu = to_dev(inp["x"], dtype), to_dev(inp["w_conv"], dtype), torch.from_numpy(inp["cu"]).cuda()
    y = gdn.conv1d(x, w, cu, s)
    ref = oracle.conv1d(inp["x"], inp["w_conv"], inp["cu"], nqk, cfg.d_k)
    assert_close(host(y), ref, TOL[dtype], "y")
    rng = np.random.default_rng(3)
    dy = rng.standard_normal(inp["x"].shape).astype(np.float32)
    if dtype == "bf16":
        dy = synth.round_bf16(dy)
    dx, dw = gdn.conv1d_bwd(to_dev(dy, dtype), x, w, cu, s)
    rdx, rdw = oracle.conv1d_bwd(inp["x"], inp["w_conv"], inp["cu"], nqk, cfg.d_k, dy)
    assert_close(host(dx), rdx, TOL[dtype], "dx")
    assert_close(host(dw), rdw, TOL[dtype], "dw_conv")


# ----------------------------------------------------------------------------- A6 norm gate
@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 128), ("bf16", 32)])
def test_norm_gate_fwd_bwd(dtype, d):
    _print_case("norm_gate", dtype=dtype, d=d)
    cfg = small_cfg(dtype=dtype, d=d, lengths=(37, 100))
    inp = synth.make_inputs(cfg)
    s = shape_of(cfg)
    rng = np.random.default_rng(5)
    o = rng.standard_normal((cfg.T, cfg.h_v, d)).astype(np.float32)
    dy = rng.standard_normal((cfg.T, cfg.h_v, d)).astype(np.float32)
    if dtype == "bf16":
        o, dy = synth.round_bf16(o), synth.round_bf16(dy)
    z, wn = inp["z"], inp["w_norm"]
    y = gdn.norm_gate(to_dev(o, dtype), to_dev(z, dtype), to_dev(wn, dtype), s)
    assert_close(host(y), oracle.norm_gate(o, z, wn), TOL[dtype], "y")
    d_o, dz, dw = gdn.norm_gate_bwd(to_dev(dy, dtype), to_dev(o, dtype), to_dev(z, dtype), to_dev(wn, dtype), s)
    rdo, rdz, rdw = oracle.norm_gate_bwd(o, z, wn, dy)
    assert_close(host(d_o), rdo, TOL[dtype], "d_o")
    assert_close(host(dz), rdz, TOL[dtype], "dz")
    assert_close(host(dw), rdw, TOL[dtype], "dw_norm")


# ----------------------------------------------------------------------------- gates
@pytest.mark.parametrize("T,Hk,Hv,workload", [(0, 1, 4, None), (1, 1, 3, None), (333, 2, 6, None), (700, 1, 1, None),
                                               (65536, 16, 32, "train")])
def test_gates_fwd_bwd(T, Hk, Hv, workload):
    """gdn_gates / gdn_gates_bwd against the oracle's fp64 gates on the same
    float32 inputs; the last case is the training workload's own gate draw."""
    _print_case("gates", T=T, Hv=Hv, workload=workload)
    if workload:
        cfg = synth.config(workload)
        raw = synth.make_inputs(cfg, keep_raw=True)
        a, b, A_log, dt = raw["a"], raw["b"], raw["A_log"], raw["dt_bias"]
    else:
        rng = np.random.default_rng(T + Hv)
        a, b = 3 * rng.standard_normal((T, Hv)), 3 * rng.standard_normal((T, Hv))
        A_log, dt = rng.uniform(-1, 2, Hv), rng.standard_normal(Hv)
    a, b, A_log, dt = (np.asarray(x, dtype=np.float32) for x in (a, b, A_log, dt))
    rng = np.random.default_rng(7)
    dg = rng.standard_normal((T, Hv)).astype(np.float32)
    dbeta = rng.standard_normal((T, Hv)).astype(np.float32)
    s = gdn.Shape(1, T, Hk, Hv, 16, 16, 16, gdn.F32, 1.0)
    g, beta = gdn.gates(f32(a), f32(b), f32(A_log), f32(dt), s)
    r = gdn.gates_bwd(f32(a), f32(b), f32(A_log), f32(dt), f32(dg), f32(dbeta), s)
    rg, rbeta = oracle.gates(a, b, A_log, dt)
    ref = oracle.gates_bwd(a, b, A_log, dt, dg, dbeta)
    if T > 0:
        # elementwise results: float32 arithmetic of well-conditioned functions
        for got, want, name in ((g, rg, "g"), (beta, rbeta, "beta"), (r["da"], ref["da"], "da"),
                                (r["db"], ref["db"], "db")):
            got = host(got)
            assert np.all(np.abs(got - want) <= 1e-5 * np.abs(want) + 1e-30), name
            assert_close(got, want, 1e-4, name)
        assert_close(host(r["dA_log"]), ref["dA_log"], 1e-4, "dA_log")
        assert_close(host(r["ddt_bias"]), ref["ddt_bias"], 1e-4, "ddt_bias")
    else:
        assert not host(r["dA_log"]).any() and not host(r["ddt_bias"]).any()


# ----------------------------------------------------------------------------- A3-A5, A7 chunk
CHUNK_CASES = [
    ("f32", 16, 16, 2, 2, (64,)),
    ("f32", 16, 16, 1, 2, (40, 1, 23)),
    ("f32", 32, 32, 2, 4, (70, 1, 33, 64, 5)),
    ("f32", 64, 32, 1, 2, (130, 7)),
    ("bf16", 16, 16, 2, 2, (40, 9)),
    ("bf16", 128, 64, 2, 4, (200, 1, 64, 63, 65)),       # 20 (sequence, v-head) chains: 16-column state tiles
    ("bf16", 128, 64, 8, 16, (100, 64, 1, 65, 20)),      # 80 chains: half-state workgroups
    ("bf16", 128, 64, 16, 32, (70, 64, 1, 65, 0, 130, 3, 40)),  # 256 chains: whole-state pass
    ("bf16", 128, 32, 1, 2, (100, 33)),
    ("bf16", 64, 16, 2, 2, (50, 17)),
    ("bf16", 32, 64, 1, 1, (129,)),
]


@pytest.mark.parametrize("dtype,d,chunk,Hk,Hv,lengths", CHUNK_CASES)
def test_chunk_fwd_bwd(dtype, d, chunk, Hk, Hv, lengths):
    _print_case("chunk", dtype=dtype, d=d, chunk=chunk, Hk=Hk, Hv=Hv, lengths=lengths)
    cfg = small_cfg(dtype=dtype, d=d, chunk=chunk, Hk=Hk, Hv=Hv, lengths=lengths)
    inp = synth.make_inputs(cfg)
    q, k, v = qkv_inputs(cfg)
    s = shape_of(cfg, scale=0.75)
    cu = torch.from_numpy(inp["cu"]).cuda()
    T = cfg.T
    qd, kd, vd = to_dev(q.reshape(T, -1), dtype), to_dev(k.reshape(T, -1), dtype), to_dev(v.reshape(T, -1), dtype)
    g, beta, h0 = f32(inp["g"]), f32(inp["beta"]), f32(inp["h0"])
    o, ht = gdn.chunk_fwd(qd, kd, vd, g, beta, cu, s, h0=h0)
    ro, rht = oracle.recurrence(q, k, v, inp["g"], inp["beta"], inp["cu"], h0=inp["h0"], scale=0.75)
    tol = TOL[dtype]
    assert_close(host(o), ro, tol, "o")
    assert_close(host(ht), rht, TOL_F32_OUT[dtype], "ht")
    rng = np.random.default_rng(9)
    d_o = rng.standard_normal(ro.shape).astype(np.float32)
    dht = rng.standard_normal(rht.shape).astype(np.float32)
    if dtype == "bf16":
        d_o = synth.round_bf16(d_o)
    r = gdn.chunk_bwd(qd, kd, vd, g, beta, cu, s, to_dev(d_o, dtype), h0=h0, dht=f32(dht))
    ref = oracle.recurrence_bwd(q, k, v, inp["g"], inp["beta"], inp["cu"], d_o, h0=inp["h0"], dht=dht, scale=0.75)
    assert_close(host(r["dq"]).reshape(ref["dq"].shape), ref["dq"], tol, "dq")
    assert_close(host(r["dk"]).reshape(ref["dk"].shape), ref["dk"], tol, "dk")
    assert_close(host(r["dv"]).reshape(ref["dv"].shape), ref["dv"], tol, "dv")
    assert_close(host(r["dg"]), ref["dg"], TOL_F32_OUT[dtype], "dg")
    assert_close(host(r["dbeta"]), ref["dbeta"], TOL_F32_OUT[dtype], "dbeta")
    assert_close(host(r["dh0"]), ref["dh0"], TOL_F32_OUT[dtype], "dh0")


@pytest.mark.parametrize("dtype,d,chunk,Hk,Hv,lengths", CHUNK_CASES)
def test_chunk_saved_pair_bit_identical(dtype, d, chunk, Hk, Hv, lengths):
    """gdn_chunk_fwd_save + gdn_chunk_bwd_saved give the same bytes as
    gdn_chunk_fwd + gdn_chunk_bwd (which recomputes the forward's products)."""
    _print_case("chunk_saved", dtype=dtype, d=d, chunk=chunk, Hk=Hk, Hv=Hv, lengths=lengths)
    cfg = small_cfg(dtype=dtype, d=d, chunk=chunk, Hk=Hk, Hv=Hv, lengths=lengths)
    inp = synth.make_inputs(cfg)
    q, k, v = qkv_inputs(cfg)
    s = shape_of(cfg, scale=0.75)
    cu = torch.from_numpy(inp["cu"]).cuda()
    T = cfg.T
    qd, kd, vd = to_dev(q.reshape(T, -1), dtype), to_dev(k.reshape(T, -1), dtype), to_dev(v.reshape(T, -1), dtype)
    g, beta, h0 = f32(inp["g"]), f32(inp["beta"]), f32(inp["h0"])
    d_o = to_dev(np.random.default_rng(9).standard_normal((T, cfg.h_v, d)).astype(np.float32), dtype)
    dht = f32(np.random.default_rng(10).standard_normal((cfg.N, cfg.h_v, d, d)))
    o1, ht1 = gdn.chunk_fwd(qd, kd, vd, g, beta, cu, s, h0=h0)
    r1 = gdn.chunk_bwd(qd, kd, vd, g, beta, cu, s, d_o, h0=h0, dht=dht)
    ws = torch.empty(gdn.chunk_bwd_workspace(s), dtype=torch.uint8, device="cuda")
    o2, ht2 = gdn.chunk_fwd(qd, kd, vd, g, beta, cu, s, h0=h0, ws=ws, save=True)
    r2 = gdn.chunk_bwd(qd, kd, vd, g, beta, cu, s, d_o, h0=h0, dht=dht, ws=ws, saved=True)
    torch.cuda.synchronize()
    same = lambda x, y: torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x.contiguous().view(torch.uint8),
                                    y.view(torch.uint8) if y.dtype == torch.bfloat16 else y.contiguous().view(torch.uint8))
    assert same(o1, o2) and same(ht1, ht2)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert same(r1[key], r2[key]), key


@pytest.mark.parametrize("d", [64, 128])
def test_chunk_weak_decay_long_range(d):
    """A_log = -6: the state is carried across many chunks (long-range path);
    at d = 128 through the 16-column state tiles that read the plain K^T."""
    cfg = small_cfg(dtype="bf16", d=d, chunk=64, Hk=1, Hv=2, lengths=(1000, 300), weak=True)
    _print_case("weak_decay", d=d, lengths=cfg.lengths)
    inp = synth.make_inputs(cfg)
    q, k, v = qkv_inputs(cfg)
    s = shape_of(cfg)
    T = cfg.T
    o, ht = gdn.chunk_fwd(to_dev(q.reshape(T, -1), "bf16"), to_dev(k.reshape(T, -1), "bf16"),
                          to_dev(v.reshape(T, -1), "bf16"), f32(inp["g"]), f32(inp["beta"]),
                          torch.from_numpy(inp["cu"]).cuda(), s, h0=f32(inp["h0"]))
    ro, rht = oracle.recurrence(q, k, v, inp["g"], inp["beta"], inp["cu"], h0=inp["h0"])
    assert_close(host(o), ro, TOL["bf16"], "o")
    assert_close(host(ht), rht, TOL["bf16"], "ht")


# ----------------------------------------------------------------------------- whole layer
@pytest.mark.parametrize("norm,h0", [(False, False), (True, True)])
def test_layer_tiny_full(norm, h0):
    cfg = synth.config("tiny").replace(norm=norm, h0=h0, bwd=True)
    _print_case("layer_tiny", norm=norm, h0=h0)
    inp = synth.make_inputs(cfg)
    fwd, bwd = layer_gpu(cfg, inp)
    ref = oracle.layer_fwd(cfg, inp)
    tol = TOL["f32"]
    assert_close(host(fwd["o"]), ref["o"], tol, "o")
    assert_close(host(fwd["ht"]), ref["ht"], tol, "ht")
    if norm:
        assert_close(host(fwd["y"]), ref["y"], tol, "y")
    dy = inp["dy"]
    rb = oracle.layer_bwd(cfg, inp, ref, dy)
    for key in ("dx", "dw_conv", "dg", "dbeta") + (("dz", "dw_norm", "dh0") if norm else ()):
        assert_close(host(bwd[key]), rb[key], tol, key)


def test_layer_small_bf16_full():
    cfg = small_cfg(dtype="bf16", d=128, chunk=64, Hk=2, Hv=4, lengths=(300, 1, 64, 65, 130))
    _print_case("layer_small_bf16", lengths=cfg.lengths)
    inp = synth.make_inputs(cfg)
    fwd, bwd = layer_gpu(cfg, inp)
    ref = oracle.layer_fwd(cfg, inp, storage="bf16")
    rb = oracle.layer_bwd(cfg, inp, ref, inp["dy"], storage="bf16")
    tol = TOL["bf16"]
    assert_close(host(fwd["y"]), ref["y"], tol, "y")
    assert_close(host(fwd["ht"]), ref["ht"], tol, "ht")
    for key in ("dx", "dw_conv", "dg", "dbeta", "dz", "dw_norm", "dh0"):
        assert_close(host(bwd[key]), rb[key], tol, key)

"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (one packed row; q, k, v and dq, dk, dv as strided views of
the [T, Cch] conv tensors; the same grids and workspaces).

The oracle cannot recompute a 65536-token, 32-head layer in seconds, so the
tests check sampled outputs: every step of the layer is independent across
sequences and across q/k-head groups (with their v-heads), so the oracle runs
on a subset (oracle.subset) and the matching slices of the GPU result are
compared element by element.

Two kinds of check:
  * stage by stage (test_fullsize_stages): each C-ABI call runs at full size
    on inputs that hold the oracle's own values (its bf16-stored intermediates)
    at the sampled positions and seeded filler elsewhere; every output is held
    to the plain bar.
  * end to end (test_fullsize_layer): the composed layer, GPU stage feeding
    GPU stage, forward and backward.  Between calls both sides round
    intermediates to bf16, and a value within float32 precision of a rounding
    boundary can round differently on the two sides (a few hundred of ~10^7
    conv outputs here); the norm divides each row of o by that row's RMS,
    which sits up to ~10^4 times below the tensor's RMS, so such a flip
    upstream is amplified there (and squared through the norm's backward).
    Two checks: every GPU stage against the oracle step fed the GPU's own
    upstream result, at the plain bars (gpu_util.check_chain); and every
    output against the pure oracle chain, with the bar calibrated by the
    oracle's own float32 build through the same storage points
    (gpu_util.assert_calibrated).

Also here: run-to-run determinism (byte-identical outputs), packed versus
separately-run sequences (byte-identical per-sequence outputs and states),
and edge lengths (empty sequences, an empty row, single tokens).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_conv1d_amd as gdn
import oracle
import synth
from gpu_util import (TOL, TOL_F32_OUT, assert_calibrated as _calibrated, assert_close, channels, check_chain, f32,
                      host, layer_gpu, shape_of, to_dev)

pytestmark = pytest.mark.gpu

SAMPLES = [
    ("dense", [0, 3], [0, 15]),                  # 4 x 2048: first and last sequence, outer heads
    ("varlen", [0, 2, 9, 17, 19], [0, 9]),       # short, the longest, mid-size, the truncated last one
    ("long", [0], [5]),                          # one 65536-token sequence: the whole inter-chunk carry
    ("train", list(range(8)), [0, 15]),          # fwd + bwd, every sequence (conv weight grads complete)
]
_INPUTS = {}


def _inputs(name):
    if name not in _INPUTS:
        _INPUTS.clear()  # hold one full-size workload at a time
        cfg = synth.config(name)
        _INPUTS[name] = (cfg, synth.make_inputs(cfg))
    return _INPUTS[name]


def _case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("name,seqs,kheads", SAMPLES)
def test_fullsize_layer(name, seqs, kheads):
    """The composed layer, GPU stage feeding GPU stage: (a) each stage against
    the oracle step fed the GPU's own upstream result (check_chain, plain
    bars); (b) every output against the pure oracle chain, calibrated by the
    oracle's float32 build (forward: largest and RMS error; backward: RMS
    error, with the largest error reported: see assert_calibrated)."""
    cfg, inp = _inputs(name)
    _case("fullsize_layer", workload=name, T=cfg.T, N=cfg.N, seqs=seqs, kheads=kheads)
    fwd, bwd = layer_gpu(cfg, inp)
    sub_cfg, sub, toks, vheads = oracle.subset(cfg, inp, seqs, kheads)
    storage = "bf16" if cfg.dtype == "bf16" else None
    ch = channels(cfg, kheads)
    sq = np.asarray(seqs)
    check_chain(cfg, sub_cfg, sub, fwd, bwd, toks, vheads, ch, seqs, len(seqs) == cfg.N)
    ref = oracle.layer_fwd(sub_cfg, sub, storage=storage)
    r32 = oracle.layer_fwd(sub_cfg, sub, storage=storage, bits=32)
    tol, tol32 = TOL[cfg.dtype], TOL_F32_OUT[cfg.dtype]
    stored = cfg.dtype == "bf16"
    _calibrated(host(fwd["y_conv"])[toks][:, ch], ref["y_conv_exact"], r32["y_conv_exact"], tol, "y_conv", stored)
    _calibrated(host(fwd["o"])[toks][:, vheads], ref["o_exact"], r32["o_exact"], tol, "o", stored)
    _calibrated(host(fwd["ht"])[sq][:, vheads], ref["ht"], r32["ht"], tol32, "ht", False)
    if cfg.norm:
        _calibrated(host(fwd["y"])[toks][:, vheads], ref["y"], r32["y"], tol, "y", stored)
    if bwd is None:
        return
    rb = oracle.layer_bwd(sub_cfg, sub, ref, sub["dy"], storage=storage)
    rb32 = oracle.layer_bwd(sub_cfg, sub, r32, sub["dy"], storage=storage, bits=32)
    bw = dict(max_bar=False)
    _calibrated(host(bwd["dx"])[toks][:, ch], rb["dx"], rb32["dx"], tol, "dx", stored, **bw)
    _calibrated(host(bwd["dz"])[toks][:, vheads], rb["dz"], rb32["dz"], tol, "dz", stored, **bw)
    _calibrated(host(bwd["dg"])[toks][:, vheads], rb["dg"], rb32["dg"], tol32, "dg", False, **bw)
    _calibrated(host(bwd["dbeta"])[toks][:, vheads], rb["dbeta"], rb32["dbeta"], tol32, "dbeta", False, **bw)
    if "h0" in inp:
        _calibrated(host(bwd["dh0"])[sq][:, vheads], rb["dh0"], rb32["dh0"], tol32, "dh0", False, **bw)
    if len(seqs) == cfg.N:  # every sequence in the sample: the conv-weight gradient sums are complete
        _calibrated(host(bwd["dw_conv"])[ch], rb["dw_conv"], rb32["dw_conv"], tol32, "dw_conv", False, **bw)


def _filled(shape, dtype, rng, rows, cols, values, scale=1.0):
    """Full-size array of seeded filler holding `values` at [rows][:, cols]."""
    a = (scale * rng.standard_normal(shape)).astype(np.float32)
    a[np.ix_(rows, cols)] = values
    return synth.round_bf16(a) if dtype == "bf16" else a


@pytest.mark.parametrize("name,seqs,kheads", SAMPLES)
def test_fullsize_stages(name, seqs, kheads):
    """Every C-ABI call at full size against the oracle, each fed the oracle's
    own (bf16-stored) intermediates at the sampled positions."""
    cfg, inp = _inputs(name)
    _case("fullsize_stages", workload=name, T=cfg.T, N=cfg.N, seqs=seqs, kheads=kheads)
    sub_cfg, sub, toks, vheads = oracle.subset(cfg, inp, seqs, kheads)
    dt, tol = cfg.dtype, TOL[cfg.dtype]
    storage = "bf16" if dt == "bf16" else None
    ref = oracle.layer_fwd(sub_cfg, sub, storage=storage)
    rng = np.random.default_rng(1234)
    T, Hk, Hv, D = cfg.T, cfg.h_qk, cfg.h_v, cfg.d_k
    Cch = 2 * Hk * D + Hv * D
    nqk = Hk * D
    ch = channels(cfg, kheads)
    s = shape_of(cfg)
    cu = torch.from_numpy(inp["cu"]).cuda()

    # conv1d + SiLU + L2 on the workload's own x
    x, w = to_dev(inp["x"], dt), to_dev(inp["w_conv"], dt)
    y = gdn.conv1d(x, w, cu, s)
    assert_close(host(y)[toks][:, ch], ref["y_conv_exact"], tol, "conv y")
    del y

    # chunked recurrence on the oracle's conv output (q, k, v as strided views)
    yc = to_dev(_filled((T, Cch), dt, rng, toks, ch, ref["y_conv"]), dt)
    q, k, v = yc[:, :nqk], yc[:, nqk:2 * nqk], yc[:, 2 * nqk:]
    g, beta = f32(inp["g"]), f32(inp["beta"])
    h0 = f32(inp["h0"]) if "h0" in inp else None
    o, ht = gdn.chunk_fwd(q, k, v, g, beta, cu, s, h0=h0)
    assert_close(host(o)[toks][:, vheads], ref["o_exact"], tol, "chunk o")
    assert_close(host(ht)[np.asarray(seqs)][:, vheads], ref["ht"], TOL_F32_OUT[dt], "chunk ht")
    del o, ht

    # RMSNormGated on the oracle's o
    o_in = _filled((T, Hv, D), dt, rng, toks, vheads, ref["o"], scale=0.05)
    z, wn = to_dev(inp["z"], dt), to_dev(inp["w_norm"], dt)
    yn = gdn.norm_gate(to_dev(o_in, dt), z, wn, s)
    assert_close(host(yn)[toks][:, vheads], ref["y"], tol, "norm y")
    del yn
    if not cfg.bwd:
        return

    rb = oracle.layer_bwd(sub_cfg, sub, ref, sub["dy"], storage=storage)
    d_o, dz, dwn = gdn.norm_gate_bwd(to_dev(inp["dy"], dt), to_dev(o_in, dt), z, wn, s)
    assert_close(host(d_o)[toks][:, vheads], rb["d_o_exact"], tol, "norm d_o")
    assert_close(host(dz)[toks][:, vheads], rb["dz"], tol, "norm dz")
    # dw_norm sums over every row: the oracle's norm backward over the whole o_in
    _, _, rdwn = oracle.norm_gate_bwd(o_in, inp["z"], inp["w_norm"], inp["dy"])
    assert_close(host(dwn), rdwn, TOL_F32_OUT[dt], "norm dw_norm")
    del d_o, dz

    # chunk backward on the oracle's d_o; gradients land in strided views of one [T, Cch] tensor
    do_in = _filled((T, Hv, D), dt, rng, toks, vheads, rb["d_o"])
    dyc = torch.empty_like(yc)
    r = gdn.chunk_bwd(q, k, v, g, beta, cu, s, to_dev(do_in, dt), h0=h0,
                      dq=dyc[:, :nqk], dk=dyc[:, nqk:2 * nqk], dv=dyc[:, 2 * nqk:])
    n, nq = len(toks), len(kheads) * D
    got = host(dyc)[toks][:, ch]
    assert_close(got[:, :nq].reshape(n, -1, D), rb["dq"], tol, "chunk dq")
    assert_close(got[:, nq:2 * nq].reshape(n, -1, D), rb["dk"], tol, "chunk dk")
    assert_close(got[:, 2 * nq:].reshape(n, -1, D), rb["dv"], tol, "chunk dv")
    assert_close(host(r["dg"])[toks][:, vheads], rb["dg"], TOL_F32_OUT[dt], "chunk dg")
    assert_close(host(r["dbeta"])[toks][:, vheads], rb["dbeta"], TOL_F32_OUT[dt], "chunk dbeta")
    del r, q, k, v, yc, dyc

    # conv backward on the oracle's (bf16-stored) [dq | dk | dv]
    dyc_ref = np.concatenate([rb["dq"].reshape(n, -1), rb["dk"].reshape(n, -1), rb["dv"].reshape(n, -1)], axis=1)
    if storage:
        dyc_ref = synth.round_bf16(dyc_ref.astype(np.float32))
    dyc_in = _filled((T, Cch), dt, rng, toks, ch, dyc_ref)
    dx, dwc = gdn.conv1d_bwd(to_dev(dyc_in, dt), x, w, cu, s)
    assert_close(host(dx)[toks][:, ch], rb["dx"], tol, "conv dx")
    if len(seqs) == cfg.N:  # every sequence in the sample: the weight-gradient sums are complete
        assert_close(host(dwc)[ch], rb["dw_conv"], TOL_F32_OUT[dt], "conv dw")


def _bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy() if t is not None else None


def test_train_deterministic():
    """Two runs of the training step give byte-identical outputs and gradients
    (no float atomics; every reduction has a fixed order)."""
    cfg, inp = _inputs("train")
    _case("determinism", workload="train")
    f1, b1 = layer_gpu(cfg, inp)
    r1 = {k: _bytes(v) for k, v in {**f1, **b1}.items() if isinstance(v, torch.Tensor)}
    del f1, b1
    f2, b2 = layer_gpu(cfg, inp)
    for k, v in {**f2, **b2}.items():
        if isinstance(v, torch.Tensor):
            assert np.array_equal(_bytes(v), r1[k]), k


def test_varlen_packed_equals_separate():
    """Each sequence's outputs, final state and gradients are byte-identical
    whether it runs inside the packed row or alone (the arithmetic of a chunk
    does not depend on where the sequence sits in the row)."""
    cfg = synth.config("varlen").replace(bwd=True, lengths=(300, 4097, 1, 64, 65, 1000), varlen_rule=None,
                                         h_qk=4, h_v=8)
    inp = synth.make_inputs(cfg)
    _case("packed_vs_separate", lengths=cfg.lengths)
    fwd, bwd = layer_gpu(cfg, inp)
    cu = inp["cu"]
    for n in (0, 1, 2, 5):
        sub_cfg, sub, _, _ = oracle.subset(cfg, inp, [n], list(range(cfg.h_qk)))
        f1, b1 = layer_gpu(sub_cfg, sub)
        sl = slice(int(cu[n]), int(cu[n + 1]))
        for key in ("y_conv", "o", "y"):
            assert np.array_equal(_bytes(fwd[key][sl]), _bytes(f1[key])), (n, key)
        assert np.array_equal(_bytes(fwd["ht"][n:n + 1]), _bytes(f1["ht"])), (n, "ht")
        for key in ("dx", "dg", "dbeta", "dz"):
            assert np.array_equal(_bytes(bwd[key][sl]), _bytes(b1[key])), (n, key)
        assert np.array_equal(_bytes(bwd["dh0"][n:n + 1]), _bytes(b1["dh0"])), (n, "dh0")


@pytest.mark.parametrize("lengths", [(0, 0, 5), (1,), (0, 129, 0), (64, 64), (0, 0)])
def test_edge_lengths(lengths):
    """Empty sequences (no rows; ht = h0), single tokens, exact chunk
    multiples and an all-empty row (weight gradients zero).  Without the norm,
    so that the whole backward is compared end to end at the plain bar."""
    cfg = synth.config("varlen").replace(lengths=lengths, varlen_rule=None, h_qk=2, h_v=4, bwd=True, norm=False)
    inp = synth.make_inputs(cfg)
    _case("edge", lengths=lengths)
    fwd, bwd = layer_gpu(cfg, inp)
    ref = oracle.layer_fwd(cfg, inp, storage="bf16")
    rb = oracle.layer_bwd(cfg, inp, ref, inp["dy"], storage="bf16")
    tol = TOL["bf16"]
    assert_close(host(fwd["ht"]), ref["ht"], tol, "ht")
    assert_close(host(bwd["dh0"]), rb["dh0"], tol, "dh0")
    if cfg.T:
        assert_close(host(fwd["o"]), ref["o_exact"], tol, "o")
        for key in ("dx", "dg", "dbeta", "dw_conv"):
            assert_close(host(bwd[key]), rb[key], tol, key)
    else:
        assert np.all(host(bwd["dw_conv"]) == 0)

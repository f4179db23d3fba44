"""Helpers for the GPU parity tests: move seeded inputs to the device and
compare with the oracle by max|diff| / RMS(oracle)."""
import numpy as np
import torch

import gated_delta_rule_conv1d_amd as gdn
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}
# Outputs the chunk stage stores in fp32 (ht, dh0, dg, dbeta): in bf16 mode the
# oracle sees the same bf16-rounded inputs, so only the kernel's own arithmetic
# (bf16 hi/lo operand splits, about 16 significant bits, fp32 sums) separates
# them: max|diff| <= 2e-3 RMS (the worst case over the small chunk cases is
# 8e-4, ht).
TOL_F32_OUT = {"f32": 1e-4, "bf16": 2e-3}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy values -> device tensor of the workload's element type
    (bf16 values are exact: the arrays hold bf16-representable numbers)."""
    if dtype == "bf16":
        bits = synth.bf16_bits(np.asarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    err = float(np.max(np.abs(got - ref)))
    return err / rms if rms > 0 else err


BF16_ULP = 2.0 ** -8   # largest relative rounding error of a bf16 value (8 significant bits, nearest)


def storage_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i (|got_i - ref_i| - 2^-8 |ref_i|) / RMS(ref): the error beyond what
    rounding ref_i itself to bf16 may cost, relative to the tensor's RMS."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    ex = np.abs(got - ref) - BF16_ULP * np.abs(ref)
    return float(np.max(ex)) / rms if rms > 0 else float(np.max(ex))


def assert_close(got, ref, tol, name):
    """fp32 storage (tol 1e-4) and fp32-stored outputs (2e-3):
    max|diff| <= tol * RMS(ref).
    bf16 storage (tol 2e-2): |diff_i| <= tol * RMS(ref) + 2^-8 |ref_i| for
    every element: the tolerance of the statement, plus the rounding of the
    element itself to bf16 (up to 2^-8 of its value), which alone exceeds
    2e-2 * RMS on elements beyond ~5 RMS."""
    got = np.asarray(got)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_err(got, ref)
    if tol >= TOL["bf16"]:
        m = storage_err(got, ref)
        print(f"  {name}: max|d|/rms={e:.3e} beyond-rounding={m:.3e}", flush=True)
        assert m <= tol, f"{name}: max(|d| - 2^-8|ref|)/rms = {m:.3e} > {tol:.0e} (max|d|/rms = {e:.3e})"
        return m
    print(f"  {name}: max|d|/rms={e:.3e}", flush=True)
    assert e <= tol, f"{name}: max|diff|/rms = {e:.3e} > {tol:.0e}"
    return e


CAL_MAX, CAL_RMS = 4.0, 2.0


def assert_calibrated(got, ref, ref32, tol, name, stored=True, max_bar=True):
    """End-to-end bar for a chain of calls: the deviation from the float64
    oracle against that of the oracle's float32 build on the same inputs and
    the same bf16 storage points.  Both chains round their intermediates to
    bf16 between calls; a value within float32 precision of a rounding boundary
    rounds differently on the two sides, and downstream steps can amplify such
    a flip (the norm divides a row by its own RMS).  The float32 build shows
    how large those flips make a correct float32 computation's error here:
    the largest element error (beyond the final bf16 rounding when `stored`)
    is held to max(tol, CAL_MAX x the float32 build's) and the RMS error to
    max(tol, CAL_RMS x the float32 build's), both relative to RMS(ref).  The
    largest error gets the wider factor because it is an extreme over the
    flips, which fall on different elements on the two sides.

    max_bar=False (outputs downstream of the norm's backward): the largest
    error is reported, not held.  There the bf16 path's own rounding of o
    (its W = U - Wk H takes Wk in bf16), which the float32 build does not
    have, is amplified by the norm in rows whose RMS sits far below the
    tensor's, so the float32 build's largest error does not bound it; those
    outputs are held element by element by check_chain instead, and here
    by their RMS error."""
    got, ref, ref32 = (np.asarray(a, dtype=np.float64) for a in (got, ref, ref32))
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    rms = rms if rms > 0 else 1.0
    d = np.abs(got - ref)
    e_max = float(np.max(d - (BF16_ULP * np.abs(ref) if stored else 0.0))) / rms
    e_rms = float(np.sqrt(np.mean(d * d))) / rms
    d32 = np.abs(ref32 - ref)
    c_max = float(np.max(d32)) / rms
    c_rms = float(np.sqrt(np.mean(d32 * d32))) / rms
    bar_max, bar_rms = max(tol, CAL_MAX * c_max), max(tol, CAL_RMS * c_rms)
    print(f"  {name}: gpu max {e_max:.3e} rms {e_rms:.3e} | fp32 oracle max {c_max:.3e} rms {c_rms:.3e} "
          f"| bar max {bar_max:.3e} rms {bar_rms:.3e}", flush=True)
    if max_bar:
        assert e_max <= bar_max, f"{name}: largest error {e_max:.3e} > {bar_max:.3e}"
    assert e_rms <= bar_rms, f"{name}: RMS error {e_rms:.3e} > {bar_rms:.3e}"


def check_chain(cfg, sub_cfg, sub, fwd, bwd, toks, vheads, ch, seqs, all_seqs):
    """The composed GPU layer, stage by stage on its own data: every oracle step
    is fed the GPU's upstream result (the conv output, o, d_o and the conv-input
    gradient the previous GPU call produced, restricted to the sample) and its
    result is compared with the GPU's next result at the plain bar.  The whole
    GPU chain is covered, including rows where the norm amplifies the bf16
    roundings of o (there the comparison is with the oracle step applied to
    the GPU's own o, so the amplification is the same on both sides).
    fwd/bwd: the GPU layer's outputs (torch); toks/vheads/ch: the sample."""
    import oracle
    Hk, Hv, D = sub_cfg.h_qk, sub_cfg.h_v, sub_cfg.d_k
    n, nq = len(toks), Hk * D
    dt = cfg.dtype
    tol, tol32 = TOL[dt], TOL_F32_OUT[dt]
    sq = np.asarray(seqs)
    yc = host(fwd["y_conv"])[toks][:, ch]
    q, k, v = yc[:, :nq].reshape(n, Hk, D), yc[:, nq:2 * nq].reshape(n, Hk, D), yc[:, 2 * nq:].reshape(n, Hv, D)
    o_ref, ht_ref = oracle.recurrence(q, k, v, sub["g"], sub["beta"], sub["cu"], h0=sub.get("h0"))
    o = host(fwd["o"])[toks][:, vheads]
    assert_close(o, o_ref, tol, "chain o")
    assert_close(host(fwd["ht"])[sq][:, vheads], ht_ref, tol32, "chain ht")
    if cfg.norm:
        assert_close(host(fwd["y"])[toks][:, vheads], oracle.norm_gate(o, sub["z"], sub["w_norm"]), tol, "chain y")
    if bwd is None:
        return
    if cfg.norm:
        do_ref, dz_ref, _ = oracle.norm_gate_bwd(o, sub["z"], sub["w_norm"], sub["dy"])
        d_o = host(bwd["d_o"])[toks][:, vheads]
        assert_close(d_o, do_ref, tol, "chain d_o")
        assert_close(host(bwd["dz"])[toks][:, vheads], dz_ref, tol, "chain dz")
    else:
        d_o = sub["dy"]
    r = oracle.recurrence_bwd(q, k, v, sub["g"], sub["beta"], sub["cu"], d_o, h0=sub.get("h0"))
    dyc = host(bwd["dy_conv"])[toks][:, ch]
    assert_close(dyc[:, :nq].reshape(n, Hk, D), r["dq"], tol, "chain dq")
    assert_close(dyc[:, nq:2 * nq].reshape(n, Hk, D), r["dk"], tol, "chain dk")
    assert_close(dyc[:, 2 * nq:].reshape(n, Hv, D), r["dv"], tol, "chain dv")
    assert_close(host(bwd["dg"])[toks][:, vheads], r["dg"], tol32, "chain dg")
    assert_close(host(bwd["dbeta"])[toks][:, vheads], r["dbeta"], tol32, "chain dbeta")
    if "h0" in sub:
        assert_close(host(bwd["dh0"])[sq][:, vheads], r["dh0"], tol32, "chain dh0")
    dx_ref, dw_ref = oracle.conv1d_bwd(sub["x"], sub["w_conv"], sub["cu"], 2 * nq, D, dyc)
    assert_close(host(bwd["dx"])[toks][:, ch], dx_ref, tol, "chain dx")
    if all_seqs:
        assert_close(host(bwd["dw_conv"])[ch], dw_ref, tol32, "chain dw_conv")


def shape_of(cfg: synth.Config, T=None, N=None, chunk=None, scale=1.0) -> gdn.Shape:
    return gdn.Shape(n_seqs=N if N is not None else cfg.N, total_tokens=T if T is not None else cfg.T,
                     h_qk=cfg.h_qk, h_v=cfg.h_v, d_k=cfg.d_k, d_v=cfg.d_v,
                     chunk=chunk if chunk is not None else cfg.chunk,
                     dtype=gdn.BF16 if cfg.dtype == "bf16" else gdn.F32, scale=scale)


def small_cfg(dtype="bf16", lengths=(70, 1, 33, 64, 5), Hk=2, Hv=4, d=32, chunk=16, norm=True, h0=True,
              bwd=True, seed=7, weak=False):
    return synth.Config(name="case", lengths=tuple(lengths), h_qk=Hk, h_v=Hv, d_k=d, d_v=d, chunk=chunk,
                        dtype=dtype, norm=norm, h0=h0, bwd=bwd, seed=seed, weak_decay=weak)


def qkv_inputs(cfg: synth.Config, seed=11):
    """Synthetic unit-norm q, k and N(0,1) v in the storage precision (used by
    the per-call chunk tests so both sides start from identical values)."""
    rng = np.random.default_rng(seed)
    T = cfg.T
    q = rng.standard_normal((T, cfg.h_qk, cfg.d_k))
    k = rng.standard_normal((T, cfg.h_qk, cfg.d_k))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, cfg.h_v, cfg.d_v))
    q, k, v = (a.astype(np.float32) for a in (q, k, v))
    if cfg.dtype == "bf16":
        q, k, v = (synth.round_bf16(a) for a in (q, k, v))
    return q, k, v


def layer_gpu(cfg, inp, layer=None, for_backward=None, max_tokens=None):
    """The whole layer through GatedDeltaNetLayer (the path bench.py times):
    forward, and backward when the workload has one (then, by default, the
    forward keeps its chunk products for the backward, as bench.py does).
    max_tokens: the bounded-memory mode (chunk calls per token segment)."""
    s = shape_of(cfg)
    dt = cfg.dtype
    L = layer or gdn.GatedDeltaNetLayer(s, cfg.width, norm=cfg.norm)
    t = dict(x=to_dev(inp["x"], dt), w=to_dev(inp["w_conv"], dt), g=f32(inp["g"]), beta=f32(inp["beta"]),
             cu=torch.from_numpy(inp["cu"]).cuda(),
             z=to_dev(inp["z"], dt) if "z" in inp else None, wn=to_dev(inp["w_norm"], dt) if "w_norm" in inp else None,
             h0=f32(inp["h0"]) if "h0" in inp else None)
    save = (cfg.bwd if for_backward is None else for_backward) and max_tokens is None
    fwd = L.forward(t["x"], t["w"], t["g"], t["beta"], t["cu"], t["z"], t["wn"], t["h0"], for_backward=save,
                    max_tokens=max_tokens)
    bwd = None
    if cfg.bwd:
        bwd = L.backward(to_dev(inp["dy"], dt), t["x"], t["w"], t["g"], t["beta"], t["cu"], fwd, t["z"], t["wn"],
                         t["h0"])
    torch.cuda.synchronize()
    return fwd, bwd


def channels(cfg, kheads):
    """Columns of the [T, Cch] conv input that belong to some q/k heads and
    their v-heads (channel blocks [q | k | v])."""
    G = cfg.h_v // cfg.h_qk
    dk, dv, Hk = cfg.d_k, cfg.d_v, cfg.h_qk
    q = np.concatenate([np.arange(j * dk, (j + 1) * dk) for j in kheads])
    v = np.concatenate([2 * Hk * dk + np.arange(h * dv, (h + 1) * dv) for j in kheads for h in range(j * G, j * G + G)])
    return np.concatenate([q, q + Hk * dk, v])

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


def mixed_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max(RMS(ref), |ref_i|)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(rms, np.abs(ref))
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den))


def assert_close(got, ref, tol, name):
    """fp32 storage (tol 1e-4): max|diff| <= tol * RMS(ref).
    bf16 storage (tol 2e-2): |diff_i| <= tol * max(RMS(ref), |ref_i|) for every
    element -- the same bound wherever |ref_i| <= RMS, and 2% relative error on
    the heavy tail, where the bf16 representation error alone (up to 2^-8 of the
    value) already exceeds 2e-2 * RMS once |ref_i| > 5 RMS."""
    got = np.asarray(got)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_err(got, ref)
    if tol >= TOL["bf16"]:
        m = mixed_err(got, ref)
        print(f"  {name}: max|d|/rms={e:.3e} mixed={m:.3e}", flush=True)
        assert m <= tol, f"{name}: max|d|/max(rms,|ref|) = {m:.3e} > {tol:.0e} (max|d|/rms = {e:.3e})"
        return m
    print(f"  {name}: max|d|/rms={e:.3e}", flush=True)
    assert e <= tol, f"{name}: max|diff|/rms = {e:.3e} > {tol:.0e}"
    return e


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


def layer_gpu(cfg, inp, layer=None, for_backward=None):
    """The whole layer through GatedDeltaNetLayer (the path bench.py times):
    forward, and backward when the workload has one (then, by default, the
    forward keeps its chunk products for the backward, as bench.py does)."""
    s = shape_of(cfg)
    dt = cfg.dtype
    L = layer or gdn.GatedDeltaNetLayer(s, cfg.width, norm=cfg.norm)
    t = dict(x=to_dev(inp["x"], dt), w=to_dev(inp["w_conv"], dt), g=f32(inp["g"]), beta=f32(inp["beta"]),
             cu=torch.from_numpy(inp["cu"]).cuda(),
             z=to_dev(inp["z"], dt) if "z" in inp else None, wn=to_dev(inp["w_norm"], dt) if "w_norm" in inp else None,
             h0=f32(inp["h0"]) if "h0" in inp else None)
    save = cfg.bwd if for_backward is None else for_backward
    fwd = L.forward(t["x"], t["w"], t["g"], t["beta"], t["cu"], t["z"], t["wn"], t["h0"], for_backward=save)
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

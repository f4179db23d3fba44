"""The layer's steps recorded into a HIP graph (gated_delta_rule_conv1d_amd.capture)
and replayed: every replay must give byte-identical results to the same step
run eagerly (the kernels are deterministic: fixed-order sums, no float
atomics), with eager work and synchronisations between the replays, and a
replay must read new values copied into the captured inputs.  The eager
results themselves are held to the oracle by the parity tests; here the graph
is checked against them bit for bit.

Cases: the training step (gates, conv, chunked forward keeping its products,
norm, and every backward call) with the gate kernels and with the gates inside
the chunk kernels, at d = 32 / chunk 16 (the general kernels) and d = 128 /
chunk 64 (the wide and 16-column state passes); the inference forward from
initial states; and three decode steps advancing the state and the conv window
in place."""
import numpy as np
import pytest
import torch

import gated_delta_rule_conv1d_amd as gdn
import synth
from gpu_util import f32, shape_of, small_cfg, to_dev

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _flat(out):
    """Tensors of a step's result, by name (nested dicts flattened)."""
    res = {}
    for key, val in out.items():
        if isinstance(val, dict):
            res.update({f"{key}.{k}": v for k, v in _flat(val).items()})
        elif isinstance(val, torch.Tensor):
            res[key] = val
        elif isinstance(val, (tuple, list)):
            res.update({f"{key}[{i}]": v for i, v in enumerate(val) if isinstance(v, torch.Tensor)})
    return res


def _snap(out):
    return {k: v.detach().contiguous().view(torch.uint8).cpu().numpy().copy() for k, v in _flat(out).items()}


def _assert_same(got, ref, what):
    assert got.keys() == ref.keys(), (what, sorted(got), sorted(ref))
    for k in ref:
        assert np.array_equal(got[k], ref[k]), f"{what}: {k} differs"


def _layer_inputs(cfg, seed_shift=0):
    inp = synth.make_inputs(cfg.replace(seed=cfg.seed + seed_shift), keep_raw=True)
    dt = cfg.dtype
    t = dict(x=to_dev(inp["x"], dt), w=to_dev(inp["w_conv"], dt), cu=torch.from_numpy(inp["cu"]).cuda(),
             a=f32(inp["a"]), b=f32(inp["b"]), A_log=f32(inp["A_log"]), dt_bias=f32(inp["dt_bias"]),
             z=to_dev(inp["z"], dt), wn=to_dev(inp["w_norm"], dt),
             h0=f32(inp["h0"]) if "h0" in inp else None,
             dy=to_dev(inp["dy"], dt) if "dy" in inp else None)
    return t


def _layer_step(cfg, layer, t, fused):
    gates = (t["a"], t["b"], t["A_log"], t["dt_bias"])

    def step():
        if fused:
            f = layer.forward(t["x"], t["w"], None, None, t["cu"], t["z"], t["wn"], t["h0"],
                              for_backward=cfg.bwd, gates=gates)
            r = layer.backward(t["dy"], t["x"], t["w"], None, None, t["cu"], f, t["z"], t["wn"], t["h0"],
                               gates=gates) if cfg.bwd else {}
            return {"fwd": f, "bwd": r}
        g, beta = layer.gates(*gates)
        f = layer.forward(t["x"], t["w"], g, beta, t["cu"], t["z"], t["wn"], t["h0"], for_backward=cfg.bwd)
        out = {"g": g, "beta": beta, "fwd": f}
        if cfg.bwd:
            r = layer.backward(t["dy"], t["x"], t["w"], g, beta, t["cu"], f, t["z"], t["wn"], t["h0"])
            out["bwd"] = r
            out["gates_bwd"] = layer.gates_backward(*gates, r["dg"], r["dbeta"])
        return out
    return step


LAYER_CASES = [
    # (d, chunk, Hk, Hv, lengths, h0, bwd, fused)
    (32, 16, 2, 4, (70, 1, 33, 64, 5), True, True, False),
    (32, 16, 2, 4, (70, 1, 33, 64, 5), True, True, True),
    (128, 64, 2, 4, (300, 1000, 65), False, True, False),   # few chains: 16-column forward tiles
    (128, 64, 2, 4, (300, 1000, 65), True, True, True),
    (128, 64, 2, 4, (300, 1000, 65, 1, 129), True, False, False),  # inference forward
]


@pytest.mark.parametrize("d,chunk,Hk,Hv,lengths,h0,bwd,fused", LAYER_CASES)
def test_graph_layer_step(d, chunk, Hk, Hv, lengths, h0, bwd, fused):
    cfg = small_cfg("bf16", lengths=lengths, Hk=Hk, Hv=Hv, d=d, chunk=chunk, h0=h0, bwd=bwd, seed=11)
    _case("graph_layer", d=d, chunk=chunk, Hk=Hk, Hv=Hv, lengths=lengths, h0=h0, bwd=bwd, fused=fused)
    layer = gdn.GatedDeltaNetLayer(shape_of(cfg), cfg.width, norm=True)
    t = _layer_inputs(cfg)
    step = _layer_step(cfg, layer, t, fused)
    gdn.profile_enable(False)

    ref = _snap(step())          # eager; also creates the layer's workspaces
    torch.cuda.synchronize()
    graph, out = gdn.capture(step)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(_snap(out), ref, f"replay {rep}")
        _assert_same(_snap(step()), ref, f"eager after replay {rep}")  # shares the workspaces
        torch.cuda.synchronize()

    # new inputs copied into the captured tensors: the replay reads them
    t2 = _layer_inputs(cfg, seed_shift=1)
    for key in ("x", "a", "b", "z") + (("dy",) if bwd else ()) + (("h0",) if h0 else ()):
        t[key].copy_(t2[key])
    graph.replay()
    torch.cuda.synchronize()
    got = _snap(out)
    ref2 = _snap(step())
    torch.cuda.synchronize()
    _assert_same(got, ref2, "replay on new inputs")
    assert not np.array_equal(got["fwd.y"], ref["fwd.y"]), "the replay did not read the new inputs"


def test_graph_decode_steps():
    """Three decode steps (gates, conv step, recurrent step, norm), the state
    and the conv window advanced in place: replay i equals eager step i."""
    cfg = synth.config("decode").replace(lengths=(1,) * 8, h_qk=2, h_v=4)
    _case("graph_decode", N=cfg.N, Hk=cfg.h_qk, Hv=cfg.h_v, d=cfg.d_k)
    inp = synth.make_inputs(cfg, keep_raw=True)
    s = shape_of(cfg)
    layer = gdn.GatedDeltaNetLayer(s, cfg.width, norm=True)
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["w_conv"], "bf16")
    z, wn = to_dev(inp["z"], "bf16"), to_dev(inp["w_norm"], "bf16")
    a, b, A_log, dt_bias = (f32(inp[k]) for k in ("a", "b", "A_log", "dt_bias"))
    state0, window0 = f32(inp["h0"]), to_dev(inp["window"], "bf16")
    state, window = state0.clone(), window0.clone()

    def step():
        g, beta = layer.gates(a, b, A_log, dt_bias)
        yc = gdn.conv1d_step(x, w, window, s)
        q, k, v = layer.split(yc)
        o, _ = gdn.recurrent_step(q, k, v, g, beta, s, state_in=state, state_out=state)
        return {"yc": yc, "o": o, "y": gdn.norm_gate(o, z, wn, s)}

    gdn.profile_enable(False)
    eager = []
    for _ in range(3):
        r = _snap(step())
        torch.cuda.synchronize()
        r.update(_snap({"state": state, "window": window}))
        eager.append(r)
    assert not np.array_equal(eager[0]["state"], eager[1]["state"])

    state.copy_(state0)
    window.copy_(window0)
    graph, out = gdn.capture(step)   # records only: the state is not advanced
    torch.cuda.synchronize()
    _assert_same(_snap({"state": state, "window": window}),
                 _snap({"state": state0, "window": window0}), "capture ran kernels")
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = _snap(out)
        got.update(_snap({"state": state, "window": window}))
        _assert_same(got, eager[i], f"decode replay {i}")
        torch.zeros(1 << 20, device="cuda").add_(1.0)  # eager work between the replays
        torch.cuda.synchronize()

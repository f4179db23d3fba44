"""gdn_norm_gate_bwd_noalloc (the backward of RMSNormGated with the library's
own device scratch instead of a caller workspace) against gdn_norm_gate_bwd,
through the C ABI: two calls in a row, the second on a smaller input, each
bit-identical to the workspace entry point and within the bar of the oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_conv1d_amd as gdn
import oracle
import synth
from gpu_util import TOL, TOL_F32_OUT, assert_close, host, shape_of, small_cfg, to_dev

pytestmark = pytest.mark.gpu


def _case(cfg, seed):
    rng = np.random.default_rng(seed)
    dt, T, Hv, d = cfg.dtype, cfg.T, cfg.h_v, cfg.d_v
    o = rng.standard_normal((T, Hv, d)).astype(np.float32)
    z = rng.standard_normal((T, Hv, d)).astype(np.float32)
    dy = rng.standard_normal((T, Hv, d)).astype(np.float32)
    w = (1 + 0.02 * rng.standard_normal(d)).astype(np.float32)
    if dt == "bf16":
        o, z, dy, w = (synth.round_bf16(a) for a in (o, z, dy, w))
    return o, z, dy, w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_norm_gate_bwd_noalloc_matches_workspace_call(dtype):
    big = small_cfg(dtype=dtype, d=128, Hk=4, Hv=8, lengths=(700, 1, 300))
    small = small_cfg(dtype=dtype, d=64, Hk=1, Hv=2, lengths=(33,))
    for n, cfg in enumerate((big, small)):
        print(f"[case] noalloc call {n} dtype={dtype} T={cfg.T} Hv={cfg.h_v} d={cfg.d_v}", flush=True)
        s = shape_of(cfg)
        o, z, dy, w = _case(cfg, 100 + n)
        od, zd, dyd, wd = (to_dev(a, dtype) for a in (o, z, dy, w))
        ref = gdn.norm_gate_bwd(dyd, od, zd, wd, s)
        got = gdn.norm_gate_bwd_noalloc(dyd, od, zd, wd, s)
        torch.cuda.synchronize()
        for name, a, b in zip(("d_o", "dz", "dw_norm"), got, ref):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name
        rdo, rdz, rdw = oracle.norm_gate_bwd(o, z, w, dy)
        assert_close(host(got[0]), rdo, TOL[dtype], "d_o")
        assert_close(host(got[1]), rdz, TOL[dtype], "dz")
        assert_close(host(got[2]), rdw, TOL_F32_OUT[dtype], "dw_norm")

"""bench.py's host-side parts (CPU): the fused-minimum byte model that prices
the whole step, and the refusal of more than one GPU.

The per-token figures are counted here item by item from the tensors the
layer takes and returns (the pre-conv q/k/v row, z, g and beta in, the norm
output out; backward: those inputs again, dy in, their gradients out), so a
dropped or double-counted item in bench.fused_minimum_bytes fails."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

BF16, F32 = 2, 4


def _state(cfg):
    return cfg.h_v * cfg.d_k * cfg.d_v * F32


@pytest.mark.parametrize("name", ["dense", "varlen", "long", "train"])
def test_fused_minimum_per_token(name):
    cfg = synth.config(name)
    Hk, Hv, d = cfg.h_qk, cfg.h_v, cfg.d_k
    q = k = Hk * d * BF16
    v = z = y = dy = dz = Hv * d * BF16
    g = beta = Hv * F32
    fwd = (q + k + v) + z + (g + beta) + y
    bwd = (q + k + v) + z + (g + beta) + dy + (q + k + v) + dz + (g + beta)
    assert fwd == 33024 and (bwd == 57856)   # d = 128, 16 q/k heads, 32 v heads
    per_token = fwd + (bwd if cfg.bwd else 0)
    states = cfg.N * _state(cfg) * (2 if cfg.h0 else 1)   # h0 read when given, ht written
    assert bench.fused_minimum_bytes(cfg) == per_token * cfg.T + states


def test_fused_minimum_totals():
    """The varlen row (20 sequences with h0 in and ht out) and the long
    sequence (ht out): 1.166 GB and 2.166 GB."""
    assert round(bench.fused_minimum_bytes(synth.config("varlen")) / 1e6) == 1166
    assert round(bench.fused_minimum_bytes(synth.config("long")) / 1e6) == 2166


def test_fused_minimum_decode_is_state_bound():
    """A decode step reads and writes every (sequence, v-head) state and conv
    window: 1 GiB of fp32 states at 256 sequences, against 8.4 MB of tokens."""
    cfg = synth.config("decode")
    Cch = 2 * cfg.h_qk * cfg.d_k + cfg.h_v * cfg.d_v
    states = 2 * cfg.N * _state(cfg)
    windows = 2 * cfg.N * (cfg.width - 1) * Cch * BF16
    assert states == 1 << 30
    assert bench.fused_minimum_bytes(cfg) == 33024 * cfg.T + states + windows


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

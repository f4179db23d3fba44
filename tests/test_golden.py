"""Regression fixtures (written by tests/golden/make_golden.py from synth and the oracle)."""
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_varlen_row_is_stable():
    rows = {r[0]: [int(x) for x in r[1:]] for r in _read("varlen_row.txt")}
    cfg = synth.config("varlen")
    assert list(cfg.lengths) == rows["lengths"]
    assert sum(cfg.lengths) == 32768 and len(cfg.lengths) == 20
    assert all(64 <= x <= 8192 for x in cfg.lengths[:-1]) and 1 <= cfg.lengths[-1] <= 8192
    cu = synth.cu_from_lengths(cfg.lengths)
    assert list(cu) == rows["cu"]
    tab, first = oracle.chunk_table(cu, 64)
    assert list(np.diff(first)) == rows["chunks"]
    assert len(tab) == rows["n_chunks"][0]
    assert list(np.diff(first)) == [-(-x // 64) for x in cfg.lengths]


def test_tiny_oracle_values_are_stable():
    cfg = synth.config("tiny")
    out = oracle.layer_fwd(cfg, synth.make_inputs(cfg))
    for name, idx, val in _read("tiny_oracle.txt"):
        got = out[name].reshape(-1)[int(idx)]
        assert abs(got - float(val)) <= 1e-12 * max(1.0, abs(float(val))), (name, idx)


def test_generator_is_deterministic_and_bf16_rounded():
    cfg = synth.config("dense").replace(lengths=(40, 24))
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    # bf16 values are exactly representable and are the nearest ones (RNE)
    x = a["x"]
    np.testing.assert_array_equal(synth.round_bf16(x), x)
    assert np.all(a["g"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_bf16_rounding_is_round_to_nearest_even():
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5], dtype=np.float32)
    got = synth.round_bf16(vals)
    np.testing.assert_array_equal(got, np.array([1.0, 1.0 + 2 * 2.0 ** -7, 1.0 + 2.0 ** -7, -2.5], dtype=np.float32))

"""C ABI checks that need no GPU: the library loads, exports every function
include/gdn.h declares, and rejects bad arguments on the host before anything
is enqueued (only failing argument sets are passed here, so nothing launches)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_conv1d_amd as gdn
from gated_delta_rule_conv1d_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: calls below fail validation first
FAKE_ODD = ctypes.c_void_p(0x10008)    # not 16-byte aligned


def header_functions():
    with open(os.path.join(ROOT, "include", "gdn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = gdn.load()
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.SYMBOLS)


def shape(**kw):
    d = dict(n_seqs=2, total_tokens=100, h_qk=2, h_v=4, d_k=32, d_v=32, chunk=16, dtype=gdn.BF16, scale=1.0)
    d.update(kw)
    return B._Shape(*[d[f] for f, _ in B._Shape._fields_])


def test_status_strings():
    lib = gdn.load()
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert lib.gdn_status_string(code).startswith(b"GDN_")


@pytest.mark.parametrize("bad,code", [
    (dict(n_seqs=0), INVALID), (dict(total_tokens=-1), INVALID), (dict(h_qk=0), INVALID),
    (dict(h_v=3), INVALID), (dict(d_k=48, d_v=48), UNSUPPORTED), (dict(d_v=64), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED), (dict(chunk=8), UNSUPPORTED), (dict(chunk=128), UNSUPPORTED),
    (dict(dtype=gdn.F32, d_k=128, d_v=128, chunk=64), UNSUPPORTED),
    (dict(dtype=gdn.F32, d_k=32, d_v=32, chunk=64), UNSUPPORTED),   # float32 runs chunks of at most 32
])
def test_chunk_fwd_rejects_shape(bad, code):
    lib = gdn.load()
    s = shape(**bad)
    rc = lib.gdn_chunk_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, 64, 128, FAKE, FAKE, FAKE, None, FAKE, None,
                           FAKE, 1 << 40, None)
    assert rc == code
    assert lib.gdn_chunk_fwd_workspace(ctypes.byref(s)) == 0


def test_chunk_fwd_rejects_pointers_strides_workspace():
    lib = gdn.load()
    s = shape()
    ws = lib.gdn_chunk_fwd_workspace(ctypes.byref(s))
    assert ws > 0

    def call(q=FAKE, k=FAKE, v=FAKE, sqk=64, sv=128, g=FAKE, b=FAKE, cu=FAKE, o=FAKE, w=FAKE, nb=ws):
        return lib.gdn_chunk_fwd(ctypes.byref(s), q, k, v, sqk, sv, g, b, cu, None, o, None, w, nb, None)

    assert call(q=None) == INVALID
    assert call(v=None) == INVALID
    assert call(g=None) == INVALID
    assert call(cu=None) == INVALID
    assert call(o=None) == INVALID
    assert call(q=FAKE_ODD) == INVALID
    assert call(sqk=63) == INVALID          # shorter than one token of q
    assert call(sqk=68) == INVALID          # rows not 16-byte aligned (bf16)
    assert call(sv=100) == INVALID
    assert call(w=None) == WORKSPACE
    assert call(nb=ws - 1) == WORKSPACE


def test_fp8_and_fused_gate_calls_reject():
    lib = gdn.load()
    s = shape(d_k=128, d_v=128, chunk=64, h_qk=1, h_v=2)
    ws = lib.gdn_chunk_fwd_workspace(ctypes.byref(s))

    def fp8(sc=(1.0, 0.5, 2.0), sh=s, sqk=128, w=FAKE, nb=ws):
        return lib.gdn_chunk_fwd_fp8(ctypes.byref(sh), FAKE, FAKE, FAKE, sqk, 256, *sc, FAKE, FAKE, FAKE, None, FAKE,
                                     None, w, nb, None)

    assert fp8(sc=(0.75, 1.0, 1.0)) == INVALID      # scales must be powers of two
    assert fp8(sc=(1.0, 0.0, 1.0)) == INVALID
    assert fp8(sc=(1.0, 1.0, float("inf"))) == INVALID
    assert fp8(sqk=136) == INVALID                  # byte stride not a multiple of 16
    assert fp8(sh=shape(d_k=64, d_v=64, chunk=64)) == UNSUPPORTED
    assert fp8(sh=shape(d_k=128, d_v=128, chunk=32)) == UNSUPPORTED
    assert fp8(sh=shape(d_k=128, d_v=128, chunk=64, dtype=gdn.F32)) == UNSUPPORTED
    assert fp8(nb=ws - 1) == WORKSPACE

    gi = B._GateInputs(FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    gi_bad = B._GateInputs(FAKE.value, None, FAKE.value, FAKE.value)
    gg = B._GateGrads(FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    gg_bad = B._GateGrads(FAKE.value, FAKE.value, None, FAKE.value)
    s2 = shape()
    ws2 = lib.gdn_chunk_bwd_workspace(ctypes.byref(s2))

    def fwd(g):
        return lib.gdn_chunk_fwd_gated(ctypes.byref(s2), FAKE, FAKE, FAKE, 64, 128, g, FAKE, None, FAKE, None, FAKE,
                                       ws2, None)

    def bwd(g, d):
        return lib.gdn_chunk_bwd_gated(ctypes.byref(s2), FAKE, FAKE, FAKE, 64, 128, g, FAKE, None, FAKE, None,
                                       FAKE, FAKE, FAKE, d, None, FAKE, ws2 - 256, None)

    assert fwd(None) == INVALID
    assert fwd(ctypes.byref(gi_bad)) == INVALID
    assert bwd(ctypes.byref(gi), None) == INVALID
    assert bwd(ctypes.byref(gi), ctypes.byref(gg_bad)) == INVALID
    assert bwd(ctypes.byref(gi), ctypes.byref(gg)) == WORKSPACE


def test_chunk_bwd_rejects():
    lib = gdn.load()
    s = shape()
    ws = lib.gdn_chunk_bwd_workspace(ctypes.byref(s))
    assert ws > lib.gdn_chunk_fwd_workspace(ctypes.byref(s))

    def call(d_o=FAKE, dq=FAKE, w=FAKE, nb=ws):
        return lib.gdn_chunk_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, 64, 128, FAKE, FAKE, FAKE, None, d_o, None,
                                 dq, FAKE, FAKE, FAKE, FAKE, None, w, nb, None)

    assert call(d_o=None) == INVALID
    assert call(dq=None) == INVALID
    assert call(dq=FAKE_ODD) == INVALID
    assert call(nb=ws - 256) == WORKSPACE


def test_conv_and_norm_reject():
    lib = gdn.load()
    s = shape()
    assert lib.gdn_conv1d(ctypes.byref(s), FAKE, FAKE, 5, 1e-6, FAKE, ctypes.c_void_p(0x20000), None) == UNSUPPORTED
    assert lib.gdn_conv1d(ctypes.byref(s), FAKE, FAKE, 1, 1e-6, FAKE, ctypes.c_void_p(0x20000), None) == UNSUPPORTED
    assert lib.gdn_conv1d(ctypes.byref(s), FAKE, FAKE, 4, 1e-6, FAKE, FAKE, None) == INVALID   # y aliases x
    assert lib.gdn_conv1d(ctypes.byref(s), FAKE, FAKE, 4, -1.0, FAKE, ctypes.c_void_p(0x20000), None) == INVALID
    assert lib.gdn_conv1d(ctypes.byref(s), None, FAKE, 4, 1e-6, FAKE, ctypes.c_void_p(0x20000), None) == INVALID
    nb = lib.gdn_conv1d_bwd_workspace(ctypes.byref(s), 4)
    assert nb > 0 and lib.gdn_conv1d_bwd_workspace(ctypes.byref(s), 9) == 0
    assert lib.gdn_conv1d_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, 4, 1e-6, FAKE, ctypes.c_void_p(0x20000), FAKE,
                              None, nb, None) == WORKSPACE
    assert lib.gdn_norm_gate(ctypes.byref(s), FAKE, FAKE, FAKE, 1e-6, None, None) == INVALID
    assert lib.gdn_norm_gate(ctypes.byref(s), FAKE, FAKE, FAKE_ODD, 1e-6, FAKE, None) == INVALID
    nb = lib.gdn_norm_gate_bwd_workspace(ctypes.byref(s))
    assert lib.gdn_norm_gate_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1e-6, FAKE, FAKE, FAKE, FAKE, nb - 4,
                                 None) == WORKSPACE
    assert lib.gdn_chunk_index(ctypes.byref(shape(chunk=24)), FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.gdn_chunk_index(ctypes.byref(s), None, FAKE, FAKE, None) == INVALID


def test_gates_reject():
    lib = gdn.load()
    s = shape()
    G, B2 = ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000)
    odd = ctypes.c_void_p(0x10002)
    assert lib.gdn_gates(ctypes.byref(s), FAKE, FAKE, FAKE, None, G, B2, None) == INVALID    # dt_bias missing
    assert lib.gdn_gates(ctypes.byref(s), None, FAKE, FAKE, FAKE, G, B2, None) == INVALID
    assert lib.gdn_gates(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, B2, None) == INVALID  # g aliases a
    assert lib.gdn_gates(ctypes.byref(s), odd, FAKE, FAKE, FAKE, G, B2, None) == INVALID
    assert lib.gdn_gates(ctypes.byref(shape(h_v=3)), FAKE, FAKE, FAKE, FAKE, G, B2, None) == INVALID
    nb = lib.gdn_gates_bwd_workspace(ctypes.byref(s))
    assert nb >= 2 * 4 * 4  # two fp32 partial rows of Hv = 4 heads at least
    args = [FAKE] * 10
    assert lib.gdn_gates_bwd(ctypes.byref(s), *args, FAKE, nb - 4, None) == WORKSPACE
    assert lib.gdn_gates_bwd(ctypes.byref(s), *args, None, nb, None) == WORKSPACE
    assert lib.gdn_gates_bwd(ctypes.byref(s), *args[:8], None, FAKE, FAKE, nb, None) == INVALID  # dA_log missing
    assert lib.gdn_gates_bwd(ctypes.byref(s), *args[:4], None, *args[5:], FAKE, nb, None) == INVALID  # dg missing


def test_decode_calls_reject():
    lib = gdn.load()
    s = shape(n_seqs=4, total_tokens=4)
    A, B2, C3 = ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000)

    def rec(sh=s, sqk=64, sv=128, st_in=FAKE, st_out=A, o=B2):
        return lib.gdn_recurrent_step(ctypes.byref(sh), FAKE, FAKE, FAKE, sqk, sv, FAKE, FAKE, st_in, st_out, o, None)

    assert rec(sh=shape(n_seqs=4, total_tokens=5)) == INVALID   # one token per sequence
    assert rec(st_out=None) == INVALID
    assert rec(o=None) == INVALID
    assert rec(st_in=FAKE_ODD) == INVALID
    assert rec(sqk=63) == INVALID
    assert rec(sh=shape(n_seqs=4, total_tokens=4, d_k=48, d_v=48)) == UNSUPPORTED
    assert lib.gdn_conv1d_step(ctypes.byref(s), FAKE, FAKE, 5, 1e-6, A, B2, None) == UNSUPPORTED
    assert lib.gdn_conv1d_step(ctypes.byref(s), FAKE, FAKE, 4, 1e-6, A, FAKE, None) == INVALID  # y aliases x
    assert lib.gdn_conv1d_step(ctypes.byref(s), FAKE, FAKE, 4, 1e-6, None, B2, None) == INVALID
    assert lib.gdn_conv1d_step(ctypes.byref(shape(n_seqs=4, total_tokens=3)), FAKE, FAKE, 4, 1e-6, A, B2,
                               None) == INVALID
    assert lib.gdn_conv1d_window(ctypes.byref(s), FAKE, 4, FAKE, A, A, None) == INVALID      # in place
    assert lib.gdn_conv1d_window(ctypes.byref(s), FAKE, 4, None, None, A, None) == INVALID   # no cu_seqlens
    assert lib.gdn_conv1d_window(ctypes.byref(s), FAKE, 1, FAKE, None, A, None) == UNSUPPORTED
    assert lib.gdn_conv1d_window(ctypes.byref(s), FAKE, 4, FAKE, FAKE_ODD, C3, None) == INVALID
    assert lib.gdn_conv1d_prefill(ctypes.byref(s), FAKE, FAKE, 4, 1e-6, FAKE, A, B2, A, None) == INVALID  # in place
    assert lib.gdn_conv1d_prefill(ctypes.byref(s), FAKE, FAKE, 4, 1e-6, FAKE, A, FAKE, C3, None) == INVALID  # y = x
    assert lib.gdn_conv1d_prefill(ctypes.byref(s), FAKE, FAKE, 4, 1e-6, FAKE, FAKE_ODD, B2, C3, None) == INVALID
    assert lib.gdn_conv1d_prefill(ctypes.byref(s), FAKE, FAKE, 5, 1e-6, FAKE, A, B2, C3, None) == UNSUPPORTED


def test_workspace_sizes_grow_with_tokens_and_max_chunks_bound():
    lib = gdn.load()
    prev_f = prev_b = 0
    for T in (0, 1, 64, 65, 1000, 65536):
        s = shape(total_tokens=T, n_seqs=3, d_k=128, d_v=128, h_qk=16, h_v=32, chunk=64)
        f = lib.gdn_chunk_fwd_workspace(ctypes.byref(s))
        b = lib.gdn_chunk_bwd_workspace(ctypes.byref(s))
        assert f >= prev_f and b >= prev_b and b > f
        prev_f, prev_b = f, b
        assert lib.gdn_max_chunks(ctypes.byref(s)) == -(-T // 64) + 3

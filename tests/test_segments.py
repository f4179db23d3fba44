"""Host logic of the bounded-memory mode: token_segments splits a packed row
into segments the chunk calls can take one at a time (CPU only)."""
import numpy as np
import pytest

from gated_delta_rule_conv1d_amd import token_segments


def _check(cu, chunk, max_tokens):
    segs = token_segments(cu, chunk, max_tokens)
    P = max(chunk, (max_tokens // chunk) * chunk)
    N = len(cu) - 1
    t = 0
    n = 0
    for t0, t1, n0, n1, piece in segs:
        assert t0 == t and t1 >= t0 and t1 - t0 <= P, (t0, t1, P)
        if piece is None:
            # whole sequences n0 .. n1-1, exactly covering [t0, t1)
            assert n0 == n and n1 > n0 and cu[n0] == t0 and cu[n1] == t1
            n = n1
        else:
            i, count = piece
            L = cu[n0 + 1] - cu[n0]
            assert n1 == n0 + 1 and L > P and count == -(-L // P)
            # pieces start at multiples of P (a multiple of the chunk) from the sequence start
            assert t0 == cu[n0] + i * P and (t0 - cu[n0]) % chunk == 0
            assert t1 == min(cu[n0] + (i + 1) * P, cu[n0 + 1])
            if i + 1 == count:
                n = n0 + 1
        t = t1
    assert t == cu[-1] and n == N
    return segs


@pytest.mark.parametrize("lengths,chunk,max_tokens", [
    ((300, 1, 64, 65, 130, 0, 700), 64, 192),
    ((0, 0, 5), 64, 64),
    ((0,), 16, 100),
    ((65536,), 64, 16384),
    ((8192,) * 8, 64, 16384),
    ((1000,), 64, 10),          # budget below one chunk: one chunk per piece
    ((64, 64, 64), 64, 128),
])
def test_token_segments_cases(lengths, chunk, max_tokens):
    cu = [0] + list(np.cumsum(lengths))
    _check([int(c) for c in cu], chunk, max_tokens)


def test_token_segments_random():
    rng = np.random.default_rng(5)
    for _ in range(300):
        N = int(rng.integers(1, 12))
        lengths = rng.integers(0, 900, N) * (rng.random(N) < 0.9)
        chunk = int(rng.choice([16, 32, 64]))
        cu = [0] + [int(c) for c in np.cumsum(lengths)]
        _check(cu, chunk, int(rng.integers(1, 1200)))


def test_token_segments_training_budget():
    """8 x 8192 tokens with a 16384-token budget: two whole sequences per segment."""
    cu = [i * 8192 for i in range(9)]
    segs = token_segments(cu, 64, 16384)
    assert [(t0, t1, n0, n1) for t0, t1, n0, n1, _ in segs] == [(i * 16384, (i + 1) * 16384, 2 * i, 2 * i + 2)
                                                                 for i in range(4)]

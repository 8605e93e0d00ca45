"""Pins of the fp64 oracle's backward (CPU only): central finite differences of
the forward on tiny inputs, and the uniform-score closed form for dSink."""

import math

import numpy as np
import pytest

import oracle


def _loss(q, k, v, sink, dout, scale, causal, window):
    o, _ = oracle.prefill(q, k, v, sink, scale, causal=causal, window=window)
    return float(np.sum(o * dout))


def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + eps
        fp = f()
        x[idx] = old - eps
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("Sq,Sk,causal,window", [
    (4, 4, True, None), (3, 5, True, None), (4, 4, False, None), (6, 6, True, (1, 2)),
])
def test_backward_matches_finite_differences(Sq, Sk, causal, window):
    rng = np.random.default_rng(20)
    B, Hq, Hkv, D = 1, 4, 2, 3
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    sink = rng.standard_normal(Hq)
    dout = rng.standard_normal((B, Sq, Hq, D))
    scale = 0.8
    dq, dk, dv, dsink, _, _ = oracle.backward(q, k, v, sink, dout, scale, causal, window)
    f = lambda: _loss(q, k, v, sink, dout, scale, causal, window)  # noqa: E731
    for got, x in ((dq, q), (dk, k), (dv, v), (dsink, sink)):
        ref = _fd(f, x)
        assert np.max(np.abs(got - ref)) < 1e-8 * max(1.0, np.max(np.abs(ref)))


def test_backward_without_sink_has_zero_dsink_and_matches_fd():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 3, 2, 2))
    k = rng.standard_normal((1, 3, 1, 2))
    v = rng.standard_normal((1, 3, 1, 2))
    dout = rng.standard_normal((1, 3, 2, 2))
    dq, dk, dv, dsink, _, _ = oracle.backward(q, k, v, None, dout, 1.1, True)
    assert np.array_equal(dsink, np.zeros(2))
    f = lambda: _loss(q, k, v, None, dout, 1.1, True, None)  # noqa: E731
    assert np.max(np.abs(dq - _fd(f, q))) < 1e-8
    assert np.max(np.abs(dk - _fd(f, k))) < 1e-8


def test_dsink_uniform_scores_closed_form():
    """Q = 0: O_i = sum(V_vis)/(n_i + e^s) and dSink = -sum_i e^s/(n_i + e^s) <dO_i, O_i>."""
    rng = np.random.default_rng(22)
    S, D = 9, 4
    q = np.zeros((1, S, 1, D))
    k = rng.standard_normal((1, S, 1, D))
    v = rng.standard_normal((1, S, 1, D))
    dout = rng.standard_normal((1, S, 1, D))
    sink = np.array([0.7])
    _, _, _, dsink, o, _ = oracle.backward(q, k, v, sink, dout, 0.125, True)
    expect = 0.0
    for i in range(S):
        n = i + 1
        oi = v[0, :n, 0].sum(axis=0) / (n + math.exp(0.7))
        expect -= math.exp(0.7) / (n + math.exp(0.7)) * float(dout[0, i, 0] @ oi)
    assert abs(dsink[0] - expect) < 1e-12


def test_dsink_row_blocking_invariant():
    """Row blocking of the oracle does not change any gradient."""
    rng = np.random.default_rng(23)
    q = rng.standard_normal((2, 7, 4, 3))
    k = rng.standard_normal((2, 7, 2, 3))
    v = rng.standard_normal((2, 7, 2, 3))
    dout = rng.standard_normal((2, 7, 4, 3))
    sink = rng.standard_normal(4)
    a = oracle.backward(q, k, v, sink, dout, 0.5, True, None, row_block=1024)
    b = oracle.backward(q, k, v, sink, dout, 0.5, True, None, row_block=3)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < 1e-12

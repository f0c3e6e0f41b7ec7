"""Pins for the oracle's front end (CPU only): the short causal convolution on
q, k, v and the low-rank decay gate ("Kimi K3: The Manos, The Mythos, The
Legendos", stability-details bullet).  Each check is fixed by the definition of
a causal FIR filter or of softplus / SiLU, not by the oracle's own code:
identity and delay filters, the impulse response, sequence isolation, exact
continuation from a saved state, and closed-form values of the logistic
family."""

import numpy as np
import pytest


def test_width_one_unit_filter_is_identity(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((20, 3, 8))
    y, fin = oracle.short_conv(x, np.ones((3, 8, 1)))
    np.testing.assert_array_equal(y, x)
    assert fin.shape == (1, 0, 3, 8)


@pytest.mark.parametrize("tap", [0, 1, 2, 3])
def test_one_hot_tap_is_a_delay(oracle, tap):
    """weight e_tap over W = 4 taps delays by 3 - tap tokens, zero-filled at the
    sequence start without a state and filled from the state with one."""
    rng = np.random.default_rng(2 + tap)
    T, H, d, W = 17, 2, 4, 4
    x = rng.standard_normal((T, H, d))
    w = np.zeros((H, d, W))
    w[:, :, tap] = 1.0
    lag = W - 1 - tap
    y, _ = oracle.short_conv(x, w)
    expect = np.zeros_like(x)
    expect[lag:] = x[:T - lag]
    np.testing.assert_array_equal(y, expect)
    st = rng.standard_normal((1, W - 1, H, d))
    y2, _ = oracle.short_conv(x, w, state=st)
    ext = np.concatenate([st[0], x])
    np.testing.assert_array_equal(y2, ext[W - 1 - lag:W - 1 - lag + T])


def test_impulse_response_is_the_reversed_filter(oracle):
    rng = np.random.default_rng(6)
    H, d, W = 2, 5, 4
    w = rng.standard_normal((H, d, W))
    x = np.zeros((9, H, d))
    x[0] = 1.0
    y, _ = oracle.short_conv(x, w)
    for t in range(W):
        np.testing.assert_array_equal(y[t], w[:, :, W - 1 - t])
    np.testing.assert_array_equal(y[W:], 0.0)


def test_packed_sequences_do_not_leak(oracle):
    rng = np.random.default_rng(7)
    lens = [5, 1, 0, 9, 2]
    H, d, W = 2, 3, 4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, W))
    st = rng.standard_normal((len(lens), W - 1, H, d))
    y, fin = oracle.short_conv(x, w, cu_seqlens=cu, state=st)
    for n in range(len(lens)):
        yn, fn = oracle.short_conv(x[cu[n]:cu[n + 1]], w, state=st[n:n + 1])
        np.testing.assert_array_equal(y[cu[n]:cu[n + 1]], yn)
        np.testing.assert_array_equal(fin[n], fn[0])
    # an empty sequence passes its state through
    np.testing.assert_array_equal(fin[2], st[2])


@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_continuation_from_the_final_state(oracle, split):
    """Running [0, split) then [split, T) from the first part's final state is
    running [0, T) (splits shorter than W - 1 carry state rows through)."""
    rng = np.random.default_rng(10 + split)
    T, H, d, W = 12, 2, 4, 4
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, W))
    st = rng.standard_normal((1, W - 1, H, d))
    y, fin = oracle.short_conv(x, w, state=st)
    y1, f1 = oracle.short_conv(x[:split], w, state=st)
    y2, f2 = oracle.short_conv(x[split:], w, state=f1)
    np.testing.assert_array_equal(np.concatenate([y1, y2]), y)
    np.testing.assert_array_equal(f2, fin)
    np.testing.assert_array_equal(fin[0], x[T - (W - 1):])


def test_silu_closed_forms(oracle):
    # width-1 unit filter, so y = silu(x): silu(0) = 0, silu(ln 3) = (3/4) ln 3,
    # silu(x) - silu(-x) = x
    xs = np.array([0.0, np.log(3.0), 1.7, -1.7, 30.0, -30.0]).reshape(6, 1, 1)
    y, _ = oracle.short_conv(xs, np.ones((1, 1, 1)), silu=True)
    y = y[:, 0, 0]
    assert y[0] == 0.0
    np.testing.assert_allclose(y[1], 0.75 * np.log(3.0), rtol=1e-15)
    np.testing.assert_allclose(y[2] - y[3], 1.7, rtol=1e-15)
    np.testing.assert_allclose(y[4], 30.0, rtol=1e-12)
    assert abs(y[5]) < 1e-11


def test_gate_closed_forms(oracle):
    H, dk, r = 2, 3, 4
    # a = 0: g = -softplus(bias); softplus(0) = ln 2, softplus(ln(e - 1)) = 1
    a = np.zeros((2, r))
    b = np.ones((H, dk, r))
    bias = np.zeros((H, dk))
    bias[1, 2] = np.log(np.e - 1.0)
    g = oracle.low_rank_gate(a, b, bias)
    np.testing.assert_allclose(g[:, 0, 0], -np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(g[:, 1, 2], -1.0, rtol=1e-15)
    # softplus(z) - softplus(-z) = z, and g < 0 with g -> -z for large z
    rng = np.random.default_rng(20)
    a = rng.standard_normal((5, r))
    b = rng.standard_normal((H, dk, r))
    gp, gm = oracle.low_rank_gate(a, b), oracle.low_rank_gate(a, -b)
    z = np.zeros((5, H, dk))
    for j in range(r):
        z += a[:, j][:, None, None] * b[None, :, :, j]
    np.testing.assert_allclose(gm - gp, z, rtol=1e-12, atol=1e-13)
    assert np.all(gp < 0) and np.all(gm < 0)
    g_big = oracle.low_rank_gate(np.full((1, 1), 40.0), np.ones((1, 1, 1)))
    np.testing.assert_allclose(g_big, -40.0, rtol=1e-15)


def test_gate_projection_brute_force(oracle):
    """The rank-r product written as explicit sums over the rank index."""
    rng = np.random.default_rng(21)
    T, H, dk, r = 3, 2, 4, 5
    a = rng.standard_normal((T, r))
    b = rng.standard_normal((H, dk, r))
    bias = rng.standard_normal((H, dk))
    g = oracle.low_rank_gate(a, b, bias)
    for t in range(T):
        for h in range(H):
            for c in range(dk):
                z = bias[h, c]
                for j in range(r):
                    z += a[t, j] * b[h, c, j]
                np.testing.assert_allclose(g[t, h, c], -np.log1p(np.exp(z)), rtol=1e-13)

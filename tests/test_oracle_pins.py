"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something fixed outside it: a worked
example derived by hand, a closed form, a special case that reduces to a
textbook operation (causal linear attention), an invariant of the recurrence,
or brute force (the explicit O(T^2) unrolling with matrix products).  Between
them a dropped term, a wrong sign, a transposed operand, the decay on the
wrong axis or at the wrong time, or output read before the write fails at
least one test; test_oracle_mutations.py checks that claim by planting such
mistakes in a copy of the oracle.

The recurrence: "From KV Cache to Depth Attention: The Bottlenecks Kimi K3 Had
to Break", Technical Details, Kimi Delta Attention bullet; "Kimi K3: The Manos,
The Mythos, The Legendos", bullets on KDA as online learning.
"""

import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_case(rng, T, H, dk, dv, g_scale=0.5, unit=True):
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((T, H, dk)))) * g_scale).astype(np.float32)
    return q, k, v, g, beta


def unit(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True))


# ---------------------------------------------------------------- worked example
def test_hand_worked_example(oracle):
    """Three tokens computed by hand (tests/golden/hand_example_dk2_dv3.json)."""
    with open(os.path.join(HERE, "golden", "hand_example_dk2_dv3.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], np.float32)[:, None, :]
    k = np.array(ex["k"], np.float32)[:, None, :]
    v = np.array(ex["v"], np.float32)[:, None, :]
    g = np.array(ex["g"], np.float32)[:, None, :]
    beta = np.array(ex["beta"], np.float32)[:, None]
    out, fin = oracle.prefill(q, k, v, g, beta, eps=ex["eps"], l2norm=ex["l2norm"])
    tol = ex["tolerance"]
    np.testing.assert_allclose(out[:, 0, :], np.array(ex["expected_out"]), atol=tol, rtol=0)
    np.testing.assert_allclose(fin[0, 0], np.array(ex["expected_final_state"]), atol=tol,
                               rtol=0)
    # the same three tokens as three decode steps
    st = np.zeros((1, 1, 2, 3))
    for t in range(3):
        o = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                               beta[t:t + 1], st, eps=ex["eps"], l2norm=ex["l2norm"])
        np.testing.assert_allclose(o[0, 0], np.array(ex["expected_out"][t]), atol=tol, rtol=0)
    np.testing.assert_allclose(st[0, 0], np.array(ex["expected_final_state"]), atol=tol, rtol=0)


# ---------------------------------------------------------------- P1 delta write
def test_p1_delta_write_recalls_value(oracle):
    """g=0, beta=1, unit key: after the step the memory returns exactly v for k
    ("predict, then write only the difference")."""
    rng = np.random.default_rng(1)
    dk, dv = 5, 3
    s0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32)
    q, k, v, g, beta = rand_case(rng, 1, 1, dk, dv)
    g[:] = 0
    beta[:] = 1
    _, fin = oracle.prefill(q, k, v, g, beta, initial_state=s0, eps=0.0)
    kb = unit(k[0, 0])
    np.testing.assert_allclose(fin[0, 0].T @ kb, v[0, 0].astype(np.float64), atol=1e-12, rtol=0)
    # and the rest of the memory is untouched: directions orthogonal to k keep S0
    P = np.eye(dk) - np.outer(kb, kb)
    np.testing.assert_allclose(P @ fin[0, 0], P @ s0[0, 0].astype(np.float64), atol=1e-12,
                               rtol=0)


# ---------------------------------------------------------------- P2 no-op
def test_p2_beta0_g0_is_identity(oracle):
    rng = np.random.default_rng(2)
    T, H, dk, dv = 10, 2, 4, 3
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    g[:] = 0
    beta[:] = 0
    s0 = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    out, fin = oracle.prefill(q, k, v, g, beta, initial_state=s0)
    assert np.array_equal(fin, s0.astype(np.float64))
    qb = q.astype(np.float64) / np.sqrt((q.astype(np.float64) ** 2).sum(-1, keepdims=True)
                                        + oracle.EPS)
    expect = np.einsum("thi,hij->thj", qb, s0[0].astype(np.float64))
    np.testing.assert_allclose(out, expect, atol=1e-13, rtol=0)


# ---------------------------------------------------------------- P3 pure retention
def test_p3_beta0_pure_channel_decay(oracle):
    """beta=0: the state decays row-wise (key channel i) by exp(sum_t g_t[i])."""
    rng = np.random.default_rng(3)
    T, H, dk, dv = 37, 3, 6, 4
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv, g_scale=1.0)
    beta[:] = 0
    s0 = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    _, fin = oracle.prefill(q, k, v, g, beta, initial_state=s0)
    decay = np.exp(g.astype(np.float64).sum(axis=0))          # [H, dk]
    expect = decay[:, :, None] * s0[0].astype(np.float64)
    np.testing.assert_allclose(fin[0], expect, rtol=1e-13, atol=0)


def test_complete_forgetting_keeps_only_the_current_write(oracle):
    """A retention of zero in every channel (g = -inf; also g = -1000, whose
    exp underflows to exactly 0 in fp64) wipes the memory before each write, so
    S_t = beta_t kb_t v_t^T and o_t = beta_t (qb_t . kb_t) v_t exactly: the
    predict-then-write step sees an empty memory.  Channels forget on their own
    timescales ("From KV Cache to Depth Attention: The Bottlenecks Kimi K3 Had
    to Break", Technical Details, KDA bullet); this is the limit of a channel
    that keeps nothing."""
    rng = np.random.default_rng(12)
    T, H, dk, dv = 7, 2, 6, 4
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    for gval in (-np.inf, -1000.0):
        g[:] = gval
        out, fin = oracle.prefill(q, k, v, g, beta, initial_state=s0, eps=0.0)
        qb, kb = unit(q), unit(k)
        want_o = (beta * (qb * kb).sum(-1))[..., None] * v.astype(np.float64)
        np.testing.assert_allclose(out, want_o, atol=1e-13, rtol=0)
        want_s = beta[-1, :, None, None] * kb[-1][:, :, None] * v[-1].astype(np.float64)[:, None, :]
        np.testing.assert_allclose(fin[0], want_s, atol=1e-13, rtol=0)


# ---------------------------------------------------------------- P4 order sensitivity
def test_p4_token_order_matters(oracle):
    """Processing A->B->C and C->B->A gives different states."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 16, 2, 8, 8
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    _, f1 = oracle.prefill(q, k, v, g, beta)
    r = slice(None, None, -1)
    _, f2 = oracle.prefill(q[r], k[r], v[r], g[r], beta[r])
    assert np.abs(f1 - f2).max() > 1e-3
    perm = rng.permutation(T)
    _, f3 = oracle.prefill(q[perm], k[perm], v[perm], g[perm], beta[perm])
    assert np.abs(f1 - f3).max() > 1e-3


# ---------------------------------------------------------------- P5 brute force
@pytest.mark.parametrize("seed,T,dk,dv", [(5, 12, 4, 3), (6, 16, 8, 5), (7, 1, 3, 2)])
def test_p5_matches_explicit_unrolling(oracle, seed, T, dk, dv):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = rand_case(rng, T, 1, dk, dv, g_scale=1.0)
    s0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32)
    out, fin = oracle.prefill(q, k, v, g, beta, initial_state=s0, scale=0.7)
    o_n, st_n = oracle.naive_expansion(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0],
                                       initial_state=s0[0, 0], scale=0.7)
    np.testing.assert_allclose(out[:, 0], o_n, atol=1e-12, rtol=0)
    np.testing.assert_allclose(fin[0, 0], st_n[-1], atol=1e-12, rtol=0)


# ---------------------------------------------------------------- P6 linear attention
def test_p6_orthonormal_keys_reduce_to_causal_linear_attention(oracle):
    """Distinct basis keys, g=0, S0=0: nothing interferes, so the delta rule is
    plain causal linear attention: o_t = sum_{s<=t} beta_s (q_t . k_s) v_s."""
    rng = np.random.default_rng(6)
    T, dk, dv = 6, 8, 5
    idx = rng.permutation(dk)[:T]
    k = np.zeros((T, 1, dk), np.float32)
    k[np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((T, 1, dk)).astype(np.float32)
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (T, 1)).astype(np.float32)
    g = np.zeros((T, 1, dk), np.float32)
    out, fin = oracle.prefill(q, k, v, g, beta, eps=0.0)
    qb = unit(q[:, 0])
    kk, vv, bb = k[:, 0].astype(np.float64), v[:, 0].astype(np.float64), beta[:, 0]
    for t in range(T):
        expect = sum(bb[s] * (qb[t] @ kk[s]) * vv[s] for s in range(t + 1))
        np.testing.assert_allclose(out[t, 0], expect, atol=1e-13, rtol=0)
    np.testing.assert_allclose(fin[0, 0], sum(bb[s] * np.outer(kk[s], vv[s]) for s in range(T)),
                               atol=1e-13, rtol=0)


# ---------------------------------------------------------------- P7 repeated key
@pytest.mark.parametrize("b", [0.3, 0.8])
def test_p7a_repeated_key_converges_without_stacking(oracle, b):
    """Same unit key and value n times, g=0: S^T k = (1-(1-b)^n) v -- the write
    corrects towards v instead of stacking n copies."""
    n, dk, dv = 9, 4, 3
    rng = np.random.default_rng(7)
    kvec = unit(rng.standard_normal(dk)).astype(np.float32)
    vvec = rng.standard_normal(dv).astype(np.float32)
    k = np.tile(kvec, (n, 1, 1))
    v = np.tile(vvec, (n, 1, 1))
    q = k.copy()
    g = np.zeros((n, 1, dk), np.float32)
    beta = np.full((n, 1), b, np.float32)
    _, fin = oracle.prefill(q, k, v, g, beta, eps=0.0)
    kb = unit(kvec)
    bf = float(np.float32(b))
    np.testing.assert_allclose(fin[0, 0].T @ kb, (1 - (1 - bf) ** n) * vvec.astype(np.float64),
                               atol=1e-12, rtol=0)


def test_p7b_scalar_gate_geometric_series(oracle):
    """Uniform g over channels (the scalar forget gate): with a repeated unit
    key, m_n = S_n^T k obeys m_n = rho m_{n-1} + b v, rho = (1-b) e^g, so
    m_n = b v (1 - rho^n) / (1 - rho)."""
    n, dk, dv = 11, 5, 2
    rng = np.random.default_rng(8)
    kvec = unit(rng.standard_normal(dk)).astype(np.float32)
    vvec = rng.standard_normal(dv).astype(np.float32)
    b, gv = np.float32(0.6), np.float32(-0.3)
    k = np.tile(kvec, (n, 1, 1))
    v = np.tile(vvec, (n, 1, 1))
    g = np.full((n, 1, dk), gv, np.float32)
    beta = np.full((n, 1), b, np.float32)
    _, fin = oracle.prefill(k, k, v, g, beta, eps=0.0)
    rho = (1 - float(b)) * np.exp(float(gv))
    expect = float(b) * vvec.astype(np.float64) * (1 - rho ** n) / (1 - rho)
    np.testing.assert_allclose(fin[0, 0].T @ unit(kvec), expect, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- P8 bounded growth
def test_p8_norm_growth_bounded_by_the_write(oracle):
    """||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||: I - b k k^T (0<=b<=1, unit k)
    and Diag(alpha<=1) are non-expansive."""
    rng = np.random.default_rng(9)
    T, H, dk, dv = 40, 2, 8, 6
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    st = rng.standard_normal((1, H, dk, dv))
    for t in range(T):
        before = np.linalg.norm(st, axis=(2, 3))
        oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], st)
        after = np.linalg.norm(st, axis=(2, 3))
        bound = before + beta[t][None, :] * np.linalg.norm(v[t].astype(np.float64), axis=-1)
        assert np.all(after <= bound + 1e-12)


# ---------------------------------------------------------------- P9 fixed size
def test_p9_state_size_independent_of_length(oracle):
    rng = np.random.default_rng(10)
    for T in (1, 7, 130):
        q, k, v, g, beta = rand_case(rng, T, 2, 4, 3)
        _, fin = oracle.prefill(q, k, v, g, beta)
        assert fin.shape == (1, 2, 4, 3)


# ---------------------------------------------------------------- P10 chunk algebra
@pytest.mark.parametrize("chunk", [1, 2, 16, 64, 1000])
def test_p10_chunk_form_equals_recurrence(oracle, chunk):
    rng = np.random.default_rng(11)
    lens = [130, 64, 1, 77]
    T = sum(lens)
    H, dk, dv = 2, 8, 6
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv, g_scale=1.0)
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    o1, f1 = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0)
    o2, f2 = oracle.chunked(q, k, v, g, beta, chunk, cu_seqlens=cu, initial_state=s0)
    np.testing.assert_allclose(o2, o1, atol=1e-11, rtol=0)
    np.testing.assert_allclose(f2, f1, atol=1e-11, rtol=0)


def test_p10_chunk_form_strong_decay(oracle):
    """Strong per-channel decay inside a 64-token chunk (exp(-gamma) far beyond
    1e20): the chunk form with direct exponentials of differences stays exact."""
    rng = np.random.default_rng(12)
    T, H, dk, dv = 64, 1, 8, 4
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    g = (g * 6.0).astype(np.float32)
    o1, f1 = oracle.prefill(q, k, v, g, beta)
    o2, f2 = oracle.chunked(q, k, v, g, beta, 64)
    np.testing.assert_allclose(o2, o1, atol=1e-11, rtol=0)
    np.testing.assert_allclose(f2, f1, atol=1e-11, rtol=0)


# ---------------------------------------------------------------- boundaries / options
def test_varlen_packing_equals_separate_runs(oracle):
    """Sequences in one packed call do not see each other: each starts from its
    own initial state."""
    rng = np.random.default_rng(13)
    lens = [5, 0, 9, 3]
    H, dk, dv = 2, 4, 3
    T = sum(lens)
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, fin = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            np.testing.assert_array_equal(fin[n], s0[n].astype(np.float64))
            continue
        o_n, f_n = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                  initial_state=s0[n:n + 1])
        np.testing.assert_array_equal(out[a:b], o_n)
        np.testing.assert_array_equal(fin[n], f_n[0])


def test_null_initial_state_is_zero(oracle):
    rng = np.random.default_rng(14)
    q, k, v, g, beta = rand_case(rng, 9, 2, 4, 4)
    o1, f1 = oracle.prefill(q, k, v, g, beta)
    o2, f2 = oracle.prefill(q, k, v, g, beta, initial_state=np.zeros((1, 2, 4, 4), np.float32))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_l2norm_makes_qk_scale_free_and_scale_is_linear(oracle):
    rng = np.random.default_rng(15)
    q, k, v, g, beta = rand_case(rng, 20, 2, 6, 5)
    o1, f1 = oracle.prefill(q, k, v, g, beta, eps=0.0)
    # power-of-two factors keep the float32 inputs exact
    o2, f2 = oracle.prefill(q * 4.0, k * 0.25, v, g, beta, eps=0.0)
    np.testing.assert_allclose(o2, o1, atol=1e-12, rtol=0)
    np.testing.assert_allclose(f2, f1, atol=1e-12, rtol=0)
    o3, f3 = oracle.prefill(q, k, v, g, beta, eps=0.0, scale=0.5)
    np.testing.assert_allclose(o3, 0.5 * o1, atol=1e-13, rtol=0)
    np.testing.assert_array_equal(f3, f1)


def test_decode_steps_equal_prefill(oracle):
    rng = np.random.default_rng(16)
    T, H, dk, dv = 12, 3, 5, 4
    q, k, v, g, beta = rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    out, fin = oracle.prefill(q, k, v, g, beta, initial_state=s0)
    st = s0.astype(np.float64).copy()
    for t in range(T):
        o = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], st)
        np.testing.assert_array_equal(o[0], out[t])
    np.testing.assert_array_equal(st, fin)


def test_thread_count_does_not_change_results(oracle):
    rng = np.random.default_rng(17)
    lens = [33, 70, 5]
    q, k, v, g, beta = rand_case(rng, sum(lens), 3, 8, 8)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o1, f1 = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, threads=1)
    o2, f2 = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, threads=5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


# ---------------------------------------------------------------- output gate
# The output forget gate ("Kimi K3: The Manos, The Mythos, The Legendos",
# stability-details bullet), read as out * sigmoid(z).  Pinned by values of the
# logistic function that follow from its definition alone.

def test_output_gate_closed_form_values(oracle):
    rng = np.random.default_rng(31)
    o = rng.standard_normal((5, 3, 4))
    # sigmoid(0) = 1/2 and sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4, per head
    np.testing.assert_allclose(oracle.apply_output_gate(o, np.zeros((5, 3))), 0.5 * o,
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.apply_output_gate(o, np.full((5, 3), np.log(3.0))),
                               0.75 * o, rtol=1e-14, atol=1e-15)
    # a strongly open gate passes the read-out, a strongly closed one blocks it
    np.testing.assert_allclose(oracle.apply_output_gate(o, np.full((5, 3), 40.0)), o,
                               rtol=1e-15, atol=0)
    assert np.abs(oracle.apply_output_gate(o, np.full((5, 3), -40.0))).max() < 1e-17


def test_output_gate_complement_and_broadcast(oracle):
    rng = np.random.default_rng(32)
    o = rng.standard_normal((6, 2, 5))
    z = rng.standard_normal((6, 2, 5)) * 3
    # sigmoid(z) + sigmoid(-z) = 1
    np.testing.assert_allclose(oracle.apply_output_gate(o, z) + oracle.apply_output_gate(o, -z),
                               o, rtol=1e-14, atol=1e-14)
    # per channel: channel c is scaled by its own gate only
    for c in range(5):
        np.testing.assert_allclose(oracle.apply_output_gate(o, z)[..., c],
                                   oracle.apply_output_gate(o[..., c:c + 1], z[..., c:c + 1])[..., 0],
                                   rtol=0, atol=0)
    # a per-head z equals the same value repeated over the channels
    zh = rng.standard_normal((6, 2))
    np.testing.assert_array_equal(oracle.apply_output_gate(o, zh),
                                  oracle.apply_output_gate(o, np.repeat(zh[..., None], 5, -1)))
    # monotone in z
    a = oracle.apply_output_gate(np.ones((1, 1, 1)), np.full((1, 1, 1), 0.3))
    b = oracle.apply_output_gate(np.ones((1, 1, 1)), np.full((1, 1, 1), 0.4))
    assert 0.5 < a[0, 0, 0] < b[0, 0, 0] < 1.0

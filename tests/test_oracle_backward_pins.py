"""Pins for the oracle's gradients (oracle.backward): checked against the
forward oracle by central finite differences, against gradients worked out
by hand, and against properties every vector-Jacobian product has.

The loss is L = sum(W_o * o) + sum(W_S * S_final) for fixed weights, so
dL/do = W_o and dL/dS_final = W_S.  A slip in the reverse recurrence (a
missing decay on the carried gradient, dk without its read term, a sign of
the correction, dg taken against the undecayed state) fails the finite
differences on every input it touches.
"""

import math

import numpy as np
import pytest

import oracle


def _rand_case(rng, lengths, H, dk, dv, init_state=True):
    T = sum(lengths)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=2, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -5.0 * rng.random((T, H, dk))
    beta = rng.random((T, H))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S0 = rng.standard_normal((len(lengths), H, dk, dv)) if init_state else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu=cu, S0=S0)


def _loss(c, Wo, WS):
    o, Sf = oracle.recurrent(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], initial_state=c["S0"])
    return float(np.sum(Wo * o) + np.sum(WS * Sf))


def _grads(c, Wo, WS, interval=64):
    return oracle.backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], Wo, initial_state=c["S0"],
                           d_final_state=WS, interval=interval)


@pytest.mark.parametrize("interval", [2, 64])
def test_backward_matches_finite_differences(interval):
    rng = np.random.default_rng(11)
    c = _rand_case(rng, [5, 0, 3], H=2, dk=4, dv=3)
    T, H, dv = c["v"].shape
    Wo = rng.standard_normal((T, H, dv))
    WS = rng.standard_normal(c["S0"].shape)
    gr = _grads(c, Wo, WS, interval)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="d_initial_state")
    eps = 1e-6
    for name, gname in names.items():
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(c, Wo, WS)
            x[idx] = keep - eps
            lm = _loss(c, Wo, WS)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.abs(fd).max()))
        np.testing.assert_allclose(gr[gname], fd, rtol=0, atol=2e-7 * scale, err_msg=gname)


def test_backward_one_token_by_hand():
    # S0 = 0, one token: the decayed state is zero, so S = beta k v^T and
    # o = beta (k.q) v.  With q = (1,2), k = (0.6,0.8), v = (1,-1), beta = 1/2,
    # alpha = (1/2, 1), dL/do = w = (1, 1/2), dL/dS = M = [[0,1],[1,0]]:
    #   dq = beta (v.w) k                       = (0.15, 0.2)
    #   dk = beta (v.w) q + beta M v            = (-0.25, 1.0)
    #   dv = beta (k.q) w + beta M^T k          = (1.5, 0.85)
    #   dbeta = (k.q)(v.w) + k^T M v            = 1.3
    #   dg = 0 (it multiplies a zero state)
    #   dS0 = diag(alpha) (q w^T + M - beta k ((k.q) w + M^T k)^T) = [[0.05, 0.495], [1.8, 0.32]]
    q = np.array([[[1.0, 2.0]]])
    k = np.array([[[0.6, 0.8]]])
    v = np.array([[[1.0, -1.0]]])
    g = np.array([[[math.log(0.5), 0.0]]])
    beta = np.array([[0.5]])
    cu = np.array([0, 1], np.int32)
    gr = oracle.backward(q, k, v, g, beta, cu, np.array([[[1.0, 0.5]]]), initial_state=np.zeros((1, 1, 2, 2)),
                         d_final_state=np.array([[[[0.0, 1.0], [1.0, 0.0]]]]))
    np.testing.assert_allclose(gr["dq"][0, 0], [0.15, 0.2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(gr["dk"][0, 0], [-0.25, 1.0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(gr["dv"][0, 0], [1.5, 0.85], rtol=0, atol=1e-14)
    assert abs(gr["dbeta"][0, 0] - 1.3) < 1e-14
    np.testing.assert_allclose(gr["dg"][0, 0], [0.0, 0.0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(gr["d_initial_state"][0, 0], [[0.05, 0.495], [1.8, 0.32]], rtol=0, atol=1e-14)


def test_backward_scalar_case_by_hand():
    # d_k = d_v = 1: S = alpha s (1 - beta k^2) + beta k v, o = S q.  With s = 2,
    # alpha = 1/2, k = 1, beta = 1/2, v = 3, q = 1, dL/do = 1, dL/dS = 0:
    #   dL/dg = (1 - beta k^2) alpha s = 0.5,  dL/ds = alpha (1 - beta k^2) = 0.25,
    #   dL/dk = -2 beta k alpha s + beta v = 0.5,  dL/dv = beta k = 0.5,
    #   dL/dbeta = -k^2 alpha s + k v = 2,  dL/dq = S = 2
    one = lambda x: np.array([[[float(x)]]])
    gr = oracle.backward(one(1), one(1), one(3), one(math.log(0.5)), np.array([[0.5]]), np.array([0, 1], np.int32),
                         one(1), initial_state=np.array([[[[2.0]]]]))
    assert abs(gr["dg"][0, 0, 0] - 0.5) < 1e-14
    assert abs(gr["d_initial_state"][0, 0, 0, 0] - 0.25) < 1e-14
    assert abs(gr["dk"][0, 0, 0] - 0.5) < 1e-14
    assert abs(gr["dv"][0, 0, 0] - 0.5) < 1e-14
    assert abs(gr["dbeta"][0, 0] - 2.0) < 1e-14
    assert abs(gr["dq"][0, 0, 0] - 2.0) < 1e-14


def test_backward_is_linear_in_the_upstream_gradients():
    rng = np.random.default_rng(5)
    c = _rand_case(rng, [30, 7], H=2, dk=6, dv=5)
    T, H, dv = c["v"].shape
    W1, W2 = rng.standard_normal((2, T, H, dv))
    S1, S2 = rng.standard_normal((2,) + c["S0"].shape)
    g1, g2 = _grads(c, W1, S1), _grads(c, W2, S2)
    g3 = _grads(c, 2.0 * W1 - 3.0 * W2, 2.0 * S1 - 3.0 * S2)
    for name in g1:
        ref = 2.0 * g1[name] - 3.0 * g2[name]
        np.testing.assert_allclose(g3[name], ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()), err_msg=name)


def test_backward_does_not_depend_on_the_checkpoint_interval():
    rng = np.random.default_rng(9)
    c = _rand_case(rng, [70, 1, 0, 33], H=2, dk=8, dv=4)
    T, H, dv = c["v"].shape
    Wo = rng.standard_normal((T, H, dv))
    WS = rng.standard_normal(c["S0"].shape)
    a, b = _grads(c, Wo, WS, interval=1), _grads(c, Wo, WS, interval=16)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def test_backward_empty_sequence_passes_the_state_gradient_through():
    # a sequence of length 0: final state = initial state, so dS0 = dL/dS_final
    rng = np.random.default_rng(2)
    c = _rand_case(rng, [0, 4], H=1, dk=3, dv=2)
    T, H, dv = c["v"].shape
    WS = rng.standard_normal(c["S0"].shape)
    gr = _grads(c, np.zeros((T, H, dv)), WS)
    np.testing.assert_array_equal(gr["d_initial_state"][0], WS[0])


def test_start_state_gradient_is_sum_of_transported_queries():
    # The outputs of a sequence are affine in its start state: S_t = M_t S_0 + N_t,
    # with M_t the state reached from S_0 = I with v = 0 (the transition through
    # token t), so o_t = S_t^T q_t and, with dL/d(final state) = 0,
    #   dL/dS_0 = sum_t (M_t^T q_t) dO_t^T.
    # M_t^T q_t is the recurrence's own output from I with v = 0 (a d_k-column
    # state); the sum is checked against the oracle's reverse recurrence.
    rng = np.random.default_rng(23)
    c = _rand_case(rng, [7, 0, 12], H=2, dk=4, dv=3)
    T, H, dv = c["v"].shape
    dk = c["k"].shape[2]
    dO = rng.standard_normal((T, H, dv))
    gr = oracle.backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], dO, initial_state=c["S0"])
    eye = np.broadcast_to(np.eye(dk), (len(c["cu"]) - 1, H, dk, dk)).copy()
    qhat, _ = oracle.recurrent(c["q"], c["k"], np.zeros((T, H, dk)), c["g"], c["beta"], c["cu"], initial_state=eye)
    for n in range(len(c["cu"]) - 1):
        a, b = c["cu"][n], c["cu"][n + 1]
        for h in range(H):
            D = qhat[a:b, h].T @ dO[a:b, h]  # sum_t q^_t dO_t^T, d_k x d_v
            np.testing.assert_allclose(gr["d_initial_state"][n, h], D, rtol=1e-12, atol=1e-12)

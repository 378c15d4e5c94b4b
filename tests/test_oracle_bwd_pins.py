"""Pins of the oracle's backward (recurrence_bwd, chunked_bwd).

The gradient of the recurrence is fixed by the forward: these tests check the
reverse recurrence against central finite differences of the forward oracle,
against closed forms of the special cases the pages name, and the chunk-form
backward against the reverse recurrence.  Citation keys are those of
oracle/gdn2_oracle.py.  None of these tests needs a GPU.
"""

import numpy as np
import pytest

import oracle as O

NAMES = ("q", "k", "v", "log_alpha", "b", "w", "S0")
GRADS = dict(q="dq", k="dk", v="dv", log_alpha="dlog_alpha", b="db", w="dw", S0="dS0")


def _inputs(rng, B, T, H, Dk, Dv, b_range=(0.0, 1.0)):
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=rng.standard_normal((B, T, H, Dk)), k=k, v=rng.standard_normal((B, T, H, Dv)),
                log_alpha=rng.uniform(-0.5, -0.01, size=(B, T, H, Dk)),
                b=rng.uniform(*b_range, size=(B, T, H, Dk)), w=rng.uniform(0.0, 1.0, size=(B, T, H, Dv)))


def _loss(x, do, dSf, cu=None):
    o, S = O.recurrence(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x.get("S0"), cu)
    return float(np.sum(o * do) + (0.0 if dSf is None else np.sum(S * dSf)))


@pytest.mark.parametrize("case", ["dense", "varlen", "no_state"])
def test_bwd_matches_finite_differences(case):
    """Every gradient of recurrence_bwd equals a central difference of the
    forward oracle (the chain rule through the read/write step [iplexlaw,
    "Decisiones independientes en dos ejes"])."""
    rng = np.random.default_rng({"dense": 1, "varlen": 2, "no_state": 3}[case])
    cu = None
    if case == "varlen":
        cu = np.array([0, 5, 6, 14])
        x = _inputs(rng, 1, 14, 2, 4, 3, b_range=(0.0, 2.0))
        N = 3
    else:
        x = _inputs(rng, 2, 11, 2, 4, 3)
        N = 2
    if case != "no_state":
        x["S0"] = 0.3 * rng.standard_normal((N, 2, 4, 3))
    do = rng.standard_normal(x["v"].shape)
    dSf = None if case == "no_state" else rng.standard_normal((N, 2, 4, 3))
    g = O.recurrence_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], do,
                         x.get("S0"), dSf, cu)
    eps = 1e-6
    for name in NAMES:
        if name not in x:
            continue
        base = x[name]
        for idx in np.ndindex(*base.shape):
            if rng.random() > 0.25:        # a quarter of the entries, all of them over the run
                continue
            xp = dict(x); xp[name] = base.copy(); xp[name][idx] += eps
            xm = dict(x); xm[name] = base.copy(); xm[name][idx] -= eps
            fd = (_loss(xp, do, dSf, cu) - _loss(xm, do, dSf, cu)) / (2 * eps)
            assert abs(fd - g[GRADS[name]][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx)


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 8, 16])
def test_chunked_bwd_equals_recurrence_bwd(chunk):
    """The chunk-form backward (chain rule through the WY factors of [gist-3])
    gives the reverse recurrence's gradients, tails included."""
    rng = np.random.default_rng(10 + chunk)
    x = _inputs(rng, 2, 19, 2, 5, 4, b_range=(0.0, 2.0))
    S0 = 0.3 * rng.standard_normal((2, 2, 5, 4))
    do = rng.standard_normal(x["v"].shape)
    dSf = rng.standard_normal((2, 2, 5, 4))
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], do, S0, dSf)
    ref = O.recurrence_bwd(*args)
    got = O.chunked_bwd(*args, chunk=chunk)
    for name in ref:
        assert O.rel_max_err(got[name], ref[name]) < 1e-12, name


def test_chunked_bwd_varlen():
    rng = np.random.default_rng(21)
    cu = np.array([0, 3, 20, 21, 40])
    x = _inputs(rng, 1, 40, 2, 4, 4)
    S0 = 0.3 * rng.standard_normal((4, 2, 4, 4))
    do = rng.standard_normal(x["v"].shape)
    dSf = rng.standard_normal((4, 2, 4, 4))
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], do, S0, dSf)
    ref = O.recurrence_bwd(*args, cu_seqlens=cu)
    got = O.chunked_bwd(*args, cu_seqlens=cu, chunk=8)
    for name in ref:
        assert O.rel_max_err(got[name], ref[name]) < 1e-12, name


def test_bwd_decay_only_closed_form():
    """b = 0, w = 0 [gist-1: the gates' domains include 0]: S_t = Diag(gamma_t) S0
    with gamma_t = exp(sum_{s<=t} log alpha_s), so with do = 0 the gradients are
    dS0 = Diag(gamma_T) dS_final and, for every token, dlog_alpha_t[c] =
    sum_v dS_final[c, v] S_T[c, v].  dq, dk and dv vanish; the gates still get
    gradients: with G_t = Diag(gamma_T / gamma_t) dS_final and du_t = G_t^T k_t,
    dw_t = du_t * v_t and db_t = -(Diag(gamma_t) S0 du_t) * k_t."""
    rng = np.random.default_rng(30)
    x = _inputs(rng, 1, 9, 1, 4, 3)
    x["b"][:] = 0.0
    x["w"][:] = 0.0
    S0 = rng.standard_normal((1, 1, 4, 3))
    dSf = rng.standard_normal((1, 1, 4, 3))
    do = np.zeros(x["v"].shape)
    g = O.recurrence_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], do, S0, dSf)
    gamma_T = np.exp(x["log_alpha"][0, :, 0].sum(axis=0))
    S_T = gamma_T[:, None] * S0[0, 0]
    np.testing.assert_allclose(g["dS0"][0, 0], gamma_T[:, None] * dSf[0, 0], rtol=1e-13)
    for t in range(9):
        np.testing.assert_allclose(g["dlog_alpha"][0, t, 0], np.sum(dSf[0, 0] * S_T, axis=1),
                                   rtol=1e-12)
    for name in ("dq", "dk", "dv"):
        assert np.max(np.abs(g[name])) == 0.0
    gamma = np.exp(np.cumsum(x["log_alpha"][0, :, 0], axis=0))
    for t in range(9):
        kt, vt = x["k"][0, t, 0], x["v"][0, t, 0]
        du = ((gamma_T / gamma[t])[:, None] * dSf[0, 0]).T @ kt
        np.testing.assert_allclose(g["dw"][0, t, 0], du * vt, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["db"][0, t, 0], -((gamma[t][:, None] * S0[0, 0]) @ du) * kt,
                                   rtol=1e-12, atol=1e-14)


def test_bwd_linear_attention_closed_form():
    """alpha = 1, b = 0 [iplexlaw: without erase the update only writes]: o =
    tril(Q K^T) Z + Q S0 with Z = w * v, a plain matrix product, whose
    gradients (with S_T = S0 + K^T Z read against dS_final) are
    dQ = tril(dO Z^T) K + dO S0^T, dK = tril(dO Z^T)^T Q + Z dS_final^T,
    dZ = tril(Q K^T)^T dO + K dS_final, dv = w dZ, dw = v dZ, dS0 = Q^T dO + dS_final,
    and dlog_alpha_t[c] = sum_v S_{t-1}[c, v] (sum_{i>=t} q_i[c] do_i[v] + dSf[c, v])."""
    rng = np.random.default_rng(31)
    T, Dk, Dv = 7, 4, 3
    x = _inputs(rng, 1, T, 1, Dk, Dv)
    x["log_alpha"][:] = 0.0
    x["b"][:] = 0.0
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    dSf = rng.standard_normal((1, 1, Dk, Dv))
    do = rng.standard_normal(x["v"].shape)
    g = O.recurrence_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], do, S0, dSf)
    Q, K, V, Wg = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["w"][0, :, 0]
    dO = do[0, :, 0]
    Z = Wg * V
    L = np.tril(np.ones((T, T)))
    dQ = (L * (dO @ Z.T)) @ K + dO @ S0[0, 0].T
    dK = (L * (dO @ Z.T)).T @ Q + Z @ dSf[0, 0].T
    dZ = (L * (Q @ K.T)).T @ dO + K @ dSf[0, 0]
    np.testing.assert_allclose(g["dq"][0, :, 0], dQ, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dk"][0, :, 0], dK, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dv"][0, :, 0], Wg * dZ, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw"][0, :, 0], V * dZ, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dS0"][0, 0], Q.T @ dO + dSf[0, 0], rtol=1e-12, atol=1e-12)
    S_prev = S0[0, 0] + np.concatenate([np.zeros((1, Dk, Dv)),
                                        np.cumsum(K[:, :, None] * Z[:, None, :], axis=0)[:-1]])
    for t in range(T):
        rhs = Q[t:].T @ dO[t:] + dSf[0, 0]
        np.testing.assert_allclose(g["dlog_alpha"][0, t, 0], np.sum(S_prev[t] * rhs, axis=1),
                                   rtol=1e-12, atol=1e-12)

"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test states the passage it checks.  Citation keys are those of
oracle/gdn2_oracle.py.  None of these tests needs a GPU.
"""

import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, H, Dk, Dv, B=1, b_range=(0.0, 1.0), la_range=(-0.5, -0.01)):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    la = rng.uniform(*la_range, size=(B, T, H, Dk))
    b = rng.uniform(*b_range, size=(B, T, H, Dk))
    w = rng.uniform(0.0, 1.0, size=(B, T, H, Dv))
    return q, k, v, la, b, w


# ---------------------------------------------------------------------------
# Golden: hand-worked two-token example
# ---------------------------------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = line.split("=")
            vals[key.strip()] = np.array([float(x) for x in rhs.split()])
    return vals


def test_golden_hand_worked_two_tokens():
    """Fixture worked by hand from the read/write rule [iplexlaw]."""
    g = _read_golden("hand_worked_two_tokens.txt")
    S = g["S0"].reshape(2, 2)
    for t in (1, 2):
        o, S = O.step(g[f"q_{t}"], g[f"k_{t}"], g[f"v_{t}"], np.log(g[f"alpha_{t}"]),
                      g[f"b_{t}"], g[f"w_{t}"], S)
        np.testing.assert_allclose(S.ravel(), g[f"S_{t}"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(o, g[f"o_{t}"], rtol=0, atol=1e-13)


def test_golden_through_recurrence_and_chunks():
    """The same fixture through the whole-sequence and chunked entry points."""
    g = _read_golden("hand_worked_two_tokens.txt")
    shp = (1, 2, 1, 2)
    q = np.stack([g["q_1"], g["q_2"]]).reshape(shp)
    k = np.stack([g["k_1"], g["k_2"]]).reshape(shp)
    v = np.stack([g["v_1"], g["v_2"]]).reshape(shp)
    la = np.log(np.stack([g["alpha_1"], g["alpha_2"]])).reshape(shp)
    b = np.stack([g["b_1"], g["b_2"]]).reshape(shp)
    w = np.stack([g["w_1"], g["w_2"]]).reshape(shp)
    S0 = g["S0"].reshape(1, 1, 2, 2)
    for fn in (O.recurrence, lambda *a, **kw: O.chunked(*a, chunk=2, **kw),
               lambda *a, **kw: O.chunked(*a, chunk=1, **kw)):
        o, S = fn(q, k, v, la, b, w, S0=S0)
        np.testing.assert_allclose(o[0, :, 0], np.stack([g["o_1"], g["o_2"]]), atol=1e-12)
        np.testing.assert_allclose(S.ravel(), g["S_2"], atol=1e-12)


# ---------------------------------------------------------------------------
# P1: read/write form equals the matrix form printed on two other pages
# ---------------------------------------------------------------------------

def test_p1_matrix_form():
    """[iplexlaw] read/write form == [gist-1]/[zubnet-1] matrix form."""
    rng = np.random.default_rng(1)
    Dk, Dv = 6, 5
    S = rng.standard_normal((Dk, Dv))
    for _ in range(8):
        q, k, v, la, b, w = (x[0, 0, 0] for x in _rand_inputs(rng, 1, 1, Dk, Dv))
        o, S_new = O.step(q, k, v, la, b, w, S)
        D = np.diag(np.exp(la))
        S_mat = (np.eye(Dk) - np.outer(k, b * k)) @ D @ S + np.outer(k, w * v)
        np.testing.assert_allclose(S_new, S_mat, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o, S_mat.T @ q, rtol=0, atol=1e-14)
        S = S_new


# ---------------------------------------------------------------------------
# P2/P3: reductions to KDA, Gated DeltaNet and DeltaNet
# ---------------------------------------------------------------------------

def test_p2_reduces_to_kda():
    """b = w = beta * 1 gives KDA's update (I - beta k k^T) Diag(alpha) S + beta k v^T
    [gist-1, reductions; iplexlaw, same section]."""
    rng = np.random.default_rng(2)
    Dk, Dv = 5, 4
    S = rng.standard_normal((Dk, Dv))
    S_kda = S.copy()
    for _ in range(10):
        q, k, v, la, _, _ = (x[0, 0, 0] for x in _rand_inputs(rng, 1, 1, Dk, Dv))
        beta = rng.uniform()
        o, S = O.step(q, k, v, la, np.full(Dk, beta), np.full(Dv, beta), S)
        S_kda = (np.eye(Dk) - beta * np.outer(k, k)) @ np.diag(np.exp(la)) @ S_kda \
            + beta * np.outer(k, v)
        np.testing.assert_allclose(S, S_kda, atol=1e-13)
        np.testing.assert_allclose(o, S_kda.T @ q, atol=1e-13)


def test_p3_reduces_to_gated_deltanet_and_deltanet():
    """Scalar decay too gives Gated DeltaNet S = alpha (I - beta k k^T) S + beta k v^T;
    alpha = 1 gives DeltaNet in its error-correction form
    S = S - beta k (S^T k - v)^T  [gist-1; iplexlaw]."""
    rng = np.random.default_rng(3)
    Dk, Dv = 5, 4
    S = rng.standard_normal((Dk, Dv))
    S_gdn = S.copy()
    for _ in range(10):
        q, k, v, _, _, _ = (x[0, 0, 0] for x in _rand_inputs(rng, 1, 1, Dk, Dv))
        beta, a = rng.uniform(), rng.uniform(0.5, 1.0)
        o, S = O.step(q, k, v, np.full(Dk, np.log(a)), np.full(Dk, beta), np.full(Dv, beta), S)
        S_gdn = a * (np.eye(Dk) - beta * np.outer(k, k)) @ S_gdn + beta * np.outer(k, v)
        np.testing.assert_allclose(S, S_gdn, atol=1e-13)
    S_dn = S.copy()
    for _ in range(10):
        q, k, v, _, _, _ = (x[0, 0, 0] for x in _rand_inputs(rng, 1, 1, Dk, Dv))
        beta = rng.uniform()
        o, S = O.step(q, k, v, np.zeros(Dk), np.full(Dk, beta), np.full(Dv, beta), S)
        S_dn = S_dn - beta * np.outer(k, S_dn.T @ k - v)
        np.testing.assert_allclose(S, S_dn, atol=1e-13)
        np.testing.assert_allclose(o, S_dn.T @ q, atol=1e-13)


# ---------------------------------------------------------------------------
# P4: linear attention closed form
# ---------------------------------------------------------------------------

def test_p4_linear_attention_closed_form():
    """alpha = 1 and b = 0 leave plain linear attention with a write gate:
    O = Q S0 + tril(Q K^T) (W*V) (diagonal included, the query reads the
    updated state [iplexlaw]) and S_T = S0 + K^T (W*V)."""
    rng = np.random.default_rng(4)
    T, H, Dk, Dv = 13, 2, 6, 5
    q, k, v, _, _, w = _rand_inputs(rng, T, H, Dk, Dv)
    la = np.zeros_like(q)
    b = np.zeros_like(q)
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, S = O.recurrence(q, k, v, la, b, w, S0=S0)
    for h in range(H):
        Q, K, Z = q[0, :, h], k[0, :, h], (w * v)[0, :, h]
        np.testing.assert_allclose(o[0, :, h], Q @ S0[0, h] + np.tril(Q @ K.T) @ Z, atol=1e-12)
        np.testing.assert_allclose(S[0, h], S0[0, h] + K.T @ Z, atol=1e-12)


# ---------------------------------------------------------------------------
# P5: exact retrieval
# ---------------------------------------------------------------------------

def test_p5_exact_retrieval_orthonormal_keys():
    """Orthonormal keys with b = 1, alpha = 1, w = 1: every stored value is read
    back exactly, and rewriting a key replaces its value."""
    rng = np.random.default_rng(5)
    Dk, Dv = 8, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm.T                                   # rows orthonormal
    vals = rng.standard_normal((Dk, Dv))
    S = rng.standard_normal((Dk, Dv))             # arbitrary prior content
    one_k, one_v, zero = np.ones(Dk), np.ones(Dv), np.zeros(Dk)
    for i in range(Dk):
        _, S = O.step(keys[i], keys[i], vals[i], zero, one_k, one_v, S)
    for i in range(Dk):
        np.testing.assert_allclose(S.T @ keys[i], vals[i], atol=1e-12)
    new = rng.standard_normal(Dv)
    o, S = O.step(keys[3], keys[3], new, zero, one_k, one_v, S)
    np.testing.assert_allclose(o, new, atol=1e-12)
    for i in range(Dk):
        np.testing.assert_allclose(S.T @ keys[i], new if i == 3 else vals[i], atol=1e-12)


def test_p5_one_step_write_is_read_back():
    """b = 1 and |k| = 1: after the step the state returns w*v for key k, for any
    decay and any prior state (the read is corrected to the gated target [gist-2]);
    with q = k the output is w*v."""
    rng = np.random.default_rng(6)
    Dk, Dv = 7, 5
    S = rng.standard_normal((Dk, Dv))
    for _ in range(10):
        _, k, v, la, _, w = (x[0, 0, 0] for x in _rand_inputs(rng, 1, 1, Dk, Dv))
        o, S = O.step(k, k, v, la, np.ones(Dk), w, S)
        np.testing.assert_allclose(S.T @ k, w * v, atol=1e-12)
        np.testing.assert_allclose(o, w * v, atol=1e-12)


# ---------------------------------------------------------------------------
# P6: decay only
# ---------------------------------------------------------------------------

def test_p6_decay_only():
    """b = 0 and w = 0: rows decay by exp(cumulative log alpha) [zubnet-1]."""
    rng = np.random.default_rng(7)
    T, H, Dk, Dv = 9, 2, 5, 4
    q, k, v, la, _, _ = _rand_inputs(rng, T, H, Dk, Dv)
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, S = O.recurrence(q, k, v, la, np.zeros_like(q), np.zeros_like(v), S0=S0)
    for h in range(H):
        G = np.cumsum(la[0, :, h], axis=0)
        for t in range(T):
            St = np.exp(G[t])[:, None] * S0[0, h]
            np.testing.assert_allclose(o[0, t, h], St.T @ q[0, t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], np.exp(G[-1])[:, None] * S0[0, h], atol=1e-12)


# ---------------------------------------------------------------------------
# P7: chunk (WY) algebra equals the recurrence
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 8, 16])
def test_p7_chunked_equals_recurrence(chunk):
    """The chunk form [gist-3] with an explicit (I+A)^-1, chunk sizes with
    ragged tails, nonzero initial state, equals the token recurrence."""
    rng = np.random.default_rng(100 + chunk)
    T, H, Dk, Dv = 16, 2, 6, 5
    q, k, v, la, b, w = _rand_inputs(rng, T - 1, H, Dk, Dv, B=2)  # T-1 = 15: ragged
    S0 = rng.standard_normal((2, H, Dk, Dv))
    o_r, S_r = O.recurrence(q, k, v, la, b, w, S0=S0)
    o_c, S_c = O.chunked(q, k, v, la, b, w, S0=S0, chunk=chunk)
    np.testing.assert_allclose(o_c, o_r, atol=1e-12)
    np.testing.assert_allclose(S_c, S_r, atol=1e-12)


def test_p7_chunk_factor_identities():
    """Internal identities of one chunk: (I + A) Tinv = I, A strictly lower,
    M lower with diagonal q_i . k_i, and the affine map of the chunk."""
    rng = np.random.default_rng(11)
    L, Dk, Dv = 12, 6, 5
    q, k, v, la, b, w = (x[0, :, 0] for x in _rand_inputs(rng, L, 1, Dk, Dv))
    f = O.chunk_factors(q, k, v, la, b, w)
    np.testing.assert_allclose((np.eye(L) + f["A"]) @ f["Tinv"], np.eye(L), atol=1e-13)
    assert np.all(np.triu(f["A"]) == 0)
    assert np.all(np.triu(f["M"], 1) == 0)
    np.testing.assert_allclose(np.diag(f["M"]), np.sum(q * k, axis=1), atol=1e-13)
    # brute force: A_ij over channels, written element by element
    g = np.cumsum(la, axis=0)
    for i in range(L):
        for j in range(i):
            ref = sum(b[i, c] * k[i, c] * k[j, c] * np.exp(g[i, c] - g[j, c]) for c in range(Dk))
            assert abs(f["A"][i, j] - ref) < 1e-13
    S_in = rng.standard_normal((Dk, Dv))
    _, S_out = O.chunk_apply(f, S_in)
    P, Qc = O.chunk_affine_map(f)
    np.testing.assert_allclose(S_out, P @ S_in + Qc, atol=1e-12)


def test_p7_padding_tokens_are_noops():
    """A token with k = 0 and log alpha = 0 leaves the state unchanged."""
    rng = np.random.default_rng(12)
    Dk, Dv = 5, 4
    S = rng.standard_normal((Dk, Dv))
    q = rng.standard_normal(Dk)
    _, S2 = O.step(q, np.zeros(Dk), rng.standard_normal(Dv), np.zeros(Dk),
                   rng.uniform(size=Dk), rng.uniform(size=Dv), S)
    np.testing.assert_array_equal(S2, S)


# ---------------------------------------------------------------------------
# P8: state passing
# ---------------------------------------------------------------------------

def test_p8_state_passing():
    """run(x1 || x2) == run(x2, S0 = run(x1).S_final)."""
    rng = np.random.default_rng(8)
    T1, T2, H, Dk, Dv = 7, 9, 2, 5, 4
    q, k, v, la, b, w = _rand_inputs(rng, T1 + T2, H, Dk, Dv)
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, S = O.recurrence(q, k, v, la, b, w, S0=S0)
    sl1 = (slice(None), slice(0, T1))
    sl2 = (slice(None), slice(T1, None))
    o1, S1 = O.recurrence(*(x[sl1] for x in (q, k, v, la, b, w)), S0=S0)
    o2, S2 = O.recurrence(*(x[sl2] for x in (q, k, v, la, b, w)), S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-12)
    np.testing.assert_allclose(S2, S, atol=1e-12)


def test_p8_varlen_equals_separate_calls():
    """A packed call equals separate calls per sequence, each with its own S0."""
    rng = np.random.default_rng(9)
    lens = [5, 1, 8, 3]
    H, Dk, Dv = 2, 4, 3
    Tt = sum(lens)
    q, k, v, la, b, w = _rand_inputs(rng, Tt, H, Dk, Dv)
    S0 = rng.standard_normal((len(lens), H, Dk, Dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = O.recurrence(q, k, v, la, b, w, S0=S0, cu_seqlens=cu)
    o_c, S_c = O.chunked(q, k, v, la, b, w, S0=S0, cu_seqlens=cu, chunk=4)
    np.testing.assert_allclose(o_c, o, atol=1e-12)
    np.testing.assert_allclose(S_c, S, atol=1e-12)
    for n in range(len(lens)):
        sl = (slice(None), slice(cu[n], cu[n + 1]))
        o_n, S_n = O.recurrence(*(x[sl] for x in (q, k, v, la, b, w)), S0=S0[n:n + 1])
        np.testing.assert_allclose(o[:, cu[n]:cu[n + 1]], o_n, atol=1e-12)
        np.testing.assert_allclose(S[n], S_n[0], atol=1e-12)


# ---------------------------------------------------------------------------
# P9: permutation equivariance
# ---------------------------------------------------------------------------

def test_p9_permutation_equivariance():
    """Permuting key channels leaves o unchanged and permutes S's rows; permuting
    value channels permutes o and S's columns [gist-1: gates act per axis]."""
    rng = np.random.default_rng(10)
    T, H, Dk, Dv = 6, 2, 5, 4
    q, k, v, la, b, w = _rand_inputs(rng, T, H, Dk, Dv)
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, S = O.recurrence(q, k, v, la, b, w, S0=S0)
    pk, pv = rng.permutation(Dk), rng.permutation(Dv)
    o2, S2 = O.recurrence(q[..., pk], k[..., pk], v[..., pv], la[..., pk], b[..., pk],
                          w[..., pv], S0=S0[:, :, pk][:, :, :, pv])
    np.testing.assert_allclose(o2, o[..., pv], atol=1e-12)
    np.testing.assert_allclose(S2, S[:, :, pk][:, :, :, pv], atol=1e-12)


def test_heads_and_batch_rows_independent():
    rng = np.random.default_rng(13)
    T, H, Dk, Dv = 5, 3, 4, 3
    q, k, v, la, b, w = _rand_inputs(rng, T, H, Dk, Dv, B=2)
    o, S = O.recurrence(q, k, v, la, b, w)
    o1, S1 = O.recurrence(q, k, v, la, b, w, heads=[1])
    np.testing.assert_allclose(o1[:, :, 1], o[:, :, 1], atol=1e-14)
    np.testing.assert_allclose(S1[:, 1], S[:, 1], atol=1e-14)
    o_b1, _ = O.recurrence(*(x[1:2] for x in (q, k, v, la, b, w)))
    np.testing.assert_allclose(o_b1[0], o[1], atol=1e-14)


def test_erase_range_widened_to_two():
    """The kernel must not assume b <= 1 (the [0, 2] erase ablation): the
    chunk form still equals the recurrence with b in [0, 2]."""
    rng = np.random.default_rng(14)
    q, k, v, la, b, w = _rand_inputs(rng, 11, 1, 5, 4, b_range=(0.0, 2.0))
    o_r, S_r = O.recurrence(q, k, v, la, b, w)
    o_c, S_c = O.chunked(q, k, v, la, b, w, chunk=4)
    np.testing.assert_allclose(o_c, o_r, atol=1e-11)
    np.testing.assert_allclose(S_c, S_r, atol=1e-11)


# ---------------------------------------------------------------------------
# Error metric
# ---------------------------------------------------------------------------

def test_rel_max_err():
    assert O.rel_max_err([1.0, -2.0], [1.0, -2.0]) == 0.0
    assert abs(O.rel_max_err([1.0, -2.1], [1.0, -2.0]) - 0.05) < 1e-12
    assert O.rel_max_err([0.0], [0.0]) == 0.0


def test_gates_from_logits_closed_forms():
    """Gates are sigmoids of their projections [iplexlaw, "Decisiones
    independientes en dos ejes"]: sigma(0) = 1/2, sigma(ln 3) = 3/4,
    sigma(-x) = 1 - sigma(x), values in (0, 1), and the erase and write
    logits map independently."""
    b, w = O.gates_from_logits(np.array([0.0, np.log(3.0), -np.log(3.0)]), np.array([40.0, -40.0]))
    np.testing.assert_allclose(b, [0.5, 0.75, 0.25], rtol=1e-15)
    assert 1.0 - w[0] < 1e-17 and 0.0 < w[1] < 1e-17
    x = np.linspace(-8, 8, 33)
    bx, wx = O.gates_from_logits(x, -x)
    np.testing.assert_allclose(bx + wx, 1.0, rtol=1e-15)
    assert np.all(np.diff(bx) > 0)

"""Pins of the fp64 layer oracle (oracle/layer_oracle.py) to things other than
itself: library routines (numpy.convolve; torch's float64 functional ops),
closed forms, and invariants of the layer (causality, sequence independence,
unit norms).  The core used inside is the token-by-token recurrence, which
has its own pins."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W
from oracle import layer_oracle as LO


def _tiny(seed=5, B=2, T=11, H=2, Dk=4, Dv=4, D=6, L=3, lengths=None, with_S0=True):
    wl = W.LayerWorkload("tiny", B, T, H, Dk, Dv, D, L, seed, with_S0=with_S0)
    return W.make_layer_inputs(wl, lengths=lengths)


def _call(inp, **kw):
    return LO.layer_fwd(inp["x"], inp["W_in"], inp["conv_w"], inp["alpha_bias"], inp["norm_w"],
                        inp["W_o"], inp["H"], inp["Dk"], inp["Dv"], S0=inp["S0"],
                        cu_seqlens=inp["cu_seqlens"], **kw)


def test_causal_conv_matches_numpy_convolve():
    # numpy.convolve(a, v)[t] = sum_j a[t-j] v[j]; the layer's tap j reads token
    # t-L+1+j, so the same filter reversed gives the layer's convolution.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 40, 5))
    cw = rng.standard_normal((5, 4))
    spans = [(0, 0, 3), (0, 3, 3), (0, 3, 17), (0, 17, 40)]   # includes an empty and a short one
    y = LO.causal_conv(x, cw, spans)
    for _, t0, t1 in spans:
        if t1 == t0:
            continue
        for c in range(5):
            ref = np.convolve(x[0, t0:t1, c], cw[c, ::-1])[:t1 - t0]
            np.testing.assert_allclose(y[0, t0:t1, c], ref, rtol=1e-13, atol=1e-13)


def test_logsigmoid_closed_forms():
    assert LO.logsigmoid(0.0) == pytest.approx(-np.log(2.0), rel=1e-15)
    # far tails: log(1/(1+e^-z)) = -log1p(e^-z) ~ -e^-z for large z; ~ z for very negative z
    assert LO.logsigmoid(40.0) == pytest.approx(-np.exp(-40.0), rel=1e-12)
    assert LO.logsigmoid(-40.0) == pytest.approx(-40.0 - np.exp(-40.0), rel=1e-15)
    z = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(LO.logsigmoid(z), np.log(1.0 / (1.0 + np.exp(-z))), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("L", [1, 3, 4])
def test_layer_matches_torch_functional(L):
    """The whole layer against a composition of torch's float64 functional
    ops (linear, grouped conv1d with left padding, silu, normalize,
    logsigmoid, sigmoid, rms_norm), with the recurrence as the core."""
    inp = _tiny(L=L)
    H, Dk, Dv, B, T = inp["H"], inp["Dk"], inp["Dv"], inp["B"], inp["T"]
    y, S = _call(inp, core=O.recurrence, l2_eps=0.0)

    t = {k_: torch.from_numpy(np.asarray(inp[k_], dtype=np.float64))
         for k_ in ("x", "W_in", "conv_w", "alpha_bias", "norm_w", "W_o")}
    HK, HV = H * Dk, H * Dv
    P = F.linear(t["x"], t["W_in"])
    q_, k_, v_, a_, g_, b_, w_ = torch.split(P, [HK, HK, HV, HK, HV, HK, HV], dim=-1)
    C = 2 * HK + HV
    qkv = torch.cat([q_, k_, v_], dim=-1).transpose(1, 2)          # [B, C, T]
    conv = F.conv1d(qkv, t["conv_w"].unsqueeze(1), padding=L - 1, groups=C)[..., :T]
    qkv = F.silu(conv).transpose(1, 2)
    q = F.normalize(qkv[..., :HK].reshape(B, T, H, Dk), dim=-1, eps=1e-300)
    k = F.normalize(qkv[..., HK:2 * HK].reshape(B, T, H, Dk), dim=-1, eps=1e-300)
    v = qkv[..., 2 * HK:].reshape(B, T, H, Dv)
    la = F.logsigmoid(a_ + t["alpha_bias"]).reshape(B, T, H, Dk)
    b = torch.sigmoid(b_).reshape(B, T, H, Dk)
    w = torch.sigmoid(w_).reshape(B, T, H, Dv)
    o, S_ref = O.recurrence(q.numpy(), k.numpy(), v.numpy(), la.numpy(), b.numpy(), w.numpy(),
                            S0=inp["S0"])
    z = F.rms_norm(torch.from_numpy(o), (Dv,), weight=t["norm_w"], eps=1e-6)
    z = z * torch.sigmoid(g_).reshape(B, T, H, Dv)
    y_ref = F.linear(z.reshape(B, T, HV), t["W_o"]).numpy()
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-13)


def test_layer_is_causal():
    inp = _tiny(T=13)
    y0, _ = _call(inp)
    t_cut = 6
    x2 = inp["x"].copy()
    x2[:, t_cut + 1:] = np.random.default_rng(9).standard_normal(x2[:, t_cut + 1:].shape)
    y1, _ = _call(dict(inp, x=x2))
    np.testing.assert_array_equal(y0[:, :t_cut + 1], y1[:, :t_cut + 1])
    assert np.abs(y0[:, t_cut + 1:] - y1[:, t_cut + 1:]).max() > 1e-3


def test_packed_call_equals_separate_sequences():
    lengths = [5, 0, 1, 9, 3]
    inp = _tiny(lengths=lengths, L=4)
    y, S = _call(inp)
    cu = inp["cu_seqlens"]
    for n, ln in enumerate(lengths):
        one = dict(inp, x=inp["x"][:, cu[n]:cu[n + 1]], cu_seqlens=None, S0=inp["S0"][n:n + 1])
        y1, S1 = _call(one)
        np.testing.assert_allclose(y[:, cu[n]:cu[n + 1]], y1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S[n], S1[0], rtol=1e-12, atol=1e-14)


def test_normalisation_invariants():
    inp = _tiny(T=20, H=3, Dk=8, Dv=8, D=12)
    _, _, parts = _call(inp, return_parts=True)
    nq = np.linalg.norm(parts["q"], axis=-1)
    nk = np.linalg.norm(parts["k"], axis=-1)
    np.testing.assert_allclose(nq, 1.0, rtol=0, atol=1e-4)   # |x|/sqrt(|x|^2+1e-6)
    np.testing.assert_allclose(nk, 1.0, rtol=0, atol=1e-4)
    P = parts["P"]
    r = LO.block_rows(3, 8, 8)
    gate = LO.sigmoid(P[..., r["gate"][0]:r["gate"][1]]).reshape(parts["z"].shape)
    unit = parts["z"] / (inp["norm_w"] * gate)
    rms = np.sqrt(np.mean(unit ** 2, axis=-1))
    o_ms = np.mean(parts["o"] ** 2, axis=-1)
    np.testing.assert_allclose(rms, np.sqrt(o_ms / (o_ms + 1e-6)), rtol=1e-12)


def test_chunked_core_agrees_with_recurrence_core():
    inp = _tiny(T=150, H=2, Dk=8, Dv=8, D=16, L=4)
    y_c, S_c = _call(inp)
    y_r, S_r = _call(inp, core=O.recurrence)
    np.testing.assert_allclose(y_c, y_r, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(S_c, S_r, rtol=1e-9, atol=1e-11)

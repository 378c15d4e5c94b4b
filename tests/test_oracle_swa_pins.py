"""Pins of the fp64 sliding-window attention oracle (oracle/swa_oracle.py):
torch's float64 scaled_dot_product_attention (causal, and with an explicit
window mask), closed forms (window 1 returns v; zero keys average v over the
window), a brute-force loop per query, and packed = separate sequences."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import swa_oracle as SO


def _inp(T=37, H=2, D=8, window=5, seed=1, lengths=None, B=2):
    wl = W.SwaWorkload("tiny", B, T, H, D, window, seed)
    return W.make_swa_inputs(wl, lengths=lengths)


def _sdpa(q, k, v, mask=None, causal=False):
    t = [torch.from_numpy(np.asarray(x, dtype=np.float64)).transpose(1, 2) for x in (q, k, v)]
    o = F.scaled_dot_product_attention(*t, attn_mask=mask, is_causal=causal)
    return o.transpose(1, 2).numpy()


def test_window_covering_sequence_is_causal_attention():
    inp = _inp(T=23, window=64)
    o, _ = SO.swa_fwd(inp["q"], inp["k"], inp["v"], 64)
    np.testing.assert_allclose(o, _sdpa(inp["q"], inp["k"], inp["v"], causal=True), rtol=1e-12,
                               atol=1e-13)


@pytest.mark.parametrize("window", [1, 3, 8])
def test_window_mask_against_sdpa(window):
    inp = _inp(T=30, window=window)
    o, _ = SO.swa_fwd(inp["q"], inp["k"], inp["v"], window)
    i = torch.arange(30)[:, None]
    j = torch.arange(30)[None, :]
    mask = (j <= i) & (j > i - window)      # torch's boolean mask: True = attend
    np.testing.assert_allclose(o, _sdpa(inp["q"], inp["k"], inp["v"], mask=mask), rtol=1e-12,
                               atol=1e-13)


def test_window_one_returns_v_and_lse_is_own_score():
    inp = _inp(T=12, window=1)
    o, lse = SO.swa_fwd(inp["q"], inp["k"], inp["v"], 1, scale=0.5)
    np.testing.assert_allclose(o, inp["v"], rtol=0, atol=0)
    own = 0.5 * np.einsum("bthd,bthd->bht", inp["q"].astype(np.float64), inp["k"].astype(np.float64))
    np.testing.assert_allclose(lse, own, rtol=1e-14, atol=1e-14)


def test_zero_keys_average_values_over_window():
    inp = _inp(T=20, window=6)
    k = np.zeros_like(inp["k"])
    o, lse = SO.swa_fwd(inp["q"], k, inp["v"], 6)
    v = inp["v"].astype(np.float64)
    for t in range(20):
        lo = max(0, t - 5)
        np.testing.assert_allclose(o[:, t], v[:, lo:t + 1].mean(axis=1), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, t], np.log(t + 1 - lo), rtol=1e-14)


def test_brute_force_loop():
    inp = _inp(T=9, H=1, D=4, window=4, B=1)
    q, k, v = (inp[x].astype(np.float64)[0, :, 0] for x in ("q", "k", "v"))
    o, _ = SO.swa_fwd(inp["q"], inp["k"], inp["v"], 4, scale=0.3)
    for i in range(9):
        js = [j for j in range(9) if i - 4 < j <= i]
        w = [np.exp(0.3 * float(q[i] @ k[j])) for j in js]
        ref = sum(wj * v[j] for wj, j in zip(w, js)) / sum(w)
        np.testing.assert_allclose(o[0, i, 0], ref, rtol=1e-13)


def test_packed_equals_separate():
    lengths = [7, 0, 1, 13, 4]
    inp = _inp(lengths=lengths, window=5)
    o, lse = SO.swa_fwd(inp["q"], inp["k"], inp["v"], 5, cu_seqlens=inp["cu_seqlens"])
    cu = inp["cu_seqlens"]
    for n in range(len(lengths)):
        sl = slice(cu[n], cu[n + 1])
        o1, l1 = SO.swa_fwd(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], 5)
        np.testing.assert_allclose(o[:, sl], o1, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse[:, :, sl], l1, rtol=1e-14, atol=1e-15)


def test_swa_layer_matches_torch_composition():
    """The layer around the attention: torch float64 linear + windowed
    scaled_dot_product_attention + linear."""
    wl = W.SwaLayerWorkload("tiny_layer", 2, 19, 2, 4, 6, 5, 77)
    inp = W.make_swa_layer_inputs(wl)
    y, _ = SO.swa_layer_fwd(inp["x"], inp["W_qkv"], inp["W_o"], 2, 4, 5)
    t = {k_: torch.from_numpy(np.asarray(inp[k_], dtype=np.float64)) for k_ in ("x", "W_qkv", "W_o")}
    P = F.linear(t["x"], t["W_qkv"])
    q, k, v = (z.reshape(2, 19, 2, 4).transpose(1, 2) for z in torch.split(P, 8, dim=-1))
    i = torch.arange(19)[:, None]
    j = torch.arange(19)[None, :]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=(j <= i) & (j > i - 5))
    y_ref = F.linear(o.transpose(1, 2).reshape(2, 19, 8), t["W_o"]).numpy()
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-13)

"""GPU parity of the token-mixer layer forward (gdn2_layer_fwd) against the
fp64 layer oracle: small dense and packed calls over several chunks with a
ragged tail, both head sizes, convolution lengths 1..8, determinism, and the
full-size layer workload checked on whole batch rows.

Tolerance: the library rounds every intermediate to bf16 (projections, the
core's inputs and output, the normalised z, y) while the oracle stays in
fp64; each rounding is 2^-9 relative and the core alone stays within 2e-2 of
max|o| (its own bound).  y is a 2048-term sum of z W_o, which averages the
per-element errors, so the core's bound also bounds max|dy| / max|y|."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import workloads as W
from gpu_util import dev, host, log
from oracle import layer_oracle as LO
import oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _upload(inp):
    return dict(x=dev(inp["x"], W.BF16), W_in=dev(inp["W_in"], W.BF16),
                conv_w=dev(inp["conv_w"]), alpha_bias=dev(inp["alpha_bias"]),
                norm_w=dev(inp["norm_w"]), W_o=dev(inp["W_o"], W.BF16), S0=dev(inp["S0"]),
                cu_seqlens=dev(inp["cu_seqlens"]))


def _run(inp, d=None):
    import torch
    d = d or _upload(inp)
    y, S = g.layer_fwd(d["x"], d["W_in"], d["conv_w"], d["alpha_bias"], d["norm_w"], d["W_o"],
                       inp["H"], inp["Dk"], inp["Dv"], S0=d["S0"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return y, S


def _oracle(inp, rows=None):
    x, S0 = inp["x"], inp["S0"]
    if rows is not None:
        x = x[rows]
        S0 = None if S0 is None else S0[rows]
    return LO.layer_fwd(x, inp["W_in"], inp["conv_w"], inp["alpha_bias"], inp["norm_w"],
                        inp["W_o"], inp["H"], inp["Dk"], inp["Dv"], S0=S0,
                        cu_seqlens=inp["cu_seqlens"], core=O.recurrence)


def _check(inp, label):
    y, S = _run(inp)
    y_ref, S_ref = _oracle(inp)
    ey, es = O.rel_max_err(host(y), y_ref), O.rel_max_err(host(S), S_ref)
    log("%s: err_y %.3e err_S %.3e" % (label, ey, es))
    assert ey <= TOL and es <= TOL
    return y, S


@pytest.mark.parametrize("D", [128, 64])
def test_layer_dense_ragged(D):
    """2 sequences of 200 tokens (3 chunks + 8), nonzero S0, model width 256."""
    H = 256 // D
    wl = W.LayerWorkload("layer_dense", 2, 200, H, D, D, 256, 4, 9100 + D, with_S0=True)
    _check(W.make_layer_inputs(wl), "layer dense D=%d" % D)


def test_layer_varlen_edge_lengths():
    """Packed lengths shorter than the convolution, empty, and over a chunk."""
    wl = W.LayerWorkload("layer_varlen", 1, 0, 2, 128, 128, 256, 4, 9200, with_S0=True)
    _check(W.make_layer_inputs(wl, lengths=[1, 3, 0, 70, 2, 130]), "layer varlen")


@pytest.mark.parametrize("L", [1, 2, 8])
def test_layer_conv_lengths(L):
    wl = W.LayerWorkload("layer_conv", 1, 96, 2, 128, 128, 256, L, 9300 + L)
    _check(W.make_layer_inputs(wl), "layer conv_len=%d" % L)


def test_layer_wide_model():
    """Model width 512 over 2 heads of 128 (D != H*Dv)."""
    wl = W.LayerWorkload("layer_wide", 1, 130, 2, 128, 128, 512, 4, 9400, with_S0=True)
    _check(W.make_layer_inputs(wl), "layer D=512")


def test_layer_deterministic():
    import torch
    wl = W.LayerWorkload("layer_det", 2, 150, 2, 128, 128, 256, 4, 9500, with_S0=True)
    inp = W.make_layer_inputs(wl)
    d = _upload(inp)
    y1, S1 = _run(inp, d)
    y2, S2 = _run(inp, d)
    assert torch.equal(y1, y2) and torch.equal(S1, S2)


def test_layer_full_size_rows():
    """The 1.3B-layer workload (B=8, T=4096, 16 heads of 128, D=2048): the whole
    batch runs on the GPU; batch row 5 (all 4096 tokens and its final state)
    is checked against the oracle."""
    inp = W.make_layer_inputs(W.LAYER_4K)
    y, S = _run(inp)
    r = 5
    y_ref, S_ref = _oracle(inp, rows=slice(r, r + 1))
    ey = O.rel_max_err(host(y[r:r + 1]), y_ref)
    es = O.rel_max_err(host(S[r:r + 1]), S_ref)
    log("%s row %d: err_y %.3e err_S %.3e" % (W.LAYER_4K.name, r, ey, es))
    assert ey <= TOL and es <= TOL
    assert np.isfinite(host(y)).all()

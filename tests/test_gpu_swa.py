"""GPU parity of sliding-window attention (gdn2_swa_fwd) against the fp64
oracle: dense and packed calls spanning several 128-query blocks and 64-key
tiles with ragged tails, window sizes from 1 to beyond the sequence, both
head sizes, determinism, and the full-size hybrid workload (B=8, T=4096,
16 heads of 128, 2048-token window) on sampled (sequence, head) pairs.

Tolerance: q, k, v are bf16 and exact on both sides; scores, softmax
statistics and accumulation are fp32, the probabilities enter the second
product as bf16 (2^-9 relative) and o is stored as bf16 (2^-9), so
max|do| / max|o| <= 1e-2 holds with margin; lse (fp32 throughout) within 1e-3
absolute."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import workloads as W
from gpu_util import dev, host, log
from oracle import swa_oracle as SO
import oracle as O

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


def _run(inp, window):
    import torch
    q, k, v = (dev(inp[x], W.BF16) for x in ("q", "k", "v"))
    o, lse = g.swa_fwd(q, k, v, window, cu_seqlens=dev(inp["cu_seqlens"]))
    torch.cuda.synchronize()
    return host(o), host(lse)


def _check(inp, window, label):
    o, lse = _run(inp, window)
    o_ref, lse_ref = SO.swa_fwd(inp["q"], inp["k"], inp["v"], window, cu_seqlens=inp["cu_seqlens"])
    eo, el = O.rel_max_err(o, o_ref), float(np.abs(lse - lse_ref).max())
    log("%s: err_o %.3e err_lse %.3e" % (label, eo, el))
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("window", [1, 37, 100, 1000])
def test_swa_dense(D, window):
    """2 sequences of 300 tokens (2 query blocks + 44), 2 heads."""
    wl = W.SwaWorkload("swa_dense", 2, 300, 2, D, window, 9600 + D + window)
    _check(W.make_swa_inputs(wl), window, "swa dense D=%d W=%d" % (D, window))


def test_swa_packed_edge_lengths():
    wl = W.SwaWorkload("swa_packed", 1, 0, 3, 128, 64, 9700)
    inp = W.make_swa_inputs(wl, lengths=[1, 127, 128, 0, 129, 300, 5])
    _check(inp, 64, "swa packed")


def test_swa_deterministic():
    import torch
    wl = W.SwaWorkload("swa_det", 1, 500, 2, 128, 200, 9800)
    inp = W.make_swa_inputs(wl)
    q, k, v = (dev(inp[x], W.BF16) for x in ("q", "k", "v"))
    o1, l1 = g.swa_fwd(q, k, v, 200)
    o2, l2 = g.swa_fwd(q, k, v, 200)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_swa_full_size_sampled():
    wl = W.SWA_4K
    inp = W.make_swa_inputs(wl)
    o, lse = _run(inp, wl.window)
    for b, h in [(0, 0), (3, 9), (7, 15)]:
        sl = slice(b, b + 1)
        o_ref, lse_ref = SO.swa_fwd(inp["q"][sl], inp["k"][sl], inp["v"][sl], wl.window, heads=[h])
        eo = O.rel_max_err(o[b, :, h], o_ref[0, :, h])
        el = float(np.abs(lse[b, h] - lse_ref[0, h]).max())
        log("%s (%d, %d): err_o %.3e err_lse %.3e" % (wl.name, b, h, eo, el))
        assert eo <= TOL_O and el <= TOL_LSE


def _run_layer(inp):
    import torch
    y, lse = g.swa_layer_fwd(dev(inp["x"], W.BF16), dev(inp["W_qkv"], W.BF16),
                             dev(inp["W_o"], W.BF16), inp["H"], inp["D"], inp["window"],
                             cu_seqlens=dev(inp["cu_seqlens"]))
    torch.cuda.synchronize()
    return host(y), host(lse)


@pytest.mark.parametrize("lengths", [None, [1, 130, 0, 300, 7]])
def test_swa_layer(lengths):
    """The projection-attention-projection layer; the projections are bf16
    GEMMs (rounded to bf16 before the attention), so the bound is the layer's
    2e-2 on y; lse within 2e-2 (its logits come from bf16-rounded q, k)."""
    wl = W.SwaLayerWorkload("swa_layer_small", 2, 200, 2, 128, 256, 64, 9900)
    inp = W.make_swa_layer_inputs(wl, lengths=lengths)
    y, lse = _run_layer(inp)
    y_ref, lse_ref = SO.swa_layer_fwd(inp["x"], inp["W_qkv"], inp["W_o"], inp["H"], inp["D"],
                                      inp["window"], cu_seqlens=inp["cu_seqlens"])
    ey, el = O.rel_max_err(y, y_ref), float(np.abs(lse - lse_ref).max())
    log("swa layer lengths=%s: err_y %.3e err_lse %.3e" % (lengths, ey, el))
    assert ey <= 2e-2 and el <= 2e-2


def test_swa_layer_full_size_row():
    inp = W.make_swa_layer_inputs(W.SWA_LAYER_4K)
    y, _ = _run_layer(inp)
    r = 6
    y_ref, _ = SO.swa_layer_fwd(inp["x"][r:r + 1], inp["W_qkv"], inp["W_o"], inp["H"], inp["D"],
                                inp["window"])
    ey = O.rel_max_err(y[r:r + 1], y_ref)
    log("%s row %d: err_y %.3e" % (W.SWA_LAYER_4K.name, r, ey))
    assert ey <= 2e-2

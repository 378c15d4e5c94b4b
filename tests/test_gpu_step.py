"""GPU parity of gdn2_step (the decode kernel) against the fp64 oracle."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import oracle as O
import workloads as W
from gpu_util import dev, host, log, tol

pytestmark = pytest.mark.gpu


def _decode_wl(B, H, D, io, steps):
    return W.DecodeWorkload("decode_test", B, H, D, D, io, 4711 + D + B, steps)


@pytest.mark.parametrize("io", [W.BF16, W.F32])
@pytest.mark.parametrize("D", [64, 128])
def test_step_small_all_chains(io, D):
    import torch
    wl = _decode_wl(3, 5, D, io, 24)
    S_ref = W.make_decode_state(wl).astype(np.float64)
    S = dev(W.make_decode_state(wl))
    log("step_small io=%s D=%d" % (io, D))
    errs_o = []
    for s in range(wl.steps):
        x = W.make_decode_step(wl, s)
        o_ref, S_ref = O.step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S_ref)
        o = g.step(dev(x["q"], io), dev(x["k"], io), dev(x["v"], io), dev(x["log_alpha"]),
                   dev(x["b"]), dev(x["w"]), S)
        torch.cuda.synchronize()
        errs_o.append(O.rel_max_err(host(o), o_ref))
    err_S = O.rel_max_err(host(S), S_ref)
    log("  err_o max %.3e  err_S %.3e" % (max(errs_o), err_S))
    assert max(errs_o) <= tol(io)
    assert err_S <= tol(io)


def test_step_full_decode_workload_128_chains():
    """B=256, H=16, d=128, 1024 consecutive steps; the oracle follows 128
    chains (all 16 heads of 8 batch rows spread over the batch): the outputs
    of every step and the state after steps 1, 256, 512 and 1024."""
    import torch
    wl = W.DECODE
    rows = np.array([0, 37, 74, 111, 148, 185, 222, 255])
    bs = np.repeat(rows, wl.H)
    hs = np.tile(np.arange(wl.H), len(rows))
    S_init = W.make_decode_state(wl)
    S = dev(S_init)
    S_ref = S_init[bs, hs].astype(np.float64)            # [128, Dk, Dv]
    o_dev = torch.empty((wl.B, wl.H, wl.Dv), dtype=torch.bfloat16, device="cuda")
    worst_o = 0.0
    check_at = {1, 256, 512, 1024}
    names = ("q", "k", "v", "log_alpha", "b", "w")
    log("decode full: B=%d H=%d steps=%d, %d chains checked" % (wl.B, wl.H, wl.steps, len(bs)))
    for s in range(wl.steps):
        x = W.make_decode_step(wl, s)
        g.step(dev(x["q"], wl.io), dev(x["k"], wl.io), dev(x["v"], wl.io), dev(x["log_alpha"]),
               dev(x["b"]), dev(x["w"]), S, o=o_dev)
        o_h = host(o_dev)
        o_r, S_ref = O.step(*(x[n][bs, hs] for n in names), S_ref)
        worst_o = max(worst_o, O.rel_max_err(o_h[bs, hs], o_r))
        if s + 1 in check_at:
            err = O.rel_max_err(host(S)[bs, hs], S_ref)
            log("  step %d: err_S %.3e  err_o so far %.3e" % (s + 1, err, worst_o))
            assert err <= tol(wl.io)
    assert worst_o <= tol(wl.io)


def test_step_equals_chunk_forward():
    """T successive decode steps equal one chunk forward over the same T tokens."""
    import torch
    inp = W.make_chunk_inputs(W.BATCH_4K, T=100, B=2, H=3)
    io = inp["io"]
    d = {k_: dev(inp[k_], io if k_ in ("q", "k", "v") else None)
         for k_ in ("q", "k", "v", "log_alpha", "b", "w", "S0")}
    o_c, S_c = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"])
    S = d["S0"].clone()
    outs = []
    for t in range(inp["T"]):
        outs.append(g.step(*(d[k_][:, t].contiguous() for k_ in
                             ("q", "k", "v", "log_alpha", "b", "w")), S))
    torch.cuda.synchronize()
    o_s = torch.stack(outs, dim=1)
    assert O.rel_max_err(host(o_s), host(o_c)) <= tol(io)
    assert O.rel_max_err(host(S), host(S_c)) <= tol(io)

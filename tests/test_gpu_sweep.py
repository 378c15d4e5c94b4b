"""A seeded sweep of small random chunk-forward and backward calls against the
fp64 oracle: each case draws its own io dtype, head width, dense or packed
layout, batch, length (ragged tails and zero-length sequences included), head
count, decay range, erase-gate range and initial state, so that combinations
the hand-picked cases do not name are also checked.  bf16 cases also run the
training pair (gdn2_chunk_fwd_train + gdn2_chunk_bwd_saved), which must equal
the plain calls bitwise.  Bounds: 2e-2 of max|ref| for bf16 I/O, 1e-4 for
fp32 I/O, on every output and gradient."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import oracle as O
import workloads as W
from gpu_util import dev, host, log, tol, upload_chunk

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")
DECAYS = [(-0.2, -0.001), (0.0, 0.0), (-1.0, -0.5), (-2.5, -2.0), (-0.05, 0.0)]


def _case(i):
    """Case i of the sweep: every choice drawn from a generator seeded by i."""
    rng = np.random.Generator(np.random.PCG64(90210 + i))
    io = W.BF16 if rng.random() < 0.7 else W.F32
    D = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 5))
    decay = DECAYS[int(rng.integers(0, len(DECAYS)))]
    b_scale = 2.0 if rng.random() < 0.3 else 1.0
    with_S0 = bool(rng.random() < 0.7)
    if rng.random() < 0.4:
        n = int(rng.integers(1, 6))
        lengths = [int(x) for x in rng.integers(0, 200, size=n)]
        wl = W.ChunkWorkload("sweep%d" % i, 1, 0, H, D, D, io, 5000 + i, with_S0=with_S0, n_seqs=n)
        inp = W.make_chunk_inputs(wl, lengths=lengths, log_alpha_range=decay, b_scale=b_scale)
        shape = "packed %s" % lengths
    else:
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 200))
        wl = W.ChunkWorkload("sweep%d" % i, B, T, H, D, D, io, 5000 + i, with_S0=with_S0)
        inp = W.make_chunk_inputs(wl, log_alpha_range=decay, b_scale=b_scale)
        shape = "B=%d T=%d" % (B, T)
    label = "case %d: %s d=%d H=%d %s log_alpha in %s b_scale %g S0 %s" % (
        i, "bf16" if io == W.BF16 else "f32", D, H, shape, decay, b_scale, with_S0)
    return inp, label


@pytest.mark.parametrize("i", range(16))
def test_random_case(i):
    import torch
    inp, label = _case(i)
    log(label)
    grads = W.make_chunk_grads(inp, 600 + i)
    d = upload_chunk(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    dout = dev(grads["dout"], inp["io"])
    dSf = dev(grads["dS_final"])
    o, S = g.chunk_fwd(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"])
    bw = g.chunk_bwd(*x, dout, S0=d["S0"], dS_final=dSf, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()

    raw = [inp[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = O.recurrence(*raw, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"])
    ref = O.recurrence_bwd(*raw, grads["dout"], inp["S0"], grads["dS_final"], inp["cu_seqlens"])
    errs = {"o": O.rel_max_err(host(o), o_ref), "S": O.rel_max_err(host(S), S_ref)}
    errs.update({n: O.rel_max_err(host(bw[n]), ref[n]) for n in NAMES})
    log("  " + " ".join("%s %.2e" % kv for kv in errs.items()))
    bound = tol(inp["io"])
    for n, e in errs.items():
        assert e <= bound, (label, n, e)

    if inp["io"] == W.BF16:
        o2, S2, ws = g.chunk_fwd_train(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"])
        bw2 = g.chunk_bwd_saved(*x, dout, ws, dS_final=dSf, cu_seqlens=d["cu_seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(S2, S), label
        for n in NAMES:
            assert torch.equal(bw2[n], bw[n]), (label, n)

"""The training pair gdn2_chunk_fwd_train + gdn2_chunk_bwd_saved: the forward
that keeps the chunk factors (with their transposes) and every chunk's
incoming state, and the backward that starts from them instead of
recomputing them.  Both run the same kernels on the same values as
gdn2_chunk_fwd and gdn2_chunk_bwd, so their results must be bitwise equal;
a second backward from the same workspace must repeat the first (the saved
data are not overwritten); and one small case is checked against the fp64
oracle's reverse recurrence directly (bound 2e-2 for bf16)."""

import pytest

import gated_delta_rule_47_amd as g
import oracle as O
import workloads as W
from gpu_util import dev, host, log, tol, upload_chunk

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _pair(inp, grads, label):
    import torch
    d = upload_chunk(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    dout = dev(grads["dout"], inp["io"])
    dSf = dev(grads["dS_final"])
    o_ref, S_ref = g.chunk_fwd(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"])
    ref = g.chunk_bwd(*x, dout, S0=d["S0"], dS_final=dSf, cu_seqlens=d["cu_seqlens"])
    o, S, ws = g.chunk_fwd_train(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"])
    got = g.chunk_bwd_saved(*x, dout, ws, dS_final=dSf, cu_seqlens=d["cu_seqlens"])
    again = g.chunk_bwd_saved(*x, dout, ws, dS_final=dSf, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref), label
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), (label, n)
        assert torch.equal(again[n], got[n]), (label, n, "second backward")
    log("%s: training forward and saved-state backward equal the recomputing calls bitwise" % label)
    return got


@pytest.mark.parametrize("D", [64, 128])
def test_train_pair_dense_ragged(D):
    """T = 150 (two full chunks and a 22-token tail), S0 and dS_final nonzero."""
    wl = W.ChunkWorkload("train_dense", 2, 150, 2, D, D, W.BF16, 7100 + D, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    _pair(inp, W.make_chunk_grads(inp, 31 + D), "train dense D=%d" % D)


def test_train_pair_packed_edge_lengths():
    """Packed lengths 1, 63, 64, 65, 130, 0 and 7 (the chunk table is saved too)."""
    wl = W.ChunkWorkload("train_varlen", 1, 0, 2, 128, 128, W.BF16, 7200, with_S0=True, n_seqs=7)
    inp = W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7])
    _pair(inp, W.make_chunk_grads(inp, 32), "train packed")


def test_train_pair_256_chains():
    """B = 16, H = 16 (256 chains: the reverse pass's 4-wave workgroups), T = 70."""
    wl = W.ChunkWorkload("train_many", 16, 70, 16, 128, 128, W.BF16, 7300, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    _pair(inp, W.make_chunk_grads(inp, 33), "train 256 chains")


def test_train_pair_batch_workload():
    """B=8, H=16, T=4096, d=128, in the launch configuration the benchmark times."""
    inp = W.make_chunk_inputs(W.BATCH_4K)
    _pair(inp, W.make_chunk_grads(inp, 1), "train batch workload")


def test_saved_backward_against_the_oracle():
    """The saved-state backward against the plain reverse recurrence."""
    wl = W.ChunkWorkload("train_oracle", 2, 150, 2, 128, 128, W.BF16, 7400, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    grads = W.make_chunk_grads(inp, 34)
    got = _pair(inp, grads, "train oracle case")
    ref = O.recurrence_bwd(*(inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")),
                           grads["dout"], inp["S0"], grads["dS_final"], inp["cu_seqlens"])
    errs = {n: O.rel_max_err(host(got[n]), ref[n]) for n in NAMES}
    log("saved backward vs oracle: %s" % " ".join("%s %.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e <= tol(W.BF16), (n, e)

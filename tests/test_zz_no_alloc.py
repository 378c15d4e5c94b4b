"""gdn2_chunk_fwd_noalloc, the chunk forward that allocates nothing, called
through the C ABI and compared with gdn2_chunk_fwd on a caller's workspace
(the same kernels, so the results must be bitwise equal) and with the fp64
oracle at the forward's parity bound.  The calls run back to back, each
smaller than the one before, so that later calls run over the intermediates
an earlier call left in the library's region."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import oracle as O
import workloads as W
from gpu_util import host, log, tol, upload_chunk

SCRATCH_BYTES = 128 << 20


def _sizes(inp):
    return inp["N"], inp["B"], inp["T"], inp["H"], inp["Dk"], inp["Dv"]


def _noalloc(d, inp, io):
    """One gdn2_chunk_fwd_noalloc call on torch-owned inputs and outputs."""
    import torch
    N, B, T, H, Dk, Dv = _sizes(inp)
    dt = torch.bfloat16 if io == g.GDN2_BF16 else torch.float32
    o = torch.full((B, T, H, Dv), float("nan"), dtype=dt, device="cuda")
    S = torch.full((N, H, Dk, Dv), float("nan"), dtype=torch.float32, device="cuda")
    p = lambda t: None if t is None else t.data_ptr()
    st = g.gdn2_chunk_fwd_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["log_alpha"]), p(d["b"]),
                                  p(d["w"]), p(d["S0"]), p(o), p(S), p(d["cu_seqlens"]), N, B, T, H,
                                  Dk, Dv, io, torch.cuda.current_stream().cuda_stream)
    assert st == g.GDN2_OK, g.gdn2_status_string(st)
    return o, S


def _compare(inp, label):
    import torch
    io = g.GDN2_BF16 if inp["io"] == W.BF16 else g.GDN2_F32
    need = g.gdn2_chunk_fwd_workspace_bytes(*_sizes(inp), io, inp["cu_seqlens"] is not None)
    assert 0 < need <= SCRATCH_BYTES
    d = upload_chunk(inp)
    o_n, S_n = _noalloc(d, inp, io)
    o_w, S_w = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                           cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w), label
    args = [inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = O.recurrence(*args, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"])
    eo, es = O.rel_max_err(host(o_n), o_ref), O.rel_max_err(host(S_n), S_ref)
    log("noalloc %s: %d workspace bytes, err_o %.3e err_S %.3e" % (label, need, eo, es))
    assert eo <= tol(inp["io"]) and es <= tol(inp["io"])


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_on_shrinking_inputs():
    # 1) the single-sequence 4K workload (B=1, H=16, T=4096, d=128): 76 MB of intermediates
    _compare(W.make_chunk_inputs(W.SEQ_4K), "seq 4K")
    # 2) smaller, dense with a ragged tail and S0: runs over the leftovers of 1)
    wl = W.ChunkWorkload("noalloc_small", 2, 200, 3, 128, 128, W.BF16, 9101, with_S0=True)
    _compare(W.make_chunk_inputs(wl), "B2 H3 T200")
    # 3) smaller still, packed (the chunk table also lives in the region), fp32
    wl = W.ChunkWorkload("noalloc_varlen", 1, 0, 2, 64, 64, W.F32, 9102, with_S0=True, n_seqs=4)
    _compare(W.make_chunk_inputs(wl, lengths=[65, 1, 0, 64]), "packed fp32 d64")


def test_noalloc_rejects_calls_beyond_its_region():
    """Sizes whose intermediates exceed the 128 MiB region are refused before
    any pointer is looked at or anything is enqueued (no GPU needed)."""
    bf = g.GDN2_BF16
    assert g.gdn2_chunk_fwd_workspace_bytes(1, 1, 7168, 16, 128, 128, bf, 0) <= SCRATCH_BYTES
    assert g.gdn2_chunk_fwd_workspace_bytes(1, 1, 7232, 16, 128, 128, bf, 0) > SCRATCH_BYTES
    st = g.gdn2_chunk_fwd_noalloc(*([None] * 10), 1, 1, 7232, 16, 128, 128, bf, None)
    assert st == g.GDN2_ERR_WORKSPACE
    st = g.gdn2_chunk_fwd_noalloc(*([None] * 10), 8, 8, 4096, 16, 128, 128, bf, None)
    assert st == g.GDN2_ERR_WORKSPACE
    # invalid sizes get the common validation's answer
    assert g.gdn2_chunk_fwd_noalloc(*([None] * 10), 1, 1, 64, 1, 96, 96, bf, None) == \
        g.GDN2_ERR_UNSUPPORTED
    assert np.isfinite(SCRATCH_BYTES)

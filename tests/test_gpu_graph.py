"""The chunk forward under HIP graph capture: gdn2_chunk_fwd (dense and packed,
the packed call's chunk table built by its own kernel) and
gdn2_chunk_fwd_noalloc, each captured once on torch's capture stream and
replayed three times, with other eager library calls and synchronisations
between the replays.  Every replay must reproduce the eager result bitwise
(the same kernels on the same inputs): the calls issue only kernel launches,
no memset or copy nodes."""

import pytest

import gated_delta_rule_47_amd as g
import workloads as W
from gpu_util import log, upload_chunk

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _other_work(seed):
    """Unrelated eager library work between replays (another forward)."""
    import torch
    inp = W.make_chunk_inputs(W.ChunkWorkload("graph_other", 1, 70, 2, 64, 64, W.BF16, seed,
                                              with_S0=True))
    d = upload_chunk(inp)
    g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"])
    torch.cuda.synchronize()


def _replay_and_check(graph, outs, refs, label):
    import torch
    for rep in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r), (label, rep)
        log("%s: replay %d matches the eager call bitwise" % (label, rep))
        _other_work(900 + rep)


def _check_chunk_fwd(inp, label):
    import torch
    d = upload_chunk(inp)
    N, B, T, H, D = inp["N"], inp["B"], inp["T"], inp["H"], inp["Dk"]
    varlen = d["cu_seqlens"] is not None
    ws = torch.empty(g.gdn2_chunk_fwd_workspace_bytes(N, B, T, H, D, D, g.GDN2_BF16, varlen),
                     dtype=torch.uint8, device="cuda")
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o_ref, S_ref = g.chunk_fwd(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"], workspace=ws)
    torch.cuda.synchronize()
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.chunk_fwd(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"], o=o, S_final=S, workspace=ws)
    _replay_and_check(graph, (o, S), (o_ref, S_ref), label)


def test_chunk_fwd_dense_graph_replays():
    """B=2, T=150 (a 22-token tail), H=2, d=128, bf16, S0 != 0."""
    wl = W.ChunkWorkload("graph_dense", 2, 150, 2, 128, 128, W.BF16, 6101, with_S0=True)
    _check_chunk_fwd(W.make_chunk_inputs(wl), "graph dense")


def test_chunk_fwd_packed_graph_replays():
    """Packed lengths 1, 63, 64, 65, 130, 0 and 7: the chunk table is built in the graph."""
    wl = W.ChunkWorkload("graph_varlen", 1, 0, 2, 128, 128, W.BF16, 6202, with_S0=True, n_seqs=7)
    _check_chunk_fwd(W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7]), "graph packed")


def test_chunk_fwd_noalloc_graph_replays():
    """gdn2_chunk_fwd_noalloc captured after one eager call (which looks up the
    library's region for this device), on B=2, T=200, H=4, d=128."""
    import torch
    wl = W.ChunkWorkload("graph_noalloc", 2, 200, 4, 128, 128, W.BF16, 6303, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    d = upload_chunk(inp)
    N, B, T, H, D = inp["N"], inp["B"], inp["T"], inp["H"], inp["Dk"]
    p = lambda t: None if t is None else t.data_ptr()

    def call(o, S):
        st = g.gdn2_chunk_fwd_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["log_alpha"]), p(d["b"]),
                                      p(d["w"]), p(d["S0"]), p(o), p(S), None, N, B, T, H, D, D,
                                      g.GDN2_BF16, torch.cuda.current_stream().cuda_stream)
        assert st == g.GDN2_OK, g.gdn2_status_string(st)

    o_ref = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    S_ref = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    call(o_ref, S_ref)
    torch.cuda.synchronize()
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o, S)
    _replay_and_check(graph, (o, S), (o_ref, S_ref), "graph noalloc")

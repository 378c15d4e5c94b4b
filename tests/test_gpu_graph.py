"""The library's calls under HIP graph capture: gdn2_chunk_fwd (dense and
packed, the packed call's chunk table built by its own kernel),
gdn2_chunk_fwd_noalloc, gdn2_chunk_bwd, the training pair
gdn2_chunk_fwd_train + gdn2_chunk_bwd_saved, and a run of gdn2_step calls,
each captured once on torch's capture stream and replayed three times, with
other eager library calls and synchronisations between the replays.  Every
replay must reproduce the eager result bitwise (the same kernels on the same
inputs): the calls issue only kernel launches, no memset or copy nodes."""

import pytest

import gated_delta_rule_47_amd as g
import workloads as W
from gpu_util import dev, log, upload_chunk

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


GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _bwd_case(inp, seed, label, train=False):
    import torch
    grads = W.make_chunk_grads(inp, seed)
    d = upload_chunk(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    dout = dev(grads["dout"], inp["io"])
    dSf = dev(grads["dS_final"])
    kw = dict(cu_seqlens=d["cu_seqlens"])
    if train:
        o_r, S_r, ws_r = g.chunk_fwd_train(*x, S0=d["S0"], **kw)
        ref = g.chunk_bwd_saved(*x, dout, ws_r, dS_final=dSf, **kw)
        refs = [o_r, S_r] + [ref[n] for n in GRADS]
    else:
        ref = g.chunk_bwd(*x, dout, S0=d["S0"], dS_final=dSf, **kw)
        refs = [ref[n] for n in GRADS]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        if train:
            o, S, ws = g.chunk_fwd_train(*x, S0=d["S0"], **kw)
            out = g.chunk_bwd_saved(*x, dout, ws, dS_final=dSf, **kw)
            outs = [o, S] + [out[n] for n in GRADS]
        else:
            out = g.chunk_bwd(*x, dout, S0=d["S0"], dS_final=dSf, **kw)
            outs = [out[n] for n in GRADS]
    _replay_and_check(graph, outs, refs, label)


def test_chunk_bwd_dense_graph_replays():
    """gdn2_chunk_bwd on B=2, T=150, H=2, d=128, bf16, S0 and dS_final != 0."""
    wl = W.ChunkWorkload("graph_bwd", 2, 150, 2, 128, 128, W.BF16, 6404, with_S0=True)
    _bwd_case(W.make_chunk_inputs(wl), 41, "graph bwd dense")


def test_chunk_bwd_packed_graph_replays():
    """gdn2_chunk_bwd on packed lengths 1, 63, 64, 65, 130, 0 and 7."""
    wl = W.ChunkWorkload("graph_bwd_varlen", 1, 0, 2, 128, 128, W.BF16, 6505, with_S0=True, n_seqs=7)
    _bwd_case(W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7]), 42, "graph bwd packed")


def test_training_pair_graph_replays():
    """gdn2_chunk_fwd_train and gdn2_chunk_bwd_saved captured together, on
    B=2, T=200, H=4, d=128, bf16."""
    wl = W.ChunkWorkload("graph_train", 2, 200, 4, 128, 128, W.BF16, 6606, with_S0=True)
    _bwd_case(W.make_chunk_inputs(wl), 43, "graph training pair", train=True)


def test_decode_steps_graph_replays():
    """Four consecutive gdn2_step calls on one state (B=4, H=2, d=128, bf16),
    captured once; before each replay the state is reset to its initial
    value, and every step's output and the final state must equal the eager
    run's."""
    import torch
    dw = W.DecodeWorkload("graph_decode", 4, 2, 128, 128, W.BF16, 6707, 4)
    S_init = dev(W.make_decode_state(dw))
    names = ("q", "k", "v", "log_alpha", "b", "w")
    xs = []
    for t in range(dw.steps):
        x = W.make_decode_step(dw, t)
        xs.append([dev(x[n], dw.io if n in ("q", "k", "v") else None) for n in names])
    S_e = S_init.clone()
    o_ref = [g.step(*xs[t], S_e) for t in range(dw.steps)]
    torch.cuda.synchronize()
    S_g = S_init.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = [g.step(*xs[t], S_g) for t in range(dw.steps)]
    for rep in range(REPLAYS):
        S_g.copy_(S_init)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(dw.steps):
            assert torch.equal(outs[t], o_ref[t]), ("decode step", t, rep)
        assert torch.equal(S_g, S_e), ("decode state", rep)
        log("graph decode: replay %d matches the eager steps bitwise" % rep)
        _other_work(950 + rep)

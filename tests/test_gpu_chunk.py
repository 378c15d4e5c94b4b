"""GPU parity of gdn2_chunk_fwd against the fp64 oracle: end to end, per stage
(the chunk intermediates kept in the workspace), varlen, edge cases and the
full-size workloads checked whole against the plain recurrence."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import oracle as O
import workloads as W
from gpu_util import dev, host, log, tol, upload_chunk

pytestmark = pytest.mark.gpu


def _run(inp, d=None, workspace=None, stages=g.GDN2_STAGE_ALL):
    import torch
    d = d or upload_chunk(inp)
    o, S = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                       cu_seqlens=d["cu_seqlens"], workspace=workspace, stages=stages)
    torch.cuda.synchronize()
    return o, S


def _check_all(inp, label):
    o, S = _run(inp)
    args = [inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = O.recurrence(*args, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"])
    eo, es = O.rel_max_err(host(o), o_ref), O.rel_max_err(host(S), S_ref)
    log("%s: err_o %.3e err_S %.3e" % (label, eo, es))
    assert eo <= tol(inp["io"]) and es <= tol(inp["io"])
    return o, S


def test_tiny_fp32_workload_full():
    """B=1, H=2, T=256, d=64, all fp32, S0 = 0: whole output against the oracle."""
    _check_all(W.make_chunk_inputs(W.TINY_F32), "tiny_f32")


@pytest.mark.parametrize("io,D", [(W.BF16, 128), (W.BF16, 64), (W.F32, 128), (W.F32, 64)])
def test_dense_ragged_with_state(io, D):
    """Several chunks and a ragged tail (T = 200 = 3*64 + 8), nonzero S0."""
    wl = W.ChunkWorkload("dense_test", 2, 200, 3, D, D, io, 555 + D, with_S0=True)
    _check_all(W.make_chunk_inputs(wl), "dense io=%s D=%d" % (io, D))


@pytest.mark.parametrize("io", [W.BF16, W.F32])
def test_varlen_edge_lengths(io):
    """Packed sequences of lengths 1, 63, 64, 65, 130, 0 and 7 with S0."""
    wl = W.ChunkWorkload("varlen_test", 1, 0, 2, 128, 128, io, 777, with_S0=True, n_seqs=7)
    _check_all(W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7]), "varlen io=%s" % io)


@pytest.mark.parametrize("io,B", [(W.BF16, 4), (W.BF16, 8), (W.F32, 4)])
def test_slab_widths(io, B):
    """H = 16 with B = 4 and 8 (64 and 128 chains): the propagation's 32- and
    64-column value slabs at a size the oracle checks whole (the cases above
    take 16-column slabs)."""
    wl = W.ChunkWorkload("slab_test", B, 70, 16, 128, 128, io, 999 + B, with_S0=True)
    _check_all(W.make_chunk_inputs(wl), "slabs io=%s chains=%d" % (io, 16 * B))


def test_erase_gate_range_zero_to_two():
    """The kernels do not assume b <= 1 (widened [0, 2] erase range)."""
    wl = W.ChunkWorkload("b2_test", 1, 192, 2, 128, 128, W.BF16, 888, with_S0=True)
    _check_all(W.make_chunk_inputs(wl, b_scale=2.0), "b in [0,2]")


def test_long_sequence():
    """One 32768-token sequence (512 chunks in one chain), H = 2, nonzero S0:
    the state carried through a long propagation, whole output checked."""
    wl = W.ChunkWorkload("long_test", 1, 32768, 2, 128, 128, W.BF16, 5151, with_S0=True)
    _check_all(W.make_chunk_inputs(wl), "long sequence T=32768")


@pytest.mark.parametrize("case", ["no_decay_no_erase", "strong_decay"])
def test_degenerate_gates(case):
    """Gate settings at the ends of their ranges: log alpha = 0 with b = 0 (the
    state only accumulates, linear attention), and per-token decay of 2 to
    2.5 nats (up to 160 nats per chunk, near the decay precondition), where the
    midpoint-scaled factors span e^{+-80}."""
    wl = W.ChunkWorkload("degen_test", 2, 200, 2, 128, 128, W.BF16, 6161, with_S0=True)
    if case == "no_decay_no_erase":
        inp = W.make_chunk_inputs(wl, log_alpha_range=(0.0, 0.0), b_scale=0.0)
    else:
        inp = W.make_chunk_inputs(wl, log_alpha_range=(-2.5, -2.0))
    _check_all(inp, "degenerate gates: %s" % case)


def test_empty_sequence_returns_initial_state():
    import torch
    wl = W.ChunkWorkload("empty_test", 2, 64, 2, 128, 128, W.BF16, 999, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    d = upload_chunk(inp)
    z = d["q"][:, :0].contiguous()
    zf = d["log_alpha"][:, :0].contiguous()
    o, S = g.chunk_fwd(z, z, z, zf, zf, zf, S0=d["S0"])
    torch.cuda.synchronize()
    assert o.shape[1] == 0
    assert torch.equal(S, d["S0"])


def test_empty_call_without_initial_state_gives_zero_state():
    """T == 0 with no S0: S_final = 0 (the token and output pointers are NULL)."""
    import torch
    z = torch.empty((2, 0, 3, 64), dtype=torch.bfloat16, device="cuda")
    zf = torch.empty((2, 0, 3, 64), dtype=torch.float32, device="cuda")
    S = torch.full((2, 3, 64, 64), 7.0, device="cuda")
    o, S = g.chunk_fwd(z, z, z, zf, zf, zf, S_final=S)
    torch.cuda.synchronize()
    assert o.shape[1] == 0
    assert torch.count_nonzero(S).item() == 0


def test_deterministic_bitwise():
    import torch
    inp = W.make_chunk_inputs(W.SEQ_4K, T=300, H=4)
    d = upload_chunk(inp)
    o1, S1 = _run(inp, d)
    o2, S2 = _run(inp, d)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_state_passing_split_sequence():
    """run(x1 || x2) == run(x2, S0 = run(x1).S_final) on the GPU (resume)."""
    import torch
    wl = W.ChunkWorkload("split_test", 2, 320, 2, 128, 128, W.BF16, 1234, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    d = upload_chunk(inp)
    o, S = _run(inp, d)
    keys = ("q", "k", "v", "log_alpha", "b", "w")
    d1 = {k_: d[k_][:, :128].contiguous() for k_ in keys}
    d2 = {k_: d[k_][:, 128:].contiguous() for k_ in keys}
    o1, S1 = g.chunk_fwd(*(d1[k_] for k_ in keys), S0=d["S0"])
    o2, S2 = g.chunk_fwd(*(d2[k_] for k_ in keys), S0=S1)
    torch.cuda.synchronize()
    assert O.rel_max_err(host(torch.cat([o1, o2], 1)), host(o)) <= 2e-2
    assert O.rel_max_err(host(S2), host(S)) <= 2e-2


def test_final_state_aliases_initial_state():
    import torch
    wl = W.ChunkWorkload("alias_test", 1, 130, 2, 128, 128, W.BF16, 4321, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    d = upload_chunk(inp)
    o_ref, S_ref = _run(inp, d)
    S_io = d["S0"].clone()
    g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=S_io, S_final=S_io)
    torch.cuda.synchronize()
    assert torch.equal(S_io, S_ref)


# ---------------------------------------------------------------------------
# Per-stage parity: the intermediates the chunk-factor kernel leaves in the
# workspace (cumulative decay via Qhat/Khat/gamma_last, the solved T, W, M)
# ---------------------------------------------------------------------------

def _ws_view(ws, off, count, dtype, shape):
    import torch
    esz = 2 if dtype == torch.bfloat16 else 4
    return ws[off:off + count * esz].view(dtype).reshape(shape)


def _frag_order(R, K, bf16):
    """Flat index of X[r][k] for an R x K matrix stored in MFMA fragment order
    (the layout the header documents)."""
    KS, KPL = (32, 8) if bf16 else (4, 1)
    r = np.arange(R)[:, None]
    k = np.arange(K)[None, :]
    return ((r // 16) * (K // KS) + k // KS) * 64 * KPL + ((r % 16) + 16 * ((k % KS) // KPL)) * KPL \
        + k % KPL


def _unfrag(flat, R, K, bf16):
    """[..., R*K] in fragment order -> [..., R, K]."""
    return flat[..., _frag_order(R, K, bf16)]


@pytest.mark.parametrize("io,D,lengths", [(W.F32, 64, None), (W.BF16, 128, None),
                                          (W.BF16, 128, [70, 5, 64])])
def test_chunk_factors_in_workspace(io, D, lengths):
    import torch
    if lengths is None:
        wl = W.ChunkWorkload("factors_test", 1, 200, 2, D, D, io, 2468)
        inp = W.make_chunk_inputs(wl)
    else:
        wl = W.ChunkWorkload("factors_vl", 1, 0, 2, D, D, io, 2469, n_seqs=len(lengths))
        inp = W.make_chunk_inputs(wl, lengths=lengths)
    varlen = inp["cu_seqlens"] is not None
    N, B, T, H = inp["N"], inp["B"], inp["T"], inp["H"]
    ioc = g.GDN2_BF16 if io == W.BF16 else g.GDN2_F32
    L = g.gdn2_chunk_fwd_workspace_layout(N, B, T, H, D, D, ioc, varlen)
    # NaN bytes everywhere first: whatever the kernel leaves unwritten shows up
    ws = torch.full((L.total_bytes_with_Tinv,), 0xFF, dtype=torch.uint8, device="cuda")
    _run(inp, workspace=ws, stages=g.GDN2_STAGE_ALL | g.GDN2_STAGE_STORE_T)
    tdt = torch.bfloat16 if io == W.BF16 else torch.float32
    nch = L.max_chunks
    Tw = host(_ws_view(ws, L.off_Tinv, nch * H * 4096, tdt, (nch, H, 64, 64)))
    bf = io == W.BF16
    Ww = _unfrag(host(_ws_view(ws, L.off_W, nch * H * 64 * D, tdt, (nch, H, 64 * D))), 64, D, bf)
    Qw = _unfrag(host(_ws_view(ws, L.off_Qhat, nch * H * 64 * D, tdt, (nch, H, 64 * D))), 64, D, bf)
    Kw = _unfrag(host(_ws_view(ws, L.off_KhatT, nch * H * 64 * D, tdt, (nch, H, 64 * D))), D, 64, bf)
    Mw = _unfrag(host(_ws_view(ws, L.off_M, nch * H * 4096, tdt, (nch, H, 4096))), 64, 64, bf)
    # M's fragments wholly above the diagonal (16-row block rb, KS-column block
    # kb with kb*KS > 16*rb + 15) are not stored; everything else is
    KS = 32 if bf else 4
    rr, cc = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    m_unused = (cc // KS) * KS > 16 * (rr // 16) + 15
    Mw = np.where(m_unused, 0.0, Mw)
    Gw = host(_ws_view(ws, L.off_gamma_last, nch * H * D, torch.float32, (nch, H, D)))
    # U is stored in MFMA accumulator order: [I][cb][lane][r] -> U[16I + 4(lane/16) + r][16cb + lane%16]
    Us = host(_ws_view(ws, L.off_U, nch * H * 64 * D, tdt, (nch, H, 4, D // 16, 4, 16, 4)))
    Uw = Us.transpose(0, 1, 2, 4, 6, 3, 5).reshape(nch, H, 64, D)
    # chunk list in id order: (row, first token, length)
    chunks = []
    if varlen:
        cu = inp["cu_seqlens"]
        for n in range(N):
            for t0 in range(int(cu[n]), int(cu[n + 1]), 64):
                chunks.append((0, t0, min(64, int(cu[n + 1]) - t0)))
    else:
        for n in range(B):
            for t0 in range(0, T, 64):
                chunks.append((n, t0, min(64, T - t0)))
    Mraw = _unfrag(host(_ws_view(ws, L.off_M, nch * H * 4096, tdt, (nch, H, 4096))), 64, 64, bf)
    assert np.isnan(Mraw[:len(chunks)][..., m_unused]).all()
    assert not np.isnan(Mraw[:len(chunks)][..., ~m_unused]).any()
    bound = 1e-2 if io == W.BF16 else 1e-5
    worst = {}
    for cid, (row, t0, ln) in enumerate(chunks):
        for h in range(H):
            sl = (row, slice(t0, t0 + ln), h)
            f = O.chunk_factors(*(inp[x][sl] for x in ("q", "k", "v", "log_alpha", "b", "w")))
            pairs = {"Tinv": (Tw[cid, h, :ln, :ln], f["Tinv"]),
                     "W": (Ww[cid, h, :ln], f["W"]),
                     "U": (Uw[cid, h, :ln], f["U"]),
                     "Qhat": (Qw[cid, h, :ln], f["Qhat"]),
                     "KhatT": (Kw[cid, h, :, :ln], f["Khat"].T),
                     "M": (Mw[cid, h, :ln, :ln], f["M"]),
                     "gamma_last": (Gw[cid, h], f["gamma_last"])}
            for name, (got, ref) in pairs.items():
                worst[name] = max(worst.get(name, 0.0), O.rel_max_err(got, ref))
            # padding rows/columns past the chunk's length
            assert np.all(Ww[cid, h, ln:] == 0) and np.all(Qw[cid, h, ln:] == 0)
            assert np.all(Uw[cid, h, ln:] == 0)
            assert np.all(Kw[cid, h, :, ln:] == 0) and np.all(Mw[cid, h, ln:] == 0)
            assert np.all(Mw[cid, h, :, ln:] == 0)
            np.testing.assert_array_equal(Tw[cid, h, ln:, ln:], np.eye(64 - ln))
            assert np.all(Tw[cid, h, :ln, ln:] == 0) and np.all(Tw[cid, h, ln:, :ln] == 0)
    log("factors io=%s D=%d: %s" % (io, D, " ".join("%s %.2e" % kv for kv in worst.items())))
    for name, e in worst.items():
        assert e <= bound, (name, e)


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times, checked
# whole against the plain recurrence (every sequence, head, token and the final
# state)
# ---------------------------------------------------------------------------

def _check_whole(wl):
    inp = W.make_chunk_inputs(wl)
    log("%s: T=%d N=%d generated" % (wl.name, inp["T"], inp["N"]))
    o, S = _run(inp)
    o_h, S_h = host(o), host(S)
    del o, S
    args = [inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = O.recurrence(*args, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"])
    eo, es = O.rel_max_err(o_h, o_ref), O.rel_max_err(S_h, S_ref)
    # the worst (sequence, head) chain, to show where the error sits
    if inp["cu_seqlens"] is None:
        per = np.abs(o_h - o_ref).max(axis=(1, 3))           # [B, H]
    else:
        per = np.abs(o_h - o_ref)[0].max(axis=2)              # [T, H]
    log("%s (whole): err_o %.3e err_S %.3e; worst |do| %.3e at %s; max|o| %.3e"
        % (wl.name, eo, es, per.max(), np.unravel_index(per.argmax(), per.shape),
           np.abs(o_ref).max()))
    assert eo <= tol(wl.io) and es <= tol(wl.io)
    assert np.isfinite(S_h).all()


def test_seq_4k_workload_whole():
    """B=1, H=16, T=4096, d=128 (16 chains of 64 dependent chunk steps)."""
    _check_whole(W.SEQ_4K)


def test_batch_4k_workload_whole():
    """B=8, H=16, T=4096, d=128, S0 != 0 (the benchmark's workload)."""
    _check_whole(W.BATCH_4K)


def test_varlen_workload_whole():
    """32 packed sequences of 512..8192 tokens, H=16, d=128."""
    _check_whole(W.VARLEN)


def _check_gate_logits(inp, label):
    import torch
    io = inp["io"]
    q, k, v = dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io)
    la, bl, wl_ = (dev(inp[x], W.BF16) for x in ("log_alpha", "b_logit", "w_logit"))
    o, S = g.chunk_fwd_gate_logits(q, k, v, la, bl, wl_, S0=dev(inp["S0"]),
                                   cu_seqlens=dev(inp["cu_seqlens"]))
    torch.cuda.synchronize()
    b, w = O.gates_from_logits(inp["b_logit"], inp["w_logit"])
    o_ref, S_ref = O.recurrence(inp["q"], inp["k"], inp["v"], inp["log_alpha"], b, w,
                                S0=inp["S0"], cu_seqlens=inp["cu_seqlens"])
    eo, es = O.rel_max_err(host(o), o_ref), O.rel_max_err(host(S), S_ref)
    log("%s: err_o %.3e err_S %.3e" % (label, eo, es))
    assert eo <= tol(io) and es <= tol(io)


@pytest.mark.parametrize("D", [64, 128])
def test_gate_logits_dense(D):
    """bf16 log alpha and gate logits, sigmoid in the kernel; ragged tail, S0."""
    wl = W.ChunkWorkload("logits_dense", 2, 200, 3, D, D, W.BF16, 666 + D, with_S0=True)
    _check_gate_logits(W.make_chunk_inputs(wl, gate_logits=True), "gate logits D=%d" % D)


def test_gate_logits_varlen():
    wl = W.ChunkWorkload("logits_varlen", 1, 0, 2, 128, 128, W.BF16, 668, with_S0=True, n_seqs=7)
    _check_gate_logits(W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7], gate_logits=True),
                       "gate logits varlen")

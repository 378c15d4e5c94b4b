"""GPU parity of gdn2_chunk_bwd against the fp64 oracle's reverse recurrence
(oracle.recurrence_bwd): every gradient, dense and packed calls, ragged tails,
with and without initial state and final-state gradient, for bf16 I/O (bound
2e-2) and fp32 I/O (bound 1e-4)."""

import numpy as np
import pytest

import gated_delta_rule_47_amd as g
import oracle as O
import workloads as W
from gpu_util import dev, host, log, tol, upload_chunk

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")
# The forward's parity bound on max|err| / max|ref| for the io dtype (2e-2
# for bf16), applied to every gradient: the bf16 factors and the bf16
# gradient outputs keep the measured agreement within about 1e-2.
TOL = tol(W.BF16)


def _run_bwd(inp, grads):
    import torch
    d = upload_chunk(inp)
    dout = dev(grads["dout"], inp["io"])
    dSf = dev(grads["dS_final"])
    out = g.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dout, S0=d["S0"],
                      dS_final=dSf, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return out


def _check(inp, grads, label):
    out = _run_bwd(inp, grads)
    ref = O.recurrence_bwd(*(inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")),
                           grads["dout"], inp["S0"], grads["dS_final"], inp["cu_seqlens"])
    errs = {n: O.rel_max_err(host(out[n]), ref[n]) for n in NAMES}
    log("%s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())))
    for n, e in errs.items():
        assert e <= TOL, (n, e)
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_dense_ragged(D):
    """T = 150 (two full chunks and a 22-token tail), S0 and dS_final nonzero."""
    wl = W.ChunkWorkload("bwd_dense", 2, 150, 2, D, D, W.BF16, 4242 + D, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    _check(inp, W.make_chunk_grads(inp, 11 + D), "bwd dense D=%d" % D)


def test_bwd_no_state_no_final_grad():
    """S0 = NULL and dS_final = NULL (zero), a single short chunk."""
    wl = W.ChunkWorkload("bwd_nostate", 1, 40, 2, 128, 128, W.BF16, 4343)
    inp = W.make_chunk_inputs(wl)
    _check(inp, W.make_chunk_grads(inp, 12, with_dS_final=False), "bwd no state")


def test_bwd_varlen_edge_lengths():
    """Packed sequences of lengths 1, 63, 64, 65, 130, 0 and 7."""
    wl = W.ChunkWorkload("bwd_varlen", 1, 0, 2, 128, 128, W.BF16, 4444, with_S0=True, n_seqs=7)
    inp = W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7])
    _check(inp, W.make_chunk_grads(inp, 13), "bwd varlen")


def test_bwd_varlen_many_chains():
    """Packed sequences of lengths 0-200 on H = 8 heads (9 sequences, 72
    chains): the reverse pass's 8-wave workgroups driven by the chunk table."""
    lengths = [200, 0, 65, 1, 128, 63, 130, 7, 64]
    wl = W.ChunkWorkload("bwd_varlen_many", 1, 0, 8, 128, 128, W.BF16, 4545, with_S0=True,
                         n_seqs=len(lengths))
    inp = W.make_chunk_inputs(wl, lengths=lengths)
    _check(inp, W.make_chunk_grads(inp, 14), "bwd varlen 72 chains")


@pytest.mark.parametrize("B,D", [(4, 128), (16, 128), (4, 64), (16, 64)])
def test_bwd_many_chains(B, D):
    """H = 16 with B = 4 and 16 (64 and 256 chains), d = 64 and 128: the
    reverse pass's 8-wave workgroups on 64-column slabs (two 32-column halves)
    and its 4-wave workgroups on 64-column slabs (the small cases above take
    32-column slabs in two 16-column halves)."""
    wl = W.ChunkWorkload("bwd_many", B, 70, 16, D, D, W.BF16, 4646 + B + D, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    _check(inp, W.make_chunk_grads(inp, 15 + B + D), "bwd %d chains d=%d" % (B * 16, D))


@pytest.mark.parametrize("case", ["no_decay_no_erase", "strong_decay"])
def test_bwd_degenerate_gates(case):
    """log alpha = 0 with b = 0, and 2 to 2.5 nats of decay per token (up to
    160 per chunk, near the decay precondition)."""
    wl = W.ChunkWorkload("bwd_degen", 2, 150, 2, 128, 128, W.BF16, 4747, with_S0=True)
    if case == "no_decay_no_erase":
        inp = W.make_chunk_inputs(wl, log_alpha_range=(0.0, 0.0), b_scale=0.0)
    else:
        inp = W.make_chunk_inputs(wl, log_alpha_range=(-2.5, -2.0))
    _check(inp, W.make_chunk_grads(inp, 16), "bwd %s" % case)


def test_bwd_erase_gate_to_two():
    wl = W.ChunkWorkload("bwd_b2", 1, 128, 2, 128, 128, W.BF16, 4545, with_S0=True)
    inp = W.make_chunk_inputs(wl, b_scale=2.0)
    _check(inp, W.make_chunk_grads(inp, 14), "bwd b in [0,2]")


def test_bwd_deterministic_bitwise():
    import torch
    wl = W.ChunkWorkload("bwd_det", 2, 200, 3, 128, 128, W.BF16, 4646, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    grads = W.make_chunk_grads(inp, 15)
    a = _run_bwd(inp, grads)
    b = _run_bwd(inp, grads)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


# ---------------------------------------------------------------------------
# fp32 I/O: the same gradients at the all-fp32 bound (1e-4 of max |ref|)
# ---------------------------------------------------------------------------

def _check_f32(inp, grads, label):
    out = _run_bwd(inp, grads)
    ref = O.recurrence_bwd(*(inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")),
                           grads["dout"], inp["S0"], grads["dS_final"], inp["cu_seqlens"])
    errs = {n: O.rel_max_err(host(out[n]), ref[n]) for n in NAMES}
    log("%s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())))
    for n, e in errs.items():
        assert e <= tol(W.F32), (n, e)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_f32_dense_ragged(D):
    """fp32: T = 150 (a 22-token tail), S0 and dS_final nonzero."""
    wl = W.ChunkWorkload("bwd_f32_dense", 2, 150, 2, D, D, W.F32, 5242 + D, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    _check_f32(inp, W.make_chunk_grads(inp, 21 + D), "bwd f32 dense D=%d" % D)


def test_bwd_f32_no_state_no_final_grad():
    wl = W.ChunkWorkload("bwd_f32_nostate", 1, 40, 2, 128, 128, W.F32, 5343)
    inp = W.make_chunk_inputs(wl)
    _check_f32(inp, W.make_chunk_grads(inp, 22, with_dS_final=False), "bwd f32 no state")


def test_bwd_f32_varlen_edge_lengths():
    wl = W.ChunkWorkload("bwd_f32_varlen", 1, 0, 2, 128, 128, W.F32, 5444, with_S0=True,
                         n_seqs=7)
    inp = W.make_chunk_inputs(wl, lengths=[1, 63, 64, 65, 130, 0, 7])
    _check_f32(inp, W.make_chunk_grads(inp, 23), "bwd f32 varlen")


def test_bwd_f32_many_chains():
    """16 chains over 3 chunks each, d = 64."""
    wl = W.ChunkWorkload("bwd_f32_many", 4, 130, 4, 64, 64, W.F32, 5545, with_S0=True)
    inp = W.make_chunk_inputs(wl)
    _check_f32(inp, W.make_chunk_grads(inp, 24), "bwd f32 16 chains")


def test_bwd_f32_erase_gate_to_two():
    wl = W.ChunkWorkload("bwd_f32_b2", 1, 128, 2, 128, 128, W.F32, 5646, with_S0=True)
    inp = W.make_chunk_inputs(wl, b_scale=2.0)
    _check_f32(inp, W.make_chunk_grads(inp, 25), "bwd f32 b in [0,2]")


@pytest.mark.parametrize("case", ["no_decay_no_erase", "strong_decay"])
def test_bwd_f32_degenerate_gates(case):
    wl = W.ChunkWorkload("bwd_f32_degen", 2, 150, 2, 128, 128, W.F32, 5747, with_S0=True)
    if case == "no_decay_no_erase":
        inp = W.make_chunk_inputs(wl, log_alpha_range=(0.0, 0.0), b_scale=0.0)
    else:
        inp = W.make_chunk_inputs(wl, log_alpha_range=(-2.5, -2.0))
    _check_f32(inp, W.make_chunk_grads(inp, 26), "bwd f32 %s" % case)


def test_bwd_f32_tiny_workload():
    """The tiny fp32 workload (B=1, H=2, T=256, d=64) with upstream gradients."""
    inp = W.make_chunk_inputs(W.TINY_F32)
    _check_f32(inp, W.make_chunk_grads(inp, 27), "bwd f32 tiny workload")


def test_bwd_full_batch_workload_sampled():
    """B=8, H=16, T=4096, d=128 (the batch workload) in the launch configuration
    the benchmark times; sampled (sequence, head) pairs against the plain
    reverse recurrence (oracle.recurrence_bwd)."""
    inp = W.make_chunk_inputs(W.BATCH_4K)
    grads = W.make_chunk_grads(inp, 1)
    out = _run_bwd(inp, grads)
    out = {n: host(t) for n, t in out.items()}
    worst = {}
    for n, h in [(0, 0), (2, 5), (5, 9), (7, 15)]:
        sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
        ref = O.recurrence_bwd(*(inp[x][sl] for x in ("q", "k", "v", "log_alpha", "b", "w")),
                               grads["dout"][sl], inp["S0"][n:n + 1, h:h + 1],
                               grads["dS_final"][n:n + 1, h:h + 1])
        errs = {}
        for name in NAMES:
            got = out[name][n:n + 1, h:h + 1] if name == "dS0" else out[name][sl]
            errs[name] = O.rel_max_err(got, ref[name])
            worst[name] = max(worst.get(name, 0.0), errs[name])
        log("bwd batch (%d,%d): %s" % (n, h, " ".join("%s %.2e" % kv for kv in errs.items())))
    for name, e in worst.items():
        assert e <= TOL, (name, e)

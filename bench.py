#!/usr/bin/env python3
"""Benchmark of libgdn2 on one MI355X.

Headline step: one gdn2_chunk_fwd over the training-batch workload
(B=8, H=16, T=4096, d_k=d_v=128, bf16 q/k/v/o, fp32 gates and state, nonzero
initial state), inputs resident in HBM.  value = tokens/s (B*T tokens per
step, 16 heads each).  The two kernels of the call (chunk factors, state
propagation) are bracketed with HIP events on the stream they run on, which
gives each kernel's duration and the roofline of the dominant one.

Also measured in the same run (each in its own object of the JSON line):
  seq / tiny: gdn2_chunk_fwd on the single-sequence 4K workload (B=1, H=16,
          16 chains of 64 dependent chunk steps) and on the tiny fp32 one;
  context_sweep: the same 16K tokens as B x T = 8 x 2K, 4 x 4K, 2 x 8K, 1 x 16K;
  decode: gdn2_step on B=256, H=16, d=128 (fp32 state, in place) over 1024
          distinct pre-generated steps, GB/s of its algorithmic traffic;
  varlen: the 32-sequence packed workload; gate_logits: the batch workload with
          bf16 gate logits; training_step: the recomputing and the saved-state
          backward after their forwards; backward, layer, swa: the backward, the
          token-mixer layer and the sliding-window attention (and its layer).
cpu_baseline: the fp64 numpy oracle over the whole batch workload, its
(sequence, head) chains spread over a process pool on this host's cores, plus
one-core figures for the tiny and single-sequence workloads.  Work that starts
worker processes (the baseline, the decode inputs) runs before the GPU is
initialised.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --calibrate-copy   (plain copy of known size, for PMC scaling)
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--only", choices=["all", "chunk", "decode", "varlen", "bwd", "layer", "swa",
                                       "seq", "sweep"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers", type=int, default=0,
                    help="host worker processes (default: the usable cores, at most 16; "
                         "1 runs the host-side work in this process, as profiled runs need)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain device copy of 1 GiB (5 times) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Algorithmic byte counts (what the operation must read and write once)
# ---------------------------------------------------------------------------

def chunk_alg_bytes(n_tok_heads, n_states, d, io_bytes):
    """Algorithmic bytes, split by the kernel that moves them: the chunk-factor
    kernel reads every per-token input (q, k, v in the io type; log_alpha, b,
    w in fp32); the propagation kernel reads the initial state and writes o
    and the final state.  The chunk factors passed between the two kernels
    through the workspace are not algorithmic bytes."""
    factors = n_tok_heads * (3 * d * io_bytes + 3 * d * 4)
    prop = n_tok_heads * d * io_bytes + n_states * 2 * d * d * 4
    return factors, prop


def decode_alg_bytes(B, H, d, io_bytes):
    per = 2 * d * d * 4 + 3 * d * io_bytes + 3 * d * 4 + d * io_bytes
    return B * H * per


def chunk_flops_dense(n_chunk_heads, d):
    """MFMA flops per chunk-head as issued (dense 64-row tiles):
    A, M (64x64xd), W (64xdx64), U (64xdx64), W S, Qhat S (64xdxd),
    M U_eff (64xdx64), Khat^T U_eff (dxdx64)."""
    c = 64
    per = 2 * (2 * c * c * d + c * d * c + c * d * c + 2 * c * d * d + c * d * c + d * d * c)
    return n_chunk_heads * per


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_47_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload, digest):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------

def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(5):
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy %d: %d bytes read, %d bytes written" % (i, n, n))
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))


def upload(inp):
    import torch
    import workloads as W

    def dev(x, io=None):
        if x is None:
            return None
        if io == W.BF16:
            return torch.from_numpy(W.bf16_bits(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    io = inp["io"]
    return dict(q=dev(inp["q"], io), k=dev(inp["k"], io), v=dev(inp["v"], io),
                log_alpha=dev(inp["log_alpha"]), b=dev(inp["b"]), w=dev(inp["w"]),
                S0=dev(inp["S0"]), cu_seqlens=dev(inp["cu_seqlens"]))


def time_chunk(d, inp, steps, warmup):
    """Time `steps` forward calls; each call's two stages bracketed by events."""
    import torch
    import gated_delta_rule_47_amd as g
    B, T, H, D = inp["B"], inp["T"], inp["H"], inp["Dk"]
    N = inp["N"]
    o = torch.empty((B, T, H, D), dtype=d["q"].dtype, device="cuda")
    S = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    io = g.GDN2_BF16 if d["q"].dtype == torch.bfloat16 else g.GDN2_F32
    varlen = d["cu_seqlens"] is not None
    ws = torch.empty(g.gdn2_chunk_fwd_workspace_bytes(N, B, T, H, D, D, io, varlen),
                     dtype=torch.uint8, device="cuda")
    args = dict(S0=d["S0"], cu_seqlens=d["cu_seqlens"], o=o, S_final=S, workspace=ws)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    first = g.GDN2_STAGE_PLAN | g.GDN2_STAGE_FACTORS
    for _ in range(warmup):
        g.chunk_fwd(*x, **args)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        g.chunk_fwd(*x, **args, stages=first)
        ev[i][1].record()
        g.chunk_fwd(*x, **args, stages=g.GDN2_STAGE_PROPAGATE)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    p_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    # one plain gdn2_chunk_fwd pass, to confirm the staged calls give its result
    o2 = torch.empty_like(o)
    S2 = torch.empty_like(S)
    g.chunk_fwd(*x, S0=d["S0"], cu_seqlens=d["cu_seqlens"], o=o2, S_final=S2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2), "staged calls differ from one call"
    return wall / steps * 1e3, f_ms, p_ms


# ---------------------------------------------------------------------------
# Host-side work done in worker processes, before the GPU is initialised
# ---------------------------------------------------------------------------

def host_workers(requested=0):
    """Worker processes for host-side work: the usable cores, at most 16."""
    n = len(os.sched_getaffinity(0))
    return max(1, min(requested or n, n, 16))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_POOL_INP = None  # inputs shared with forked workers (read only)


def _oracle_chain(nh):
    """The oracle on one (sequence, head) chain of _POOL_INP."""
    import oracle as O
    n, h = nh
    inp = _POOL_INP
    sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
    S0 = None if inp["S0"] is None else inp["S0"][n:n + 1, h:h + 1]
    _, S = O.recurrence(*(inp[x][sl] for x in ("q", "k", "v", "log_alpha", "b", "w")), S0=S0)
    return float(abs(S).sum())


def cpu_baseline(inp, workers):
    """The oracle as it stands, timed on this host: every (sequence, head)
    chain of the dense workload `inp`, spread over a pool of forked worker
    processes (one numpy thread each).  Returns (tokens/s, seconds, tokens)."""
    import multiprocessing as mp
    global _POOL_INP
    _POOL_INP = inp
    units = [(n, h) for n in range(inp["B"]) for h in range(inp["H"])]
    t0 = time.perf_counter()
    if workers == 1:  # in this process (profiled runs: no worker processes)
        for u in units:
            _oracle_chain(u)
    else:
        with mp.get_context("fork").Pool(workers) as pool:
            pool.map(_oracle_chain, units, chunksize=1)
    dt = time.perf_counter() - t0
    _POOL_INP = None
    n_tokens = inp["B"] * inp["T"]
    return n_tokens / dt, dt, n_tokens


def cpu_one_core(inp):
    """The oracle on a whole workload in this process (one core)."""
    import oracle as O
    t0 = time.perf_counter()
    O.recurrence(*(inp[x] for x in ("q", "k", "v", "log_alpha", "b", "w")), S0=inp["S0"],
                 cu_seqlens=inp["cu_seqlens"])
    dt = time.perf_counter() - t0
    return inp["B"] * inp["T"] / dt, dt


def _decode_step_packed(s):
    """Decode step s of the decode workload: bf16 bits of q, k, v (uint16) and
    the fp32 gates."""
    import workloads as W
    x = W.make_decode_step(W.DECODE, s)
    return (s, W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]), x["log_alpha"],
            x["b"], x["w"])


def pregenerate_decode(steps, workers):
    """All `steps` decode inputs (each step its own seeded stream), made by a
    pool of forked workers: uint16 [steps, B, H, D] for q, k, v and float32
    for log_alpha, b, w."""
    import multiprocessing as mp
    import workloads as W
    wl = W.DECODE
    shp = (steps, wl.B, wl.H, wl.Dk)
    out = dict(q=np.empty(shp, np.uint16), k=np.empty(shp, np.uint16), v=np.empty(shp, np.uint16),
               log_alpha=np.empty(shp, np.float32), b=np.empty(shp, np.float32),
               w=np.empty(shp, np.float32))
    def keep(s, *arrs):
        for name, arr in zip(("q", "k", "v", "log_alpha", "b", "w"), arrs):
            out[name][s] = arr
    if workers == 1:  # in this process (profiled runs: no worker processes)
        for s in range(steps):
            keep(*_decode_step_packed(s))
        return out
    with mp.get_context("fork").Pool(workers) as pool:
        for res in pool.imap_unordered(_decode_step_packed, range(steps), chunksize=4):
            keep(*res)
    return out


def time_decode(pre):
    """gdn2_step over the decode workload: every step reads its own
    pre-generated inputs (uploaded before timing); each launch is bracketed
    by events on the launch stream."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W
    wl = W.DECODE
    steps = pre["q"].shape[0]
    S = torch.from_numpy(W.make_decode_state(wl)).to("cuda")
    dev = {}
    for name in ("q", "k", "v"):
        dev[name] = torch.from_numpy(pre[name].view(np.int16)).to("cuda").view(torch.bfloat16)
    for name in ("log_alpha", "b", "w"):
        dev[name] = torch.from_numpy(pre[name]).to("cuda")
    xs = [tuple(dev[n][i] for n in ("q", "k", "v", "log_alpha", "b", "w")) for i in range(steps)]
    o = torch.empty((wl.B, wl.H, wl.Dv), dtype=torch.bfloat16, device="cuda")
    S_warm = S.clone()
    for i in range(3):
        g.step(*xs[i], S_warm, o=o)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i].record()
        g.step(*xs[i], S, o=o)
    ev[steps].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    assert torch.isfinite(S).all()
    return wall, float(np.mean(per)), float(np.median(per))


def time_gate_logits(inp, steps, warmup):
    """gdn2_chunk_fwd_gate_logits over the batch workload.  Returns the whole call's
    time, the chunk-factor part (whole call minus propagation) and the propagation
    alone, timed as the PROPAGATE stage on the workspace the call filled."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W

    def bf(x):
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    q, k, v = bf(inp["q"]), bf(inp["k"]), bf(inp["v"])
    la, bl, wl = bf(inp["log_alpha"]), bf(inp["b_logit"]), bf(inp["w_logit"])
    S0 = torch.from_numpy(inp["S0"]).to("cuda")
    B, T, H, D, N = inp["B"], inp["T"], inp["H"], inp["Dk"], inp["N"]
    ws = torch.empty(g.gdn2_chunk_fwd_workspace_bytes(N, B, T, H, D, D, g.GDN2_BF16, 0),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        g.chunk_fwd_gate_logits(q, k, v, la, bl, wl, S0=S0, o=o, S_final=S, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.chunk_fwd_gate_logits(q, k, v, la, bl, wl, S0=S0, o=o, S_final=S, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # propagation alone (it reads only the workspace the call above filled)
    e0.record()
    for _ in range(steps):
        g.gdn2_chunk_fwd_stages(q.data_ptr(), k.data_ptr(), v.data_ptr(), la.data_ptr(),
                                bl.data_ptr(), wl.data_ptr(), S0.data_ptr(), o.data_ptr(),
                                S.data_ptr(), None, N, B, T, H, D, D, g.GDN2_BF16, ws.data_ptr(),
                                ws.numel(), torch.cuda.current_stream().cuda_stream,
                                g.GDN2_STAGE_PROPAGATE)
    e1.record()
    torch.cuda.synchronize()
    p_ms = e0.elapsed_time(e1) / steps
    return ms, ms - p_ms, p_ms


def bwd_alg_bytes(n_th, chains, D, io_bytes):
    """Backward: reads q, k, v, dout (io) and log_alpha, b, w (fp32), writes dq, dk, dv (io)
    and dlog_alpha, db, dw (fp32), per token-head; S0 and dS_final in, dS0 out per chain."""
    per_th = D * (7 * io_bytes + 6 * 4)
    return n_th * per_th + chains * 3 * D * D * 4


def time_bwd(d, inp, steps, warmup):
    """Time `steps` gdn2_chunk_bwd calls (events on the launch stream)."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W
    B, T, H, D, N = inp["B"], inp["T"], inp["H"], inp["Dk"], inp["N"]
    gr = W.make_chunk_grads(inp, 1)
    dout = torch.from_numpy(W.bf16_bits(gr["dout"]).view(np.int16)).to("cuda").view(torch.bfloat16)
    dSf = torch.from_numpy(gr["dS_final"]).to("cuda")
    varlen = d["cu_seqlens"] is not None
    ws = torch.empty(g.gdn2_chunk_bwd_workspace_bytes(N, B, T, H, D, D, g.GDN2_BF16, varlen),
                     dtype=torch.uint8, device="cuda")
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dout)
    kw = dict(S0=d["S0"], dS_final=dSf, cu_seqlens=d["cu_seqlens"], workspace=ws)
    for _ in range(warmup):
        g.chunk_bwd(*x, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.chunk_bwd(*x, **kw)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, ws.numel()


def time_train(d, inp, steps, warmup):
    """A training step's chunk core both ways: gdn2_chunk_fwd + gdn2_chunk_bwd
    (the backward recomputes the forward's factors and states) against
    gdn2_chunk_fwd_train + gdn2_chunk_bwd_saved (the backward reuses them).
    Events on the launch stream around each call; returns a dict of ms."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W
    gr = W.make_chunk_grads(inp, 1)
    dout = torch.from_numpy(W.bf16_bits(gr["dout"]).view(np.int16)).to("cuda").view(torch.bfloat16)
    dSf = torch.from_numpy(gr["dS_final"]).to("cuda")
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    B, T, H, D, N = inp["B"], inp["T"], inp["H"], inp["Dk"], inp["N"]
    varlen = d["cu_seqlens"] is not None
    o = torch.empty((B, T, H, D), dtype=d["q"].dtype, device="cuda")
    S = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    ws_f = torch.empty(g.gdn2_chunk_fwd_workspace_bytes(N, B, T, H, D, D, g.GDN2_BF16, varlen),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(g.gdn2_chunk_bwd_workspace_bytes(N, B, T, H, D, D, g.GDN2_BF16, varlen),
                       dtype=torch.uint8, device="cuda")
    ws_t = torch.empty(g.gdn2_chunk_train_workspace_bytes(N, B, T, H, D, D, g.GDN2_BF16, varlen),
                       dtype=torch.uint8, device="cuda")
    kw = dict(S0=d["S0"], cu_seqlens=d["cu_seqlens"])

    def recompute():
        g.chunk_fwd(*x, **kw, o=o, S_final=S, workspace=ws_f)
        return g.chunk_bwd(*x, dout, **kw, dS_final=dSf, workspace=ws_b)

    def saved():
        g.chunk_fwd_train(*x, **kw, o=o, S_final=S, workspace=ws_t)
        return g.chunk_bwd_saved(*x, dout, ws_t, dS_final=dSf, cu_seqlens=d["cu_seqlens"])

    def timed(f0, f1):
        for _ in range(warmup):
            f0()
            f1()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            f0()
            ev[i][1].record()
            f1()
            ev[i][2].record()
        torch.cuda.synchronize()
        return (float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
                float(np.mean([e[1].elapsed_time(e[2]) for e in ev])))

    fwd_ms, bwd_ms = timed(lambda: g.chunk_fwd(*x, **kw, o=o, S_final=S, workspace=ws_f),
                           lambda: g.chunk_bwd(*x, dout, **kw, dS_final=dSf, workspace=ws_b))
    ftr_ms, bsv_ms = timed(lambda: g.chunk_fwd_train(*x, **kw, o=o, S_final=S, workspace=ws_t),
                           lambda: g.chunk_bwd_saved(*x, dout, ws_t, dS_final=dSf,
                                                     cu_seqlens=d["cu_seqlens"]))
    # the two ways give the same gradients
    a, b = recompute(), saved()
    torch.cuda.synchronize()
    assert all(torch.equal(a[n], b[n]) for n in a if a[n] is not None), "training pair differs"
    return dict(fwd_ms=fwd_ms, bwd_ms=bwd_ms, step_ms=fwd_ms + bwd_ms, fwd_train_ms=ftr_ms,
                bwd_saved_ms=bsv_ms, train_step_ms=ftr_ms + bsv_ms, workspace_bytes=ws_t.numel())


def time_layer(inp, steps, warmup):
    """Time `steps` gdn2_layer_fwd calls on the token-mixer layer workload
    (events on the launch stream).  Returns (ms, workspace bytes)."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W

    def bf(x):
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).to("cuda").view(torch.bfloat16)

    def f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    x, W_in, W_o = bf(inp["x"]), bf(inp["W_in"]), bf(inp["W_o"])
    cw, ab, nw = f32(inp["conv_w"]), f32(inp["alpha_bias"]), f32(inp["norm_w"])
    B, T, H, D, Dm, N = inp["B"], inp["T"], inp["H"], inp["Dk"], inp["D"], inp["N"]
    ws = torch.empty(g.gdn2_layer_fwd_workspace_bytes(N, B, T, H, D, D, Dm, 0), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((B, T, Dm), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    call = lambda: g.layer_fwd(x, W_in, cw, ab, nw, W_o, H, D, D, y=y, S_final=S, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, ws.numel()


def swa_useful_flops(lengths, H, D, window):
    """Flops of the unmasked score pairs: 2 D for q.k and 2 D for p v per pair."""
    pairs = 0
    for L in lengths:
        L = int(L)
        full = max(0, L - window)
        tri = min(L, window)
        pairs += tri * (tri + 1) // 2 + full * window
    return pairs * H * 4 * D


def time_swa(inp, steps, warmup):
    """Time `steps` gdn2_swa_fwd calls (events on the launch stream)."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W

    def bf(x):
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    q, k, v = bf(inp["q"]), bf(inp["k"]), bf(inp["v"])
    o = torch.empty_like(q)
    lse = torch.empty((inp["B"], inp["H"], inp["T"]), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        g.swa_fwd(q, k, v, inp["window"], o=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.swa_fwd(q, k, v, inp["window"], o=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_swa_layer(inp, steps, warmup):
    """Time `steps` gdn2_swa_layer_fwd calls (events on the launch stream)."""
    import torch
    import gated_delta_rule_47_amd as g
    import workloads as W

    def bf(x):
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    x, Wq, Wo = bf(inp["x"]), bf(inp["W_qkv"]), bf(inp["W_o"])
    B, T, H, D, Dm = inp["B"], inp["T"], inp["H"], inp["D"], inp["Dm"]
    ws = torch.empty(g.gdn2_swa_layer_fwd_workspace_bytes(B, B, T, H, D, Dm, 0), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((B, T, Dm), dtype=torch.bfloat16, device="cuda")
    call = lambda: g.swa_layer_fwd(x, Wq, Wo, H, D, inp["window"], y=y, return_lse=False,
                                   workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: libgdn2 has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import workloads as W

    # Host-side work that starts worker processes comes first: nothing below
    # it initialises the GPU until it is done.
    workers = host_workers(a.workers)
    do_chunk = a.only in ("all", "chunk")
    inp = None
    cpu = None
    if do_chunk and not a.calibrate_copy:
        log("generating %s" % W.BATCH_4K.name)
        inp = W.make_chunk_inputs(W.BATCH_4K)
        if not a.no_cpu_baseline:
            tps, dt, n = cpu_baseline(inp, workers)
            log("cpu oracle: %.1f tokens/s (%d tokens, %d workers, %.1f s)" % (tps, n, workers, dt))
            one = {}
            for wl in (W.TINY_F32, W.SEQ_4K):
                t1, d1 = cpu_one_core(W.make_chunk_inputs(wl))
                one[wl.name] = {"tokens_per_s": t1, "seconds": d1}
                log("cpu oracle, one core, %s: %.1f tokens/s (%.1f s)" % (wl.name, t1, d1))
            cpu = {"value": tps, "unit": "tokens/s", "cores": workers, "kind": "oracle",
                   "cpu_model": cpu_model(),
                   "sample": "fp64 numpy token recurrence over the whole %s workload (%d tokens "
                             "x 16 heads, S0 as in the workload): its %d (sequence, head) chains "
                             "on a pool of %d worker processes, one numpy thread each, %.1f s"
                             % (W.BATCH_4K.name, n, inp["B"] * inp["H"], workers, dt),
                   "one_core": one}
    decode_pre = None
    if a.only in ("all", "decode") and not a.calibrate_copy:
        t0 = time.perf_counter()
        decode_pre = pregenerate_decode(a.decode_steps, workers)
        log("decode inputs: %d steps generated in %.1f s" % (a.decode_steps,
                                                             time.perf_counter() - t0))

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.calibrate_copy:
        calibrate_copy()
        return
    import gated_delta_rule_47_amd as g
    g.load_library()
    out = {"metric": "tokens/s and MFMA util for gdn2_chunk_fwd (H16, d128, T4K); decode GB/s",
           "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; shapes of a 1.3B-parameter layer: 16 heads, 128x128 state)"}
    # The part's own figures beside the published peaks used in the rooflines:
    # a gfx950 CU retires 4096 dense bf16 MFMA flops and 256 fp32 vector flops
    # per clock.
    props = torch.cuda.get_device_properties(0)
    cus, khz = g.device_info(0)
    out["device"] = {"name": props.name, "arch": props.gcnArchName, "compute_units": cus,
                     "peak_clock_mhz": khz / 1e3, "hbm_gib": props.total_memory / 2**30,
                     "bf16_mfma_peak_tflops_from_clock": cus * 4096 * khz * 1e3 / 1e12,
                     "fp32_vector_peak_tflops_from_clock": cus * 256 * khz * 1e3 / 1e12,
                     "published_peaks": {"hbm_GBps": HBM_PEAK_GBS, "bf16_mfma_tflops": MFMA_BF16_PEAK_TFLOPS}}
    log("device: %s, %d CUs at %.0f MHz -> bf16 MFMA %.0f TFLOP/s from the clock"
        % (props.gcnArchName, cus, khz / 1e3, out["device"]["bf16_mfma_peak_tflops_from_clock"]))

    if do_chunk:
        wl = W.BATCH_4K
        d = upload(inp)
        ms, f_ms, p_ms = time_chunk(d, inp, a.steps, a.warmup)
        tokens = inp["B"] * inp["T"]
        n_th = tokens * inp["H"]
        fa, pa = chunk_alg_bytes(n_th, inp["N"] * inp["H"], inp["Dk"], 2)
        digest = source_digest("gdn2_chunk_prep.hip", "gdn2_chunk_prop.hip", "gdn2_device.h")
        kernels = {"chunk_factors": (f_ms, fa), "chunk_propagate": (p_ms, pa)}
        dom = max(kernels, key=lambda k: kernels[k][0])
        dms, dbytes = kernels[dom]
        achieved = dbytes / (dms * 1e-3) / 1e9
        flops = chunk_flops_dense(inp["B"] * (inp["T"] // 64) * inp["H"], inp["Dk"])
        out.update({
            "value": tokens / (ms * 1e-3),
            "ms_per_step": ms,
            "config": {"workload": wl.name, "B": inp["B"], "T": inp["T"], "H": inp["H"],
                       "d_k": inp["Dk"], "d_v": inp["Dv"], "chunk": 64, "io": "bf16",
                       "gates_state": "fp32", "S0": "N(0, 0.02^2)"},
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": stored_traffic(dom, wl.name, digest),
                         "traffic_source": "committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary "
                                           "of the same kernel source (null if it changed)",
                         "alg_bytes_per_launch": dbytes, "avg_launch_ms": dms},
            "kernels_ms": {"chunk_factors": f_ms, "chunk_propagate": p_ms},
            "path": {"alg_bytes": fa + pa, "alg_GBps": (fa + pa) / (ms * 1e-3) / 1e9,
                     "hbm_frac": (fa + pa) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "mfma_flops_issued": flops,
                     "mfma_frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
            "kernel_source_digest": digest,
        })
        log("chunk: %.3f ms/step (factors %.3f, propagate %.3f) -> %.3e tokens/s"
            % (ms, f_ms, p_ms, out["value"]))
        if cpu is not None:
            out["cpu_baseline"] = cpu
        del d, inp

    if a.only in ("all", "chunk", "seq"):
        # The single-sequence 4K workload (16 chains of 64 dependent chunk steps)
        # and the tiny fp32 one.
        for key, wl in (("seq", W.SEQ_4K), ("tiny", W.TINY_F32)):
            inp_s = W.make_chunk_inputs(wl)
            ms, f_ms, p_ms = time_chunk(upload(inp_s), inp_s, a.steps, a.warmup)
            tokens = inp_s["B"] * inp_s["T"]
            nchunks = (inp_s["T"] + 63) // 64
            out[key] = {"workload": wl.name, "io": wl.io, "ms": ms,
                        "tokens_per_s": tokens / (ms * 1e-3),
                        "kernels_ms": {"chunk_factors": f_ms, "chunk_propagate": p_ms},
                        "chunk_steps_per_chain": nchunks,
                        "us_per_chunk_step": p_ms * 1e3 / nchunks}
            log("%s: %.3f ms (factors %.3f, propagate %.3f = %.2f us per chunk step)"
                % (wl.name, ms, f_ms, p_ms, p_ms * 1e3 / nchunks))
            del inp_s

    if a.only in ("all", "sweep"):
        # The same 16K tokens (16 heads) as B x T = 8 x 2K, 4 x 4K, 2 x 8K, 1 x 16K.
        sweep = []
        for B, T in ((8, 2048), (4, 4096), (2, 8192), (1, 16384)):
            inp_s = W.make_chunk_inputs(W.BATCH_4K, B=B, T=T)
            ms, f_ms, p_ms = time_chunk(upload(inp_s), inp_s, max(5, a.steps // 2), 2)
            sweep.append({"B": B, "T": T, "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
                          "kernels_ms": {"chunk_factors": f_ms, "chunk_propagate": p_ms}})
            log("sweep B=%d T=%d: %.3f ms (factors %.3f, propagate %.3f) -> %.3e tokens/s"
                % (B, T, ms, f_ms, p_ms, B * T / (ms * 1e-3)))
            del inp_s
        out["context_sweep"] = {"workload": "B x T = 16384 tokens, H16 d128, bf16, S0 != 0",
                                "points": sweep}

    if a.only in ("all", "chunk"):
        # The same batch workload with bf16 gate inputs (log alpha and the b, w logits).
        wl = W.BATCH_4K
        log("generating %s (bf16 gate logits)" % wl.name)
        inp = W.make_chunk_inputs(wl, gate_logits=True)
        ms, f_ms, p_ms = time_gate_logits(inp, max(3, a.steps // 2), 2)
        tokens = inp["B"] * inp["T"]
        n_th = tokens * inp["H"]
        fbytes = n_th * inp["Dk"] * 6 * 2   # q, k, v, log_alpha, b_logit, w_logit in bf16
        out["gate_logits"] = {"workload": wl.name, "entry": "gdn2_chunk_fwd_gate_logits",
                              "ms": ms, "tokens_per_s": tokens / (ms * 1e-3),
                              "kernels_ms": {"chunk_factors": f_ms, "chunk_propagate": p_ms},
                              "chunk_factors_alg_bytes": fbytes,
                              "chunk_factors_GBps": fbytes / (f_ms * 1e-3) / 1e9}
        log("gate logits: %.3f ms (factors %.3f, propagate %.3f) -> %.3e tokens/s"
            % (ms, f_ms, p_ms, tokens / (ms * 1e-3)))
        del inp

    if a.only in ("all", "bwd"):
        wl = W.BATCH_4K
        log("generating %s (backward)" % wl.name)
        inp = W.make_chunk_inputs(wl)
        d = upload(inp)
        ms, ws_bytes = time_bwd(d, inp, max(3, a.steps // 4), 2)
        tokens = inp["B"] * inp["T"]
        nb = bwd_alg_bytes(tokens * inp["H"], inp["N"] * inp["H"], inp["Dk"], 2)
        tr = time_train(d, inp, max(3, a.steps // 4), 2)
        tokens_ = inp["B"] * inp["T"]
        out["training_step"] = {
            "workload": wl.name,
            "recompute": {"entries": "gdn2_chunk_fwd + gdn2_chunk_bwd", "fwd_ms": tr["fwd_ms"],
                          "bwd_ms": tr["bwd_ms"], "step_ms": tr["step_ms"]},
            "saved": {"entries": "gdn2_chunk_fwd_train + gdn2_chunk_bwd_saved",
                      "fwd_ms": tr["fwd_train_ms"], "bwd_ms": tr["bwd_saved_ms"],
                      "step_ms": tr["train_step_ms"], "workspace_bytes": tr["workspace_bytes"],
                      "tokens_per_s": tokens_ / (tr["train_step_ms"] * 1e-3)}}
        log("training step: forward + recomputing backward %.3f + %.3f = %.3f ms; "
            "training forward + saved-state backward %.3f + %.3f = %.3f ms (%.2f GB kept)"
            % (tr["fwd_ms"], tr["bwd_ms"], tr["step_ms"], tr["fwd_train_ms"], tr["bwd_saved_ms"],
               tr["train_step_ms"], tr["workspace_bytes"] / 1e9))
        out["backward"] = {"workload": wl.name, "entry": "gdn2_chunk_bwd", "ms": ms,
                           "tokens_per_s": tokens / (ms * 1e-3), "alg_bytes": nb,
                           "alg_GBps": nb / (ms * 1e-3) / 1e9,
                           "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "workspace_bytes": ws_bytes}
        log("backward: %.3f ms -> %.3e tokens/s (%.1f%% of HBM by algorithmic bytes)"
            % (ms, tokens / (ms * 1e-3), 100 * out["backward"]["hbm_frac"]))
        if "value" not in out:
            out.update({"value": tokens / (ms * 1e-3), "ms_per_step": ms,
                        "config": {"workload": wl.name, "pass": "backward"}})
        del d, inp

    if a.only in ("all", "layer"):
        wl = W.LAYER_4K
        log("generating %s" % wl.name)
        inp = W.make_layer_inputs(wl)
        ms, ws_bytes = time_layer(inp, max(3, a.steps // 2), 2)
        M, H, D, Dm = inp["B"] * inp["T"], inp["H"], inp["Dk"], inp["D"]
        gemm_flops = 2 * M * Dm * 7 * H * D + 2 * M * H * D * Dm
        core_flops = chunk_flops_dense(inp["B"] * (inp["T"] // 64) * H, D)
        out["layer"] = {"workload": wl.name, "entry": "gdn2_layer_fwd", "ms": ms,
                        "tokens_per_s": M / (ms * 1e-3), "D_model": Dm, "conv_len": inp["L"],
                        "gemm_flops": gemm_flops, "core_mfma_flops": core_flops,
                        "mfma_TFLOPs_over_whole_layer": (gemm_flops + core_flops) / (ms * 1e-3) / 1e12,
                        "workspace_bytes": ws_bytes}
        log("layer: %.3f ms -> %.3e tokens/s (%.0f TFLOP/s of MFMA work over the whole call)"
            % (ms, M / (ms * 1e-3), out["layer"]["mfma_TFLOPs_over_whole_layer"]))
        if "value" not in out:
            out.update({"value": M / (ms * 1e-3), "ms_per_step": ms,
                        "config": {"workload": wl.name, "pass": "layer forward"}})
        del inp

    if a.only in ("all", "swa"):
        wl = W.SWA_4K
        log("generating %s" % wl.name)
        inp = W.make_swa_inputs(wl)
        ms = time_swa(inp, max(3, a.steps // 2), 2)
        fl = swa_useful_flops([inp["T"]] * inp["B"], inp["H"], inp["D"], inp["window"])
        swa_tokens = inp["B"] * inp["T"]
        tf = fl / (ms * 1e-3) / 1e12
        out["swa"] = {"workload": wl.name, "entry": "gdn2_swa_fwd", "ms": ms,
                      "tokens_per_s": inp["B"] * inp["T"] / (ms * 1e-3),
                      "roofline": {"bound": "mfma", "kernel": "swa_fwd", "achieved": tf,
                                   "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                                   "alg_flops_per_launch": fl, "avg_launch_ms": ms}}
        log("swa: %.3f ms -> %.1f TFLOP/s of unmasked attention (%.1f%% of bf16 MFMA peak)"
            % (ms, tf, 100 * tf / MFMA_BF16_PEAK_TFLOPS))
        del inp
        # the attention layer around it (projections on hipBLASLt)
        lw = W.SWA_LAYER_4K
        li = W.make_swa_layer_inputs(lw)
        lms = time_swa_layer(li, max(3, a.steps // 2), 2)
        M = li["B"] * li["T"]
        gemm = 2 * M * li["Dm"] * 3 * li["H"] * li["D"] + 2 * M * li["H"] * li["D"] * li["Dm"]
        out["swa"]["layer"] = {"workload": lw.name, "entry": "gdn2_swa_layer_fwd", "ms": lms,
                               "tokens_per_s": M / (lms * 1e-3), "gemm_flops": gemm,
                               "mfma_TFLOPs_over_whole_layer": (gemm + fl) / (lms * 1e-3) / 1e12}
        log("swa layer: %.3f ms -> %.3e tokens/s" % (lms, M / (lms * 1e-3)))
        del li
        if "value" not in out:
            out.update({"value": swa_tokens / (ms * 1e-3), "ms_per_step": ms,
                        "config": {"workload": wl.name, "pass": "swa forward"}})

    if a.only in ("all", "decode"):
        wl = W.DECODE
        wall, mean_ms, med_ms = time_decode(decode_pre)
        del decode_pre
        nbytes = decode_alg_bytes(wl.B, wl.H, wl.Dk, 2)
        ddig = source_digest("gdn2_step.hip", "gdn2_device.h")
        dec = {"workload": wl.name, "steps": a.decode_steps, "us_per_step": mean_ms * 1e3,
               "GBps": nbytes / (mean_ms * 1e-3) / 1e9,
               "hbm_frac": nbytes / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "roofline": {"bound": "hbm", "kernel": "decode_step",
                            "achieved": nbytes / (mean_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": nbytes / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "traffic": stored_traffic("decode_step", wl.name, ddig),
                            "alg_bytes_per_launch": nbytes, "avg_launch_ms": mean_ms},
               "alg_bytes_per_step": nbytes, "loop_wall_s": wall,
               "inputs": "%d distinct pre-generated steps, uploaded before timing"
                         % a.decode_steps,
               "tokens_per_s": wl.B * a.decode_steps / wall}
        out["decode"] = dec
        log("decode: %.1f us/step, %.0f GB/s (%.1f%% of HBM)"
            % (dec["us_per_step"], dec["GBps"], 100 * dec["hbm_frac"]))
        if "value" not in out:
            out.update({"value": dec["GBps"], "unit": "GB/s", "ms_per_step": mean_ms,
                        "config": {"workload": wl.name}})

    if a.only in ("all", "varlen"):
        wl = W.VARLEN
        log("generating %s" % wl.name)
        inp = W.make_chunk_inputs(wl)
        d = upload(inp)
        ms, f_ms, p_ms = time_chunk(d, inp, max(3, a.steps // 4), 2)
        out["varlen"] = {"workload": wl.name, "tokens": inp["T"], "ms": ms,
                         "tokens_per_s": inp["T"] / (ms * 1e-3),
                         "kernels_ms": {"plan+chunk_factors": f_ms, "chunk_propagate": p_ms}}
        log("varlen: %d tokens, %.3f ms -> %.3e tokens/s" % (inp["T"], ms, inp["T"] / (ms * 1e-3)))
        if "value" not in out:
            out.update({"value": inp["T"] / (ms * 1e-3), "ms_per_step": ms,
                        "config": {"workload": wl.name}})
        del d, inp

    print(json.dumps(out))


if __name__ == "__main__":
    main()

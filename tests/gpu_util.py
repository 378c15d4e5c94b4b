"""Helpers for the GPU parity tests: upload seeded inputs, run the library,
evaluate the oracle on sampled (sequence, head) pairs."""

import sys

import numpy as np

import oracle as O
import workloads as W


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(x, io=None):
    """numpy float32 array -> device tensor (bfloat16 when io == BF16)."""
    import torch
    if x is None:
        return None
    if io == W.BF16:
        bits = W.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    if x.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def upload_chunk(inp):
    io = inp["io"]
    return dict(q=dev(inp["q"], io), k=dev(inp["k"], io), v=dev(inp["v"], io),
                log_alpha=dev(inp["log_alpha"]), b=dev(inp["b"]), w=dev(inp["w"]),
                S0=dev(inp["S0"]), cu_seqlens=dev(inp["cu_seqlens"]))


def tol(io):
    """Parity bound on max|err| / max|ref|: 2e-2 for bf16 I/O, 1e-4 all-fp32."""
    return 2e-2 if io == W.BF16 else 1e-4


def oracle_sampled(inp, pairs):
    """Oracle outputs for (sequence n, head h) pairs.

    Returns {(n, h): (o [L, Dv], S_final [Dk, Dv])}, where o covers the
    sequence's tokens only.
    """
    cu = inp["cu_seqlens"]
    out = {}
    for n, h in pairs:
        if cu is None:
            row, t0, t1 = n, 0, inp["T"]
        else:
            row, t0, t1 = 0, int(cu[n]), int(cu[n + 1])
        sl = (slice(row, row + 1), slice(t0, t1), slice(h, h + 1))
        S0 = None if inp["S0"] is None else inp["S0"][n:n + 1, h:h + 1]
        o, S = O.recurrence(*(inp[x][sl] for x in ("q", "k", "v", "log_alpha", "b", "w")), S0=S0)
        out[(n, h)] = (o[0, :, 0], S[0, 0])
    return out


def gpu_slices(inp, o_gpu, S_gpu, n, h):
    """The GPU outputs matching oracle_sampled's (n, h) entry, as float64 arrays."""
    cu = inp["cu_seqlens"]
    if cu is None:
        o = o_gpu[n, :, h]
    else:
        o = o_gpu[0, int(cu[n]):int(cu[n + 1]), h]
    return host(o), host(S_gpu[n, h])

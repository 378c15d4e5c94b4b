"""Helpers for the GPU parity tests: upload seeded inputs and the parity bound."""

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

"""fp64 CPU oracle for sliding-window softmax attention (forward).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the package smoke check and the CPU-baseline leg of the benchmark script use
it.  It shares no code with the HIP library.

The hybrid model interleaves the Gated DeltaNet-2 mixer with sliding-window
attention over a 2K window, the attention taking the precise local
interactions and the recurrence the long range (iplexlaw digest, section
"Condiciones de comparación": the hybrid family adds 2K sliding-window
attention and keeps a bounded local cache; gist.science summary, part
"4. Architecture": SWA interleaved with the mixer).  The pages give nothing
more, so this is the plainest reading, each point also listed in the design
notes:

  * multi-head softmax attention, one key/value head per query head;
  * query i of a sequence attends to the keys j of the same sequence with
    i - window < j <= i (a causal window of `window` tokens, itself included);
  * scores are scaled by `scale` (1/sqrt(d) by default); no positional
    encoding is applied here (a caller applies one to q and k);
  * lse_i = log sum_j exp(scale * q_i . k_j) over the window, also returned.

Layouts: q, k, v, o are [B, T, H, D]; lse is [B, H, T].  A packed call has
B == 1 and cu_seqlens of length N+1.  All math is float64.
"""

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _spans(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(n, 0, T) for n in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def window_mask(L, window):
    """[L, L] boolean: True where query i may attend to key j (i - window < j <= i)."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return (j <= i) & (j > i - window)


def swa_fwd(q, k, v, window, scale=None, cu_seqlens=None, heads=None):
    """Dense masked softmax attention per sequence and head.

    Returns (o [B, T, H, D], lse [B, H, T]).  heads: optional list of head
    indices to evaluate (the others stay zero), for spot checks at large sizes.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    hs = range(H) if heads is None else heads
    o = np.zeros(q.shape)
    lse = np.zeros((B, H, T))
    for row, t0, t1 in _spans(B, T, cu_seqlens):
        L = t1 - t0
        if L == 0:
            continue
        allowed = window_mask(L, window)
        for h in hs:
            s = scale * (q[row, t0:t1, h] @ k[row, t0:t1, h].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            den = p.sum(axis=1, keepdims=True)
            o[row, t0:t1, h] = (p / den) @ v[row, t0:t1, h]
            lse[row, h, t0:t1] = (m + np.log(den))[:, 0]
    return o, lse


def swa_layer_fwd(x, W_qkv, W_o, H, D, window, scale=None, cu_seqlens=None):
    """The attention layer of the hybrid model around swa_fwd: q, k, v are
    the three row blocks of one projection x W_qkv^T (W_qkv [3 H D, Dm], rows
    q | k | v, no biases), attention over the window, then y = o W_o^T
    (W_o [Dm, H D]).  Reading: the pages name only the window, so the layer
    is the plain projection-attention-projection form with no positional
    encoding, normalisation or gate.  Returns (y [B, T, Dm], lse [B, H, T])."""
    x, W_qkv, W_o = _f64(x), _f64(W_qkv), _f64(W_o)
    B, T, Dm = x.shape
    HD = H * D
    P = x @ W_qkv.T
    q = P[..., :HD].reshape(B, T, H, D)
    k = P[..., HD:2 * HD].reshape(B, T, H, D)
    v = P[..., 2 * HD:].reshape(B, T, H, D)
    o, lse = swa_fwd(q, k, v, window, scale=scale, cu_seqlens=cu_seqlens)
    return o.reshape(B, T, HD) @ W_o.T, lse

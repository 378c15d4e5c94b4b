"""fp64 CPU oracle for the Gated DeltaNet-2 token-mixer layer (forward).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the package smoke check and the CPU-baseline leg of the benchmark script use
it.  It shares no code with the HIP library.

The layer around the core recurrence follows the iplexlaw digest, section
"Procesamiento del token y entrenamiento paralelo": queries and keys go
through a linear projection, a short causal convolution, SiLU and an L2
normalisation; values through a projection, the convolution and SiLU; the
recurrent output is RMS-normalised, multiplied by an output gate of its own
(not the write gate) and projected back.  The erase and write gates are
sigmoids of their own linear projections (same digest, section "Decisiones
independientes en dos ejes").  The core is gdn2_oracle.chunked (or any
function with the signature of gdn2_oracle.recurrence).

Readings taken where the page is silent (each also listed in the design
notes):
  * one input weight W_in [7 blocks, D] stacked in the order
    q | k | v | alpha | output gate | b | w, each block H*Dk (q, k, alpha, b)
    or H*Dv (v, output gate, w) rows; no projection biases;
  * the decay is log alpha = logsigmoid(x W_alpha^T + alpha_bias), a per-channel
    sigmoid gate like b and w, with a per-channel bias so that a layer can
    start near alpha = 1;
  * the short convolution is depthwise and causal over the q, k and v channels:
    y_t = sum_{j<L} conv_w[c, j] x_{t-L+1+j}, with x = 0 before the sequence's
    first token (each packed sequence starts afresh);
  * L2 normalisation is per head over Dk: x / sqrt(|x|^2 + 1e-6);
  * RMS normalisation is per head over Dv with one weight vector [Dv] shared
    by the heads: o / sqrt(mean(o^2) + eps) * norm_w;
  * the output gate is a sigmoid of its own projection;
  * the output projection W_o is [D, H*Dv], no bias.

All math is float64.  x is [B, T, D]; a packed call has B == 1 and
cu_seqlens of length N+1.
"""

import numpy as np

from .gdn2_oracle import chunked

L2_EPS = 1e-6
BLOCKS = ("q", "k", "v", "alpha", "gate", "b", "w")


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def block_rows(H, Dk, Dv):
    """Row ranges of the seven blocks of W_in, in the order of BLOCKS."""
    sizes = {"q": H * Dk, "k": H * Dk, "v": H * Dv, "alpha": H * Dk, "gate": H * Dv,
             "b": H * Dk, "w": H * Dv}
    out, r = {}, 0
    for name in BLOCKS:
        out[name] = (r, r + sizes[name])
        r += sizes[name]
    return out


def sequence_spans(B, T, cu_seqlens):
    """(batch row, start, stop) of every sequence of the call."""
    if cu_seqlens is None:
        return [(n, 0, T) for n in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def causal_conv(x, conv_w, spans):
    """Depthwise causal convolution over the token axis of x [B, T, C] with
    taps conv_w [C, L]: y_t = sum_j conv_w[:, j] * x_{t-L+1+j}, taps before
    the first token of the token's own sequence read zero."""
    x, conv_w = _f64(x), _f64(conv_w)
    L = conv_w.shape[1]
    y = np.zeros_like(x)
    for row, t0, t1 in spans:
        seg = x[row, t0:t1]
        for j in range(L):
            shift = L - 1 - j  # this tap reads the token `shift` steps back
            if shift >= t1 - t0:
                continue
            y[row, t0 + shift:t1] += conv_w[:, j] * seg[:t1 - t0 - shift]
    return y


def silu(z):
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def logsigmoid(z):
    """log(1 / (1 + e^-z)), evaluated without overflow for either sign."""
    z = _f64(z)
    return np.minimum(z, 0.0) - np.log1p(np.exp(-np.abs(z)))


def l2_normalize(x, eps=L2_EPS):
    """x / sqrt(|x|^2 + eps) along the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def rms_normalize(x, eps):
    """x / sqrt(mean(x^2) + eps) along the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def layer_fwd(x, W_in, conv_w, alpha_bias, norm_w, W_o, H, Dk, Dv, norm_eps=1e-6, S0=None,
              cu_seqlens=None, core=chunked, return_parts=False, l2_eps=L2_EPS):
    """Forward of the token-mixer layer.

    x [B, T, D]; W_in [2*H*Dk + H*Dv + H*Dk + H*Dv + H*Dk + H*Dv, D] (blocks in
    the order of BLOCKS); conv_w [2*H*Dk + H*Dv, L] (q, k, v channels);
    alpha_bias [H*Dk]; norm_w [Dv]; W_o [D, H*Dv].
    Returns (y [B, T, D], S_final [N, H, Dk, Dv]) and, with return_parts,
    a dict of the intermediates as a third element.
    """
    x, W_in, W_o = _f64(x), _f64(W_in), _f64(W_o)
    alpha_bias, norm_w = _f64(alpha_bias), _f64(norm_w)
    B, T, D = x.shape
    rows = block_rows(H, Dk, Dv)
    spans = sequence_spans(B, T, cu_seqlens)

    P = x @ W_in.T  # every projection at once: [B, T, rows]
    proj = {name: P[..., r0:r1] for name, (r0, r1) in rows.items()}

    qkv = np.concatenate([proj["q"], proj["k"], proj["v"]], axis=-1)
    qkv = silu(causal_conv(qkv, conv_w, spans))
    HK, HV = H * Dk, H * Dv
    q = l2_normalize(qkv[..., :HK].reshape(B, T, H, Dk), l2_eps)
    k = l2_normalize(qkv[..., HK:2 * HK].reshape(B, T, H, Dk), l2_eps)
    v = qkv[..., 2 * HK:].reshape(B, T, H, Dv)

    log_alpha = logsigmoid(proj["alpha"] + alpha_bias).reshape(B, T, H, Dk)
    b = sigmoid(proj["b"]).reshape(B, T, H, Dk)
    w = sigmoid(proj["w"]).reshape(B, T, H, Dv)

    o, S_final = core(q, k, v, log_alpha, b, w, S0=S0, cu_seqlens=cu_seqlens)

    z = rms_normalize(o, norm_eps) * norm_w * sigmoid(proj["gate"]).reshape(B, T, H, Dv)
    y = z.reshape(B, T, HV) @ W_o.T
    if return_parts:
        parts = dict(q=q, k=k, v=v, log_alpha=log_alpha, b=b, w=w, o=o, z=z, P=P)
        return y, S_final, parts
    return y, S_final

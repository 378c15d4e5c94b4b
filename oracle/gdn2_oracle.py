"""fp64 CPU oracle for the Gated DeltaNet-2 core recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test suite, the package smoke check and the CPU-baseline leg
of the benchmark script use it.  It shares no code with the HIP library.

Citation keys used below (each names a web page and the part of it followed):

  [iplexlaw]   iplexlaw.co.kr blog post "Gated DeltaNet-2 erase/write"
               (Spanish digest of arXiv 2605.22791), section
               "Decisiones independientes en dos ejes" (read/write form) and
               "Procesamiento del token y entrenamiento paralelo" (64-token
               WY chunks, fp32 decay).
  [gist-1]     gist.science summary of arXiv 2605.22791, technical summary,
               part "1. Gated Delta Rule-2" (matrix-form state update, gate
               domains, reductions to KDA / Gated DeltaNet).
  [gist-2]     same page, part "2. Fast-weight update perspective" (the read
               is taken from the decayed state with the erase vector).
  [gist-3]     same page, part "3. Efficient chunkwise parallel training"
               (decay absorbed into erase/write factors, lower-triangular
               system (I+T)^-1, erase-side Y and write-side U).
  [zubnet-1]   zubnet.ai news item, first paragraph (matrix-form update,
               D_t = Diag(alpha_t), gate domains).

What is computed (state S is d_k x d_v, rows are key channels):

    alpha_t = exp(log_alpha_t)                 per key channel
    Sbar    = Diag(alpha_t) S_{t-1}            decay first            [iplexlaw]
    e_t     = b_t * k_t,  z_t = w_t * v_t      erase on keys, write on values
    r_t     = Sbar^T e_t                       read the decayed state [iplexlaw][gist-2]
    S_t     = Sbar + k_t (z_t - r_t)^T         erase along k, write z [iplexlaw]
    o_t     = S_t^T q_t                        the query reads S_t    [iplexlaw]

which is the same map as S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1}
+ k_t (w_t*v_t)^T  [gist-1][zubnet-1].  No query scale is applied (the pages
print none; a caller may fold one into q).

Readings taken where the pages are silent (each also listed in the design
notes): decay enters as log alpha in fp32 and alpha = exp(log alpha); a
missing initial state is zero; in a packed variable-length batch every
sequence starts from its own initial state and is chunked from its own first
token; the last chunk of a sequence may be shorter than 64.

Array conventions: q, k, log_alpha, b are [B, T, H, Dk]; v, w are
[B, T, H, Dv]; o is [B, T, H, Dv]; states are [N, H, Dk, Dv].  All math is
float64.
"""

import numpy as np

CHUNK = 64  # tokens per WY chunk [iplexlaw, "Procesamiento del token y entrenamiento paralelo"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Token-by-token recurrence (the definition)
# ---------------------------------------------------------------------------

def step(q, k, v, log_alpha, b, w, S):
    """One recurrent token for independent (batch, head) pairs.

    q, k, log_alpha, b: [..., Dk]; v, w: [..., Dv]; S: [..., Dk, Dv].
    Returns (o [..., Dv], S_new [..., Dk, Dv]) in float64.

    Follows the read/write decomposition [iplexlaw, "Decisiones
    independientes en dos ejes"]: decay, read with the erase vector from the
    decayed state [gist-2], write k (z - r)^T, then read the updated state
    with the query.
    """
    q, k, v, log_alpha, b, w, S = map(_f64, (q, k, v, log_alpha, b, w, S))
    alpha = np.exp(log_alpha)                      # per-key-channel decay [zubnet-1]
    S_bar = alpha[..., :, None] * S                # Diag(alpha) acts on rows (key axis)
    e = b * k                                      # erase vector, key axis [gist-1]
    z = w * v                                      # write vector, value axis [gist-1]
    r = np.einsum("...kv,...k->...v", S_bar, e)    # r = Sbar^T e
    S_new = S_bar + k[..., :, None] * (z - r)[..., None, :]
    o = np.einsum("...kv,...k->...v", S_new, q)    # o = S_t^T q_t (updated state)
    return o, S_new


def _sequences(B, T, cu_seqlens):
    """Yield (n, batch_row, start, stop) for every sequence of the call."""
    if cu_seqlens is None:
        for n in range(B):
            yield n, n, 0, T
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        for n in range(len(cu) - 1):
            yield n, 0, int(cu[n]), int(cu[n + 1])


def recurrence(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, heads=None):
    """Whole-sequence forward by the plain recurrence, one token at a time.

    Dense call: cu_seqlens is None and each of the B rows is one sequence of
    length T.  Packed call: B == 1 and cu_seqlens (length N+1) gives the
    token offsets of N sequences; each starts from S0[n] (or zero).

    heads: optional list of head indices to evaluate (others are left 0 in
    o and in the returned state), so that large shapes can be spot-checked.

    Returns (o [B,T,H,Dv] float64, S_final [N,H,Dk,Dv] float64).
    """
    q, k, v, log_alpha, b, w, S0 = map(_f64, (q, k, v, log_alpha, b, w, S0))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, Dv))
    S_final = np.zeros((N, H, Dk, Dv))
    for n, row, t0, t1 in _sequences(B, T, cu_seqlens):
        S = np.zeros((len(hs), Dk, Dv)) if S0 is None else S0[n, hs].copy()
        for t in range(t0, t1):
            o_t, S = step(q[row, t, hs], k[row, t, hs], v[row, t, hs],
                          log_alpha[row, t, hs], b[row, t, hs], w[row, t, hs], S)
            o[row, t, hs] = o_t
        S_final[n, hs] = S
    return o, S_final


# ---------------------------------------------------------------------------
# Chunk-parallel (WY) form, in fp64 with an explicit inverse
# ---------------------------------------------------------------------------

def chunk_factors(q, k, v, log_alpha, b, w):
    """WY factors of one chunk of one head (L <= 64 tokens).

    Inputs are [L, Dk] / [L, Dv] arrays.  The chunk form follows [gist-3]
    and [iplexlaw, "Procesamiento del token y entrenamiento paralelo"]: the
    cumulative per-channel decay inside the chunk (computed from the start of
    the chunk) is absorbed into an erase-side factor and a key-side factor,
    which turns the decayed recurrence into a pure asymmetric delta update
    of the normalised state Diag(gamma_i)^-1 S_i with key k_i / gamma_i and
    erase vector gamma_i * b_i * k_i.  Unrolling that update gives a unit
    lower-triangular system whose inverse yields the erase-side and write-side
    auxiliaries.

    Returns a dict (all float64):
      g       [L, Dk]  inclusive cumulative sum of log alpha within the chunk
      A       [L, L]   strictly lower: A_ij = sum_c b_i k_i k_j exp(g_i - g_j)
                       (the pages' "T" interaction matrix)
      Tinv    [L, L]   (I + A)^-1  (the pages' "(I+T)^-1")
      W       [L, Dk]  Tinv @ (gamma * b * k)   (erase side, the pages' Y)
      U       [L, Dv]  Tinv @ (w * v)           (write side, the pages' U)
      M       [L, L]   lower incl. diagonal: M_ij = sum_c q_i k_j exp(g_i - g_j)
      Qhat    [L, Dk]  gamma * q
      Khat    [L, Dk]  exp(g_last - g) * k
      gamma_last [Dk]  exp(g_last)
    """
    q, k, v, log_alpha, b, w = map(_f64, (q, k, v, log_alpha, b, w))
    L = k.shape[0]
    g = np.cumsum(log_alpha, axis=0)                   # fp32 in the kernels, fp64 here
    gamma = np.exp(g)
    E = gamma * b * k                                  # erase side, decay absorbed
    Kt = k / gamma                                     # key side, decay absorbed
    A = np.tril(E @ Kt.T, -1)                          # strictly lower
    Tinv = np.linalg.inv(np.eye(L) + A)
    W = Tinv @ E
    U = Tinv @ (w * v)
    M = np.tril((gamma * q) @ Kt.T)                    # inclusive diagonal: query reads S_t
    g_last = g[-1]
    return dict(g=g, A=A, Tinv=Tinv, W=W, U=U, M=M, Qhat=gamma * q,
                Khat=np.exp(g_last - g) * k, gamma_last=np.exp(g_last))


def chunk_apply(f, S_in):
    """Propagate one chunk given its factors and the incoming state.

    U_eff = U - W S_in are the per-token corrected values; the chunk output is
    O = Qhat S_in + M U_eff and the outgoing state is
    S_out = Diag(gamma_last) S_in + Khat^T U_eff.
    """
    U_eff = f["U"] - f["W"] @ S_in
    O = f["Qhat"] @ S_in + f["M"] @ U_eff
    S_out = f["gamma_last"][:, None] * S_in + f["Khat"].T @ U_eff
    return O, S_out


def chunk_affine_map(f):
    """The chunk as an affine map of the state: S_out = P S_in + Qc."""
    P = np.diag(f["gamma_last"]) - f["Khat"].T @ f["W"]
    Qc = f["Khat"].T @ f["U"]
    return P, Qc


def chunked(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, chunk=CHUNK):
    """Whole-sequence forward by the chunk form (fp64, explicit inverse).

    Same signature and result as recurrence(); each sequence is cut into
    chunks of `chunk` tokens from its own first token, the last one possibly
    shorter.
    """
    q, k, v, log_alpha, b, w, S0 = map(_f64, (q, k, v, log_alpha, b, w, S0))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, Dv))
    S_final = np.zeros((N, H, Dk, Dv))
    for n, row, t0, t1 in _sequences(B, T, cu_seqlens):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else S0[n, h].copy()
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                sl = (row, slice(c0, c1), h)
                f = chunk_factors(q[sl], k[sl], v[sl], log_alpha[sl], b[sl], w[sl])
                O, S = chunk_apply(f, S)
                o[sl] = O
            S_final[n, h] = S
    return o, S_final


# ---------------------------------------------------------------------------
# Error metric used by every parity check
# ---------------------------------------------------------------------------

def rel_max_err(got, ref):
    """max |got - ref| / max |ref| over the whole array (0 if both are 0)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(num)
    return float(num / denom)

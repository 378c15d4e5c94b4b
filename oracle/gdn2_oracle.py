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
# Gate-logit inputs
# ---------------------------------------------------------------------------

def gates_from_logits(b_logit, w_logit):
    """The erase and write gates from their pre-activations: each gate is the
    sigmoid of its own linear projection of the token [iplexlaw, "Decisiones
    independientes en dos ejes"], so b = 1 / (1 + exp(-b_logit)) and likewise
    w.  Returns (b, w) in float64."""
    b_logit, w_logit = _f64(b_logit), _f64(w_logit)
    return 1.0 / (1.0 + np.exp(-b_logit)), 1.0 / (1.0 + np.exp(-w_logit))


# ---------------------------------------------------------------------------
# Backward: gradients of the recurrence
# ---------------------------------------------------------------------------
#
# The pages name a gate-aware backward as one of the method's contributions
# ([gist-3], item on the backward pass: the channel-wise gates b and w enter
# the gradients of the auxiliary matrices directly; [iplexlaw], "El artículo
# y su pregunta": gradients that include the gates) but print no formulas.
# The gradient of the recurrence has a plain definition, the chain rule taken
# backwards through the token steps, which recurrence_bwd writes out.

def recurrence_bwd(q, k, v, log_alpha, b, w, do, S0=None, dS_final=None, cu_seqlens=None):
    """Reverse-mode gradients of recurrence() for upstream gradients do
    (of o) and dS_final (of S_final; None means zero).

    Returns a dict of float64 arrays: dq, dk, dv, dlog_alpha, db, dw (shapes
    of the inputs) and dS0 [N, H, Dk, Dv].

    One token of the forward (see step) is  Sbar = Diag(alpha) S_prev,
    r = Sbar^T e, u = z - r, S = Sbar + k u^T, o = S^T q  with e = b*k and
    z = w*v.  Going backwards with G = dL/dS (the output gradient folded in):
        G     += q do^T,        dq = S do
        du     = G^T k,         dk = G u
        dSbar  = G - e du^T,    de = -Sbar du        (u = z - Sbar^T e)
        dlog_alpha = rowsum(dSbar * Sbar),   G_prev = Diag(alpha) dSbar
        db = de * k,  dk += de * b,  dw = du * v,  dv = du * w.
    """
    q, k, v, log_alpha, b, w, do, S0, dS_final = map(
        _f64, (q, k, v, log_alpha, b, w, do, S0, dS_final))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dlog_alpha=np.zeros_like(log_alpha), db=np.zeros_like(b), dw=np.zeros_like(w),
               dS0=np.zeros((N, H, Dk, Dv)))
    for n, row, t0, t1 in _sequences(B, T, cu_seqlens):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else S0[n, h].copy()
            states = [S]                               # states[i] = S after i tokens
            for t in range(t0, t1):
                _, S = step(q[row, t, h], k[row, t, h], v[row, t, h], log_alpha[row, t, h],
                            b[row, t, h], w[row, t, h], S)
                states.append(S)
            G = np.zeros((Dk, Dv)) if dS_final is None else dS_final[n, h].copy()
            for t in range(t1 - 1, t0 - 1, -1):
                i = t - t0
                S_prev, S_t = states[i], states[i + 1]
                qt, kt, vt = q[row, t, h], k[row, t, h], v[row, t, h]
                bt, wt = b[row, t, h], w[row, t, h]
                alpha = np.exp(log_alpha[row, t, h])
                S_bar = alpha[:, None] * S_prev
                e, z = bt * kt, wt * vt
                u = z - S_bar.T @ e
                G = G + np.outer(qt, do[row, t, h])
                out["dq"][row, t, h] = S_t @ do[row, t, h]
                du = G.T @ kt
                dk = G @ u
                dS_bar = G - np.outer(e, du)
                de = -(S_bar @ du)
                out["dlog_alpha"][row, t, h] = np.sum(dS_bar * S_bar, axis=1)
                G = alpha[:, None] * dS_bar
                out["db"][row, t, h] = de * kt
                out["dk"][row, t, h] = dk + de * bt
                out["dw"][row, t, h] = du * vt
                out["dv"][row, t, h] = du * wt
            out["dS0"][n, h] = G
    return out


def chunk_bwd(f, q, k, v, b, w, S_in, dO, dS_out):
    """Gradients of one chunk (fp64, explicit inverse), given its factors f
    (chunk_factors), the incoming state S_in, the output gradient dO [L, Dv]
    and the gradient dS_out of the outgoing state.

    This is the chain rule applied to the chunk form (chunk_factors and
    chunk_apply), written factor by factor; the unit tests check it against
    recurrence_bwd.  Returns (grads dict for the chunk's tokens, dS_in) with
    dlog_alpha already accumulated over the chunk's cumulative sum.
    """
    q, k, v, b, w, S_in, dO, dS_out = map(_f64, (q, k, v, b, w, S_in, dO, dS_out))
    g = f["g"]
    gamma = np.exp(g)
    gl = f["gamma_last"]
    E = gamma * b * k                                  # erase side (W = Tinv E)
    Kt = k / gamma                                     # key side of A and M
    Z = w * v
    T_ = f["Tinv"]
    U_eff = f["U"] - f["W"] @ S_in
    # chunk_apply:  O = Qhat S + M U_eff,  S_out = Diag(gl) S + Khat^T U_eff
    dU_eff = f["M"].T @ dO + f["Khat"] @ dS_out
    dS_in = f["Qhat"].T @ dO + gl[:, None] * dS_out - f["W"].T @ dU_eff
    dQhat = dO @ S_in.T
    dM = np.tril(dO @ U_eff.T)
    dKhat = U_eff @ dS_out.T
    dgl = np.sum(dS_out * S_in, axis=1)
    dW = -dU_eff @ S_in.T
    dU = dU_eff
    # W = Tinv E,  U = Tinv Z,  Tinv = (I + A)^-1:  dA = -Tinv^T dTinv Tinv^T,
    # and Tinv^T (dU Z^T + dW E^T) Tinv^T = dZ U^T + dE W^T.
    dZ = T_.T @ dU
    dE = T_.T @ dW
    dA = -np.tril(dZ @ f["U"].T + dE @ f["W"].T, -1)
    # A = tril(E Kt^T, -1),  M = tril(Qhat Kt^T),  Khat = gl * Kt
    dE = dE + dA @ Kt
    dKt = dA.T @ E + dM.T @ f["Qhat"] + gl * dKhat
    dQhat = dQhat + dM @ Kt
    dgl = dgl + np.sum(Kt * dKhat, axis=0)
    # E = gamma b k,  Qhat = gamma q,  Kt = k / gamma,  Z = w v
    grads = dict(dq=gamma * dQhat, db=gamma * k * dE, dk=gamma * b * dE + dKt / gamma,
                 dw=v * dZ, dv=w * dZ)
    dg = E * dE + f["Qhat"] * dQhat - Kt * dKt          # d/dg_i of the token-i factors
    dg_last = gl * dgl                                  # gamma_last = exp(g_last)
    # g_i = sum_{j<=i} log_alpha_j:  dlog_alpha_j = sum_{i>=j} dg_i  (+ dg_last for all j)
    grads["dlog_alpha"] = np.cumsum(dg[::-1], axis=0)[::-1] + dg_last[None, :]
    return grads, dS_in


def chunked_bwd(q, k, v, log_alpha, b, w, do, S0=None, dS_final=None, cu_seqlens=None,
                chunk=CHUNK):
    """Same result as recurrence_bwd, by the chunk form: a forward pass that
    keeps each chunk's incoming state, then the chunks in reverse with
    chunk_bwd carrying the state gradient."""
    q, k, v, log_alpha, b, w, do, S0, dS_final = map(
        _f64, (q, k, v, log_alpha, b, w, do, S0, dS_final))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dlog_alpha=np.zeros_like(log_alpha), db=np.zeros_like(b), dw=np.zeros_like(w),
               dS0=np.zeros((N, H, Dk, Dv)))
    for n, row, t0, t1 in _sequences(B, T, cu_seqlens):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else S0[n, h].copy()
            spans, fs, S_ins = [], [], []
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                sl = (row, slice(c0, c1), h)
                f = chunk_factors(q[sl], k[sl], v[sl], log_alpha[sl], b[sl], w[sl])
                spans.append(sl)
                fs.append(f)
                S_ins.append(S)
                _, S = chunk_apply(f, S)
            dS = np.zeros((Dk, Dv)) if dS_final is None else dS_final[n, h].copy()
            for sl, f, S_in in zip(spans[::-1], fs[::-1], S_ins[::-1]):
                grads, dS = chunk_bwd(f, q[sl], k[sl], v[sl], b[sl], w[sl], S_in, do[sl], dS)
                for name, val in grads.items():
                    out[name][sl] = val
            out["dS0"][n, h] = dS
    return out


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

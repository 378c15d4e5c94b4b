"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers, L2-normalises q and k, applies a sigmoid to the gate logits and rounds
to bfloat16.  Both the HIP path and the fp64 oracle consume exactly the arrays
returned here (bfloat16 values are carried as float32 arrays whose values are
exactly representable in bfloat16, plus their raw bit patterns).

Shapes stand in for a 1.3B-parameter token-mixer layer with 16 heads and a
128 x 128 state per head (iplexlaw blog, "Condiciones de comparación": 16
heads, 128 x 128 state, 262,144 state values per layer and batch element;
4K training context).  Distributions:
  q, k ~ N(0, 1), then L2-normalised per (token, head) (norm accumulated in
  float64, scaling in float32);
  v ~ N(0, 1);
  log alpha ~ U[-0.2, -0.001] per key channel;
  b = sigmoid(N(0, 1)) over d_k;  w = sigmoid(N(0, 1)) over d_v;
  initial states ~ N(0, 0.02^2) (standard deviation 0.02) where present.
Draw order: (lengths) -> q -> k -> v -> log alpha -> b logits -> w logits ->
(state).  Generator: numpy PCG64.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class ChunkWorkload:
    name: str
    B: int
    T: int            # tokens per batch row (dense) or total packed tokens (varlen)
    H: int
    Dk: int
    Dv: int
    io: str           # dtype of q, k, v, o
    seed: int
    with_S0: bool = False
    n_seqs: int = 0   # > 0: packed variable-length batch of this many sequences
    len_lo: int = 0
    len_hi: int = 0


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    Dk: int
    Dv: int
    io: str
    seed: int
    steps: int


TINY_F32 = ChunkWorkload("tiny_f32_B1_H2_T256_d64", 1, 256, 2, 64, 64, F32, 47000)
SEQ_4K = ChunkWorkload("seq_B1_H16_T4096_d128", 1, 4096, 16, 128, 128, BF16, 47001)
BATCH_4K = ChunkWorkload("batch_B8_H16_T4096_d128", 8, 4096, 16, 128, 128, BF16, 47002,
                         with_S0=True)
VARLEN = ChunkWorkload("varlen_N32_L512-8192_H16_d128", 1, 0, 16, 128, 128, BF16, 47003,
                       n_seqs=32, len_lo=512, len_hi=8192)
DECODE = DecodeWorkload("decode_B256_H16_d128", 256, 16, 128, 128, BF16, 47004, 1024)

CHUNK_WORKLOADS = (TINY_F32, SEQ_4K, BATCH_4K, VARLEN)


# ---------------------------------------------------------------------------
# bfloat16 helpers (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x):
    """Round a float array to the nearest bfloat16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float32)
    out = np.exp(-x)
    out += np.float32(1.0)
    np.reciprocal(out, out=out)
    return out


def _l2norm(x):
    x = np.asarray(x, dtype=np.float32)
    inv = 1.0 / np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float64))
    return (x * inv[..., None].astype(np.float32)).astype(np.float32)


def _io_cast(x, io):
    return bf16_round(x) if io == BF16 else np.asarray(x, dtype=np.float32)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _l2norm_blocked(x, block=1 << 16):
    """L2-normalise the last axis of a [..., D] array in row blocks."""
    flat = x.reshape(-1, x.shape[-1])
    for i in range(0, flat.shape[0], block):
        flat[i:i + block] = _l2norm(flat[i:i + block])
    return x


# ---------------------------------------------------------------------------
# Chunk-forward inputs
# ---------------------------------------------------------------------------

def varlen_lengths(wl: ChunkWorkload):
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    return rng.integers(wl.len_lo, wl.len_hi, size=wl.n_seqs, endpoint=True)


def make_chunk_inputs(wl: ChunkWorkload, lengths=None, T: Optional[int] = None,
                      B: Optional[int] = None, H: Optional[int] = None,
                      seed: Optional[int] = None, log_alpha_range=(-0.2, -0.001),
                      b_scale: float = 1.0, gate_logits: bool = False):
    """Draw the inputs of one chunk-forward call.

    Optional overrides (T, B, H, lengths, seed) shrink a workload for
    oracle-sized tests while keeping its distributions.  b_scale multiplies
    the erase gate (b_scale = 2 gives the widened [0, 2] erase range).

    Returns a dict with float32 arrays q, k, v, log_alpha, b, w, S0 (or None),
    cu_seqlens (int32 [N+1] or None) and meta fields B, T, H, Dk, Dv, N, io.
    With gate_logits, the gates are handed over as bfloat16 values instead:
    log_alpha rounded to bfloat16 and the N(0, 1) logits b_logit, w_logit
    (rounded to bfloat16); b and w are then None (the sigmoid belongs to the
    computation under test).
    """
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    H = wl.H if H is None else H
    cu = None
    if wl.n_seqs or lengths is not None:
        if lengths is None:
            lengths = rng.integers(wl.len_lo, wl.len_hi, size=wl.n_seqs, endpoint=True)
        else:
            lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B_, T_ = 1, int(cu[-1])
        N = len(lengths)
    else:
        B_ = wl.B if B is None else B
        T_ = wl.T if T is None else T
        N = B_
    Dk, Dv = wl.Dk, wl.Dv
    q = _io_cast(_l2norm_blocked(_normal(rng, (B_, T_, H, Dk))), wl.io)
    k = _io_cast(_l2norm_blocked(_normal(rng, (B_, T_, H, Dk))), wl.io)
    v = _io_cast(_normal(rng, (B_, T_, H, Dv)), wl.io)
    lo, hi = log_alpha_range
    log_alpha = (lo + (hi - lo) * rng.random((B_, T_, H, Dk), dtype=np.float32)).astype(np.float32)
    b_logit = _normal(rng, (B_, T_, H, Dk))
    w_logit = _normal(rng, (B_, T_, H, Dv))
    extra = {}
    if gate_logits:
        log_alpha = bf16_round(log_alpha)
        extra = dict(b_logit=bf16_round(b_logit), w_logit=bf16_round(w_logit))
        b = w = None
    else:
        b = _sigmoid(b_logit)
        if b_scale != 1.0:
            b = (b * np.float32(b_scale)).astype(np.float32)
        w = _sigmoid(w_logit)
    S0 = None
    if wl.with_S0:
        S0 = (0.02 * _normal(rng, (N, H, Dk, Dv))).astype(np.float32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, b=b, w=w, S0=S0, cu_seqlens=cu,
                B=B_, T=T_, H=H, Dk=Dk, Dv=Dv, N=N, io=wl.io, **extra)


def make_chunk_grads(inp, seed: int, with_dS_final: bool = True):
    """Upstream gradients for a backward call on `inp` (a make_chunk_inputs
    result), from their own PCG64 stream: dout ~ N(0, 1) [B, T, H, Dv] in the
    io dtype and dS_final ~ N(0, 1) [N, H, Dk, Dv] float32 (or None)."""
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    dout = _io_cast(_normal(rng, (inp["B"], inp["T"], inp["H"], inp["Dv"])), inp["io"])
    dSf = None
    if with_dS_final:
        dSf = _normal(rng, (inp["N"], inp["H"], inp["Dk"], inp["Dv"])).astype(np.float32)
    return dict(dout=dout, dS_final=dSf)


# ---------------------------------------------------------------------------
# Decode inputs
# ---------------------------------------------------------------------------

def make_decode_state(wl: DecodeWorkload, B: Optional[int] = None, H: Optional[int] = None):
    """Initial decode state S ~ N(0, 0.02^2), float32 [B, H, Dk, Dv]."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    return (0.02 * _normal(rng, (B, H, wl.Dk, wl.Dv))).astype(np.float32)


def make_decode_step(wl: DecodeWorkload, step: int, B: Optional[int] = None,
                     H: Optional[int] = None):
    """Inputs of decode step `step` (its own PCG64 stream seeded by (seed, step)).

    Returns float32 arrays q, k, v [B, H, D*] (bf16-exact when io is bf16)
    and log_alpha, b, w.
    """
    rng = np.random.Generator(np.random.PCG64([wl.seed, step + 1]))
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    q = _io_cast(_l2norm(_normal(rng, (B, H, wl.Dk))), wl.io)
    k = _io_cast(_l2norm(_normal(rng, (B, H, wl.Dk))), wl.io)
    v = _io_cast(_normal(rng, (B, H, wl.Dv)), wl.io)
    log_alpha = (-0.2 + 0.199 * rng.random((B, H, wl.Dk), dtype=np.float32)).astype(np.float32)
    b = _sigmoid(_normal(rng, (B, H, wl.Dk)))
    w = _sigmoid(_normal(rng, (B, H, wl.Dv)))
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, b=b, w=w)


# ---------------------------------------------------------------------------
# Token-mixer layer inputs
# ---------------------------------------------------------------------------
#
# The layer's width D = H * Dv (16 heads of 128 make the 2048-wide hidden
# state of a 1.3B-parameter model).  Distributions (all weights drawn here are
# random initialisations, not trained values):
#   x ~ N(0, 1) [B, T, D], bf16;
#   W_in ~ N(0, 1/D) [7 blocks, D], bf16 (projections come out ~ N(0, 1));
#   conv_w ~ U(-1, 1) / sqrt(L) [2*H*Dk + H*Dv, L], fp32;
#   alpha_bias ~ U(3, 6) [H*Dk], fp32 (alpha = sigmoid(~N(4.5, 1)) ~ 0.95..0.999);
#   norm_w = 1 + 0.1 N(0, 1) [Dv], fp32;
#   W_o ~ N(0, 1/(H*Dv)) [D, H*Dv], bf16;
#   S0 ~ N(0, 0.02^2) where present.
# Draw order: (lengths) -> x -> W_in -> conv_w -> alpha_bias -> norm_w -> W_o
# -> (state).  Generator: numpy PCG64.

@dataclass(frozen=True)
class LayerWorkload:
    name: str
    B: int
    T: int            # tokens per batch row (dense) or total packed tokens (varlen)
    H: int
    Dk: int
    Dv: int
    D: int            # model width
    conv_len: int
    seed: int
    with_S0: bool = False
    n_seqs: int = 0
    len_lo: int = 0
    len_hi: int = 0


LAYER_4K = LayerWorkload("layer_batch_B8_H16_T4096_d128_D2048", 8, 4096, 16, 128, 128, 2048, 4,
                         47005)


def layer_in_rows(H, Dk, Dv):
    """Rows of the stacked input weight: q, k, v, alpha, output gate, b, w."""
    return 4 * H * Dk + 3 * H * Dv


def make_layer_inputs(wl: LayerWorkload, lengths=None, T: Optional[int] = None,
                      B: Optional[int] = None, seed: Optional[int] = None):
    """Draw the inputs and weights of one layer-forward call.  bf16 values are
    float32 arrays holding bf16-representable numbers.  Returns a dict with
    x, W_in, conv_w, alpha_bias, norm_w, W_o, S0 (or None), cu_seqlens (or
    None) and meta fields B, T, H, Dk, Dv, D, L, N."""
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = None
    if wl.n_seqs or lengths is not None:
        if lengths is None:
            lengths = rng.integers(wl.len_lo, wl.len_hi, size=wl.n_seqs, endpoint=True)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B_, T_, N = 1, int(cu[-1]), len(lengths)
    else:
        B_ = wl.B if B is None else B
        T_ = wl.T if T is None else T
        N = B_
    H, Dk, Dv, D, L = wl.H, wl.Dk, wl.Dv, wl.D, wl.conv_len
    rows = layer_in_rows(H, Dk, Dv)
    x = bf16_round(_normal(rng, (B_, T_, D)))
    W_in = bf16_round(_normal(rng, (rows, D)) * np.float32(1.0 / np.sqrt(D)))
    conv_w = ((2.0 * rng.random((2 * H * Dk + H * Dv, L), dtype=np.float32) - 1.0)
              / np.float32(np.sqrt(L))).astype(np.float32)
    alpha_bias = (3.0 + 3.0 * rng.random(H * Dk, dtype=np.float32)).astype(np.float32)
    norm_w = (1.0 + 0.1 * _normal(rng, (Dv,))).astype(np.float32)
    W_o = bf16_round(_normal(rng, (D, H * Dv)) * np.float32(1.0 / np.sqrt(H * Dv)))
    S0 = None
    if wl.with_S0:
        S0 = (0.02 * _normal(rng, (N, H, Dk, Dv))).astype(np.float32)
    return dict(x=x, W_in=W_in, conv_w=conv_w, alpha_bias=alpha_bias, norm_w=norm_w, W_o=W_o,
                S0=S0, cu_seqlens=cu, B=B_, T=T_, H=H, Dk=Dk, Dv=Dv, D=D, L=L, N=N)


# ---------------------------------------------------------------------------
# Sliding-window attention inputs
# ---------------------------------------------------------------------------
#
# The hybrid model's attention layer over the same 16 heads of 128 and a
# 2048-token window.  q, k, v ~ N(0, 1) in bf16 (the scale 1/sqrt(d) keeps the
# logits ~ N(0, 1)).  Draw order: (lengths) -> q -> k -> v.  PCG64.

@dataclass(frozen=True)
class SwaWorkload:
    name: str
    B: int
    T: int
    H: int
    D: int
    window: int
    seed: int
    n_seqs: int = 0
    len_lo: int = 0
    len_hi: int = 0


SWA_4K = SwaWorkload("swa_batch_B8_H16_T4096_d128_W2048", 8, 4096, 16, 128, 2048, 47006)


def make_swa_inputs(wl: SwaWorkload, lengths=None, T: Optional[int] = None,
                    B: Optional[int] = None, seed: Optional[int] = None):
    """q, k, v (float32 arrays of bf16 values, [B, T, H, D]), cu_seqlens (or
    None) and meta fields B, T, H, D, N, window."""
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = None
    if wl.n_seqs or lengths is not None:
        if lengths is None:
            lengths = rng.integers(wl.len_lo, wl.len_hi, size=wl.n_seqs, endpoint=True)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B_, T_, N = 1, int(cu[-1]), len(lengths)
    else:
        B_ = wl.B if B is None else B
        T_ = wl.T if T is None else T
        N = B_
    shape = (B_, T_, wl.H, wl.D)
    q = bf16_round(_normal(rng, shape))
    k = bf16_round(_normal(rng, shape))
    v = bf16_round(_normal(rng, shape))
    return dict(q=q, k=k, v=v, cu_seqlens=cu, B=B_, T=T_, H=wl.H, D=wl.D, N=N, window=wl.window)


# Sliding-window attention layer: x ~ N(0, 1) [B, T, Dm] bf16; W_qkv ~
# N(0, 1/Dm) [3 H D, Dm] bf16; W_o ~ N(0, 1/(H D)) [Dm, H D] bf16.  Draw order:
# (lengths) -> x -> W_qkv -> W_o.  PCG64.

@dataclass(frozen=True)
class SwaLayerWorkload:
    name: str
    B: int
    T: int
    H: int
    D: int
    Dm: int
    window: int
    seed: int


SWA_LAYER_4K = SwaLayerWorkload("swa_layer_B8_H16_T4096_d128_D2048_W2048", 8, 4096, 16, 128, 2048,
                                2048, 47007)


def make_swa_layer_inputs(wl: SwaLayerWorkload, lengths=None, T: Optional[int] = None,
                          B: Optional[int] = None):
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    cu = None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B_, T_, N = 1, int(cu[-1]), len(lengths)
    else:
        B_ = wl.B if B is None else B
        T_ = wl.T if T is None else T
        N = B_
    HD = wl.H * wl.D
    x = bf16_round(_normal(rng, (B_, T_, wl.Dm)))
    W_qkv = bf16_round(_normal(rng, (3 * HD, wl.Dm)) * np.float32(1.0 / np.sqrt(wl.Dm)))
    W_o = bf16_round(_normal(rng, (wl.Dm, HD)) * np.float32(1.0 / np.sqrt(HD)))
    return dict(x=x, W_qkv=W_qkv, W_o=W_o, cu_seqlens=cu, B=B_, T=T_, H=wl.H, D=wl.D, Dm=wl.Dm,
                N=N, window=wl.window)

"""Python binding of libgdn2 (Gated DeltaNet-2 core recurrence on MI355X).

Thin ctypes marshalling over the C ABI declared in include/libgdn2.h: the
gdn2_* functions take raw device pointers and sizes exactly like their C
counterparts; chunk_fwd(), chunk_fwd_gate_logits(), chunk_bwd() and step() accept
torch tensors, allocate outputs and the workspace with torch, and pass torch's
current stream.  Every step of the
computation runs in the HIP library; if libgdn2.so is missing, loading fails
with an error (there is no fallback).
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn2.so")

GDN2_OK = 0
GDN2_ERR_INVALID_ARGUMENT = 1
GDN2_ERR_UNSUPPORTED = 2
GDN2_ERR_WORKSPACE = 3
GDN2_ERR_HIP = 4
GDN2_F32 = 0
GDN2_BF16 = 1
CHUNK = 64

GDN2_STAGE_PLAN = 1
GDN2_STAGE_FACTORS = 2
GDN2_STAGE_PROPAGATE = 4
GDN2_STAGE_ALL = 7
GDN2_STAGE_STORE_T = 8

EXPORTED = ("gdn2_abi_version", "gdn2_status_string", "gdn2_chunk_fwd_workspace_bytes",
            "gdn2_chunk_fwd_workspace_layout", "gdn2_chunk_fwd", "gdn2_chunk_fwd_stages",
            "gdn2_chunk_fwd_gate_logits", "gdn2_chunk_bwd_workspace_bytes", "gdn2_chunk_bwd",
            "gdn2_step", "gdn2_layer_fwd_workspace_bytes", "gdn2_layer_fwd",
            "gdn2_swa_fwd_workspace_bytes", "gdn2_swa_fwd", "gdn2_swa_layer_fwd_workspace_bytes",
            "gdn2_swa_layer_fwd")


class Gdn2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s" % (where, gdn2_status_string(status)))


class LayerWeights(ctypes.Structure):
    """gdn2_layer_weights: device addresses of the layer's weights."""
    _fields_ = [("W_in", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
                ("alpha_bias", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("W_o", ctypes.c_void_p)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("max_chunks", ctypes.c_int),
                ("off_Tinv", ctypes.c_size_t), ("off_W", ctypes.c_size_t),
                ("off_Qhat", ctypes.c_size_t), ("off_KhatT", ctypes.c_size_t),
                ("off_M", ctypes.c_size_t), ("off_U", ctypes.c_size_t),
                ("off_gamma_last", ctypes.c_size_t),
                ("off_plan", ctypes.c_size_t)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libgdn2.so (once).  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libgdn2.so not found at %s; build it with "
                          "`python -m gated_delta_rule_47_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn2_abi_version.restype = I
    lib.gdn2_abi_version.argtypes = []
    lib.gdn2_status_string.restype = ctypes.c_char_p
    lib.gdn2_status_string.argtypes = [I]
    lib.gdn2_chunk_fwd_workspace_bytes.restype = Z
    lib.gdn2_chunk_fwd_workspace_bytes.argtypes = [I] * 8
    lib.gdn2_chunk_fwd_workspace_layout.restype = I
    lib.gdn2_chunk_fwd_workspace_layout.argtypes = [I] * 8 + [ctypes.POINTER(WorkspaceLayout)]
    lib.gdn2_chunk_fwd.restype = I
    lib.gdn2_chunk_fwd.argtypes = [P] * 10 + [I] * 7 + [P, Z, P]
    lib.gdn2_chunk_fwd_stages.restype = I
    lib.gdn2_chunk_fwd_stages.argtypes = [P] * 10 + [I] * 7 + [P, Z, P, I]
    lib.gdn2_chunk_fwd_gate_logits.restype = I
    lib.gdn2_chunk_fwd_gate_logits.argtypes = [P] * 10 + [I] * 7 + [P, Z, P]
    lib.gdn2_chunk_bwd_workspace_bytes.restype = Z
    lib.gdn2_chunk_bwd_workspace_bytes.argtypes = [I] * 8
    lib.gdn2_chunk_bwd.restype = I
    lib.gdn2_chunk_bwd.argtypes = [P] * 17 + [I] * 7 + [P, Z, P]
    lib.gdn2_step.restype = I
    lib.gdn2_step.argtypes = [P] * 8 + [I] * 5 + [P]
    lib.gdn2_layer_fwd_workspace_bytes.restype = Z
    lib.gdn2_layer_fwd_workspace_bytes.argtypes = [I] * 8
    lib.gdn2_layer_fwd.restype = I
    lib.gdn2_layer_fwd.argtypes = ([P, ctypes.POINTER(LayerWeights), I, ctypes.c_float] + [P] * 4
                                   + [I] * 7 + [P, Z, P])
    lib.gdn2_swa_fwd_workspace_bytes.restype = Z
    lib.gdn2_swa_fwd_workspace_bytes.argtypes = [I, I]
    lib.gdn2_swa_fwd.restype = I
    lib.gdn2_swa_fwd.argtypes = [P] * 6 + [I] * 6 + [ctypes.c_float, P, Z, P]
    lib.gdn2_swa_layer_fwd_workspace_bytes.restype = Z
    lib.gdn2_swa_layer_fwd_workspace_bytes.argtypes = [I] * 7
    lib.gdn2_swa_layer_fwd.restype = I
    lib.gdn2_swa_layer_fwd.argtypes = [P] * 6 + [I] * 7 + [ctypes.c_float, P, Z, P]
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# Raw C-ABI wrappers (same names and arguments as the C functions)
# ---------------------------------------------------------------------------

def gdn2_abi_version():
    return load_library().gdn2_abi_version()


def gdn2_status_string(status):
    return load_library().gdn2_status_string(int(status)).decode()


def gdn2_chunk_fwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen):
    return load_library().gdn2_chunk_fwd_workspace_bytes(N, B, T, H, Dk, Dv, io, int(varlen))


def gdn2_chunk_fwd_workspace_layout(N, B, T, H, Dk, Dv, io, varlen):
    out = WorkspaceLayout()
    st = load_library().gdn2_chunk_fwd_workspace_layout(N, B, T, H, Dk, Dv, io, int(varlen),
                                                        ctypes.byref(out))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_fwd_workspace_layout")
    return out


def gdn2_chunk_fwd(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk, Dv,
                   io, workspace, workspace_bytes, stream):
    """Raw call: every pointer argument is an int (device address) or None."""
    return load_library().gdn2_chunk_fwd(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens,
                                          N, B, T, H, Dk, Dv, io, workspace, workspace_bytes,
                                          stream)


def gdn2_layer_fwd_workspace_bytes(N, B, T, H, Dk, Dv, D, varlen):
    return load_library().gdn2_layer_fwd_workspace_bytes(N, B, T, H, Dk, Dv, D, int(varlen))


def gdn2_layer_fwd(x, weights, conv_len, norm_eps, S0, y, S_final, cu_seqlens, N, B, T, H, Dk,
                   Dv, D, workspace, workspace_bytes, stream):
    """Raw call: weights is a LayerWeights; other pointers are ints or None."""
    return load_library().gdn2_layer_fwd(x, ctypes.byref(weights), conv_len, norm_eps, S0, y,
                                          S_final, cu_seqlens, N, B, T, H, Dk, Dv, D, workspace,
                                          workspace_bytes, stream)


def gdn2_swa_fwd_workspace_bytes(N, varlen):
    return load_library().gdn2_swa_fwd_workspace_bytes(N, int(varlen))


def gdn2_swa_fwd(q, k, v, o, lse, cu_seqlens, N, B, T, H, D, window, scale, workspace,
                 workspace_bytes, stream):
    """Raw call: pointers are ints or None."""
    return load_library().gdn2_swa_fwd(q, k, v, o, lse, cu_seqlens, N, B, T, H, D, window,
                                        scale, workspace, workspace_bytes, stream)


def gdn2_swa_layer_fwd_workspace_bytes(N, B, T, H, D, Dm, varlen):
    return load_library().gdn2_swa_layer_fwd_workspace_bytes(N, B, T, H, D, Dm, int(varlen))


def gdn2_swa_layer_fwd(x, W_qkv, W_o, y, lse, cu_seqlens, N, B, T, H, D, Dm, window, scale,
                       workspace, workspace_bytes, stream):
    """Raw call: pointers are ints or None."""
    return load_library().gdn2_swa_layer_fwd(x, W_qkv, W_o, y, lse, cu_seqlens, N, B, T, H, D, Dm,
                                              window, scale, workspace, workspace_bytes, stream)


def gdn2_chunk_fwd_stages(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk,
                          Dv, io, workspace, workspace_bytes, stream, stages):
    """Raw call of a subset of the chunk-forward stages (GDN2_STAGE_* bits)."""
    return load_library().gdn2_chunk_fwd_stages(q, k, v, log_alpha, b, w, S0, o, S_final,
                                                 cu_seqlens, N, B, T, H, Dk, Dv, io, workspace,
                                                 workspace_bytes, stream, stages)


def gdn2_chunk_fwd_gate_logits(q, k, v, log_alpha, b_logit, w_logit, S0, o, S_final, cu_seqlens,
                               N, B, T, H, Dk, Dv, io, workspace, workspace_bytes, stream):
    """Raw call: every pointer argument is an int (device address) or None."""
    return load_library().gdn2_chunk_fwd_gate_logits(q, k, v, log_alpha, b_logit, w_logit, S0, o,
                                                      S_final, cu_seqlens, N, B, T, H, Dk, Dv, io,
                                                      workspace, workspace_bytes, stream)


def gdn2_chunk_bwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen):
    return load_library().gdn2_chunk_bwd_workspace_bytes(N, B, T, H, Dk, Dv, io, int(varlen))


def gdn2_chunk_bwd(q, k, v, log_alpha, b, w, S0, dout, dS_final, dq, dk, dv, dlog_alpha, db, dw,
                   dS0, cu_seqlens, N, B, T, H, Dk, Dv, io, workspace, workspace_bytes, stream):
    """Raw call: every pointer argument is an int (device address) or None."""
    return load_library().gdn2_chunk_bwd(q, k, v, log_alpha, b, w, S0, dout, dS_final, dq, dk,
                                          dv, dlog_alpha, db, dw, dS0, cu_seqlens, N, B, T, H,
                                          Dk, Dv, io, workspace, workspace_bytes, stream)


def gdn2_step(q, k, v, log_alpha, b, w, S, o, B, H, Dk, Dv, io, stream):
    """Raw call: every pointer argument is an int (device address) or None."""
    return load_library().gdn2_step(q, k, v, log_alpha, b, w, S, o, B, H, Dk, Dv, io, stream)


# ---------------------------------------------------------------------------
# torch-tensor marshalling
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _io_of(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN2_BF16
    if t.dtype == torch.float32:
        return GDN2_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def chunk_fwd(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, o=None, S_final=None,
              output_final_state=True, workspace=None, stream=None, stages=GDN2_STAGE_ALL):
    """Chunk-parallel forward.  Shapes: q, k, log_alpha, b [B,T,H,Dk]; v, w [B,T,H,Dv].

    cu_seqlens (int32 device tensor [N+1]) selects a packed call (B must be 1).
    stages (GDN2_STAGE_* bits) runs only part of the forward, see the header.
    Returns (o [B,T,H,Dv] in q's dtype, S_final [N,H,Dk,Dv] float32 or None).
    """
    import torch
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_of(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype)
    for name, t in (("log_alpha", log_alpha), ("b", b), ("w", w), ("S0", S0)):
        _check(t, name, torch.float32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if S_final is None and output_final_state:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    varlen = cu_seqlens is not None
    nbytes = gdn2_chunk_fwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(o),
            _ptr(S_final), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, io, _ptr(workspace),
            workspace.numel(), _stream(stream))
    if stages == GDN2_STAGE_ALL:
        st = gdn2_chunk_fwd(*args)
    else:
        st = gdn2_chunk_fwd_stages(*args, stages)
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_fwd")
    return o, S_final


def step(q, k, v, log_alpha, b, w, S, o=None, stream=None):
    """One decode token: q, k, log_alpha, b [B,H,Dk]; v, w [B,H,Dv]; S [B,H,Dk,Dv] f32 in place."""
    import torch
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_of(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype)
    for name, t in (("log_alpha", log_alpha), ("b", b), ("w", w), ("S", S)):
        _check(t, name, torch.float32)
    if o is None:
        o = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    st = gdn2_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S), _ptr(o),
                   B, H, Dk, Dv, io, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_step")
    return o


def chunk_bwd(q, k, v, log_alpha, b, w, dout, S0=None, dS_final=None, cu_seqlens=None,
              need_dS0=True, workspace=None, stream=None):
    """Gradients of chunk_fwd for upstream gradients dout (of o) and dS_final
    (of S_final, None = zero).  Same shapes as chunk_fwd; bfloat16 q/k/v only.
    Returns a dict: dq, dk, dv (q's dtype), dlog_alpha, db, dw (float32) and
    dS0 ([N,H,Dk,Dv] float32, or None when need_dS0 is False).
    """
    import torch
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_of(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, q.dtype)
    for name, t in (("log_alpha", log_alpha), ("b", b), ("w", w), ("S0", S0),
                    ("dS_final", dS_final)):
        _check(t, name, torch.float32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dlog_alpha=torch.empty_like(log_alpha), db=torch.empty_like(b),
               dw=torch.empty_like(w),
               dS0=torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
               if need_dS0 else None)
    varlen = cu_seqlens is not None
    nbytes = gdn2_chunk_bwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = gdn2_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0),
                        _ptr(dout), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                        _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]),
                        _ptr(out["dw"]), _ptr(out["dS0"]), _ptr(cu_seqlens), N, B, T, H, Dk, Dv,
                        io, _ptr(workspace), workspace.numel(), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_bwd")
    return out


def chunk_fwd_gate_logits(q, k, v, log_alpha, b_logit, w_logit, S0=None, cu_seqlens=None,
                          o=None, S_final=None, output_final_state=True, workspace=None,
                          stream=None):
    """chunk_fwd with bfloat16 gate inputs: log_alpha itself and the logits of b
    and w (sigmoid taken in the kernel).  q, k, v must be bfloat16."""
    import torch
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_of(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("b_logit", b_logit),
                    ("w_logit", w_logit)):
        _check(t, name, torch.bfloat16)
    _check(S0, "S0", torch.float32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if S_final is None and output_final_state:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    varlen = cu_seqlens is not None
    nbytes = gdn2_chunk_fwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = gdn2_chunk_fwd_gate_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b_logit),
                                    _ptr(w_logit), _ptr(S0), _ptr(o), _ptr(S_final),
                                    _ptr(cu_seqlens), N, B, T, H, Dk, Dv, io, _ptr(workspace),
                                    workspace.numel(), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_fwd_gate_logits")
    return o, S_final


def layer_fwd(x, W_in, conv_w, alpha_bias, norm_w, W_o, H, Dk, Dv, norm_eps=1e-6, S0=None,
              cu_seqlens=None, y=None, S_final=None, output_final_state=True, workspace=None,
              stream=None):
    """Token-mixer layer forward (gdn2_layer_fwd).  x [B, T, D], W_in
    [7*H*Dk, D] and W_o [D, H*Dv] are bfloat16; conv_w [3*H*Dk, L],
    alpha_bias [H*Dk] and norm_w [Dv] float32.  Returns (y, S_final)."""
    import torch
    B, T, D = x.shape
    for name, t in (("x", x), ("W_in", W_in), ("W_o", W_o)):
        _check(t, name, torch.bfloat16)
    for name, t in (("conv_w", conv_w), ("alpha_bias", alpha_bias), ("norm_w", norm_w)):
        _check(t, name, torch.float32)
    _check(S0, "S0", torch.float32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    if W_in.shape != (7 * H * Dk, D) or W_o.shape != (D, H * Dv) or conv_w.dim() != 2 \
            or conv_w.shape[0] != 3 * H * Dk or alpha_bias.numel() != H * Dk \
            or norm_w.numel() != Dv:
        raise ValueError("layer weight shapes do not match H=%d, Dk=%d, Dv=%d, D=%d"
                         % (H, Dk, Dv, D))
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if y is None:
        y = torch.empty((B, T, D), dtype=torch.bfloat16, device=x.device)
    if S_final is None and output_final_state:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=x.device)
    nbytes = gdn2_layer_fwd_workspace_bytes(N, B, T, H, Dk, Dv, D, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    wts = LayerWeights(_ptr(W_in), _ptr(conv_w), _ptr(alpha_bias), _ptr(norm_w), _ptr(W_o))
    st = gdn2_layer_fwd(_ptr(x), wts, conv_w.shape[1], float(norm_eps), _ptr(S0), _ptr(y),
                        _ptr(S_final), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, D, _ptr(workspace),
                        workspace.numel(), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_layer_fwd")
    return y, S_final


def swa_fwd(q, k, v, window, scale=None, cu_seqlens=None, o=None, lse=None, return_lse=True,
            workspace=None, stream=None):
    """Sliding-window attention forward (gdn2_swa_fwd).  q, k, v bfloat16
    [B, T, H, D]; returns (o, lse) with lse float32 [B, H, T] (None if
    return_lse is False)."""
    import torch
    B, T, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, torch.bfloat16)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    nbytes = gdn2_swa_fwd_workspace_bytes(N, cu_seqlens is not None)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    st = gdn2_swa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), N, B, T,
                      H, D, int(window), float(scale), _ptr(workspace),
                      0 if workspace is None else workspace.numel(), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_swa_fwd")
    return o, lse


def swa_layer_fwd(x, W_qkv, W_o, H, D, window, scale=None, cu_seqlens=None, y=None, lse=None,
                  return_lse=True, workspace=None, stream=None):
    """Sliding-window attention layer (gdn2_swa_layer_fwd).  x [B, T, Dm],
    W_qkv [3 H D, Dm], W_o [Dm, H D], all bfloat16.  Returns (y, lse)."""
    import torch
    B, T, Dm = x.shape
    for name, t in (("x", x), ("W_qkv", W_qkv), ("W_o", W_o)):
        _check(t, name, torch.bfloat16)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    if W_qkv.shape != (3 * H * D, Dm) or W_o.shape != (Dm, H * D):
        raise ValueError("weight shapes do not match H=%d, D=%d, Dm=%d" % (H, D, Dm))
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if scale is None:
        scale = D ** -0.5
    if y is None:
        y = torch.empty((B, T, Dm), dtype=torch.bfloat16, device=x.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=x.device)
    nbytes = gdn2_swa_layer_fwd_workspace_bytes(N, B, T, H, D, Dm, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    st = gdn2_swa_layer_fwd(_ptr(x), _ptr(W_qkv), _ptr(W_o), _ptr(y), _ptr(lse), _ptr(cu_seqlens),
                            N, B, T, H, D, Dm, int(window), float(scale), _ptr(workspace),
                            workspace.numel(), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_swa_layer_fwd")
    return y, lse

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
# The ABI revision these argument lists are written for (gdn2_abi_version()).
ABI_VERSION = 3

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
            "gdn2_swa_layer_fwd", "gdn2_chunk_fwd_noalloc", "gdn2_device_info",
            "gdn2_chunk_train_workspace_bytes", "gdn2_chunk_fwd_train", "gdn2_chunk_bwd_saved")


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
                ("off_plan", ctypes.c_size_t), ("total_bytes_with_Tinv", ctypes.c_size_t)]


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
    if lib.gdn2_abi_version() != ABI_VERSION:
        raise ImportError("%s reports ABI %d, this binding expects %d; rebuild it with "
                          "`python -m gated_delta_rule_47_amd.build`"
                          % (path, lib.gdn2_abi_version(), ABI_VERSION))
    lib.gdn2_status_string.restype = ctypes.c_char_p
    lib.gdn2_status_string.argtypes = [I]
    lib.gdn2_device_info.restype = I
    lib.gdn2_device_info.argtypes = [I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.gdn2_chunk_fwd_workspace_bytes.restype = Z
    lib.gdn2_chunk_fwd_workspace_bytes.argtypes = [I] * 8
    lib.gdn2_chunk_fwd_workspace_layout.restype = I
    lib.gdn2_chunk_fwd_workspace_layout.argtypes = [I] * 8 + [ctypes.POINTER(WorkspaceLayout)]
    lib.gdn2_chunk_fwd.restype = I
    lib.gdn2_chunk_fwd.argtypes = [P] * 10 + [I] * 7 + [P, Z, P]
    lib.gdn2_chunk_fwd_noalloc.restype = I
    lib.gdn2_chunk_fwd_noalloc.argtypes = [P] * 10 + [I] * 7 + [P]
    lib.gdn2_chunk_fwd_stages.restype = I
    lib.gdn2_chunk_fwd_stages.argtypes = [P] * 10 + [I] * 7 + [P, Z, P, I]
    lib.gdn2_chunk_fwd_gate_logits.restype = I
    lib.gdn2_chunk_fwd_gate_logits.argtypes = [P] * 10 + [I] * 7 + [P, Z, P]
    lib.gdn2_chunk_bwd_workspace_bytes.restype = Z
    lib.gdn2_chunk_bwd_workspace_bytes.argtypes = [I] * 8
    lib.gdn2_chunk_bwd.restype = I
    lib.gdn2_chunk_bwd.argtypes = [P] * 17 + [I] * 7 + [P, Z, P]
    lib.gdn2_chunk_train_workspace_bytes.restype = Z
    lib.gdn2_chunk_train_workspace_bytes.argtypes = [I] * 8
    lib.gdn2_chunk_fwd_train.restype = I
    lib.gdn2_chunk_fwd_train.argtypes = [P] * 10 + [I] * 7 + [P, Z, P]
    lib.gdn2_chunk_bwd_saved.restype = I
    lib.gdn2_chunk_bwd_saved.argtypes = [P] * 16 + [I] * 7 + [P, Z, P]
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


def device_info(device=0):
    """(compute units, peak engine clock in kHz) of a device, from the HIP runtime."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    st = load_library().gdn2_device_info(int(device), ctypes.byref(cus), ctypes.byref(khz))
    if st != 0:
        raise Gdn2Error(st, "gdn2_device_info")
    return cus.value, khz.value


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


def gdn2_chunk_fwd_noalloc(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk,
                           Dv, io, stream):
    """Raw call of the chunk forward that allocates nothing (no workspace
    argument; the library's own fixed device region holds the intermediates)."""
    return load_library().gdn2_chunk_fwd_noalloc(q, k, v, log_alpha, b, w, S0, o, S_final,
                                                  cu_seqlens, N, B, T, H, Dk, Dv, io, stream)


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


def gdn2_chunk_train_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen):
    return load_library().gdn2_chunk_train_workspace_bytes(N, B, T, H, Dk, Dv, io, int(varlen))


def gdn2_chunk_fwd_train(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, N, B, T, H, Dk,
                         Dv, io, workspace, workspace_bytes, stream):
    """Raw call: every pointer argument is an int (device address) or None."""
    return load_library().gdn2_chunk_fwd_train(q, k, v, log_alpha, b, w, S0, o, S_final,
                                                cu_seqlens, N, B, T, H, Dk, Dv, io, workspace,
                                                workspace_bytes, stream)


def gdn2_chunk_bwd_saved(q, k, v, log_alpha, b, w, dout, dS_final, dq, dk, dv, dlog_alpha, db, dw,
                         dS0, cu_seqlens, N, B, T, H, Dk, Dv, io, workspace, workspace_bytes,
                         stream):
    """Raw call: every pointer argument is an int (device address) or None."""
    return load_library().gdn2_chunk_bwd_saved(q, k, v, log_alpha, b, w, dout, dS_final, dq, dk,
                                                dv, dlog_alpha, db, dw, dS0, cu_seqlens, N, B, T,
                                                H, Dk, Dv, io, workspace, workspace_bytes, stream)


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


def _validate(specs, device=None):
    """Validate tensor arguments before their addresses reach the library.

    specs: (name, tensor or None, expected shape or None, dtype or None).
    Every tensor's shape and dtype is checked first, then that each lives on
    `device` and is contiguous: a tensor of the wrong size would otherwise
    become out-of-bounds device reads or writes.
    """
    for name, t, shape, dtype in specs:
        if t is None:
            continue
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if dtype is not None and t.dtype != dtype:
            raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    for name, t, _, _ in specs:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if device is not None and t.device != device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _check(t, name, shape=None, dtype=None, device=None):
    _validate([(name, t, shape, dtype)], device)


def _check_cu_seqlens(cu_seqlens, B, device):
    """Packed calls: int32 [N+1] offsets on the device, with B == 1.  Returns N."""
    import torch
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N+1 offsets")
    if B != 1:
        raise ValueError("a packed call (cu_seqlens given) needs B == 1, got B = %d" % B)
    _check(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=device)
    return cu_seqlens.numel() - 1


def _workspace(workspace, nbytes, device):
    """The caller's workspace (any dtype, contiguous, on the device) or a new one;
    returns (tensor, size in bytes)."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _check(workspace, "workspace", device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _chunk_shapes(q, v, cu_seqlens):
    """(B, T, H, Dk, Dv, N) of a chunk call, from q [B,T,H,Dk] and v [B,T,H,Dv]."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, T, H, D] tensors")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else _check_cu_seqlens(cu_seqlens, B, q.device)
    return B, T, H, Dk, Dv, N


def chunk_fwd(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, o=None, S_final=None,
              output_final_state=True, workspace=None, stream=None, stages=GDN2_STAGE_ALL):
    """Chunk-parallel forward.  Shapes: q, k, log_alpha, b [B,T,H,Dk]; v, w [B,T,H,Dv].

    cu_seqlens (int32 device tensor [N+1]) selects a packed call (B must be 1).
    stages (GDN2_STAGE_* bits) runs only part of the forward, see the header.
    Returns (o [B,T,H,Dv] in q's dtype, S_final [N,H,Dk,Dv] float32 or None).
    """
    import torch
    B, T, H, Dk, Dv, N = _chunk_shapes(q, v, cu_seqlens)
    io = _io_of(q)
    dev = q.device
    tk, tv, st_shape = (B, T, H, Dk), (B, T, H, Dv), (N, H, Dk, Dv)
    f32 = torch.float32
    _validate([("q", q, tk, q.dtype), ("k", k, tk, q.dtype), ("v", v, tv, q.dtype),
               ("o", o, tv, q.dtype), ("log_alpha", log_alpha, tk, f32), ("b", b, tk, f32),
               ("w", w, tv, f32), ("S0", S0, st_shape, f32), ("S_final", S_final, st_shape, f32)],
              dev)
    if o is None:
        o = torch.empty(tv, dtype=q.dtype, device=dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(st_shape, dtype=torch.float32, device=dev)
    varlen = cu_seqlens is not None
    nbytes = gdn2_chunk_fwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen)
    if stages & GDN2_STAGE_STORE_T:
        nbytes = gdn2_chunk_fwd_workspace_layout(N, B, T, H, Dk, Dv, io,
                                                 varlen).total_bytes_with_Tinv
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(o),
            _ptr(S_final), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, io, _ptr(workspace),
            ws_bytes, _stream(stream))
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
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [B, H, D] tensors")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_of(q)
    dev = q.device
    f32, dt = torch.float32, q.dtype
    _validate([("q", q, (B, H, Dk), dt), ("k", k, (B, H, Dk), dt), ("v", v, (B, H, Dv), dt),
               ("o", o, (B, H, Dv), dt), ("log_alpha", log_alpha, (B, H, Dk), f32),
               ("b", b, (B, H, Dk), f32), ("w", w, (B, H, Dv), f32),
               ("S", S, (B, H, Dk, Dv), f32)], dev)
    if S is None:
        raise ValueError("S (the state updated in place) is required")
    if o is None:
        o = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    st = gdn2_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S), _ptr(o),
                   B, H, Dk, Dv, io, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_step")
    return o


def chunk_bwd(q, k, v, log_alpha, b, w, dout, S0=None, dS_final=None, cu_seqlens=None,
              need_dS0=True, workspace=None, stream=None):
    """Gradients of chunk_fwd for upstream gradients dout (of o) and dS_final
    (of S_final, None = zero).  Same shapes and dtypes as chunk_fwd (bf16 or
    fp32 q/k/v/dout).
    Returns a dict: dq, dk, dv (q's dtype), dlog_alpha, db, dw (float32) and
    dS0 ([N,H,Dk,Dv] float32, or None when need_dS0 is False).
    """
    import torch
    B, T, H, Dk, Dv, N = _chunk_shapes(q, v, cu_seqlens)
    io = _io_of(q)
    dev = q.device
    tk, tv, st_shape = (B, T, H, Dk), (B, T, H, Dv), (N, H, Dk, Dv)
    f32 = torch.float32
    _validate([("q", q, tk, q.dtype), ("k", k, tk, q.dtype), ("v", v, tv, q.dtype),
               ("dout", dout, tv, q.dtype), ("log_alpha", log_alpha, tk, f32),
               ("b", b, tk, f32), ("w", w, tv, f32), ("S0", S0, st_shape, f32),
               ("dS_final", dS_final, st_shape, f32)], dev)
    if dout is None:
        raise ValueError("dout is required")
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dlog_alpha=torch.empty_like(log_alpha), db=torch.empty_like(b),
               dw=torch.empty_like(w),
               dS0=torch.empty(st_shape, dtype=torch.float32, device=dev) if need_dS0 else None)
    varlen = cu_seqlens is not None
    nbytes = gdn2_chunk_bwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen)
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    st = gdn2_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0),
                        _ptr(dout), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                        _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]),
                        _ptr(out["dw"]), _ptr(out["dS0"]), _ptr(cu_seqlens), N, B, T, H, Dk, Dv,
                        io, _ptr(workspace), ws_bytes, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_bwd")
    return out


def chunk_fwd_train(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, o=None, S_final=None,
                    output_final_state=True, workspace=None, stream=None):
    """chunk_fwd (bf16 only) that also keeps, in `workspace`, what
    chunk_bwd_saved needs.  Returns (o, S_final, workspace); hold the
    workspace until the backward."""
    import torch
    B, T, H, Dk, Dv, N = _chunk_shapes(q, v, cu_seqlens)
    io = _io_of(q)
    dev = q.device
    tk, tv, st_shape = (B, T, H, Dk), (B, T, H, Dv), (N, H, Dk, Dv)
    f32 = torch.float32
    _validate([("q", q, tk, q.dtype), ("k", k, tk, q.dtype), ("v", v, tv, q.dtype),
               ("o", o, tv, q.dtype), ("log_alpha", log_alpha, tk, f32), ("b", b, tk, f32),
               ("w", w, tv, f32), ("S0", S0, st_shape, f32), ("S_final", S_final, st_shape, f32)],
              dev)
    if o is None:
        o = torch.empty(tv, dtype=q.dtype, device=dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(st_shape, dtype=torch.float32, device=dev)
    nbytes = gdn2_chunk_train_workspace_bytes(N, B, T, H, Dk, Dv, io, cu_seqlens is not None)
    if nbytes == 0:
        raise Gdn2Error(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_train_workspace_bytes")
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    st = gdn2_chunk_fwd_train(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                              _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens), N, B, T, H, Dk,
                              Dv, io, _ptr(workspace), ws_bytes, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_fwd_train")
    return o, S_final, workspace


def chunk_bwd_saved(q, k, v, log_alpha, b, w, dout, workspace, dS_final=None, cu_seqlens=None,
                    need_dS0=True, stream=None):
    """chunk_bwd's gradients from the workspace of a chunk_fwd_train call on the
    same inputs (S0 entered through the saved states).  Returns the dict of
    chunk_bwd."""
    import torch
    B, T, H, Dk, Dv, N = _chunk_shapes(q, v, cu_seqlens)
    io = _io_of(q)
    dev = q.device
    tk, tv, st_shape = (B, T, H, Dk), (B, T, H, Dv), (N, H, Dk, Dv)
    f32 = torch.float32
    _validate([("q", q, tk, q.dtype), ("k", k, tk, q.dtype), ("v", v, tv, q.dtype),
               ("dout", dout, tv, q.dtype), ("log_alpha", log_alpha, tk, f32),
               ("b", b, tk, f32), ("w", w, tv, f32), ("dS_final", dS_final, st_shape, f32)], dev)
    if dout is None or workspace is None:
        raise ValueError("dout and the training forward's workspace are required")
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dlog_alpha=torch.empty_like(log_alpha), db=torch.empty_like(b),
               dw=torch.empty_like(w),
               dS0=torch.empty(st_shape, dtype=torch.float32, device=dev) if need_dS0 else None)
    nbytes = gdn2_chunk_train_workspace_bytes(N, B, T, H, Dk, Dv, io, cu_seqlens is not None)
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    st = gdn2_chunk_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                              _ptr(dout), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                              _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]),
                              _ptr(out["dw"]), _ptr(out["dS0"]), _ptr(cu_seqlens), N, B, T, H, Dk,
                              Dv, io, _ptr(workspace), ws_bytes, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_chunk_bwd_saved")
    return out


def chunk_fwd_gate_logits(q, k, v, log_alpha, b_logit, w_logit, S0=None, cu_seqlens=None,
                          o=None, S_final=None, output_final_state=True, workspace=None,
                          stream=None):
    """chunk_fwd with bfloat16 gate inputs: log_alpha itself and the logits of b
    and w (sigmoid taken in the kernel).  q, k, v must be bfloat16."""
    import torch
    B, T, H, Dk, Dv, N = _chunk_shapes(q, v, cu_seqlens)
    io = _io_of(q)
    dev = q.device
    tk, tv, st_shape = (B, T, H, Dk), (B, T, H, Dv), (N, H, Dk, Dv)
    bf, f32 = torch.bfloat16, torch.float32
    _validate([("q", q, tk, bf), ("k", k, tk, bf), ("v", v, tv, bf),
               ("log_alpha", log_alpha, tk, bf), ("b_logit", b_logit, tk, bf),
               ("w_logit", w_logit, tv, bf), ("o", o, tv, bf), ("S0", S0, st_shape, f32),
               ("S_final", S_final, st_shape, f32)], dev)
    if o is None:
        o = torch.empty(tv, dtype=q.dtype, device=dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(st_shape, dtype=torch.float32, device=dev)
    varlen = cu_seqlens is not None
    nbytes = gdn2_chunk_fwd_workspace_bytes(N, B, T, H, Dk, Dv, io, varlen)
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    st = gdn2_chunk_fwd_gate_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b_logit),
                                    _ptr(w_logit), _ptr(S0), _ptr(o), _ptr(S_final),
                                    _ptr(cu_seqlens), N, B, T, H, Dk, Dv, io, _ptr(workspace),
                                    ws_bytes, _stream(stream))
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
    if x.dim() != 3:
        raise ValueError("x must be a [B, T, D] tensor")
    B, T, D = x.shape
    dev = x.device
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be a [3*H*Dk, L] tensor")
    N = B if cu_seqlens is None else _check_cu_seqlens(cu_seqlens, B, dev)
    bf, f32 = torch.bfloat16, torch.float32
    _validate([("x", x, (B, T, D), bf), ("W_in", W_in, (7 * H * Dk, D), bf),
               ("W_o", W_o, (D, H * Dv), bf), ("y", y, (B, T, D), bf),
               ("conv_w", conv_w, (3 * H * Dk, conv_w.shape[1]), f32),
               ("alpha_bias", alpha_bias, (H * Dk,), f32), ("norm_w", norm_w, (Dv,), f32),
               ("S0", S0, (N, H, Dk, Dv), f32), ("S_final", S_final, (N, H, Dk, Dv), f32)], dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=torch.bfloat16, device=dev)
    if S_final is None and output_final_state:
        S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    nbytes = gdn2_layer_fwd_workspace_bytes(N, B, T, H, Dk, Dv, D, cu_seqlens is not None)
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    wts = LayerWeights(_ptr(W_in), _ptr(conv_w), _ptr(alpha_bias), _ptr(norm_w), _ptr(W_o))
    st = gdn2_layer_fwd(_ptr(x), wts, conv_w.shape[1], float(norm_eps), _ptr(S0), _ptr(y),
                        _ptr(S_final), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, D, _ptr(workspace),
                        ws_bytes, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_layer_fwd")
    return y, S_final


def swa_fwd(q, k, v, window, scale=None, cu_seqlens=None, o=None, lse=None, return_lse=True,
            workspace=None, stream=None):
    """Sliding-window attention forward (gdn2_swa_fwd).  q, k, v bfloat16
    [B, T, H, D]; returns (o, lse) with lse float32 [B, H, T] (None if
    return_lse is False)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be a [B, T, H, D] tensor")
    B, T, H, D = q.shape
    dev = q.device
    N = B if cu_seqlens is None else _check_cu_seqlens(cu_seqlens, B, dev)
    bf = torch.bfloat16
    _validate([("q", q, (B, T, H, D), bf), ("k", k, (B, T, H, D), bf),
               ("v", v, (B, T, H, D), bf), ("o", o, (B, T, H, D), bf),
               ("lse", lse, (B, H, T), torch.float32)], dev)
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    nbytes = gdn2_swa_fwd_workspace_bytes(N, cu_seqlens is not None)
    ws_bytes = 0
    if workspace is not None or nbytes:
        workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    st = gdn2_swa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), N, B, T,
                      H, D, int(window), float(scale), _ptr(workspace), ws_bytes,
                      _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_swa_fwd")
    return o, lse


def swa_layer_fwd(x, W_qkv, W_o, H, D, window, scale=None, cu_seqlens=None, y=None, lse=None,
                  return_lse=True, workspace=None, stream=None):
    """Sliding-window attention layer (gdn2_swa_layer_fwd).  x [B, T, Dm],
    W_qkv [3 H D, Dm], W_o [Dm, H D], all bfloat16.  Returns (y, lse)."""
    import torch
    if x.dim() != 3:
        raise ValueError("x must be a [B, T, Dm] tensor")
    B, T, Dm = x.shape
    dev = x.device
    N = B if cu_seqlens is None else _check_cu_seqlens(cu_seqlens, B, dev)
    bf = torch.bfloat16
    _validate([("x", x, (B, T, Dm), bf), ("W_qkv", W_qkv, (3 * H * D, Dm), bf),
               ("W_o", W_o, (Dm, H * D), bf), ("y", y, (B, T, Dm), bf),
               ("lse", lse, (B, H, T), torch.float32)], dev)
    if scale is None:
        scale = D ** -0.5
    if y is None:
        y = torch.empty((B, T, Dm), dtype=torch.bfloat16, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    nbytes = gdn2_swa_layer_fwd_workspace_bytes(N, B, T, H, D, Dm, cu_seqlens is not None)
    workspace, ws_bytes = _workspace(workspace, nbytes, dev)
    st = gdn2_swa_layer_fwd(_ptr(x), _ptr(W_qkv), _ptr(W_o), _ptr(y), _ptr(lse), _ptr(cu_seqlens),
                            N, B, T, H, D, Dm, int(window), float(scale), _ptr(workspace),
                            ws_bytes, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st, "gdn2_swa_layer_fwd")
    return y, lse

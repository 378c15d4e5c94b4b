"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before launching anything."""

import ctypes
import os
import re

import pytest

import gated_delta_rule_47_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgdn2.h")

P16 = 1 << 20  # a 16-byte aligned fake address; never dereferenced (validation fails first)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = g.load_library()
    declared = _declared_functions()
    assert set(declared) == set(g.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_version_and_status_strings():
    assert g.gdn2_abi_version() == g.ABI_VERSION == 3
    assert g.gdn2_status_string(g.GDN2_OK) == "GDN2_OK"
    assert g.gdn2_status_string(g.GDN2_ERR_WORKSPACE) == "GDN2_ERR_WORKSPACE"
    assert g.gdn2_status_string(99) == "GDN2_ERR_UNKNOWN"


def test_workspace_size_and_layout():
    n = g.gdn2_chunk_fwd_workspace_bytes(8, 8, 4096, 16, 128, 128, g.GDN2_BF16, 0)
    L = g.gdn2_chunk_fwd_workspace_layout(8, 8, 4096, 16, 128, 128, g.GDN2_BF16, 0)
    assert L.total_bytes == n and L.max_chunks == 8 * 64
    chd = 8 * 64 * 16
    # W, Qhat, KhatT, M, U in bf16 plus gamma_last in f32, each 256-byte aligned;
    # the optional T slot comes after everything else and is not in total_bytes
    assert L.off_Qhat - L.off_W == chd * 64 * 128 * 2
    assert L.off_M - L.off_KhatT == chd * 128 * 64 * 2
    assert L.off_Tinv == L.total_bytes
    assert L.total_bytes_with_Tinv == L.total_bytes + chd * 64 * 64 * 2
    for off in (L.off_Tinv, L.off_W, L.off_Qhat, L.off_KhatT, L.off_M, L.off_gamma_last):
        assert off % 256 == 0
    # the backward's workspace has no T, Qhat or M slots of its own
    nb = g.gdn2_chunk_bwd_workspace_bytes(8, 8, 4096, 16, 128, 128, g.GDN2_BF16, 0)
    assert 0 < nb < 2_000_000_000
    Lv = g.gdn2_chunk_fwd_workspace_layout(32, 1, 139000, 16, 128, 128, g.GDN2_BF16, 1)
    assert Lv.max_chunks == (139000 + 63) // 64 + 32
    assert Lv.total_bytes >= Lv.off_plan + 4 * (33 + 3 * Lv.max_chunks)
    assert g.gdn2_chunk_fwd_workspace_bytes(1, 1, 64, 1, 96, 96, g.GDN2_BF16, 0) == 0
    assert g.gdn2_chunk_fwd_workspace_bytes(1, 1, 64, 1, 128, 128, 7, 0) == 0
    assert g.gdn2_chunk_fwd_workspace_bytes(1, 1, 0, 1, 64, 64, g.GDN2_F32, 0) == 0


def _chunk(**kw):
    args = dict(q=P16, k=P16, v=P16, log_alpha=P16, b=P16, w=P16, S0=None, o=P16 + 4096,
                S_final=None, cu_seqlens=None, N=1, B=1, T=64, H=1, Dk=128, Dv=128,
                io=g.GDN2_BF16, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return g.gdn2_chunk_fwd(**args)


def test_chunk_fwd_validation():
    assert _chunk(q=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _chunk(w=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _chunk(k=P16 + 8) == g.GDN2_ERR_INVALID_ARGUMENT          # misaligned
    assert _chunk(Dk=96, Dv=96) == g.GDN2_ERR_UNSUPPORTED
    assert _chunk(Dk=128, Dv=64) == g.GDN2_ERR_UNSUPPORTED
    assert _chunk(io=5) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _chunk(T=-1) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _chunk(N=2, B=1) == g.GDN2_ERR_INVALID_ARGUMENT           # dense needs N == B
    assert _chunk(cu_seqlens=P16, N=2, B=2) == g.GDN2_ERR_INVALID_ARGUMENT  # varlen needs B == 1
    assert _chunk(S_final=P16 + 4096) == g.GDN2_ERR_INVALID_ARGUMENT   # o aliases S_final
    assert _chunk() == g.GDN2_ERR_WORKSPACE                           # workspace missing
    need = g.gdn2_chunk_fwd_workspace_bytes(1, 1, 64, 1, 128, 128, g.GDN2_BF16, 0)
    assert _chunk(workspace=P16, workspace_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
    assert _chunk(workspace=P16 + 16, workspace_bytes=need) == g.GDN2_ERR_WORKSPACE  # not 256-aligned
    # the T slot is required only when the stages ask for T
    L = g.gdn2_chunk_fwd_workspace_layout(1, 1, 64, 1, 128, 128, g.GDN2_BF16, 0)
    assert g.gdn2_chunk_fwd_stages(P16, P16, P16, P16, P16, P16, None, P16 + 4096, None, None, 1, 1,
                                   64, 1, 128, 128, g.GDN2_BF16, P16, L.total_bytes, None,
                                   g.GDN2_STAGE_ALL | g.GDN2_STAGE_STORE_T) == g.GDN2_ERR_WORKSPACE
    # empty calls succeed without touching the GPU
    assert _chunk(N=0, B=0) == g.GDN2_OK
    assert _chunk(H=0) == g.GDN2_OK


def test_chunk_fwd_empty_call_without_buffers():
    """T == 0 with o, S0 and the token pointers all NULL is a valid call (it
    writes S_final = 0).  Validation must accept it; without a GPU the launch
    that writes S_final is what fails here."""
    none = dict(q=None, k=None, v=None, log_alpha=None, b=None, w=None, o=None, S0=None)
    st = _chunk(T=0, S_final=P16 + 8192, **none)
    assert st in (g.GDN2_OK, g.GDN2_ERR_HIP)
    assert _chunk(T=0, S_final=None, **none) in (g.GDN2_OK, g.GDN2_ERR_HIP)
    # a non-empty call still needs every token pointer
    assert _chunk(T=64, S_final=P16 + 8192, **none) == g.GDN2_ERR_INVALID_ARGUMENT


def _bwd(fn, **kw):
    args = dict(q=P16, k=P16, v=P16, log_alpha=P16, b=P16, w=P16, dout=P16, dS_final=None,
                dq=P16 + 4096, dk=P16 + 8192, dv=P16 + 12288, dlog_alpha=P16 + 16384,
                db=P16 + 20480, dw=P16 + 24576, dS0=None, cu_seqlens=None, N=1, B=1, T=64, H=1,
                Dk=128, Dv=128, io=g.GDN2_BF16, workspace=None, workspace_bytes=0, stream=None)
    if fn is g.gdn2_chunk_bwd:
        args["S0"] = None
    args.update(kw)
    return fn(**args)


def test_chunk_bwd_validation():
    """gdn2_chunk_bwd and gdn2_chunk_bwd_saved reject bad arguments before any launch."""
    sizes = (1, 1, 64, 1, 128, 128, g.GDN2_BF16, 0)
    for fn, need in ((g.gdn2_chunk_bwd, g.gdn2_chunk_bwd_workspace_bytes(*sizes)),
                     (g.gdn2_chunk_bwd_saved, g.gdn2_chunk_train_workspace_bytes(*sizes))):
        assert _bwd(fn, q=None) == g.GDN2_ERR_INVALID_ARGUMENT
        assert _bwd(fn, dout=None) == g.GDN2_ERR_INVALID_ARGUMENT
        assert _bwd(fn, dq=P16 + 4104) == g.GDN2_ERR_INVALID_ARGUMENT      # misaligned
        assert _bwd(fn, dk=P16 + 4096) == g.GDN2_ERR_INVALID_ARGUMENT      # dk aliases dq
        assert _bwd(fn, dq=P16) == g.GDN2_ERR_INVALID_ARGUMENT             # dq aliases the inputs
        assert _bwd(fn, Dk=96, Dv=96) == g.GDN2_ERR_UNSUPPORTED
        assert _bwd(fn, N=2, B=1) == g.GDN2_ERR_INVALID_ARGUMENT
        assert _bwd(fn) == g.GDN2_ERR_WORKSPACE                          # workspace missing
        assert _bwd(fn, workspace=P16, workspace_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
        assert _bwd(fn, workspace=P16 + 16, workspace_bytes=need) == g.GDN2_ERR_WORKSPACE
        assert _bwd(fn, N=0, B=0) == g.GDN2_OK and _bwd(fn, H=0) == g.GDN2_OK
    # the saved-state backward is bf16 only
    assert _bwd(g.gdn2_chunk_bwd_saved, io=g.GDN2_F32) == g.GDN2_ERR_UNSUPPORTED


def test_chunk_fwd_train_validation_and_workspace():
    """The training forward's workspace is the forward's (without T) plus the
    backward's slots and a dKhat slot of its own; bf16 only."""
    fwd = g.gdn2_chunk_fwd_workspace_bytes(8, 8, 4096, 16, 128, 128, g.GDN2_BF16, 0)
    tr = g.gdn2_chunk_train_workspace_bytes(8, 8, 4096, 16, 128, 128, g.GDN2_BF16, 0)
    chd = 8 * 64 * 16
    # M^T, Qhat^T, T^T, Sc, dSc, dKhat (bf16) per chunk-head
    assert tr == fwd + chd * 2 * (64 * 64 + 128 * 64 + 64 * 64 + 128 * 128 + 128 * 128 + 64 * 128)
    assert g.gdn2_chunk_train_workspace_bytes(8, 8, 4096, 16, 128, 128, g.GDN2_F32, 0) == 0
    args = dict(q=P16, k=P16, v=P16, log_alpha=P16, b=P16, w=P16, S0=None, o=P16 + 4096,
                S_final=None, cu_seqlens=None, N=1, B=1, T=64, H=1, Dk=128, Dv=128,
                io=g.GDN2_BF16, workspace=None, workspace_bytes=0, stream=None)
    call = lambda **kw: g.gdn2_chunk_fwd_train(**dict(args, **kw))
    need = g.gdn2_chunk_train_workspace_bytes(1, 1, 64, 1, 128, 128, g.GDN2_BF16, 0)
    assert call(io=g.GDN2_F32) == g.GDN2_ERR_UNSUPPORTED
    assert call(q=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert call() == g.GDN2_ERR_WORKSPACE
    assert call(workspace=P16, workspace_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
    assert call(N=0, B=0) == g.GDN2_OK


def _step(**kw):
    args = dict(q=P16, k=P16, v=P16, log_alpha=P16, b=P16, w=P16, S=P16 + 8192, o=P16 + 4096,
                B=1, H=1, Dk=128, Dv=128, io=g.GDN2_BF16, stream=None)
    args.update(kw)
    return g.gdn2_step(**args)


def test_step_validation():
    assert _step(S=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _step(o=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _step(v=P16 + 4) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _step(o=P16 + 8192) == g.GDN2_ERR_INVALID_ARGUMENT         # o aliases S
    assert _step(Dk=32, Dv=32) == g.GDN2_ERR_UNSUPPORTED
    assert _step(io=-1) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _step(B=-1) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _step(B=0) == g.GDN2_OK


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("gated_delta_rule_47_amd")
    with pytest.raises(ImportError):
        mod._lib_backup = mod._lib
        try:
            mod._lib = None
            mod.load_library(str(tmp_path / "missing.so"))
        finally:
            mod._lib = mod._lib_backup


def _layer(weights=None, **kw):
    w = weights or g.LayerWeights(P16, P16 + 1024, P16 + 2048, P16 + 3072, P16 + 4096)
    args = dict(x=P16 + 8192, weights=w, conv_len=4, norm_eps=1e-6, S0=None, y=P16 + 16384,
                S_final=None, cu_seqlens=None, N=1, B=1, T=64, H=1, Dk=128, Dv=128, D=256,
                workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return g.gdn2_layer_fwd(**args)


def test_layer_fwd_validation():
    assert _layer(x=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _layer(y=P16 + 8) == g.GDN2_ERR_INVALID_ARGUMENT               # misaligned
    assert _layer(y=P16 + 8192) == g.GDN2_ERR_INVALID_ARGUMENT            # y aliases x
    assert _layer(y=P16) == g.GDN2_ERR_INVALID_ARGUMENT                   # y aliases W_in
    bad_w = g.LayerWeights(P16, None, P16 + 2048, P16 + 3072, P16 + 4096)
    assert _layer(weights=bad_w) == g.GDN2_ERR_INVALID_ARGUMENT           # conv_w missing
    assert _layer(conv_len=0) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _layer(conv_len=9) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _layer(norm_eps=-1.0) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _layer(norm_eps=float("nan")) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _layer(D=100) == g.GDN2_ERR_UNSUPPORTED                        # D % 8 != 0
    assert _layer(Dk=96, Dv=96) == g.GDN2_ERR_UNSUPPORTED
    assert _layer(N=2, B=1) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _layer() == g.GDN2_ERR_WORKSPACE
    need = g.gdn2_layer_fwd_workspace_bytes(1, 1, 64, 1, 128, 128, 256, 0)
    assert need > g.gdn2_chunk_fwd_workspace_bytes(1, 1, 64, 1, 128, 128, g.GDN2_BF16, 0)
    assert _layer(workspace=P16, workspace_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
    assert g.gdn2_layer_fwd_workspace_bytes(1, 1, 64, 1, 128, 128, 100, 0) == 0
    assert _layer(N=0, B=0) == g.GDN2_OK
    assert _layer(H=0) == g.GDN2_OK


def _swa(**kw):
    args = dict(q=P16, k=P16 + 4096, v=P16 + 8192, o=P16 + 12288, lse=None, cu_seqlens=None, N=1,
                B=1, T=64, H=1, D=128, window=16, scale=0.088, workspace=None, workspace_bytes=0,
                stream=None)
    args.update(kw)
    return g.gdn2_swa_fwd(**args)


def test_swa_fwd_validation():
    assert _swa(q=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _swa(o=P16 + 12296) == g.GDN2_ERR_INVALID_ARGUMENT       # misaligned
    assert _swa(o=P16) == g.GDN2_ERR_INVALID_ARGUMENT               # o aliases q
    assert _swa(window=0) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _swa(scale=0.0) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _swa(scale=float("nan")) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _swa(D=96) == g.GDN2_ERR_UNSUPPORTED
    assert _swa(N=2) == g.GDN2_ERR_INVALID_ARGUMENT                 # dense needs N == B
    assert _swa(cu_seqlens=P16, N=2, B=2) == g.GDN2_ERR_INVALID_ARGUMENT
    need = g.gdn2_swa_fwd_workspace_bytes(3, 1)
    assert need >= 16 and g.gdn2_swa_fwd_workspace_bytes(3, 0) == 0
    assert _swa(cu_seqlens=P16, N=3) == g.GDN2_ERR_WORKSPACE        # packed needs a workspace
    assert _swa(cu_seqlens=P16, N=3, workspace=P16 + 16, workspace_bytes=need) == g.GDN2_ERR_WORKSPACE
    assert _swa(T=0) == g.GDN2_OK and _swa(H=0) == g.GDN2_OK and _swa(N=0, B=0) == g.GDN2_OK


def _swa_layer(**kw):
    args = dict(x=P16, W_qkv=P16 + 4096, W_o=P16 + 8192, y=P16 + 12288, lse=None, cu_seqlens=None,
                N=1, B=1, T=64, H=1, D=128, Dm=256, window=16, scale=0.088, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(kw)
    return g.gdn2_swa_layer_fwd(**args)


def test_swa_layer_fwd_validation():
    assert _swa_layer(x=None) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _swa_layer(y=P16) == g.GDN2_ERR_INVALID_ARGUMENT          # y aliases x
    assert _swa_layer(Dm=100) == g.GDN2_ERR_UNSUPPORTED
    assert _swa_layer(D=96) == g.GDN2_ERR_UNSUPPORTED
    assert _swa_layer(window=0) == g.GDN2_ERR_INVALID_ARGUMENT
    assert _swa_layer() == g.GDN2_ERR_WORKSPACE
    need = g.gdn2_swa_layer_fwd_workspace_bytes(1, 1, 64, 1, 128, 256, 0)
    assert need > 0 and g.gdn2_swa_layer_fwd_workspace_bytes(1, 1, 64, 1, 128, 100, 0) == 0
    assert _swa_layer(workspace=P16, workspace_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
    assert _swa_layer(T=0) == g.GDN2_OK and _swa_layer(H=0) == g.GDN2_OK


# ---------------------------------------------------------------------------
# The binding's own checks: every tensor's shape, dtype and device is compared
# with the sizes taken from q (or x) before an address reaches the library.
# Metadata is checked before the device, so CPU tensors exercise these paths.
# ---------------------------------------------------------------------------

def _chunk_tensors(B=2, T=8, H=3, D=64, dtype="bfloat16"):
    import torch
    dt = getattr(torch, dtype)
    tk = torch.zeros(B, T, H, D, dtype=dt)
    f = torch.zeros(B, T, H, D, dtype=torch.float32)
    return dict(q=tk, k=tk.clone(), v=tk.clone(), log_alpha=f, b=f.clone(), w=f.clone())


@pytest.mark.parametrize("name,shape", [("k", (2, 8, 3, 32)), ("v", (2, 8, 2, 64)),
                                        ("log_alpha", (2, 8, 3, 1)), ("b", (2, 7, 3, 64)),
                                        ("w", (1, 8, 3, 64))])
def test_binding_chunk_fwd_rejects_wrong_shapes(name, shape):
    import torch
    x = _chunk_tensors()
    x[name] = torch.zeros(shape, dtype=x[name].dtype)
    with pytest.raises(ValueError, match=name):
        g.chunk_fwd(**x)


def test_binding_chunk_fwd_rejects_wrong_outputs_and_states():
    import torch
    x = _chunk_tensors()
    with pytest.raises(ValueError, match="S0"):
        g.chunk_fwd(**x, S0=torch.zeros(2, 3, 64, 32))
    with pytest.raises(TypeError, match="S0"):
        g.chunk_fwd(**x, S0=torch.zeros(2, 3, 64, 64, dtype=torch.float64))
    with pytest.raises(TypeError, match="o"):
        g.chunk_fwd(**x, o=torch.zeros(2, 8, 3, 64, dtype=torch.float32))     # fp32 o, bf16 q
    with pytest.raises(ValueError, match="S_final"):
        g.chunk_fwd(**x, S_final=torch.zeros(1, 3, 64, 64))
    with pytest.raises(TypeError, match="log_alpha"):
        g.chunk_fwd(**dict(x, log_alpha=x["log_alpha"].to(torch.bfloat16)))
    with pytest.raises(ValueError, match="device tensor"):   # right sizes, but host memory
        g.chunk_fwd(**x)


def test_binding_packed_calls_need_one_row():
    import torch
    x = _chunk_tensors()
    with pytest.raises(ValueError, match="B == 1"):
        g.chunk_fwd(**x, cu_seqlens=torch.tensor([0, 4, 8], dtype=torch.int32))


def test_binding_step_and_bwd_reject_wrong_shapes():
    import torch
    bf = torch.bfloat16
    q = torch.zeros(4, 2, 64, dtype=bf)
    f = torch.zeros(4, 2, 64)
    with pytest.raises(ValueError, match="S"):
        g.step(q, q, q, f, f, f, torch.zeros(4, 2, 64, 32))
    with pytest.raises(ValueError, match="b"):
        g.step(q, q, q, f, torch.zeros(4, 1, 64), f, torch.zeros(4, 2, 64, 64))
    with pytest.raises(TypeError, match="o"):
        g.step(q, q, q, f, f, f, torch.zeros(4, 2, 64, 64), o=torch.zeros(4, 2, 64))
    x = _chunk_tensors()
    with pytest.raises(ValueError, match="dout"):
        g.chunk_bwd(**x, dout=torch.zeros(2, 8, 3, 32, dtype=bf))
    with pytest.raises(ValueError, match="dS_final"):
        g.chunk_bwd(**x, dout=torch.zeros(2, 8, 3, 64, dtype=bf), dS_final=torch.zeros(3, 64, 64))
    with pytest.raises(TypeError, match="w_logit"):
        g.chunk_fwd_gate_logits(x["q"], x["k"], x["v"], x["q"], x["q"], x["w"])

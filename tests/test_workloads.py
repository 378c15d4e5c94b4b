"""Seeded input generators: determinism, shapes, distributions, bf16 rounding."""

import numpy as np
import pytest

import workloads as W


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact ties: low 16 bits == 0x8000
                        (rng.integers(0, 0x7F80, 1000).astype(np.uint32) << 16 | 0x8000)
                        .astype(np.uint32).view(np.float32),
                        np.array([0.0, -0.0, 1e-40, -3e38, np.inf, -np.inf], np.float32)])
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_workload_shapes_and_determinism():
    a = W.make_chunk_inputs(W.TINY_F32)
    b = W.make_chunk_inputs(W.TINY_F32)
    for key in ("q", "k", "v", "log_alpha", "b", "w"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].shape == (1, 256, 2, 64) and a["v"].shape == (1, 256, 2, 64)
    assert a["S0"] is None and a["cu_seqlens"] is None
    np.testing.assert_allclose(np.linalg.norm(a["k"].astype(np.float64), axis=-1), 1.0, atol=1e-6)
    assert a["log_alpha"].min() >= -0.2 and a["log_alpha"].max() <= -0.001
    assert 0.0 < a["b"].min() and a["b"].max() < 1.0


def test_bf16_workload_values_are_bf16_exact():
    a = W.make_chunk_inputs(W.SEQ_4K, T=128, H=2)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(W.bf16_round(a[key]), a[key])
    assert a["log_alpha"].dtype == np.float32


def test_varlen_workload_lengths():
    lens = W.varlen_lengths(W.VARLEN)
    assert len(lens) == 32 and lens.min() >= 512 and lens.max() <= 8192
    small = W.make_chunk_inputs(W.VARLEN, lengths=[3, 70, 64, 1], H=2)
    np.testing.assert_array_equal(small["cu_seqlens"], [0, 3, 73, 137, 138])
    assert small["q"].shape == (1, 138, 2, 128) and small["N"] == 4


def test_batch_workload_has_initial_state():
    a = W.make_chunk_inputs(W.BATCH_4K, T=64, B=2, H=2)
    assert a["S0"].shape == (2, 2, 128, 128)
    assert 0.015 < a["S0"].std() < 0.025


def test_decode_steps_are_independent_streams():
    s3a = W.make_decode_step(W.DECODE, 3, B=4, H=2)
    s3b = W.make_decode_step(W.DECODE, 3, B=4, H=2)
    s4 = W.make_decode_step(W.DECODE, 4, B=4, H=2)
    np.testing.assert_array_equal(s3a["q"], s3b["q"])
    assert not np.array_equal(s3a["q"], s4["q"])
    S = W.make_decode_state(W.DECODE, B=4, H=2)
    assert S.shape == (4, 2, 128, 128) and S.dtype == np.float32

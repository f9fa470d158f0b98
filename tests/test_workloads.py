"""Seeded input generators: shapes, value ranges, determinism (CPU only)."""
import numpy as np
import torch

from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled


def test_prefill_shapes_and_ranges():
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=96, heads=3)
    x = generate(w, seed=3)
    T = 2 * 96
    assert x["q"].shape == (T, 3, 128) and x["q"].dtype == torch.bfloat16
    assert x["v"].shape == (T, 3, 128)
    assert x["log_a"].shape == (T, 3, 128) and x["log_a"].dtype == torch.float32
    assert float(x["log_a"].max()) <= 0.0 and float(x["log_a"].min()) >= -8.0
    assert x["beta"].shape == (T, 3) and 0 < float(x["beta"].min()) and float(x["beta"].max()) < 1
    nrm = torch.linalg.vector_norm(x["k"].float(), dim=-1)
    assert torch.allclose(nrm, torch.ones_like(nrm), atol=1e-2)
    assert x["S0"].shape == (2, 3, 128, 128)
    assert abs(float(x["S0"].std()) - 0.02) < 2e-3
    assert x["cu_seqlens"].tolist() == [0, 96, 192]


def test_scalar_decay_and_no_state():
    w = scaled(WORKLOADS["gdn_h16_t4096_d128_bf16"], seqlen=64, heads=2)
    x = generate(w, seed=1)
    assert x["log_a"].shape == (64, 2)
    assert x["S0"] is None


def test_varlen_lengths_seeded():
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=5, len_range=(3, 40), heads=1, dk=32, dv=32)
    a = generate(w, seed=7)
    b = generate(w, seed=7)
    assert np.array_equal(a["lengths"], b["lengths"])
    assert all(3 <= n <= 40 for n in a["lengths"])
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["log_a"], b["log_a"])
    c = generate(w, seed=8)
    assert not torch.equal(a["q"][:3], c["q"][:3])


def test_decode_shapes():
    w = scaled(WORKLOADS["kda_decode_b256_h32_d128"], n_seqs=4, heads=2, steps=3)
    x = generate(w, seed=0)
    assert x["q"].shape == (3, 4, 2, 128)
    assert x["log_a"].shape == (3, 4, 2, 128)
    assert x["beta"].shape == (3, 4, 2)
    assert x["S"].shape == (4, 2, 128, 128) and x["S"].dtype == torch.float32
